/*
 * msda.h — C ABI of the multi-scale deformable attention (MSDeformAttn) core
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation ("Deformable DETR: Deformable Transformers for End-to-End
 * Object Detection" paper notes, phdsky.com, "Core insights / Insight 2",
 * the MSDeformAttn equation; tensor semantics from the xdnf.cn "Deformable DETR
 * model walkthrough", "encoder" section):
 *
 *   out[b,q,m*D+d] = sum_{l<L} sum_{k<K} A[b,q,m,l,k] *
 *                    bilinear(value[b, level l, :, :, m, d], loc[b,q,m,l,k,:])
 *
 * with bilinear sampling in the align_corners=False pixel convention (a
 * normalised coordinate u maps to the pixel coordinate u*W_l - 0.5), zero
 * padding outside the map, and A normalised over the L*K samples of one query
 * and head.
 *
 * Conventions shared by every entry point:
 *  - Tensors are dense, row-major, batch-first, and live in DEVICE memory,
 *    except spatial_shapes and level_start_index, which are HOST arrays
 *    (the launch configuration needs them; reading device copies would force a
 *    device-to-host sync).
 *  - value is [B, S, M, D] with S = sum_l H_l*W_l; level l occupies rows
 *    level_start_index[l] .. +H_l*W_l, row-major (y, x) inside a level.
 *  - Locations are (x, y): x along the width. spatial_shapes is (H, W).
 *  - The caller (PyTorch) allocates and owns all memory; the library allocates
 *    no device memory and keeps no data between calls. All entry points are
 *    reentrant. The one resource it keeps: msda_backward creates, on first
 *    use per device and host thread, one more HIP stream (default priority)
 *    and two events, kept for the life of the process; see msda_backward.
 *  - Every call validates its arguments on the host BEFORE any device work, so
 *    an error never leaves partial output. On success the work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream) and the call returns
 *    without synchronising; faults surface at the caller's next sync.
 *  - Non-finite or far-outside sampling locations contribute zero and receive
 *    zero gradients.
 *  - batch == 0 or num_query == 0 is an empty call: it succeeds and touches
 *    no tensor (NULL is accepted for the empty ones), except that
 *    msda_backward with num_query == 0 and batch > 0 still zero-fills
 *    grad_value (no contributions).
 *  - Return value: MSDA_OK (0) or a negative msda_status; msda_last_error()
 *    gives a human-readable detail for the calling thread's last failure.
 */
#ifndef MSDA_H
#define MSDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MSDA_API __attribute__((visibility("default")))
#else
#define MSDA_API
#endif

#define MSDA_ABI_VERSION 11
#define MSDA_MAX_LEVELS 16

typedef enum {
    MSDA_OK = 0,
    MSDA_E_NULL = -1,        /* a required pointer is NULL                                */
    MSDA_E_DIM = -2,         /* a size is negative, zero where it must not be, or too
                                large for 32-bit indexing                                 */
    MSDA_E_SHAPE = -3,       /* sum_l H_l*W_l != num_value, or encoder refs with Nq != S  */
    MSDA_E_LEVEL_INDEX = -4, /* level_start_index is not the exclusive prefix sum         */
    MSDA_E_UNSUPPORTED = -5, /* dtype, level count or flags outside what is compiled      */
    MSDA_E_ALIGN = -6,       /* a device pointer is not aligned to its element size       */
    MSDA_E_HIP = -7,         /* the HIP runtime reported an error at launch               */
    MSDA_E_WORKSPACE = -8    /* msda_backward's workspace is NULL or smaller than needed  */
} msda_status;

typedef enum {
    MSDA_F32 = 0,  /* IEEE binary32                                       */
    MSDA_BF16 = 1  /* bfloat16 (value only; arithmetic is still fp32)     */
} msda_dtype;

/* Sizes of one call. */
typedef struct {
    int32_t batch;                      /* B                                           */
    int32_t heads;                      /* M                                           */
    int32_t channels;                   /* D, channels per head                        */
    int32_t levels;                     /* L, 1..MSDA_MAX_LEVELS                       */
    int32_t points;                     /* K, sampling points per head and level       */
    int64_t num_value;                  /* S = sum_l H_l*W_l                           */
    int64_t num_query;                  /* Nq                                          */
    const int64_t *spatial_shapes;      /* HOST [L][2] = (H_l, W_l)                    */
    const int64_t *level_start_index;   /* HOST [L], exclusive prefix sum of H_l*W_l   */
} msda_shape;

/* Flag for msda_backward: add into grad_value instead of overwriting it. */
#define MSDA_BWD_ACCUMULATE 1u

/* Host helper: level_start_index as the exclusive prefix sum of H_l*W_l
 * (walkthrough page, "transformer" section: the start of each level in the
 * flattened sequence). Writes lsi_out[L] and *num_value_out = S. No device
 * work. */
MSDA_API int msda_level_start_index(int32_t levels, const int64_t *spatial_shapes,
                           int64_t *lsi_out, int64_t *num_value_out);

/* Reference points, [B, Nq, L, 2] fp32 (x, y).
 *  Encoder mode (query_ref == NULL; requires num_query == num_value): query q
 *  is pixel (i, j) of level lq, q = level_start_index[lq] + i*W_lq + j, and
 *    ref[b,q,l] = ((j+0.5)/(vr[b,lq,x]*W_lq) * vr[b,l,x],
 *                  (i+0.5)/(vr[b,lq,y]*H_lq) * vr[b,l,y])
 *  (juhe.plus debug-build notes, "Key point 1: get_reference_points"; the
 *  walkthrough page's "encoder" section).
 *  Decoder mode (query_ref = u [B, Nq, 2]): ref[b,q,l] = u[b,q] * vr[b,l]
 *  (the notes' "decoder data flow"; the walkthrough page's "Decoder").
 *  valid_ratios: [B, L, 2] fp32, (x = width ratio, y = height ratio), or NULL
 *  for all ones (no padding masks). ref_out is fully overwritten. */
MSDA_API int msda_reference_points(const msda_shape *shape, const float *valid_ratios,
                          const float *query_ref, float *ref_out, void *stream);

/* Sampling locations from 2-d reference points (walkthrough page, "encoder";
 * paper notes, "Key code"): offsets are in pixels of level l and are
 * normalised by (W_l, H_l):
 *   loc[b,q,m,l,k,:] = ref[b,q,l,:] + offset_px[b,q,m,l,k,:] / (W_l, H_l)
 * ref [B,Nq,L,2], offset_px and loc_out [B,Nq,M,L,K,2], all fp32. */
MSDA_API int msda_sampling_locations(const msda_shape *shape, const float *ref,
                            const float *offset_px, float *loc_out, void *stream);

/* Attention weights: softmax of logits [B,Nq,M,L*K] over the L*K samples of
 * each (b, q, m), so that they sum to 1 over all levels and points (paper
 * notes, "Insight 2"). weights_out [B,Nq,M,L,K] fp32; may alias logits. */
MSDA_API int msda_attention_softmax(const msda_shape *shape, const float *logits,
                           float *weights_out, void *stream);

/* The three calls above in one: reference points (as msda_reference_points,
 * into ref_out [B,Nq,L,2]), the sampling locations from them (as
 * msda_sampling_locations, offset_px -> loc_out [B,Nq,M,L,K,2]) and the
 * softmax of logits [B,Nq,M,L*K] (as msda_attention_softmax, into
 * weights_out [B,Nq,M,L,K]); all fp32, with the same arguments and rules
 * as those three, and bit for bit the same results. For K in {2, 4, 8},
 * L*K in {4, 8, 16, 32} and 16-byte aligned offset_px, loc_out, logits and
 * weights_out it is a single kernel launch (each location thread forms its
 * reference point itself instead of reading ref_out back); otherwise the
 * three kernels run in turn on `stream`. weights_out may alias logits; no
 * other output may alias an input. */
MSDA_API int msda_prologue(const msda_shape *shape, const float *valid_ratios, const float *query_ref,
                           const float *offset_px, const float *logits, float *ref_out, float *loc_out,
                           float *weights_out, void *stream);

/* Forward of the core (the bracketed sum of the MSDeformAttn equation).
 *  value              [B,S,M,D]        fp32 or bf16 (value_dtype), 4-byte
 *                                      (fp32) / 2-byte (bf16) aligned
 *  sampling_locations [B,Nq,M,L,K,2]   fp32, normalised (x, y)
 *  attention_weights  [B,Nq,M,L,K]     fp32
 *  output             [B,Nq,M*D]       fp32, fully overwritten (m-major)
 * Accumulation is fp32 for both value dtypes. */
MSDA_API int msda_forward(const msda_shape *shape, const void *value, msda_dtype value_dtype,
                 const float *sampling_locations, const float *attention_weights,
                 float *output, void *stream);

/* Bytes of device workspace msda_backward needs for these sizes (0 when the
 * sizes have no tiled fast path; the call then needs none). Host only. */
MSDA_API int msda_backward_workspace_size(const msda_shape *shape, size_t *bytes);

/* How msda_backward's tiled fast path would treat each level of these sizes
 * (host only; for diagnostics and tests). Bit l of *dense_levels: level l is
 * summed from its samples directly (at least 24 samples per pixel, per batch
 * and head, and at most 2048 pixels). Bit l of *direct_levels: its tiles are
 * so small (at most 4 pixels) that they skip the per-cell sort. Bit l of
 * *split_levels: those small tiles share their records among several
 * workgroups, whose partial sums meet in float atomics. All three are 0 when
 * the sizes take the generic path (msda_backward_workspace_size reports 0).
 * Any output pointer may be NULL. */
MSDA_API int msda_backward_plan(const msda_shape *shape, uint32_t *dense_levels, uint32_t *direct_levels,
                                uint32_t *split_levels);

/* Backward of the core: the exact derivative of msda_forward given
 * grad_output [B,Nq,M*D] fp32 (the op is trained end to end through autograd:
 * walkthrough page, "encoder"; paper notes, "Key code").
 *  grad_value              [B,S,M,D]      fp32 (also for bf16 value); fully
 *                                         overwritten, or added into when flags
 *                                         has MSDA_BWD_ACCUMULATE
 *  grad_sampling_locations [B,Nq,M,L,K,2] fp32, fully overwritten
 *  grad_attention_weights  [B,Nq,M,L,K]   fp32, fully overwritten
 *  workspace               device scratch of at least
 *                          msda_backward_workspace_size() bytes, 256-byte
 *                          aligned, owned by the caller; its contents on entry
 *                          do not matter and are clobbered. Calls that overlap
 *                          in time must use different workspaces.
 * At an integer pixel coordinate the location gradient is the right
 * derivative (the cell [floor(x), floor(x)+1] is used).
 * On the tiled fast path (value and gradient rows 16-byte aligned,
 * M*D == 256 and compiled (L, K)) grad_value is gathered per pixel tile; only
 * the tiles of the densest levels, whose sample lists are split over several
 * workgroups, merge their partial sums with float atomics. Other sizes scatter
 * with float atomics. The fast path also orders each pixel's contributions
 * by integer LDS atomics racing between waves. So the summation order, and
 * with it the last bits of grad_value, can vary from run to run;
 * grad_sampling_locations and grad_attention_weights are reproducible.
 * On the fast path the dense levels' accumulation runs on the library's own
 * stream, forked from `stream` by an event and joined back into it by another
 * before the kernels that need it, so the call stays ordered on `stream`
 * (later work on `stream` sees all of its results) and can be captured into a
 * HIP graph from `stream`. */
MSDA_API int msda_backward(const msda_shape *shape, const void *value, msda_dtype value_dtype,
                  const float *sampling_locations, const float *attention_weights,
                  const float *grad_output, float *grad_value,
                  float *grad_sampling_locations, float *grad_attention_weights,
                  void *workspace, size_t workspace_bytes, unsigned flags, void *stream);

/* Bytes of device scratch that msda_backward_noalloc holds (per GPU). */
#define MSDA_NOALLOC_SCRATCH_BYTES (160u * 1024u * 1024u)

/* msda_backward for callers that cannot allocate device memory during the
 * call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments, results and status codes as
 * msda_backward, without the workspace. Its scratch is a device array inside
 * the library, MSDA_NOALLOC_SCRATCH_BYTES (160 MiB) per GPU, which each GPU
 * the library runs on holds until the process ends; its address is resolved
 * on the first call per device. Sizes whose workspace
 * (msda_backward_workspace_size) exceeds it return MSDA_E_WORKSPACE before
 * any device work. The call allocates nothing, creates no stream or event
 * (the dense levels run on `stream` too, and the timing aid records nothing
 * for it) and leaves no state in the scratch that a later call relies on.
 * All calls on one GPU share that GPU's scratch: calls that may overlap in
 * time on one GPU (other streams, other host threads) race and must not be
 * made. */
MSDA_API int msda_backward_noalloc(const msda_shape *shape, const void *value, msda_dtype value_dtype,
                                   const float *sampling_locations, const float *attention_weights,
                                   const float *grad_output, float *grad_value, float *grad_sampling_locations,
                                   float *grad_attention_weights, unsigned flags, void *stream);

/* Fused forward (the adjacent steps formed inside the core): for every sample
 *   loc = reference_points[b,q,l] + sampling_offsets[b,q,m,l,k] / (W_l, H_l)
 *         (reference_dims 2: points, offsets in pixels of level l), or
 *   loc = ref[b,q,l,0:2] + sampling_offsets / K * ref[b,q,l,2:4] * 0.5
 *         (reference_dims 4: boxes (cx, cy, w, h), the iterative-refinement
 *          branch of the module source)
 *   A[b,q,m,:] = softmax over the L*K logits attention_logits[b,q,m,:]
 * and then output as msda_forward (walkthrough page, "encoder" and the
 * MSDeformAttn module source; paper notes, "Insight 2" and "Key code").
 *  reference_points        [B,Nq,L,reference_dims] fp32, normalised
 *  sampling_offsets        [B,Nq,M,L,K,2] fp32 (x, y)
 *  attention_logits        [B,Nq,M,L*K]   fp32
 *  key_padding_mask        [B,S] bytes, nonzero = padded position, or NULL:
 *                          the value rows of padded positions read as zero
 *                          (the module fills the projected value with zeros
 *                          there before the core: paper notes, "Key code",
 *                          MSDeformAttn.forward; walkthrough page, "encoder")
 *  output                  [B,Nq,M*D]     fp32, fully overwritten
 *  sampling_locations_out  [B,Nq,M,L,K,2] fp32, fully overwritten (for the
 *  attention_weights_out   [B,Nq,M,L,K]   fp32   backward; never NULL)
 * Shapes whose L*K does not divide 64 run the three steps one after the other
 * through the two side outputs. reference_dims other than 2 or 4:
 * MSDA_E_UNSUPPORTED; otherwise the status codes of msda_forward. */
MSDA_API int msda_forward_fused(const msda_shape *shape, const void *value, msda_dtype value_dtype,
                                const float *reference_points, int reference_dims, const float *sampling_offsets,
                                const float *attention_logits, const uint8_t *key_padding_mask, float *output,
                                float *sampling_locations_out, float *attention_weights_out, void *stream);

/* Backward of msda_forward_fused, given the locations and weights it wrote:
 * grad_value as msda_backward, and, by the chain rule through the two fused
 * steps,
 *   grad_sampling_offsets = grad_loc / (W_l, H_l)            (points)
 *                         = grad_loc * ref_wh * 0.5 / K       (boxes)
 *   grad_attention_logits[b,q,m,i] = A_i * (grad_A_i - sum_j A_j grad_A_j)
 *   grad_reference_points[b,q,l]   = sum over m, k of grad_loc, and for boxes
 *                                    sum of grad_loc * offset * 0.5 / K for
 *                                    (w, h)  (if not NULL)
 * reference_points and sampling_offsets are read for boxes only (NULL allowed
 * for points). Shapes [B,Nq,M,L,K,2], [B,Nq,M,L*K], [B,Nq,L,reference_dims],
 * fp32, fully overwritten. key_padding_mask: the forward's [B,S] mask or
 * NULL; padded value rows read as zero and get zero grad_value (with
 * MSDA_BWD_ACCUMULATE they are left as they were). Workspace, flags, stream
 * use and status codes as msda_backward. */
MSDA_API int msda_backward_fused(const msda_shape *shape, const void *value, msda_dtype value_dtype,
                                 const float *sampling_locations, const float *attention_weights,
                                 const float *reference_points, const float *sampling_offsets, int reference_dims,
                                 const uint8_t *key_padding_mask, const float *grad_output, float *grad_value,
                                 float *grad_sampling_offsets, float *grad_attention_logits,
                                 float *grad_reference_points, void *workspace, size_t workspace_bytes,
                                 unsigned flags, void *stream);

/* Static English name of a status code. */
MSDA_API const char *msda_status_string(int status);

/* Detail text for the calling thread's most recent failed call ("" if none). */
MSDA_API const char *msda_last_error(void);

/* MSDA_ABI_VERSION of the built library. */
MSDA_API int msda_abi_version(void);

/* Per-kernel timing, a profiling aid for the caller's benchmark (not part of
 * the op). While enabled (on != 0), every kernel this library launches on a
 * stream that is not being captured into a graph is bracketed by two HIP
 * events recorded on that stream; the elapsed time between them is added to
 * the kernel's entry. While it is on, the backward runs all of its kernels on
 * the caller's stream (the dense levels too, which otherwise run on a second
 * stream beside the others), so that each pair times its kernel alone.
 * Enabling adds a little launch overhead; it is off by default. Host only,
 * thread safe. Returns MSDA_OK. */
MSDA_API int msda_timing_enable(int on);

/* Drops all timing entries and unread event pairs (waits for the latter). */
MSDA_API int msda_timing_reset(void);

/* Waits for the recorded event pairs and folds them into the entries, then
 * reports entry `index` (0 .. count-1, in order of first launch): *name is a
 * static string, the kernel's name as the compiler and profilers show it
 * (without template arguments), valid for the life of the process;
 * *total_ms the summed elapsed time and *launches the number of launches.
 * Any output pointer may be NULL. *count, if given, receives the number of
 * entries; index -1 reports only that. Another index out of range:
 * MSDA_E_DIM (with *count still set). A HIP error while waiting: MSDA_E_HIP. */
MSDA_API int msda_timing_read(int index, int *count, const char **name, double *total_ms,
                              int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_H */
