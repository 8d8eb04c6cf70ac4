// Internal declarations shared by the HIP translation units of libmsda.
// Not part of the public ABI (include/msda.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "msda.h"

namespace msda {

// Per-level sizes, passed to kernels by value (kernel arguments are
// wave-uniform and land in scalar registers).
struct Levels {
    int32_t H[MSDA_MAX_LEVELS];
    int32_t W[MSDA_MAX_LEVELS];
    int32_t start[MSDA_MAX_LEVELS];
};

// A validated call geometry. Every tensor of the call has fewer than 2^31
// elements and one batch of value fewer than 2^31 bytes, so 32-bit offsets
// suffice inside a batch.
struct Geometry {
    int32_t B, M, D, L, K;
    int32_t S, Nq;
    Levels lv;
    __host__ __device__ int64_t samples() const { return (int64_t)B * Nq * M * L * K; }
    __host__ __device__ int64_t queries() const { return (int64_t)B * Nq; }
    __host__ __device__ int32_t channels() const { return M * D; }
};

// Pixel tiling of grad_value for the scatter-free backward (per level: tile
// height/width, tiles per row of tiles, first tile index), tiles per
// (batch, head), and the query ranges of the binning workgroups.
struct TilePlan {
    int32_t th[MSDA_MAX_LEVELS];
    int32_t tw[MSDA_MAX_LEVELS];
    int32_t ntw[MSDA_MAX_LEVELS];
    int32_t tbase[MSDA_MAX_LEVELS];
    int32_t nchunk[MSDA_MAX_LEVELS];  // workgroups sharing one tile's records
    int32_t ibase[MSDA_MAX_LEVELS];   // first work item of the level within (batch, head)
    int32_t ipb;  // work items (tile, chunk) per (batch, head)
    int32_t tpb;  // tiles per (batch, head)
    int32_t qpw;  // queries per workgroup
    int32_t wpb;  // workgroups per batch
    // per-head path (one workgroup per batch, head and range of queries)
    int32_t hqr;   // query ranges per (batch, head)
    int32_t hqpr;  // queries per range
    // record slots per (batch, query, head): a sample of a sparse level has a
    // record in each tile its in-map corners touch, at most four
    int32_t rslots;
    // Dense levels (bit l of dense_mask; adjacent levels) have no tiles and no
    // records: their grad_value is accumulated from the samples directly, per
    // (pixel part, query split) work item. Their pixels are numbered one level
    // after the other: level l's from dbase[l], ndpix in all.
    int32_t dense_mask;
    int32_t ndl;     // dense levels
    int32_t ndpix;   // their pixels (per batch and head)
    int32_t dbase[MSDA_MAX_LEVELS];
    int32_t dparts;  // pixel parts of the dense numbering
    int32_t dsplits; // query splits
    int32_t dipb;    // dense items per (batch, head): dparts * dsplits (0 without dense levels)
    // the query splits' sums (dsplits > 1): per (batch, head) ppb = dsplits *
    // ndpix rows of D channels, split s's from s * ndpix
    int32_t ppb;
    // 1/tw and 1/th as floats: floor((c + 0.5) * (1/t)) is c / t exactly for
    // 0 <= c < 2^20 and t <= 128 (checked exhaustively), without a division
    float tinv_w[MSDA_MAX_LEVELS];
    float tinv_h[MSDA_MAX_LEVELS];
};

// Whether level l's grad_value rows are summed with float atomics (they must
// then be zeroed first unless the call accumulates): the split tiles of the
// direct mode. Dense levels sum their query splits in a second pass.
__host__ __device__ inline bool level_uses_atomics(const TilePlan &tp, int l)
{
    return !((tp.dense_mask >> l) & 1) && tp.nchunk[l] > 1;
}

// Whether the backward takes the tiled fast path for this call (it then needs
// backward_workspace_bytes(g) bytes of workspace), and that size (0 when the
// shape has no fast path).
bool make_tile_plan(const Geometry &g, TilePlan &tp);
bool backward_uses_workspace(const Geometry &g, const void *value, msda_dtype vt, const float *go,
                             const float *gv);
size_t backward_workspace_bytes(const Geometry &g);
// The per-level path masks of the tiled fast path (false: generic path).
bool backward_plan_masks(const Geometry &g, uint32_t &dense, uint32_t &direct, uint32_t &split);

// Brackets the launches made during its lifetime with a timing event pair on
// `st` while msda_timing_enable is on (and `st` is not being captured).
// `name` must be a string literal.
class KernelScope {
  public:
    KernelScope(const char *name, hipStream_t st);
    ~KernelScope();
    KernelScope(const KernelScope &) = delete;
    KernelScope &operator=(const KernelScope &) = delete;

  private:
    const char *name_;
    hipStream_t st_;
    hipEvent_t start_;
};

// Inputs and side outputs of the fused forward: reference points [B,Nq,L,2]
// (or 4-d boxes [B,Nq,L,4]), offsets [B,Nq,M,L,K,2] and logits [B,Nq,M,L*K]
// in; the sampling locations and attention weights it forms out (for the
// backward).
struct FusedInputs {
    const float *ref;
    int ref_dims;  // 2: offsets in pixels of level l; 4: relative to the box size
    const float2 *off;
    const float *logits;
    float2 *loc_out;
    float *attn_out;
    const uint8_t *mask;  // key padding mask [B,S] (nonzero = padded, reads zero), or null
};

// One sample's location from its reference and offset.
__host__ __device__ inline float2 fused_location(const float *ref, int ref_dims, int64_t ref_row, float2 o,
                                                 float Wf, float Hf, float Kf)
{
    if (ref_dims == 4) {
        const float4 r = reinterpret_cast<const float4 *>(ref)[ref_row];
        return make_float2(r.x + o.x / Kf * r.z * 0.5f, r.y + o.y / Kf * r.w * 0.5f);
    }
    const float2 r = reinterpret_cast<const float2 *>(ref)[ref_row];
    return make_float2(r.x + o.x / Wf, r.y + o.y / Hf);
}

// What the fused backward needs besides the plain one: the references and
// offsets (4-d boxes only) and the optional reference gradient [B,Nq,L,dims].
struct FusedGrads {
    const float *ref;
    const float2 *off;
    int ref_dims;
    float *grad_ref;
    const uint8_t *mask;  // key padding mask [B,S] of the fused forward, or null
};

// The fused kernels form the L*K softmax across adjacent lanes of a wave.
inline bool fused_forward_supported(const Geometry &g)
{
    const int lk = g.L * g.K;
    return lk <= 64 && (64 % lk) == 0;
}

// Largest workspace msda_backward_noalloc serves from its device array.
constexpr size_t kNoAllocScratchBytes = (size_t)MSDA_NOALLOC_SCRATCH_BYTES;

// The calling device's address of that array (resolved with
// hipGetSymbolAddress on the first call per device, then cached).
hipError_t noalloc_scratch(void **out);

// Whether launches on `st` from this thread are being timed now (timing
// enabled, not suppressed, `st` not capturing).
bool timing_on(hipStream_t st);

// While an object of this type lives, the calling thread's launches record no
// timing events (the allocation-free entry point creates no events).
class TimingOff {
  public:
    TimingOff();
    ~TimingOff();
    TimingOff(const TimingOff &) = delete;
    TimingOff &operator=(const TimingOff &) = delete;
};

// Launchers (each returns a hipError_t from the launch).
hipError_t launch_reference_points(const Geometry &g, const float *valid_ratios,
                                   const float *query_ref, float *ref_out, hipStream_t st);
hipError_t launch_sampling_locations(const Geometry &g, const float *ref, const float *off,
                                     float *loc, hipStream_t st);
hipError_t launch_softmax(const Geometry &g, const float *logits, float *w, hipStream_t st);
// The three above in one launch where the shapes allow (else in turn).
hipError_t launch_prologue(const Geometry &g, const float *valid_ratios, const float *query_ref,
                           const float *offset_px, const float *logits, float *ref, float *loc, float *w,
                           hipStream_t st);
hipError_t launch_forward(const Geometry &g, const void *value, msda_dtype vt, const float *loc,
                          const float *attn, float *out, hipStream_t st);
hipError_t launch_forward_fused(const Geometry &g, const void *value, msda_dtype vt, const FusedInputs &fi,
                                float *out, hipStream_t st);
hipError_t launch_zero_fill(float *p, int64_t n, hipStream_t st);
// grad_value is fully overwritten unless `accumulate`. `workspace` must hold
// backward_workspace_bytes(g) bytes when backward_uses_workspace(...) holds.
// `side_ok`: the dense levels may run on the library's side stream (else
// everything runs on `st`, and no stream or event is created).
hipError_t launch_backward(const Geometry &g, const void *value, msda_dtype vt, const float *loc,
                           const float *attn, const float *grad_out, float *grad_value,
                           float *grad_loc, float *grad_attn, void *workspace, bool accumulate,
                           bool side_ok, hipStream_t st);
// The same, carried back to the fused forward's inputs: grad_offsets,
// grad_logits and (if fg.grad_ref is not null) grad_ref instead of grad_loc
// and grad_attn.
hipError_t launch_backward_fused(const Geometry &g, const void *value, msda_dtype vt, const float *loc,
                                 const float *attn, const float *grad_out, float *grad_value,
                                 float *grad_offsets, float *grad_logits, const FusedGrads &fg, void *workspace,
                                 bool accumulate, bool side_ok, hipStream_t st);
hipError_t launch_sampling_locations_box(const Geometry &g, const float *ref, const float *off, float *loc,
                                         hipStream_t st);

}  // namespace msda
