// Host side of the C ABI declared in include/msda.h: argument validation
// (always before any device work), geometry packing and kernel dispatch.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "msda_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok()
{
    g_last_error.clear();
    return MSDA_OK;
}

constexpr int64_t kMax32 = 0x7fffffffLL;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validate the sizes and host metadata of a call and pack them into a
// Geometry. Checks: non-NULL, positive sizes (batch and num_query may be 0:
// an empty call), at most MSDA_MAX_LEVELS levels,
// sum_l H_l*W_l == S (the mmcv module asserts the same), level_start_index
// equal to the exclusive prefix sum, every tensor below 2^31 elements and one
// batch of value (as fp32) below 2^31 bytes.
int make_geometry(const msda_shape *sh, msda::Geometry &g)
{
    if (!sh) return fail(MSDA_E_NULL, "shape is NULL");
    if (!sh->spatial_shapes) return fail(MSDA_E_NULL, "spatial_shapes is NULL");
    if (!sh->level_start_index) return fail(MSDA_E_NULL, "level_start_index is NULL");
    if (sh->batch < 0 || sh->heads <= 0 || sh->channels <= 0 || sh->levels <= 0 || sh->points <= 0 ||
        sh->num_value <= 0 || sh->num_query < 0)
        return fail(MSDA_E_DIM, "non-positive size (B=%d M=%d D=%d L=%d K=%d S=%lld Nq=%lld)", sh->batch,
                    sh->heads, sh->channels, sh->levels, sh->points, (long long)sh->num_value,
                    (long long)sh->num_query);
    if (sh->levels > MSDA_MAX_LEVELS)
        return fail(MSDA_E_UNSUPPORTED, "levels=%d exceeds MSDA_MAX_LEVELS=%d", sh->levels, MSDA_MAX_LEVELS);
    int64_t start = 0;
    for (int l = 0; l < sh->levels; ++l) {
        const int64_t H = sh->spatial_shapes[2 * l], W = sh->spatial_shapes[2 * l + 1];
        if (H <= 0 || W <= 0 || H > kMax32 || W > kMax32)
            return fail(MSDA_E_DIM, "level %d has shape (%lld, %lld)", l, (long long)H, (long long)W);
        if (sh->level_start_index[l] != start)
            return fail(MSDA_E_LEVEL_INDEX, "level_start_index[%d]=%lld, expected %lld", l,
                        (long long)sh->level_start_index[l], (long long)start);
        start += H * W;
        if (start > kMax32) return fail(MSDA_E_DIM, "sum of H*W exceeds 2^31-1");
    }
    if (start != sh->num_value)
        return fail(MSDA_E_SHAPE, "sum of H_l*W_l = %lld but num_value = %lld", (long long)start,
                    (long long)sh->num_value);
    const int64_t B = sh->batch, M = sh->heads, D = sh->channels, L = sh->levels, K = sh->points;
    const int64_t S = sh->num_value, Nq = sh->num_query;
    const int64_t C = M * D;
    if (C > kMax32 || S * C * 4 > kMax32)
        return fail(MSDA_E_DIM, "one batch of value is %lld elements; limit is 2^29", (long long)(S * C));
    if (B * S * C > kMax32 || B * Nq * C > kMax32 || B * Nq * M * L * K * 2 > kMax32 || Nq > kMax32 ||
        B * Nq * L * 2 > kMax32)
        return fail(MSDA_E_DIM, "a tensor of the call has 2^31 elements or more");
    g.B = sh->batch;
    g.M = sh->heads;
    g.D = sh->channels;
    g.L = sh->levels;
    g.K = sh->points;
    g.S = (int32_t)S;
    g.Nq = (int32_t)Nq;
    memset(&g.lv, 0, sizeof g.lv);
    for (int l = 0; l < sh->levels; ++l) {
        g.lv.H[l] = (int32_t)sh->spatial_shapes[2 * l];
        g.lv.W[l] = (int32_t)sh->spatial_shapes[2 * l + 1];
        g.lv.start[l] = (int32_t)sh->level_start_index[l];
    }
    return MSDA_OK;
}

int launched(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(MSDA_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int msda_abi_version(void) { return MSDA_ABI_VERSION; }

const char *msda_last_error(void) { return g_last_error.c_str(); }

const char *msda_status_string(int status)
{
    switch (status) {
    case MSDA_OK: return "ok";
    case MSDA_E_NULL: return "null pointer";
    case MSDA_E_DIM: return "bad dimension";
    case MSDA_E_SHAPE: return "shape mismatch";
    case MSDA_E_LEVEL_INDEX: return "level_start_index mismatch";
    case MSDA_E_UNSUPPORTED: return "unsupported";
    case MSDA_E_ALIGN: return "misaligned pointer";
    case MSDA_E_HIP: return "HIP runtime error";
    case MSDA_E_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
    }
}

int msda_level_start_index(int32_t levels, const int64_t *spatial_shapes, int64_t *lsi_out,
                           int64_t *num_value_out)
{
    if (!spatial_shapes || !lsi_out) return fail(MSDA_E_NULL, "NULL argument");
    if (levels <= 0 || levels > MSDA_MAX_LEVELS) return fail(MSDA_E_DIM, "levels=%d", levels);
    int64_t start = 0;
    for (int l = 0; l < levels; ++l) {
        const int64_t H = spatial_shapes[2 * l], W = spatial_shapes[2 * l + 1];
        if (H <= 0 || W <= 0) return fail(MSDA_E_DIM, "level %d has shape (%lld, %lld)", l, (long long)H, (long long)W);
        lsi_out[l] = start;
        start += H * W;
    }
    if (num_value_out) *num_value_out = start;
    return ok();
}

int msda_reference_points(const msda_shape *shape, const float *valid_ratios, const float *query_ref,
                          float *ref_out, void *stream)
{
    msda::Geometry g;
    if (int st = make_geometry(shape, g)) return st;
    if (g.B == 0 || g.Nq == 0) return ok();
    if (!ref_out) return fail(MSDA_E_NULL, "ref_out is NULL");
    if (!query_ref && g.Nq != g.S)
        return fail(MSDA_E_SHAPE, "encoder reference points need num_query == num_value (%d != %d)", g.Nq, g.S);
    if (!aligned(ref_out, 8) || (query_ref && !aligned(query_ref, 8)) || (valid_ratios && !aligned(valid_ratios, 4)))
        return fail(MSDA_E_ALIGN, "ref_out/query_ref need 8-byte, valid_ratios 4-byte alignment");
    return launched(msda::launch_reference_points(g, valid_ratios, query_ref, ref_out, (hipStream_t)stream),
                    "reference_points");
}

int msda_sampling_locations(const msda_shape *shape, const float *ref, const float *offset_px,
                            float *loc_out, void *stream)
{
    msda::Geometry g;
    if (int st = make_geometry(shape, g)) return st;
    if (g.B == 0 || g.Nq == 0) return ok();
    if (!ref || !offset_px || !loc_out) return fail(MSDA_E_NULL, "NULL tensor");
    if (!aligned(ref, 8) || !aligned(offset_px, 8) || !aligned(loc_out, 8))
        return fail(MSDA_E_ALIGN, "(x, y) tensors need 8-byte alignment");
    return launched(msda::launch_sampling_locations(g, ref, offset_px, loc_out, (hipStream_t)stream),
                    "sampling_locations");
}

int msda_attention_softmax(const msda_shape *shape, const float *logits, float *weights_out, void *stream)
{
    msda::Geometry g;
    if (int st = make_geometry(shape, g)) return st;
    if (g.B == 0 || g.Nq == 0) return ok();
    if (!logits || !weights_out) return fail(MSDA_E_NULL, "NULL tensor");
    if (!aligned(logits, 4) || !aligned(weights_out, 4)) return fail(MSDA_E_ALIGN, "fp32 tensors need 4-byte alignment");
    return launched(msda::launch_softmax(g, logits, weights_out, (hipStream_t)stream), "attention_softmax");
}

int msda_prologue(const msda_shape *shape, const float *valid_ratios, const float *query_ref,
                  const float *offset_px, const float *logits, float *ref_out, float *loc_out, float *weights_out,
                  void *stream)
{
    msda::Geometry g;
    if (int st = make_geometry(shape, g)) return st;
    if (g.B == 0 || g.Nq == 0) return ok();
    if (!offset_px || !logits || !ref_out || !loc_out || !weights_out) return fail(MSDA_E_NULL, "NULL tensor");
    if (!query_ref && g.Nq != g.S)
        return fail(MSDA_E_SHAPE, "encoder reference points need num_query == num_value (%d != %d)", g.Nq, g.S);
    if (!aligned(ref_out, 8) || !aligned(loc_out, 8) || !aligned(offset_px, 8) || (query_ref && !aligned(query_ref, 8)))
        return fail(MSDA_E_ALIGN, "(x, y) tensors need 8-byte alignment");
    if (!aligned(logits, 4) || !aligned(weights_out, 4) || (valid_ratios && !aligned(valid_ratios, 4)))
        return fail(MSDA_E_ALIGN, "fp32 tensors need 4-byte alignment");
    return launched(msda::launch_prologue(g, valid_ratios, query_ref, offset_px, logits, ref_out, loc_out,
                                          weights_out, (hipStream_t)stream),
                    "prologue");
}

static int check_core(const msda::Geometry &g, const void *value, msda_dtype vt, const float *loc,
                      const float *attn)
{
    if (vt != MSDA_F32 && vt != MSDA_BF16) return fail(MSDA_E_UNSUPPORTED, "value dtype %d", (int)vt);
    if (!value || !loc || !attn) return fail(MSDA_E_NULL, "NULL tensor");
    if (!aligned(value, vt == MSDA_F32 ? 4 : 2) || !aligned(loc, 8) || !aligned(attn, 4))
        return fail(MSDA_E_ALIGN, "value needs element alignment, locations 8 bytes, weights 4 bytes");
    (void)g;
    return MSDA_OK;
}

int msda_forward(const msda_shape *shape, const void *value, msda_dtype value_dtype,
                 const float *sampling_locations, const float *attention_weights, float *output, void *stream)
{
    msda::Geometry g;
    if (int st = make_geometry(shape, g)) return st;
    if (g.B == 0 || g.Nq == 0) return ok();
    if (int st = check_core(g, value, value_dtype, sampling_locations, attention_weights)) return st;
    if (!output) return fail(MSDA_E_NULL, "output is NULL");
    if (!aligned(output, 4)) return fail(MSDA_E_ALIGN, "output needs 4-byte alignment");
    return launched(msda::launch_forward(g, value, value_dtype, sampling_locations, attention_weights, output,
                                         (hipStream_t)stream),
                    "forward");
}

int msda_backward_workspace_size(const msda_shape *shape, size_t *bytes)
{
    msda::Geometry g;
    if (!bytes) return fail(MSDA_E_NULL, "bytes is NULL");
    if (int st = make_geometry(shape, g)) return st;
    *bytes = (g.B == 0 || g.Nq == 0) ? 0 : msda::backward_workspace_bytes(g);
    return ok();
}

int msda_backward_plan(const msda_shape *shape, uint32_t *dense_levels, uint32_t *direct_levels,
                       uint32_t *split_levels)
{
    msda::Geometry g;
    if (int st = make_geometry(shape, g)) return st;
    uint32_t d = 0, r = 0, sp = 0;
    if (g.B > 0 && g.Nq > 0) msda::backward_plan_masks(g, d, r, sp);
    if (dense_levels) *dense_levels = d;
    if (direct_levels) *direct_levels = r;
    if (split_levels) *split_levels = sp;
    return ok();
}

int msda_backward(const msda_shape *shape, const void *value, msda_dtype value_dtype,
                  const float *sampling_locations, const float *attention_weights, const float *grad_output,
                  float *grad_value, float *grad_sampling_locations, float *grad_attention_weights,
                  void *workspace, size_t workspace_bytes, unsigned flags, void *stream)
{
    msda::Geometry g;
    if (int st = make_geometry(shape, g)) return st;
    if (flags & ~MSDA_BWD_ACCUMULATE)
        return fail(MSDA_E_UNSUPPORTED, "unknown flags 0x%x", flags);
    const bool accumulate = (flags & MSDA_BWD_ACCUMULATE) != 0;
    if (g.B == 0) return ok();
    if (g.Nq == 0) {  // no queries: grad_value is all zeros (or left as is when accumulating)
        if (accumulate) return ok();
        if (!grad_value) return fail(MSDA_E_NULL, "grad_value is NULL");
        if (!aligned(grad_value, 4)) return fail(MSDA_E_ALIGN, "grad_value needs 4-byte alignment");
        return launched(msda::launch_zero_fill(grad_value, (int64_t)g.B * g.S * g.M * g.D, (hipStream_t)stream),
                        "zero_fill");
    }
    if (int st = check_core(g, value, value_dtype, sampling_locations, attention_weights)) return st;
    if (!grad_output || !grad_value || !grad_sampling_locations || !grad_attention_weights)
        return fail(MSDA_E_NULL, "NULL gradient tensor");
    if (!aligned(grad_output, 4) || !aligned(grad_value, 4) || !aligned(grad_sampling_locations, 8) ||
        !aligned(grad_attention_weights, 4))
        return fail(MSDA_E_ALIGN, "gradient tensors need 4-byte (locations 8-byte) alignment");
    if (msda::backward_uses_workspace(g, value, value_dtype, grad_output, grad_value)) {
        const size_t need = msda::backward_workspace_bytes(g);
        if (!workspace || workspace_bytes < need)
            return fail(MSDA_E_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                        need);
        if (!aligned(workspace, 256)) return fail(MSDA_E_ALIGN, "workspace needs 256-byte alignment");
    }
    return launched(msda::launch_backward(g, value, value_dtype, sampling_locations, attention_weights, grad_output,
                                          grad_value, grad_sampling_locations, grad_attention_weights, workspace,
                                          accumulate, true, (hipStream_t)stream),
                    "backward");
}

int msda_backward_noalloc(const msda_shape *shape, const void *value, msda_dtype value_dtype,
                          const float *sampling_locations, const float *attention_weights, const float *grad_output,
                          float *grad_value, float *grad_sampling_locations, float *grad_attention_weights,
                          unsigned flags, void *stream)
{
    msda::Geometry g;
    if (int st = make_geometry(shape, g)) return st;
    if (flags & ~MSDA_BWD_ACCUMULATE) return fail(MSDA_E_UNSUPPORTED, "unknown flags 0x%x", flags);
    const bool accumulate = (flags & MSDA_BWD_ACCUMULATE) != 0;
    if (g.B == 0) return ok();
    msda::TimingOff no_events;
    if (g.Nq == 0) {  // no queries: grad_value is all zeros (or left as is when accumulating)
        if (accumulate) return ok();
        if (!grad_value) return fail(MSDA_E_NULL, "grad_value is NULL");
        if (!aligned(grad_value, 4)) return fail(MSDA_E_ALIGN, "grad_value needs 4-byte alignment");
        return launched(msda::launch_zero_fill(grad_value, (int64_t)g.B * g.S * g.M * g.D, (hipStream_t)stream),
                        "zero_fill");
    }
    if (int st = check_core(g, value, value_dtype, sampling_locations, attention_weights)) return st;
    if (!grad_output || !grad_value || !grad_sampling_locations || !grad_attention_weights)
        return fail(MSDA_E_NULL, "NULL gradient tensor");
    if (!aligned(grad_output, 4) || !aligned(grad_value, 4) || !aligned(grad_sampling_locations, 8) ||
        !aligned(grad_attention_weights, 4))
        return fail(MSDA_E_ALIGN, "gradient tensors need 4-byte (locations 8-byte) alignment");
    void *scratch = nullptr;
    if (msda::backward_uses_workspace(g, value, value_dtype, grad_output, grad_value)) {
        const size_t need = msda::backward_workspace_bytes(g);
        if (need > msda::kNoAllocScratchBytes)
            return fail(MSDA_E_WORKSPACE, "these sizes need %zu bytes of scratch; msda_backward_noalloc holds %zu",
                        need, msda::kNoAllocScratchBytes);
        const hipError_t e = msda::noalloc_scratch(&scratch);
        if (e != hipSuccess) return fail(MSDA_E_HIP, "scratch address: %s", hipGetErrorString(e));
    }
    return launched(msda::launch_backward(g, value, value_dtype, sampling_locations, attention_weights, grad_output,
                                          grad_value, grad_sampling_locations, grad_attention_weights, scratch,
                                          accumulate, false, (hipStream_t)stream),
                    "backward_noalloc");
}

int msda_forward_fused(const msda_shape *shape, const void *value, msda_dtype value_dtype,
                       const float *reference_points, int reference_dims, const float *sampling_offsets,
                       const float *attention_logits, const uint8_t *key_padding_mask, float *output,
                       float *sampling_locations_out, float *attention_weights_out, void *stream)
{
    msda::Geometry g;
    if (int st = make_geometry(shape, g)) return st;
    if (reference_dims != 2 && reference_dims != 4)
        return fail(MSDA_E_UNSUPPORTED, "reference_dims %d (2 or 4)", reference_dims);
    if (g.B == 0 || g.Nq == 0) return ok();
    if (value_dtype != MSDA_F32 && value_dtype != MSDA_BF16) return fail(MSDA_E_UNSUPPORTED, "value dtype %d", (int)value_dtype);
    if (!value || !reference_points || !sampling_offsets || !attention_logits || !output || !sampling_locations_out ||
        !attention_weights_out)
        return fail(MSDA_E_NULL, "NULL tensor");
    if (!aligned(value, value_dtype == MSDA_F32 ? 4 : 2) || !aligned(reference_points, 4 * reference_dims) ||
        !aligned(sampling_offsets, 8) || !aligned(attention_logits, 4) || !aligned(output, 4) ||
        !aligned(sampling_locations_out, 8) || !aligned(attention_weights_out, 4))
        return fail(MSDA_E_ALIGN, "value needs element alignment, (x, y) tensors 8 bytes, boxes 16, the others 4");
    msda::FusedInputs fi{reference_points, reference_dims, reinterpret_cast<const float2 *>(sampling_offsets),
                         attention_logits,
                         reinterpret_cast<float2 *>(sampling_locations_out), attention_weights_out,
                         key_padding_mask};
    return launched(msda::launch_forward_fused(g, value, value_dtype, fi, output, (hipStream_t)stream),
                    "forward_fused");
}

int msda_backward_fused(const msda_shape *shape, const void *value, msda_dtype value_dtype,
                        const float *sampling_locations, const float *attention_weights,
                        const float *reference_points, const float *sampling_offsets, int reference_dims,
                        const uint8_t *key_padding_mask, const float *grad_output, float *grad_value, float *grad_sampling_offsets,
                        float *grad_attention_logits, float *grad_reference_points, void *workspace,
                        size_t workspace_bytes, unsigned flags, void *stream)
{
    msda::Geometry g;
    if (int st = make_geometry(shape, g)) return st;
    if (reference_dims != 2 && reference_dims != 4)
        return fail(MSDA_E_UNSUPPORTED, "reference_dims %d (2 or 4)", reference_dims);
    if (flags & ~MSDA_BWD_ACCUMULATE)
        return fail(MSDA_E_UNSUPPORTED, "unknown flags 0x%x", flags);
    const bool accumulate = (flags & MSDA_BWD_ACCUMULATE) != 0;
    if (g.B == 0) return ok();
    if (g.Nq == 0) {  // no queries: grad_value is all zeros (or left as is when accumulating)
        if (accumulate) return ok();
        if (!grad_value) return fail(MSDA_E_NULL, "grad_value is NULL");
        if (!aligned(grad_value, 4)) return fail(MSDA_E_ALIGN, "grad_value needs 4-byte alignment");
        return launched(msda::launch_zero_fill(grad_value, (int64_t)g.B * g.S * g.M * g.D, (hipStream_t)stream),
                        "zero_fill");
    }
    if (int st = check_core(g, value, value_dtype, sampling_locations, attention_weights)) return st;
    if (!grad_output || !grad_value || !grad_sampling_offsets || !grad_attention_logits)
        return fail(MSDA_E_NULL, "NULL gradient tensor");
    if (reference_dims == 4 && (!reference_points || !sampling_offsets))
        return fail(MSDA_E_NULL, "box references need reference_points and sampling_offsets");
    if (!aligned(grad_output, 4) || !aligned(grad_value, 4) || !aligned(grad_sampling_offsets, 8) ||
        !aligned(grad_attention_logits, 4) ||
        (grad_reference_points && !aligned(grad_reference_points, 4 * reference_dims)) ||
        (reference_dims == 4 && (!aligned(reference_points, 16) || !aligned(sampling_offsets, 8))))
        return fail(MSDA_E_ALIGN, "gradient tensors need 4-byte ((x, y) 8-byte, boxes 16-byte) alignment");
    if (msda::backward_uses_workspace(g, value, value_dtype, grad_output, grad_value)) {
        const size_t need = msda::backward_workspace_bytes(g);
        if (!workspace || workspace_bytes < need)
            return fail(MSDA_E_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                        need);
        if (!aligned(workspace, 256)) return fail(MSDA_E_ALIGN, "workspace needs 256-byte alignment");
    }
    const msda::FusedGrads fg{reference_points, reinterpret_cast<const float2 *>(sampling_offsets), reference_dims,
                              grad_reference_points, key_padding_mask};
    return launched(msda::launch_backward_fused(g, value, value_dtype, sampling_locations, attention_weights,
                                                grad_output, grad_value, grad_sampling_offsets, grad_attention_logits,
                                                fg, workspace, accumulate, true, (hipStream_t)stream),
                    "backward_fused");
}

}  // extern "C"
