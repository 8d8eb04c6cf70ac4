// Kernels that prepare the core's inputs: reference points, sampling
// locations, the L*K softmax, and the zero fill of grad_value.
//
// All four are elementwise and bound by HBM bandwidth; they use plain global
// loads/stores, one thread per output row.
#include "msda_device.h"
#include "msda_internal.h"

namespace msda {
namespace {

constexpr int kBlock = 256;

// Reference points (juhe.plus debug-build notes, "Key point 1:
// get_reference_points"; xdnf.cn walkthrough, "encoder" and "Decoder").
// Query t = (b, q)'s position relative to the valid extent of the image, in
// [0, 1] when inside; reference point at level l = that position scaled by
// level l's valid ratios.
__device__ __forceinline__ float2 query_position(const Geometry &g, const float *__restrict__ vr,
                                                 const float *__restrict__ u, int b, int q, int64_t t)
{
    if (u) {
        // decoder: u is already relative to the valid region of the image
        return make_float2(u[2 * t + 0], u[2 * t + 1]);
    }
    // encoder: q is pixel (i, j) of level lq; its centre, normalised by the
    // valid extent of its own level
    int lq = 0;
    for (int l = 1; l < g.L; ++l)
        if (q >= g.lv.start[l]) lq = l;
    const int local = q - g.lv.start[lq];
    const int W = g.lv.W[lq];
    const int i = local / W;
    const int j = local - i * W;
    const float vx = vr ? vr[(b * g.L + lq) * 2 + 0] : 1.0f;
    const float vy = vr ? vr[(b * g.L + lq) * 2 + 1] : 1.0f;
    return make_float2(((float)j + 0.5f) / (vx * (float)W), ((float)i + 0.5f) / (vy * (float)g.lv.H[lq]));
}

__device__ __forceinline__ float2 level_point(const Geometry &g, const float *__restrict__ vr, float2 p, int b,
                                              int l)
{
    const float sx = vr ? vr[(b * g.L + l) * 2 + 0] : 1.0f;
    const float sy = vr ? vr[(b * g.L + l) * 2 + 1] : 1.0f;
    return make_float2(p.x * sx, p.y * sy);
}

// One thread per (b, q), writing the L (x, y) pairs of that query.
__global__ void __launch_bounds__(kBlock)
reference_points_kernel(Geometry g, const float *__restrict__ vr, const float *__restrict__ u,
                        float *__restrict__ ref)
{
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (t >= (int64_t)g.B * g.Nq) return;
    const int b = (int)(t / g.Nq);
    const int q = (int)(t - (int64_t)b * g.Nq);
    const float2 p = query_position(g, vr, u, b, q, t);
    float2 *out = reinterpret_cast<float2 *>(ref) + t * g.L;
    for (int l = 0; l < g.L; ++l) out[l] = level_point(g, vr, p, b, l);
}

// loc = ref + offset_px / (W_l, H_l) (walkthrough page, "encoder"; paper
// notes, "Key code"). For even K the (x, y) pairs of one (b, q, m, l) are
// contiguous, so consecutive threads take consecutive pairs of points.
template <int K>
__global__ void __launch_bounds__(kBlock)
sampling_locations_kernel(Geometry g, const float2 *__restrict__ ref, const float4 *__restrict__ off,
                          float4 *__restrict__ loc)
{
    // one thread per pair of points of one (b, q, m, l): a 16-byte load and
    // store each; 32-bit index math (the host keeps the pair count < 2^32)
    constexpr int KP = K / 2;
    static_assert(K % 2 == 0, "pairs of points");
    const uint32_t t = blockIdx.x * kBlock + threadIdx.x;
    if (t >= (uint32_t)(g.queries() * g.M * g.L * KP)) return;
    const uint32_t row = t / KP;  // (b, q, m, l)
    const int l = (int)(row % (uint32_t)g.L);
    const uint32_t bq = row / (uint32_t)(g.L * g.M);
    int W = 1, H = 1;
#pragma unroll
    for (int i = 0; i < MSDA_MAX_LEVELS; ++i)
        if (i == l) {
            W = g.lv.W[i];
            H = g.lv.H[i];
        }
    const float Wf = (float)W, Hf = (float)H;
    const float2 r = ref[(int64_t)bq * g.L + l];
    const float4 v = off[t];
    loc[t] = make_float4(r.x + v.x / Wf, r.y + v.y / Hf, r.x + v.z / Wf, r.y + v.w / Hf);
}

// Any K: one thread per sample.
__global__ void __launch_bounds__(kBlock)
sampling_locations_any_kernel(Geometry g, const float2 *__restrict__ ref, const float2 *__restrict__ off,
                              float2 *__restrict__ loc)
{
    const int64_t s = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (s >= g.samples()) return;
    const int64_t row = s / g.K;  // (b, q, m, l)
    const int l = (int)(row % g.L);
    const int64_t bq = row / ((int64_t)g.L * g.M);
    int W = 1, H = 1;
#pragma unroll
    for (int i = 0; i < MSDA_MAX_LEVELS; ++i)
        if (i == l) {
            W = g.lv.W[i];
            H = g.lv.H[i];
        }
    const float2 r = ref[bq * g.L + l];
    const float2 v = off[s];
    loc[s] = make_float2(r.x + v.x / (float)W, r.y + v.y / (float)H);
}

// Locations from 4-d box references (cx, cy, w, h): ref_xy + offset / K *
// ref_wh / 2 (the 4-d reference branch of the module source on the
// walkthrough page). One thread per sample.
__global__ void __launch_bounds__(kBlock)
sampling_locations_box_kernel(Geometry g, const float *__restrict__ ref, const float2 *__restrict__ off,
                              float2 *__restrict__ loc)
{
    const int64_t s = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (s >= g.samples()) return;
    const int64_t row = s / g.K;  // (b, q, m, l)
    const int l = (int)(row % g.L);
    const int64_t bq = row / ((int64_t)g.L * g.M);
    loc[s] = fused_location(ref, 4, bq * g.L + l, off[s], 1.0f, 1.0f, (float)g.K);
}

// Softmax over the L*K logits of one (b, q, m) (paper notes, "Insight 2": the
// weights of a query and head sum to 1 over all levels and points). Rows of N
// (a multiple of 4) take N/4 adjacent lanes, one 16-byte load and store each;
// the max and the sum go across the row's lanes by DPP butterflies, so that
// many rows are in flight per wave.
template <int N>
__global__ void __launch_bounds__(kBlock)
softmax_vec_kernel(int64_t rows, const float4 *x, float4 *y)  // y may alias x
{
    constexpr int C = N / 4;  // lanes per row (divides 64: rows never straddle a wave)
    static_assert(N % 4 == 0 && kWave % C == 0, "row lanes");
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    // a row's lanes are all in range or all out of it, so the butterflies
    // below only ever combine lanes of one live row
    if (t >= rows * C) return;
    const float4 v = x[t];
    const float mx = group_max<C>(fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    const float e0 = expf(v.x - mx), e1 = expf(v.y - mx), e2 = expf(v.z - mx), e3 = expf(v.w - mx);
    const float sum = group_sum<C>((e0 + e1) + (e2 + e3));
    y[t] = make_float4(e0 / sum, e1 / sum, e2 / sum, e3 / sum);
}

__global__ void __launch_bounds__(kBlock)
softmax_kernel(int64_t rows, int n, const float *x, float *y)  // y may alias x
{
    const int64_t row = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (row >= rows) return;
    const float *xr = x + row * n;
    float *yr = y + row * n;
    float mx = xr[0];
    for (int i = 1; i < n; ++i) mx = fmaxf(mx, xr[i]);
    float sum = 0.0f;
    for (int i = 0; i < n; ++i) {
        const float e = expf(xr[i] - mx);
        yr[i] = e;
        sum += e;
    }
    for (int i = 0; i < n; ++i) yr[i] = yr[i] / sum;
}

// Reference points, sampling locations and the softmax in one launch (K in
// {2, 4, 8}, L*K in {4, 8, 16, 32}, 16-byte aligned tensors). The first loc_blocks
// workgroups form the locations, one thread per pair of points as in
// sampling_locations_kernel, each forming its query's reference point itself
// instead of reading it back; the next sm_blocks take the softmax rows as in
// softmax_vec_kernel; the rest write the reference points. Every output
// takes the same operations in the same order as in the separate kernels,
// so the bits agree (no contraction of the reference point's product into
// the location's sum).
template <int K, int N>
__global__ void __launch_bounds__(kBlock)
prologue_kernel(Geometry g, const float *__restrict__ vr, const float *__restrict__ u,
                const float4 *__restrict__ off, float4 *__restrict__ loc, const float4 *logits, float4 *w,
                float *__restrict__ ref, uint32_t loc_blocks, uint32_t sm_blocks)  // w may alias logits
{
#pragma clang fp contract(off)
    if (blockIdx.x < loc_blocks) {
        constexpr int KP = K / 2;
        const uint32_t row = blockIdx.x * kBlock + threadIdx.x;  // (b, q, m, l)
        if (row >= (uint32_t)(g.queries() * g.M * g.L)) return;
        const int l = (int)(row % (uint32_t)g.L);
        const uint32_t bq = row / (uint32_t)(g.L * g.M);
        const int b = (int)(bq / (uint32_t)g.Nq);
        const int q = (int)(bq - (uint32_t)b * (uint32_t)g.Nq);
        int W = 1, H = 1;
#pragma unroll
        for (int i = 0; i < MSDA_MAX_LEVELS; ++i)
            if (i == l) {
                W = g.lv.W[i];
                H = g.lv.H[i];
            }
        const float Wf = (float)W, Hf = (float)H;
        float4 v[KP];
#pragma unroll
        for (int p = 0; p < KP; ++p) v[p] = off[row * KP + p];
        const float2 r = level_point(g, vr, query_position(g, vr, u, b, q, (int64_t)bq), b, l);
#pragma unroll
        for (int p = 0; p < KP; ++p)
            loc[row * KP + p] = make_float4(r.x + v[p].x / Wf, r.y + v[p].y / Hf, r.x + v[p].z / Wf, r.y + v[p].w / Hf);
        return;
    }
    if (blockIdx.x < loc_blocks + sm_blocks) {
        constexpr int C = N / 4;  // lanes per row (divides 64: rows never straddle a wave)
        static_assert(N % 4 == 0 && kWave % C == 0, "row lanes");
        // the softmax part starts on a workgroup boundary, so a row's lanes
        // are all in range or all out of it, as in softmax_vec_kernel
        const int64_t t = (int64_t)(blockIdx.x - loc_blocks) * kBlock + threadIdx.x;
        if (t >= g.queries() * g.M * C) return;
        const float4 v = logits[t];
        const float mx = group_max<C>(fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
        const float e0 = expf(v.x - mx), e1 = expf(v.y - mx), e2 = expf(v.z - mx), e3 = expf(v.w - mx);
        const float sum = group_sum<C>((e0 + e1) + (e2 + e3));
        w[t] = make_float4(e0 / sum, e1 / sum, e2 / sum, e3 / sum);
        return;
    }
    const int64_t t = (int64_t)(blockIdx.x - loc_blocks - sm_blocks) * kBlock + threadIdx.x;
    if (t >= g.queries()) return;
    const int b = (int)(t / g.Nq);
    const int q = (int)(t - (int64_t)b * g.Nq);
    const float2 p = query_position(g, vr, u, b, q, t);
    float2 *out = reinterpret_cast<float2 *>(ref) + t * g.L;
    for (int l = 0; l < g.L; ++l) out[l] = level_point(g, vr, p, b, l);
}

// Zero n floats; vector stores when p is 16-byte aligned.
__global__ void __launch_bounds__(kBlock) zero_fill_kernel(float *__restrict__ p, int64_t n)
{
    const int64_t n4 = (reinterpret_cast<uintptr_t>(p) & 15u) ? 0 : n / 4;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    float4 *p4 = reinterpret_cast<float4 *>(p);
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n4; i += stride)
        p4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        p[i] = 0.0f;
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + kBlock - 1) / kBlock); }

}  // namespace

hipError_t launch_reference_points(const Geometry &g, const float *vr, const float *u, float *ref,
                                   hipStream_t st)
{
    {
        KernelScope ks_("reference_points_kernel", st);
        hipLaunchKernelGGL(reference_points_kernel, dim3(blocks_for(g.queries())), dim3(kBlock), 0, st,
                           g, vr, u, ref);
    }
    return hipGetLastError();
}

hipError_t launch_sampling_locations(const Geometry &g, const float *ref, const float *off,
                                     float *loc, hipStream_t st)
{
    const auto r = reinterpret_cast<const float2 *>(ref);
    const auto o = reinterpret_cast<const float2 *>(off);
    const auto d = reinterpret_cast<float2 *>(loc);
    const auto o4 = reinterpret_cast<const float4 *>(off);
    const auto d4 = reinterpret_cast<float4 *>(loc);
    const bool a16 = (reinterpret_cast<uintptr_t>(off) % 16) == 0 && (reinterpret_cast<uintptr_t>(loc) % 16) == 0;
    const int64_t pairs = g.samples() / 2;  // float4 = two points
    const bool vec = a16 && g.K % 2 == 0 && pairs + kBlock < (int64_t(1) << 32);
    const unsigned blocks = blocks_for(pairs);
    if (vec && g.K == 4) {
        KernelScope ks_("sampling_locations_kernel", st);
        hipLaunchKernelGGL(sampling_locations_kernel<4>, dim3(blocks), dim3(kBlock), 0, st, g, r, o4, d4);
    } else if (vec && g.K == 2) {
        KernelScope ks_("sampling_locations_kernel", st);
        hipLaunchKernelGGL(sampling_locations_kernel<2>, dim3(blocks), dim3(kBlock), 0, st, g, r, o4, d4);
    } else if (vec && g.K == 8) {
        KernelScope ks_("sampling_locations_kernel", st);
        hipLaunchKernelGGL(sampling_locations_kernel<8>, dim3(blocks), dim3(kBlock), 0, st, g, r, o4, d4);
    } else {
        KernelScope ks_("sampling_locations_any_kernel", st);
        hipLaunchKernelGGL(sampling_locations_any_kernel, dim3(blocks_for(g.samples())), dim3(kBlock), 0, st, g, r,
                           o, d);
    }
    return hipGetLastError();
}

hipError_t launch_sampling_locations_box(const Geometry &g, const float *ref, const float *off, float *loc,
                                         hipStream_t st)
{
    {
        KernelScope ks_("sampling_locations_box_kernel", st);
        hipLaunchKernelGGL(sampling_locations_box_kernel, dim3(blocks_for(g.samples())), dim3(kBlock), 0, st, g, ref,
                           reinterpret_cast<const float2 *>(off), reinterpret_cast<float2 *>(loc));
    }
    return hipGetLastError();
}

hipError_t launch_softmax(const Geometry &g, const float *logits, float *w, hipStream_t st)
{
    const int64_t rows = g.queries() * g.M;
    const int n = g.L * g.K;
    const bool a16 = (reinterpret_cast<uintptr_t>(logits) % 16) == 0 && (reinterpret_cast<uintptr_t>(w) % 16) == 0;
    const auto x4 = reinterpret_cast<const float4 *>(logits);
    const auto y4 = reinterpret_cast<float4 *>(w);
    if (a16 && n == 16) {
        KernelScope ks_("softmax_vec_kernel", st);
        hipLaunchKernelGGL(softmax_vec_kernel<16>, dim3(blocks_for(rows * 4)), dim3(kBlock), 0, st, rows, x4, y4);
    } else if (a16 && n == 32) {
        KernelScope ks_("softmax_vec_kernel", st);
        hipLaunchKernelGGL(softmax_vec_kernel<32>, dim3(blocks_for(rows * 8)), dim3(kBlock), 0, st, rows, x4, y4);
    } else if (a16 && n == 8) {
        KernelScope ks_("softmax_vec_kernel", st);
        hipLaunchKernelGGL(softmax_vec_kernel<8>, dim3(blocks_for(rows * 2)), dim3(kBlock), 0, st, rows, x4, y4);
    } else if (a16 && n == 4) {
        KernelScope ks_("softmax_vec_kernel", st);
        hipLaunchKernelGGL(softmax_vec_kernel<4>, dim3(blocks_for(rows * 1)), dim3(kBlock), 0, st, rows, x4, y4);
    } else {
        KernelScope ks_("softmax_kernel", st);
        hipLaunchKernelGGL(softmax_kernel, dim3(blocks_for(rows)), dim3(kBlock), 0, st, rows, n, logits, w);
    }
    return hipGetLastError();
}

hipError_t launch_prologue(const Geometry &g, const float *vr, const float *u, const float *off,
                           const float *logits, float *ref, float *loc, float *w, hipStream_t st)
{
    const int n = g.L * g.K;
    const bool a16 = (reinterpret_cast<uintptr_t>(off) % 16) == 0 && (reinterpret_cast<uintptr_t>(loc) % 16) == 0 &&
                     (reinterpret_cast<uintptr_t>(logits) % 16) == 0 && (reinterpret_cast<uintptr_t>(w) % 16) == 0;
    const int64_t pairs = g.samples() / 2;
    const int64_t loc_rows = g.queries() * g.M * g.L;  // (b, q, m, l)
    const int64_t sm_threads = g.queries() * g.M * (n / 4);
    const int64_t blocks = blocks_for(loc_rows) + blocks_for(sm_threads) + blocks_for(g.queries());
    const bool one = a16 && (g.K == 2 || g.K == 4 || g.K == 8) && (n == 4 || n == 8 || n == 16 || n == 32) &&
                     pairs + kBlock < (int64_t(1) << 32) && blocks < (int64_t(1) << 31);
    if (!one) {
        // the separate kernels, in turn
        hipError_t e = launch_reference_points(g, vr, u, ref, st);
        if (e == hipSuccess) e = launch_sampling_locations(g, ref, off, loc, st);
        if (e == hipSuccess) e = launch_softmax(g, logits, w, st);
        return e;
    }
    const uint32_t lb = blocks_for(loc_rows), sb = blocks_for(sm_threads);
    const auto o4 = reinterpret_cast<const float4 *>(off);
    const auto l4 = reinterpret_cast<float4 *>(loc);
    const auto x4 = reinterpret_cast<const float4 *>(logits);
    const auto w4 = reinterpret_cast<float4 *>(w);
    KernelScope ks_("prologue_kernel", st);
#define MSDA_PROLOGUE(KK, NN)                                                                                      \
    if (g.K == KK && n == NN) {                                                                                    \
        hipLaunchKernelGGL((prologue_kernel<KK, NN>), dim3((unsigned)blocks), dim3(kBlock), 0, st, g, vr, u, o4,  \
                           l4, x4, w4, ref, lb, sb);                                                               \
        return hipGetLastError();                                                                                  \
    }
    MSDA_PROLOGUE(4, 16)
    MSDA_PROLOGUE(4, 4)
    MSDA_PROLOGUE(4, 8)
    MSDA_PROLOGUE(4, 32)
    MSDA_PROLOGUE(2, 4)
    MSDA_PROLOGUE(2, 8)
    MSDA_PROLOGUE(2, 16)
    MSDA_PROLOGUE(2, 32)
    MSDA_PROLOGUE(8, 8)
    MSDA_PROLOGUE(8, 16)
    MSDA_PROLOGUE(8, 32)
#undef MSDA_PROLOGUE
    return hipErrorInvalidValue;  // every K in {2, 4, 8} with n in {4, 8, 16, 32} is listed above
}

hipError_t launch_zero_fill(float *p, int64_t n, hipStream_t st)
{
    int64_t blocks = (n / 4 + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    {
        KernelScope ks_("zero_fill_kernel", st);
        hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, p, n);
    }
    return hipGetLastError();
}

}  // namespace msda
