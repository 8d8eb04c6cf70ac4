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
// One thread per (b, q), writing the L (x, y) pairs of that query.
__global__ void __launch_bounds__(kBlock)
reference_points_kernel(Geometry g, const float *__restrict__ vr, const float *__restrict__ u,
                        float *__restrict__ ref)
{
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (t >= (int64_t)g.B * g.Nq) return;
    const int b = (int)(t / g.Nq);
    const int q = (int)(t - (int64_t)b * g.Nq);
    float px, py;  // position relative to the valid extent, in [0, 1] when inside
    if (u) {
        // decoder: u is already relative to the valid region of the image
        px = u[2 * t + 0];
        py = u[2 * t + 1];
    } else {
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
        px = ((float)j + 0.5f) / (vx * (float)W);
        py = ((float)i + 0.5f) / (vy * (float)g.lv.H[lq]);
    }
    float2 *out = reinterpret_cast<float2 *>(ref) + t * g.L;
    for (int l = 0; l < g.L; ++l) {
        const float sx = vr ? vr[(b * g.L + l) * 2 + 0] : 1.0f;
        const float sy = vr ? vr[(b * g.L + l) * 2 + 1] : 1.0f;
        out[l] = make_float2(px * sx, py * sy);
    }
}

// loc = ref + offset_px / (W_l, H_l) (walkthrough page, "encoder"; paper
// notes, "Key code"). One thread per (b, q, m).
__global__ void __launch_bounds__(kBlock)
sampling_locations_kernel(Geometry g, const float2 *__restrict__ ref,
                          const float2 *__restrict__ off, float2 *__restrict__ loc)
{
    const int64_t row = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (row >= (int64_t)g.B * g.Nq * g.M) return;
    const int64_t bq = row / g.M;
    for (int l = 0; l < g.L; ++l) {
        const float2 r = ref[bq * g.L + l];
        const float Wf = (float)g.lv.W[l], Hf = (float)g.lv.H[l];
        const int64_t base = (row * g.L + l) * g.K;
        for (int k = 0; k < g.K; ++k) {
            const float2 o = off[base + k];
            loc[base + k] = make_float2(r.x + o.x / Wf, r.y + o.y / Hf);
        }
    }
}

// Softmax over the L*K logits of one (b, q, m) (paper notes, "Insight 2": the
// weights of a query and head sum to 1 over all levels and points).
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
    hipLaunchKernelGGL(reference_points_kernel, dim3(blocks_for(g.queries())), dim3(kBlock), 0, st,
                       g, vr, u, ref);
    return hipGetLastError();
}

hipError_t launch_sampling_locations(const Geometry &g, const float *ref, const float *off,
                                     float *loc, hipStream_t st)
{
    hipLaunchKernelGGL(sampling_locations_kernel, dim3(blocks_for(g.queries() * g.M)), dim3(kBlock),
                       0, st, g, reinterpret_cast<const float2 *>(ref),
                       reinterpret_cast<const float2 *>(off), reinterpret_cast<float2 *>(loc));
    return hipGetLastError();
}

hipError_t launch_softmax(const Geometry &g, const float *logits, float *w, hipStream_t st)
{
    const int64_t rows = g.queries() * g.M;
    hipLaunchKernelGGL(softmax_kernel, dim3(blocks_for(rows)), dim3(kBlock), 0, st, rows, g.L * g.K,
                       logits, w);
    return hipGetLastError();
}

hipError_t launch_zero_fill(float *p, int64_t n, hipStream_t st)
{
    int64_t blocks = (n / 4 + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace msda
