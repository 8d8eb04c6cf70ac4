// Backward of the MSDeformAttn core on gfx950: the exact derivative of the
// forward (the op is trained end to end through autograd: xdnf.cn walkthrough,
// "encoder"; paper notes, "Key code"). Per sample with bilinear weights
// w_c = wx_c * wy_c and corner values v_c (0 off the map):
//   grad_attn        = sum_d G_d * sum_c w_c v_c[d]
//   grad_loc.x       = A * W_l * sum_d G_d * sum_c (d wx_c/d fx) wy_c v_c[d]
//   grad_loc.y       = A * H_l * sum_d G_d * sum_c wx_c (d wy_c/d fy) v_c[d]
//   grad_value[row_c] += A * w_c * G        (scattered, device atomics)
//
// Fast path (C = M*D = 256): the forward's wave-per-query layout. Phase 1
// parks each sample's corner offsets and (fx, fy, A) in LDS; phase 2 gathers
// the four corners, forms the per-lane partial dot products with the lane's
// four channels of G, reduces them over the lanes of the head (DPP/permute),
// and scatters A*w_c*G with buffer atomics whose out-of-range offsets (corners
// off the map) are dropped by the hardware range check.
#include "msda_device.h"
#include "msda_internal.h"

namespace msda {
namespace {

constexpr int kWaves = 4;
constexpr int kBlock = kWaves * kWave;

struct LevelRec {
    float Wf, Hf;
    int32_t W, start;
};

__device__ __forceinline__ float dot4(const float4 &a, const float4 &b)
{
    return __builtin_fmaf(a.w, b.w, __builtin_fmaf(a.z, b.z, __builtin_fmaf(a.y, b.y, a.x * b.x)));
}

__device__ __forceinline__ void atomic_add4(__amdgpu_buffer_rsrc_t r, uint32_t off, float s,
                                            const float4 &g)
{
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(s * g.x, r, off + 0u, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(s * g.y, r, off + 4u, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(s * g.z, r, off + 8u, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(s * g.w, r, off + 12u, 0, 0);
}

template <typename VT, int M, int L, int K>
__global__ void __launch_bounds__(kBlock)
backward_c256_kernel(Geometry g, const VT *__restrict__ value, const float2 *__restrict__ loc,
                     const float *__restrict__ attn, const float4 *__restrict__ grad_out,
                     float *__restrict__ grad_value, float2 *__restrict__ grad_loc,
                     float *__restrict__ grad_attn, uint32_t grid)
{
    constexpr int C = 256;
    constexpr int D = C / M;
    constexpr int LPH = D / 4;
    constexpr int LK = L * K;
    constexpr int NS = M * LK;
    constexpr int PAD = LK + 1;  // per-head LDS stride in records (breaks bank aliasing)
    constexpr uint32_t RB = C * sizeof(VT);
    constexpr uint32_t GRB = C * sizeof(float);  // grad_value row bytes
    static_assert(GRB % RB == 0, "value rows are no wider than grad_value rows");
    // value byte offset from a grad_value byte offset (a shift for bf16; the
    // out-of-range marker 2^31 becomes 2^30, still beyond S*RB < 2^30)
    auto vbytes = [](uint32_t o) { return o / (GRB / RB); };

    __shared__ LevelRec s_lv[L];
    __shared__ int4 s_off[kWaves][M * PAD];
    __shared__ float4 s_geo[kWaves][M * PAD];   // (fx, fy, A, -)
    __shared__ float4 s_res[kWaves][M * PAD];   // (grad_attn, grad_x, grad_y, -)

    const int lane = threadIdx.x % kWave;
    // wave-uniform by construction; readfirstlane lets the compiler keep the
    // per-wave query, batch and buffer descriptor in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (threadIdx.x < L) {
        const int l = threadIdx.x;
        s_lv[l] = LevelRec{(float)g.lv.W[l], (float)g.lv.H[l], g.lv.W[l], g.lv.start[l]};
    }
    __syncthreads();

    const int64_t gq = (int64_t)xcd_tile(blockIdx.x, grid) * kWaves + wave;
    const bool active = gq < (int64_t)g.B * g.Nq;

    if (active) {
#pragma unroll
        for (int s0 = 0; s0 < NS; s0 += kWave) {
            const int s = s0 + lane;
            if (NS % kWave == 0 || s < NS) {
                const int l = (s / K) % L;
                const int p = s + s / LK;  // padded slot
                const LevelRec lv = s_lv[l];
                float2 u = loc[gq * NS + s];
                const float a = attn[gq * NS + s];
                const bool in = sample_in_range(u.x, u.y, lv.Wf, lv.Hf);
                u.x = in ? u.x : 0.0f;
                u.y = in ? u.y : 0.0f;
                float cx, fx, cy, fy;
                cell_1d(u.x, lv.Wf, cx, fx);
                cell_1d(u.y, lv.Hf, cy, fy);
                const bool x0ok = (cx >= 0.0f) & (cx < lv.Wf);
                const bool x1ok = (cx >= -1.0f) & (cx + 1.0f < lv.Wf);
                const bool y0ok = in & (cy >= 0.0f) & (cy < lv.Hf);
                const bool y1ok = in & (cy >= -1.0f) & (cy + 1.0f < lv.Hf);
                // byte offsets into grad_value rows (fp32, GRB bytes per row);
                // value rows are addressed with the same offsets scaled by
                // RB/GRB. Off-map corners get an offset that stays out of
                // range of both resources after that scaling.
                const uint32_t o00 = (uint32_t)(lv.start + (int)cy * lv.W + (int)cx) * GRB;
                const uint32_t o10 = o00 + (uint32_t)lv.W * GRB;
                int4 o;
                o.x = (int)((y0ok & x0ok) ? o00 : kOutOfRange);
                o.y = (int)((y0ok & x1ok) ? o00 + GRB : kOutOfRange);
                o.z = (int)((y1ok & x0ok) ? o10 : kOutOfRange);
                o.w = (int)((y1ok & x1ok) ? o10 + GRB : kOutOfRange);
                s_off[wave][p] = o;
                s_geo[wave][p] = make_float4(fx, fy, a, 0.0f);
            }
        }
    }
    __syncthreads();
    if (active) {
        const int b = (int)(gq / g.Nq);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(value + (int64_t)b * g.S * C, (uint32_t)g.S * RB);
        const __amdgpu_buffer_rsrc_t gr =
            make_rsrc(grad_value + (int64_t)b * g.S * C, (uint32_t)g.S * GRB);
        const uint32_t vlane = (uint32_t)lane * 4u * sizeof(VT);
        const uint32_t glane = (uint32_t)lane * 16u;
        const int m = lane / LPH;
        const float4 G = grad_out[gq * (C / 4) + lane];
        const int4 *offs = &s_off[wave][m * PAD];
        const float4 *geo = &s_geo[wave][m * PAD];
        float4 *res = &s_res[wave][m * PAD];
        for (int l = 0; l < L; ++l) {
            const float Wf = (float)g.lv.W[l], Hf = (float)g.lv.H[l];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int i = l * K + k;
                const int4 o = offs[i];
                const float4 f = geo[i];
                const uint32_t o00 = (uint32_t)o.x, o01 = (uint32_t)o.y;
                const uint32_t o10 = (uint32_t)o.z, o11 = (uint32_t)o.w;
                const float4 v00 = ValueTraits<VT>::load4(vr, vbytes(o00) + vlane);
                const float4 v01 = ValueTraits<VT>::load4(vr, vbytes(o01) + vlane);
                const float4 v10 = ValueTraits<VT>::load4(vr, vbytes(o10) + vlane);
                const float4 v11 = ValueTraits<VT>::load4(vr, vbytes(o11) + vlane);
                const float d00 = dot4(G, v00), d01 = dot4(G, v01);
                const float d10 = dot4(G, v10), d11 = dot4(G, v11);
                const float fx = f.x, fy = f.y, a = f.z;
                const float hx = 1.0f - fx, hy = 1.0f - fy;
                float ga = hy * (hx * d00 + fx * d01) + fy * (hx * d10 + fx * d11);
                float gx = hy * (d01 - d00) + fy * (d11 - d10);
                float gy = hx * (d10 - d00) + fx * (d11 - d01);
                ga = group_sum<LPH>(ga);
                gx = group_sum<LPH>(gx);
                gy = group_sum<LPH>(gy);
                if (lane % LPH == 0) res[i] = make_float4(ga, a * Wf * gx, a * Hf * gy, 0.0f);
                const float ay0 = a * hy, ay1 = a * fy;
                atomic_add4(gr, o00 + glane, ay0 * hx, G);
                atomic_add4(gr, o01 + glane, ay0 * fx, G);
                atomic_add4(gr, o10 + glane, ay1 * hx, G);
                atomic_add4(gr, o11 + glane, ay1 * fx, G);
            }
        }
    }
    __syncthreads();
    if (!active) return;
#pragma unroll
    for (int s0 = 0; s0 < NS; s0 += kWave) {
        const int s = s0 + lane;
        if (NS % kWave == 0 || s < NS) {
            const float4 r = s_res[wave][s + s / LK];
            grad_attn[gq * NS + s] = r.x;
            grad_loc[gq * NS + s] = make_float2(r.y, r.z);
        }
    }
}

// Generic path: one thread per (b, q, m), looping over the D channels.
template <typename VT>
__device__ __forceinline__ float vload(const VT *p);
template <> __device__ __forceinline__ float vload<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float vload<uint16_t>(const uint16_t *p)
{
    return __uint_as_float((uint32_t)*p << 16);
}

template <typename VT>
__global__ void __launch_bounds__(256)
backward_generic_kernel(Geometry g, const VT *__restrict__ value, const float2 *__restrict__ loc,
                        const float *__restrict__ attn, const float *__restrict__ grad_out,
                        float *__restrict__ grad_value, float2 *__restrict__ grad_loc,
                        float *__restrict__ grad_attn)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)g.B * g.Nq * g.M) return;
    const int C = g.M * g.D;
    const int64_t bq = t / g.M;
    const int m = (int)(t - bq * g.M);
    const int b = (int)(bq / g.Nq);
    const VT *vb = value + (int64_t)b * g.S * C + m * g.D;
    float *gvb = grad_value + (int64_t)b * g.S * C + m * g.D;
    const float *G = grad_out + bq * C + m * g.D;
    for (int l = 0; l < g.L; ++l) {
        const int W = g.lv.W[l], H = g.lv.H[l];
        const float Wf = (float)W, Hf = (float)H;
        for (int k = 0; k < g.K; ++k) {
            const int64_t s = (t * g.L + l) * g.K + k;
            const float2 u = loc[s];
            const float a = attn[s];
            float ga = 0.0f, gx = 0.0f, gy = 0.0f;
            if (sample_in_range(u.x, u.y, Wf, Hf)) {
                float cx, fx, cy, fy;
                cell_1d(u.x, Wf, cx, fx);
                cell_1d(u.y, Hf, cy, fy);
                const int x0 = (int)cx, y0 = (int)cy;
                for (int dy = 0; dy < 2; ++dy)
                    for (int dx = 0; dx < 2; ++dx) {
                        const int xi = x0 + dx, yi = y0 + dy;
                        if (xi < 0 || xi >= W || yi < 0 || yi >= H) continue;
                        const float wx = dx ? fx : 1.0f - fx, wy = dy ? fy : 1.0f - fy;
                        const int64_t row = (g.lv.start[l] + (int64_t)yi * W + xi) * C;
                        float gv = 0.0f;
                        for (int d = 0; d < g.D; ++d) {
                            gv = __builtin_fmaf(G[d], vload<VT>(vb + row + d), gv);
                            atomicAdd(gvb + row + d, a * wx * wy * G[d]);
                        }
                        ga += wx * wy * gv;
                        gx += (dx ? 1.0f : -1.0f) * wy * gv;
                        gy += wx * (dy ? 1.0f : -1.0f) * gv;
                    }
            }
            grad_attn[s] = ga;
            grad_loc[s] = make_float2(a * Wf * gx, a * Hf * gy);
        }
    }
}

template <typename VT, int M, int L, int K>
hipError_t launch_c256(const Geometry &g, const void *value, const float *loc, const float *attn,
                       const float *go, float *gv, float *gl, float *ga, hipStream_t st)
{
    const uint32_t tiles = (uint32_t)((g.queries() + kWaves - 1) / kWaves);
    const uint32_t grid = round_up8(tiles);
    hipLaunchKernelGGL((backward_c256_kernel<VT, M, L, K>), dim3(grid), dim3(kBlock), 0, st, g,
                       static_cast<const VT *>(value), reinterpret_cast<const float2 *>(loc), attn,
                       reinterpret_cast<const float4 *>(go), gv, reinterpret_cast<float2 *>(gl), ga,
                       grid);
    return hipGetLastError();
}

template <typename VT>
hipError_t launch_typed(const Geometry &g, const void *value, const float *loc, const float *attn,
                        const float *go, float *gv, float *gl, float *ga, hipStream_t st)
{
    const bool c256 = g.M * g.D == 256 &&
                      (reinterpret_cast<uintptr_t>(value) % (4 * sizeof(VT))) == 0 &&
                      (reinterpret_cast<uintptr_t>(go) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(gv) % 16) == 0;
    if (c256 && g.L == 4 && g.K == 4) {
        switch (g.M) {
        case 8: return launch_c256<VT, 8, 4, 4>(g, value, loc, attn, go, gv, gl, ga, st);
        case 4: return launch_c256<VT, 4, 4, 4>(g, value, loc, attn, go, gv, gl, ga, st);
        case 16: return launch_c256<VT, 16, 4, 4>(g, value, loc, attn, go, gv, gl, ga, st);
        default: break;
        }
    }
    if (c256 && g.M == 8) {
        if (g.L == 1 && g.K == 4) return launch_c256<VT, 8, 1, 4>(g, value, loc, attn, go, gv, gl, ga, st);
        if (g.L == 4 && g.K == 8) return launch_c256<VT, 8, 4, 8>(g, value, loc, attn, go, gv, gl, ga, st);
        if (g.L == 3 && g.K == 4) return launch_c256<VT, 8, 3, 4>(g, value, loc, attn, go, gv, gl, ga, st);
        if (g.L == 4 && g.K == 1) return launch_c256<VT, 8, 4, 1>(g, value, loc, attn, go, gv, gl, ga, st);
    }
    const int64_t n = g.queries() * g.M;
    hipLaunchKernelGGL((backward_generic_kernel<VT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       st, g, static_cast<const VT *>(value), reinterpret_cast<const float2 *>(loc),
                       attn, go, gv, reinterpret_cast<float2 *>(gl), ga);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Geometry &g, const void *value, msda_dtype vt, const float *loc,
                           const float *attn, const float *go, float *gv, float *gl, float *ga,
                           hipStream_t st)
{
    if (vt == MSDA_BF16) return launch_typed<uint16_t>(g, value, loc, attn, go, gv, gl, ga, st);
    return launch_typed<float>(g, value, loc, attn, go, gv, gl, ga, st);
}

}  // namespace msda
