// Device-side helpers for the gfx950 kernels of libmsda.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {

constexpr int kWave = 64;

// Buffer resource over [base, base + bytes). Buffer loads whose byte offset is
// at or beyond `bytes` return 0 and buffer atomics there are dropped; the
// kernels use that hardware range check to implement zero padding.
// Word 3 selects 32-bit raw data, as for every CDNA raw buffer access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// An offset that is out of range for every resource the kernels build
// (each covers fewer than 2^31 bytes).
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ float4 load_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Four bf16 values (8 bytes) widened exactly to fp32.
__device__ __forceinline__ float4 load_bf16x4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    const uint32_t lo = u[0], hi = u[1];
    float4 f;
    f.x = __uint_as_float(lo << 16);
    f.y = __uint_as_float(lo & 0xffff0000u);
    f.z = __uint_as_float(hi << 16);
    f.w = __uint_as_float(hi & 0xffff0000u);
    return f;
}

template <typename VT> struct ValueTraits;
template <> struct ValueTraits<float> {
    static constexpr int kBytes = 4;
    __device__ static float4 load4(__amdgpu_buffer_rsrc_t r, uint32_t off) { return load_f32x4(r, off); }
};
template <> struct ValueTraits<uint16_t> {  // bf16 bit patterns
    static constexpr int kBytes = 2;
    __device__ static float4 load4(__amdgpu_buffer_rsrc_t r, uint32_t off) { return load_bf16x4(r, off); }
};

// Four channels of one value row as staged in LDS (fp32: 16 bytes; bf16: 8
// bytes, widened to fp32 when read).
template <typename VT> struct StageChunk;
template <> struct StageChunk<float> {
    using type = float4;
    __device__ static float4 zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ static float4 widen(const float4 &v) { return v; }
};
template <> struct StageChunk<uint16_t> {
    using type = uint2;
    __device__ static uint2 zero() { return make_uint2(0u, 0u); }
    __device__ static float4 widen(const uint2 &v)
    {
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
    }
};

// One axis of a bilinear sample in the align_corners=False convention:
// the continuous pixel coordinate is x = u*n - 0.5; returns the cell start
// c = floor(x) (as float) and the fraction f = x - c in [0, 1].
//
// x is formed with one fma, and then the fraction is re-formed exactly with a
// second fma around the candidate cell (u*n is exact in the fma, and so is
// c + 0.5), so floor(x) is decided on the exact value of u*n - 0.5 — the same
// decision an exact (fp64) evaluation makes — and f carries an absolute error
// below 2^-24 instead of one ulp of x.
__device__ __forceinline__ void cell_1d(float u, float n, float &c, float &f)
{
    const float x = __builtin_fmaf(u, n, -0.5f);
    c = __builtin_floorf(x);
    f = __builtin_fmaf(u, n, -(c + 0.5f));
    const bool below = f < 0.0f;  // x rounded up onto the next integer
    c = below ? c - 1.0f : c;
    f = below ? f + 1.0f : f;
}

// Whether a sample can touch the map at all. Non-finite and far-outside
// locations are rejected here, before any conversion to integer.
__device__ __forceinline__ bool sample_in_range(float u, float v, float Wf, float Hf)
{
    const float x = __builtin_fmaf(u, Wf, -0.5f);
    const float y = __builtin_fmaf(v, Hf, -0.5f);
    return (x > -2.0f) & (x < Wf + 1.0f) & (y > -2.0f) & (y < Hf + 1.0f);
}

// The key padding mask for a sample's four corners: a corner whose value row
// is padded (mask byte nonzero) is treated like an off-map corner (reads zero,
// receives no gradient). `mask_b` is the mask row of the sample's batch,
// `row` the flat value row of the top-left corner, `W` the level width; only
// corners still marked valid are looked up.
__device__ __forceinline__ void unmask_corners(const uint8_t *mask_b, int row, int W, bool &k00, bool &k01,
                                               bool &k10, bool &k11)
{
    if (k00) k00 = mask_b[row] == 0;
    if (k01) k01 = mask_b[row + 1] == 0;
    if (k10) k10 = mask_b[row + W] == 0;
    if (k11) k11 = mask_b[row + W + 1] == 0;
}

// Workgroup barrier that orders LDS accesses only. Unlike __syncthreads it
// does not wait for the wave's outstanding global loads, so loads issued
// before it (a prefetch) stay in flight across it. Use it only where the
// threads exchange data through LDS.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// DPP lane moves (VALU, no LDS traffic): within quads, lanes swapped by
// xor 1 and xor 2; within half-rows of 8, lane i <-> 7-i; within rows of 16,
// lane i <-> 15-i.
template <int CTRL> __device__ __forceinline__ float dpp_move(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
constexpr int kDppQuadXor1 = 0xb1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;      // quad_perm [2,3,0,1]
constexpr int kDppHalfRowMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over the lanes of aligned groups of N lanes (N a power of two <= 64);
// every lane of a group ends with the group's sum. Groups of up to 16 lanes
// use DPP only (after the quad steps every lane of a quad holds the quad sum,
// so a mirror adds the partner quad's sum, and likewise for half-rows).
template <int N> __device__ __forceinline__ float group_sum(float v)
{
    if constexpr (N >= 2) v += dpp_move<kDppQuadXor1>(v);
    if constexpr (N >= 4) v += dpp_move<kDppQuadXor2>(v);
    if constexpr (N >= 8) v += dpp_move<kDppHalfRowMirror>(v);
    if constexpr (N >= 16) v += dpp_move<kDppRowMirror>(v);
#pragma unroll
    for (int o = 16; o < N; o <<= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// The same butterfly for the maximum.
template <int N> __device__ __forceinline__ float group_max(float v)
{
    if constexpr (N >= 2) v = fmaxf(v, dpp_move<kDppQuadXor1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp_move<kDppQuadXor2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp_move<kDppHalfRowMirror>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp_move<kDppRowMirror>(v));
#pragma unroll
    for (int o = 16; o < N; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// data (one wavefront's LDS instructions execute in order).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Map a workgroup id to a logical tile so that each of the 8 XCDs (which
// receive workgroups round-robin and have private L2 caches) processes one
// contiguous range of tiles. `n` is the grid size and must be a multiple of 8
// (the map is then a permutation of [0, n)); tiles at or beyond the real tile
// count are skipped by the caller.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t bid, uint32_t n)
{
    const uint32_t per = n / 8u;
    return (bid % 8u) * per + bid / 8u;
}

__host__ __device__ constexpr uint32_t round_up8(uint32_t n) { return (n + 7u) & ~7u; }

}  // namespace msda
