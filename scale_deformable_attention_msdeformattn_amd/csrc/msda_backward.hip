// Backward of the MSDeformAttn core on gfx950: the exact derivative of the
// forward (the op is trained end to end through autograd: xdnf.cn walkthrough,
// "encoder"; paper notes, "Key code"). Per sample with bilinear weights
// w_c = wx_c * wy_c and corner values v_c (0 off the map):
//   grad_attn        = sum_d G_d * sum_c w_c v_c[d]
//   grad_loc.x       = A * W_l * sum_d G_d * sum_c (d wx_c/d fx) wy_c v_c[d]
//   grad_loc.y       = A * H_l * sum_d G_d * sum_c wx_c (d wy_c/d fy) v_c[d]
//   grad_value[pix]  = sum over the samples with a corner c at pix of A * w_c * G
//
// grad_value is a scatter: every sample adds to four pixels. On gfx950 float
// atomics (global and LDS alike) sustain only a small fraction of the
// required rate, so the fast path turns the scatter into a gather owned by
// pixel tiles (float atomics remain only where the records of one crowded
// tile are split over several workgroups, one add per pixel and channel per
// workgroup):
//
//  0. dense_accum : the dense levels (few pixels, many samples each) skip the
//                   records: workgroups read the samples of a query range
//                   directly and sort their (sample, corner) pairs by pixel in
//                   LDS. It runs on a second stream, beside steps 1 and 2.
//  1. bin_count   : each workgroup takes a fixed range of queries and counts,
//                   in an LDS histogram (integer LDS atomics), how many of its
//                   samples touch each pixel tile of each (head, sparse level);
//                   each non-zero count reserves the workgroup's range inside
//                   the tile's record list with one global atomic add.
//  2. main        : one wavefront per query (as the forward) computes
//                   grad_attn and grad_loc, and writes each sample's index into
//                   the record list of every tile it touches (positions from
//                   an LDS cursor per tile: no global atomics). Each workgroup
//                   first scans its batch's tile totals into the list bases.
//  3. tile_accum  : one workgroup per tile sorts its records by cell in LDS
//                   (with each record's four corner weights and G row offset),
//                   then each lane group takes a cell and sums A*w_c*G into
//                   the slots of the cell's four corner pixels; every pixel
//                   adds its slots and is written once with a plain store.
//                   Every pixel of a sparse level belongs to exactly one tile,
//                   so no zero fill is needed. Extra work items of the same
//                   launch add the dense levels' query splits in a fixed order.
//
// Tiles are sized on the host from the expected sample density so that one
// tile's records fit one LDS chunk; denser tiles take several chunks in turn,
// and the densest (a few pixels with many records) skip the sort and split
// their records over several workgroups whose partials meet in atomics.
// Shapes outside the fast path use one thread per (b, q, m) with float atomics.
#include <algorithm>
#include <mutex>

#include "msda_device.h"
#include "msda_internal.h"

namespace msda {
namespace {

constexpr int kWaves = 4;
constexpr int kBlock = kWaves * kWave;
constexpr int kQueriesPerGroup = 32;     // queries per workgroup of bin_count and main
constexpr int kMinQueryWGs = 256;        // workgroups the per-query path aims at, at least
constexpr int kMainAhead = 2;            // samples whose gathers run ahead in the main kernel
constexpr int kChunk = 512;              // records per LDS chunk in tile_accum
constexpr int kTileTarget = 768;         // expected records per tile the planner aims at
constexpr int kTilePix = 32;             // pixels per tile
constexpr int kTileCells = 2 * kWave;    // cells per tile (the tile plus one row and column of halo)
constexpr int kTaskSlots = 2;            // (cell, split) tasks per lane group in tile_accum
constexpr int kBatch = 4;                // records in flight per task
constexpr int kDirectPix = 4;            // tiles this small skip the per-cell sort
constexpr int kDirectRecords = 768;      // records per workgroup in direct mode
constexpr int kMaxSplit = 64;            // workgroups sharing one direct-mode tile

struct LevelRec {
    float Wf, Hf;
    int32_t W, start;
};

__device__ __forceinline__ float dot4(const float4 &a, const float4 &b)
{
    return __builtin_fmaf(a.w, b.w, __builtin_fmaf(a.z, b.z, __builtin_fmaf(a.y, b.y, a.x * b.x)));
}

// The pixel tiles (of one head and level) that a sample's in-map corners fall
// in: up to four distinct ids, -1 for none, and the sample's cell numbered
// within each of those tiles. (cx, cy) is the sample's cell: its top-left
// corner pixel (-1 when that corner is off the map).
struct SampleTiles {
    int t[4];
    int cell[4];
};

// One level's tiling, staged in LDS: a lane-varying level index into the
// kernel-argument TilePlan would turn into a memory load per lane.
struct TileLevel {
    float iw, ih;     // 1/tw, 1/th
    int32_t ntw, base;
    int32_t tw, th;
};

__device__ __forceinline__ TileLevel tile_level(const TilePlan &tp, int l)
{
    return TileLevel{tp.tinv_w[l], tp.tinv_h[l], tp.ntw[l], tp.tbase[l], tp.tw[l], tp.th[l]};
}

// A tile record: everything tile_accum needs of one (sample, tile) pair, 16 B.
//   x: (b*Nq + q) << kCellBits | the sample's cell within the tile
//   y, z, w: fx, A*(1-fy), A*fy as float bits (the corner weights are
//            (1-fx, fx) times these)
// A tile's cells are its pixels plus one halo row above and one halo column
// to the left, numbered row by row: cell (ry, rx) has its top-left corner at
// tile pixel (ry-1, rx-1).
constexpr int kCellBits = 7;
static_assert(kTileCells <= (1 << kCellBits), "cell numbers fit the record");
// The main kernels carry a record's cell in a key's bits from kKeyBits up
// (keys, the LDS cursor indices, stay below 2^kKeyBits: checked by the plan).
constexpr int kKeyBits = 24;
constexpr int kKeyMask = (1 << kKeyBits) - 1;

__device__ __forceinline__ uint4 tile_record(uint32_t bq, int cell, float fx, float fy, float a)
{
    return make_uint4((bq << kCellBits) | (uint32_t)cell, __float_as_uint(fx), __float_as_uint(a * (1.0f - fy)),
                      __float_as_uint(a * fy));
}

// n / d for 0 <= n < 2^20 and 1 <= d <= 128, given inv_d = 1.0f / d (float
// division, rounded to nearest): floor((n + 0.5) * inv_d) is exact over that
// range (every pair checked on the host in float32), and costs two VALU
// operations and a conversion instead of an integer division.
__device__ __forceinline__ int small_div(int n, float inv_d) { return (int)(((float)n + 0.5f) * inv_d); }

__device__ __forceinline__ SampleTiles sample_tiles(const TileLevel &tl, int W, int H, int cx, int cy)
{
    const int ntw = tl.ntw, base = tl.base;
    const float iw = tl.iw, ih = tl.ih;
    const bool x0 = cx >= 0 && cx < W, x1 = cx + 1 >= 0 && cx + 1 < W;
    const bool y0 = cy >= 0 && cy < H, y1 = cy + 1 >= 0 && cy + 1 < H;
    // c / t for in-map c (0 <= c < W or H < 2^20) by the float reciprocal
    const float fcx = (float)cx + 0.5f, fcy = (float)cy + 0.5f;
    const int tx0 = x0 ? (int)(fcx * iw) : -1, tx1 = x1 ? (int)((fcx + 1.0f) * iw) : -1;
    const int ty0 = y0 ? (int)(fcy * ih) : -1, ty1 = y1 ? (int)((fcy + 1.0f) * ih) : -1;
    // tile rows: ty0, and ty1 when it differs; tile columns likewise. The four
    // combinations are distinct; slot (i, j) is fixed so nothing is indexed
    // dynamically.
    const int r0 = ty0, r1 = ty1 != ty0 ? ty1 : -1;
    const int c0 = tx0, c1 = tx1 != tx0 ? tx1 : -1;
    SampleTiles r;
    // (every product below is of values under 2^20 in magnitude, or unused:
    // 24-bit multiplies, full rate where a 32-bit one is quarter rate)
    r.t[0] = (r0 >= 0 && c0 >= 0) ? base + __mul24(r0, ntw) + c0 : -1;
    r.t[1] = (r0 >= 0 && c1 >= 0) ? base + __mul24(r0, ntw) + c1 : -1;
    r.t[2] = (r1 >= 0 && c0 >= 0) ? base + __mul24(r1, ntw) + c0 : -1;
    r.t[3] = (r1 >= 0 && c1 >= 0) ? base + __mul24(r1, ntw) + c1 : -1;
    // the cell within tile (ty, tx): row cy - ty*th + 1, column cx - tx*tw + 1,
    // in rows of (pixel columns of the tile) + 1 cells
    const int ry0 = cy - __mul24(r0, tl.th) + 1, ry1 = cy - __mul24(r1, tl.th) + 1;
    const int rx0 = cx - __mul24(c0, tl.tw) + 1, rx1 = cx - __mul24(c1, tl.tw) + 1;
    const int cw0 = min(tl.tw, W - __mul24(c0, tl.tw)) + 1, cw1 = min(tl.tw, W - __mul24(c1, tl.tw)) + 1;
    r.cell[0] = __mul24(ry0, cw0) + rx0;
    r.cell[1] = __mul24(ry0, cw1) + rx1;
    r.cell[2] = __mul24(ry1, cw0) + rx0;
    r.cell[3] = __mul24(ry1, cw1) + rx1;
    return r;
}

// Cell (cx, cy) of a sample, or false if no corner can be on the map.
__device__ __forceinline__ bool sample_cell(float2 u, float Wf, float Hf, int &cx, int &cy, float &fx, float &fy)
{
    const bool in = sample_in_range(u.x, u.y, Wf, Hf);
    float cxf, cyf;
    cell_1d(in ? u.x : 0.0f, Wf, cxf, fx);
    cell_1d(in ? u.y : 0.0f, Hf, cyf, fy);
    cx = (int)cxf;
    cy = (int)cyf;
    return in;
}

// ---------------------------------------------------------------- 1. bin_count

constexpr int kBinThreads = 512;
constexpr int kBinBatch = 2;  // (query, level) blocks per bin_count_head thread in flight at once

// Clear the per-tile record totals before bin_count adds into them.
__global__ void __launch_bounds__(kBlock) clear_totals_kernel(int nkeys, uint32_t *__restrict__ totals)
{
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i < nkeys) totals[i] = 0;
}

// Workgroup w takes queries [q0, q1) of batch b. One thread per (query, head,
// sparse level) block of K samples: every sample adds one to the LDS
// histogram entry of each distinct tile its in-map corners fall in. Then
// every non-zero (w, tile) count reserves its range of the tile's record
// list with one global atomic add; the returned offset is stored at
// offsets[w][tile] (entries with a zero count are never read).
template <int M, int L, int K>
__global__ void __launch_bounds__(kBinThreads)
bin_count_kernel(Geometry g, TilePlan tp, const float2 *__restrict__ loc, uint32_t *__restrict__ offsets,
                 uint32_t *__restrict__ totals)
{
    extern __shared__ uint32_t s_hist[];  // [M * tpb]
    __shared__ LevelRec s_lv[L];
    __shared__ TileLevel s_tl[L];
    __shared__ int s_sparse[L];            // the levels that keep records
    const int nkeys = M * tp.tpb;
    for (int i = threadIdx.x; i < nkeys; i += kBinThreads) s_hist[i] = 0;
    if (threadIdx.x < L) {
        const int l = threadIdx.x;
        s_lv[l] = LevelRec{(float)g.lv.W[l], (float)g.lv.H[l], g.lv.W[l], g.lv.start[l]};
        s_tl[l] = tile_level(tp, l);
    }
    int nsl = 0;
#pragma unroll
    for (int l = 0; l < L; ++l)
        if (!((tp.dense_mask >> l) & 1)) {
            if (threadIdx.x == 0) s_sparse[nsl] = l;
            ++nsl;
        }
    __syncthreads();
    const int w = blockIdx.x;
    const int b = w / tp.wpb;
    const int q0 = (w - b * tp.wpb) * tp.qpw;
    const int q1 = min(q0 + tp.qpw, g.Nq);
    const int per_q = M * nsl;
    const int nblk = (q1 - q0) * per_q;
    for (int i = threadIdx.x; i < nblk; i += kBinThreads) {
        const int qi = i / per_q, rem = i - qi * per_q;
        const int m = rem / nsl;
        const int l = s_sparse[rem - m * nsl];
        const LevelRec lv = s_lv[l];
        const int H = (int)lv.Hf;
        const float2 *u = loc + ((((int64_t)b * g.Nq + q0 + qi) * M + m) * L + l) * K;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            int cx, cy;
            float fx, fy;
            if (!sample_cell(u[k], lv.Wf, lv.Hf, cx, cy, fx, fy)) continue;
            const SampleTiles st = sample_tiles(s_tl[l], lv.W, H, cx, cy);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (st.t[j] >= 0) atomicAdd(&s_hist[m * tp.tpb + st.t[j]], 1u);
        }
    }
    __syncthreads();
    uint32_t *row = offsets + (int64_t)w * nkeys;
    uint32_t *tot = totals + (int64_t)b * nkeys;
    // kKeysInFlight atomics per thread are issued before any result is
    // stored, so their round trips overlap instead of running one by one
    constexpr int kKeysInFlight = 8;
    for (int i0 = threadIdx.x; i0 < nkeys; i0 += kBinThreads * kKeysInFlight) {
        uint32_t r[kKeysInFlight];
#pragma unroll
        for (int j = 0; j < kKeysInFlight; ++j) {
            const int i = i0 + j * kBinThreads;
            const uint32_t c = i < nkeys ? s_hist[i] : 0u;
            r[j] = c ? atomicAdd(&tot[i], c) : 0u;
        }
#pragma unroll
        for (int j = 0; j < kKeysInFlight; ++j) {
            const int i = i0 + j * kBinThreads;
            if (i < nkeys && s_hist[i]) row[i] = r[j];
        }
    }
}

// --------------------------------------------------------------------- 2. main

// Waves per workgroup of the main kernel: as many (16, 8 or 4) as fit 56 KB of
// per-wave LDS staging, so that several workgroups share a CU.
template <int M, int L, int K> struct MainWaves {
    static constexpr int kPerWave = 2 * M * (L * K + 1) * 16;
    static constexpr int kBudget = 56 * 1024;
    static constexpr int kValue = kBudget / kPerWave >= 16 ? 16 : kBudget / kPerWave >= 8 ? 8 : 4;
};

// Four waves per SIMD: with the eight-wave workgroups of the usual shapes a
// fifth would not admit another workgroup, and the 128-register budget this
// allows keeps every instantiation free of spills.
//
// FUSED: the gradients go one step further back, to the inputs of the fused
// forward: grad_loc becomes the gradient of the offsets (divided by (W_l, H_l),
// or times ref_wh / (2K) for box references), grad_attn that of the logits
// (through the L*K softmax, across the LK adjacent lanes of one head), and
// grad_ref (if not null) sums grad_loc over heads and points (box references:
// also grad_loc * offset / (2K) for the box size).
template <typename VT, int M, int L, int K, bool FUSED>
__global__ void __launch_bounds__((MainWaves<M, L, K>::kValue * kWave)) __attribute__((amdgpu_waves_per_eu(4, 4)))
backward_c256_kernel(Geometry g, TilePlan tp, const VT *__restrict__ value, const float2 *__restrict__ loc,
                     const float *__restrict__ attn, const float4 *__restrict__ grad_out,
                     float2 *__restrict__ grad_loc, float *__restrict__ grad_attn,
                     const uint32_t *__restrict__ offsets, const uint32_t *__restrict__ totals,
                     uint32_t *__restrict__ bases, uint4 *__restrict__ records, uint32_t grid, FusedGrads fg,
                     const uint8_t *__restrict__ mask)
{
    constexpr int C = 256;
    constexpr int D = C / M;
    constexpr int LPH = D / 4;
    constexpr int LK = L * K;
    constexpr int NS = M * LK;
    constexpr int PAD = LK + 1;  // per-head LDS stride in records (breaks bank aliasing)
    constexpr uint32_t RB = C * sizeof(VT);
    constexpr int MW = MainWaves<M, L, K>::kValue;
    constexpr int NT = MW * kWave;

    extern __shared__ uint32_t s_cursor[];  // [M * tpb + kWave]; then one slot per lane for its idle adds
    __shared__ LevelRec s_lv[L];
    __shared__ TileLevel s_tl[L];
    __shared__ int4 s_off[MW][M * PAD];
    // (fx, fy, A*W_l, A*H_l) per sample; each entry is overwritten in place by its
    // (grad_attn, grad_x, grad_y, -) once the wave has read it (a wave's LDS
    // accesses execute in program order)
    __shared__ float4 s_geo[MW][M * PAD];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t w = xcd_tile(blockIdx.x, grid);
    const bool wg_active = w < (uint32_t)(g.B * tp.wpb);
    const int b = wg_active ? (int)(w / tp.wpb) : 0;
    const int q0 = wg_active ? (int)(w - b * tp.wpb) * tp.qpw : 0;
    const int q1 = wg_active ? min(q0 + tp.qpw, g.Nq) : 0;
    const int nkeys = M * tp.tpb;
    const uint32_t rcap = (uint32_t)g.B * (uint32_t)(g.Nq * M * tp.rslots);  // record slots
    if (threadIdx.x < L) {
        const int l = threadIdx.x;
        s_lv[l] = LevelRec{(float)g.lv.W[l], (float)g.lv.H[l], g.lv.W[l], g.lv.start[l]};
        s_tl[l] = tile_level(tp, l);
    }
    if (wg_active) {
        // The record ranges of batch b's tiles: batch b owns records from
        // b * 4 * (its samples) on (a sample lands in at most 4 tiles), tile i
        // from there plus the exclusive prefix of the tile totals. Every
        // workgroup of the batch scans the totals itself; its first one
        // publishes the bases for tile_accum.
        __shared__ uint32_t s_wsum[MW];
        const uint32_t *tot = totals + (int64_t)b * nkeys;
        for (int i = threadIdx.x; i < nkeys; i += NT) s_cursor[i] = tot[i];
        __syncthreads();
        const int per = (nkeys + NT - 1) / NT;
        const int i0 = min((int)threadIdx.x * per, nkeys), i1 = min(i0 + per, nkeys);
        uint32_t sum = 0;
        for (int i = i0; i < i1; ++i) sum += s_cursor[i];
        uint32_t incl = sum;  // inclusive scan over the wave
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t t = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += t;
        }
        if (lane == kWave - 1) s_wsum[wave] = incl;
        __syncthreads();
        uint32_t run = (uint32_t)b * (uint32_t)(g.Nq * M * tp.rslots) + incl - sum;
        for (int v = 0; v < wave; ++v) run += s_wsum[v];
        for (int i = i0; i < i1; ++i) {
            const uint32_t c = s_cursor[i];
            s_cursor[i] = run;
            run += c;
        }
        __syncthreads();
        const uint32_t *off = offsets + (int64_t)w * nkeys;
        const bool publish = (w % tp.wpb) == 0;
        for (int i = threadIdx.x; i < nkeys; i += NT) {
            const uint32_t base = s_cursor[i];
            if (publish) bases[(int64_t)b * nkeys + i] = base;
            s_cursor[i] = base + off[i];
        }
    }
    __syncthreads();
    if (!wg_active) return;

    const __amdgpu_buffer_rsrc_t vr = make_rsrc(value + (int64_t)b * g.S * C, (uint32_t)g.S * RB);
    const uint32_t vlane = (uint32_t)lane * 4u * sizeof(VT);
    const int m = lane / LPH;

    constexpr int NP = (NS + kWave - 1) / kWave;  // samples per lane and query

    for (int q = q0 + wave; q < q1; q += MW) {
        const int64_t gq = (int64_t)b * g.Nq + q;
        // the lane index, opaque to the compiler within each query: what phase
        // 1 derives from it (sample, level, LDS slots) is recomputed per query
        // instead of being held in registers across the loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        // ---- phase 1: per-sample geometry, one sample per lane per pass ----
        // record keys (head * tiles + tile) of the sparse-level samples, or
        // the lane's idle slot
        int keys[NP][4];
        float rfx[NP], rfy[NP], ra[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int s = p * kWave + ln;
            rfx[p] = rfy[p] = ra[p] = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) keys[p][j] = nkeys + ln;
            if (NS % kWave == 0 || s < NS) {
                const int sm = s / LK;
                const int l = (s / K) % L;
                const int pp = s + s / LK;
                const LevelRec lv = s_lv[l];
                int cx, cy;
                float fx, fy;
                const bool in = sample_cell(loc[gq * NS + s], lv.Wf, lv.Hf, cx, cy, fx, fy);
                const float a = attn[gq * NS + s];
                const int H = (int)lv.Hf;
                const bool x0ok = in & (cx >= 0) & (cx < lv.W);
                const bool x1ok = in & (cx + 1 >= 0) & (cx + 1 < lv.W);
                const bool y0ok = (cy >= 0) & (cy < H);
                const bool y1ok = (cy + 1 >= 0) & (cy + 1 < H);
                const int row = lv.start + __mul24(cy, lv.W) + cx;  // |cy|, W < 2^20
                bool k00 = y0ok & x0ok, k01 = y0ok & x1ok, k10 = y1ok & x0ok, k11 = y1ok & x1ok;
                if (mask) unmask_corners(mask + (int64_t)b * g.S, row, lv.W, k00, k01, k10, k11);
                const uint32_t o00 = (uint32_t)row * RB;
                const uint32_t o10 = o00 + (uint32_t)lv.W * RB;
                int4 o;
                o.x = (int)(k00 ? o00 : kOutOfRange);
                o.y = (int)(k01 ? o00 + RB : kOutOfRange);
                o.z = (int)(k10 ? o10 : kOutOfRange);
                o.w = (int)(k11 ? o10 + RB : kOutOfRange);
                s_off[wave][pp] = o;
                s_geo[wave][pp] = make_float4(fx, fy, a * lv.Wf, a * lv.Hf);
                if (in && !((tp.dense_mask >> l) & 1)) {
                    const SampleTiles st = sample_tiles(s_tl[l], lv.W, H, cx, cy);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (st.t[j] >= 0) keys[p][j] = (sm * tp.tpb + st.t[j]) | (st.cell[j] << kKeyBits);
                    rfx[p] = fx;
                    rfy[p] = fy;
                    ra[p] = a;
                }
            }
        }
        wave_lds_sync();
        // ---- phase 2: gathers, dot products with G, reductions over a head ----
        const float4 G = grad_out[gq * (C / 4) + lane];
        const int4 *offs = &s_off[wave][m * PAD];
        const float4 *geo = &s_geo[wave][m * PAD];
        float4 *res = &s_geo[wave][m * PAD];
        // software-pipelined over the L*K samples: the gathers of the next
        // kMainAhead samples are in flight during each one's arithmetic (the
        // in-place result writes below would otherwise keep the compiler from
        // hoisting them); kMainAhead + 1 register slots, indexed at compile
        // time (the loops are unrolled)
        constexpr int NSLOT = kMainAhead + 1;
        float4 fb[NSLOT], vb[NSLOT][4];
        auto gather = [&](int i, int slot) {
            const int4 o = offs[i];
            fb[slot] = geo[i];
            vb[slot][0] = ValueTraits<VT>::load4(vr, (uint32_t)o.x + vlane);
            vb[slot][1] = ValueTraits<VT>::load4(vr, (uint32_t)o.y + vlane);
            vb[slot][2] = ValueTraits<VT>::load4(vr, (uint32_t)o.z + vlane);
            vb[slot][3] = ValueTraits<VT>::load4(vr, (uint32_t)o.w + vlane);
        };
#pragma unroll
        for (int i = 0; i < kMainAhead; ++i)
            if (i < LK) gather(i, i);
        // the records, after the first gathers (a wait on a load also waits on
        // every store issued before it): a position per key from the LDS
        // cursor, all adds in flight at once
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            uint32_t pos[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) pos[j] = atomicAdd(&s_cursor[keys[p][j] & kKeyMask], 1u);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                // the bound keeps a record write inside the workspace whatever
                // the counts hold
                if ((keys[p][j] & kKeyMask) < nkeys && pos[j] < rcap)
                    records[pos[j]] = tile_record((uint32_t)gq, keys[p][j] >> kKeyBits, rfx[p], rfy[p], ra[p]);
        }
#pragma unroll
        for (int l = 0; l < L; ++l) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int i = l * K + k;
                if (i + kMainAhead < LK) gather(i + kMainAhead, (i + kMainAhead) % NSLOT);
                const int slot = i % NSLOT;
                const float4 f = fb[slot];
                const float4 v00 = vb[slot][0], v01 = vb[slot][1], v10 = vb[slot][2], v11 = vb[slot][3];
                const float d00 = dot4(G, v00), d01 = dot4(G, v01);
                const float d10 = dot4(G, v10), d11 = dot4(G, v11);
                const float fx = f.x, fy = f.y;
                const float hx = 1.0f - fx, hy = 1.0f - fy;
                float ga = hy * (hx * d00 + fx * d01) + fy * (hx * d10 + fx * d11);
                float gx = hy * (d01 - d00) + fy * (d11 - d10);
                float gy = hx * (d10 - d00) + fx * (d11 - d01);
                ga = group_sum<LPH>(ga);
                gx = group_sum<LPH>(gx);
                gy = group_sum<LPH>(gy);
                // every lane of the head holds the sums: all write the same
                // value (no branch, so the loop stays one basic block)
                res[i] = make_float4(ga, f.z * gx, f.w * gy, 0.0f);
            }
        }
        wave_lds_sync();
        // fused: grad_ref sums over the heads and points of each level, kept in
        // the lanes of the pass's first head (lane l*K holds level l)
        float4 ref_acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int s0 = 0; s0 < NS; s0 += kWave) {
            const int s = s0 + ln;
            if (NS % kWave == 0 || s < NS) {
                const float4 r = s_geo[wave][s + s / LK];
                if constexpr (FUSED) {
                    // grad_logit = A * (grad_A - sum over the head's L*K samples of A * grad_A)
                    const float a = attn[gq * NS + s];
                    const float t = group_sum<LK>(a * r.x);
                    const int l = (s / K) % L;
                    grad_attn[gq * NS + s] = a * (r.x - t);
                    if (fg.ref_dims == 4) {
                        const float4 bx = reinterpret_cast<const float4 *>(fg.ref)[gq * L + l];
                        grad_loc[gq * NS + s] = make_float2(r.y * (bx.z * 0.5f / (float)K), r.z * (bx.w * 0.5f / (float)K));
                    } else {
                        const LevelRec lv = s_lv[l];
                        grad_loc[gq * NS + s] = make_float2(r.y / lv.Wf, r.z / lv.Hf);
                    }
                    if (fg.grad_ref) {
                        // (x, y) from grad_loc; for boxes (w, h) from grad_loc * offset / (2K)
                        float4 p = make_float4(r.y, r.z, 0.f, 0.f);
                        if (fg.ref_dims == 4) {
                            const float2 o = fg.off[gq * NS + s];
                            p.z = r.y * o.x * 0.5f / (float)K;
                            p.w = r.z * o.y * 0.5f / (float)K;
                        }
                        // over the K points (adjacent lanes), then over the
                        // heads of this pass (lanes LK apart); levels stay apart
                        p.x = group_sum<K>(p.x);
                        p.y = group_sum<K>(p.y);
                        if (fg.ref_dims == 4) {
                            p.z = group_sum<K>(p.z);
                            p.w = group_sum<K>(p.w);
                        }
                        constexpr int kSpan = NS < kWave ? NS : kWave;  // lanes of one pass
#pragma unroll
                        for (int w = LK; w < kSpan; w <<= 1) {
                            p.x += __shfl_xor(p.x, w, kWave);
                            p.y += __shfl_xor(p.y, w, kWave);
                            if (fg.ref_dims == 4) {
                                p.z += __shfl_xor(p.z, w, kWave);
                                p.w += __shfl_xor(p.w, w, kWave);
                            }
                        }
                        ref_acc.x += p.x;
                        ref_acc.y += p.y;
                        ref_acc.z += p.z;
                        ref_acc.w += p.w;
                    }
                } else {
                    grad_attn[gq * NS + s] = r.x;
                    grad_loc[gq * NS + s] = make_float2(r.y, r.z);
                }
            }
        }
        if constexpr (FUSED) {
            if (fg.grad_ref && lane < LK && lane % K == 0) {
                const int l = lane / K;
                if (fg.ref_dims == 4)
                    reinterpret_cast<float4 *>(fg.grad_ref)[gq * L + l] = ref_acc;
                else
                    reinterpret_cast<float2 *>(fg.grad_ref)[gq * L + l] = make_float2(ref_acc.x, ref_acc.y);
            }
        }
        wave_lds_sync();
    }
}

// ------------------------------------------- 2b. per-head path (8x4x4 shapes)

// The main kernel above serves a query with all its heads, so every corner of
// every level comes through the cache-side gather path. On the shapes the
// forward stages (8 heads, 4 levels, 4 points, many queries) the backward
// takes this path instead: one workgroup per (batch, head, range of queries),
// the head's coarse-level rows staged in LDS as in the forward, QPW queries
// of the head side by side in a wave. Its binning is grouped the same way, so
// each workgroup's record cursors cover the tiles of its own head only.
constexpr int kHeadWaves = 16;
constexpr int kHeadTeam = 4;              // lanes per value row in the per-head kernel's gathers
constexpr int kHeadThreads = kHeadWaves * kWave;
constexpr int kHeadTargetWGs = 512;       // as the forward: two rounds of one workgroup per CU
constexpr int kHeadMinQueries = 1024;     // fewer queries per (batch, head) do not repay the staging
constexpr size_t kHeadLds = 160 * 1024;   // gfx950

// Workgroup (b, m, r) counts, for head m, the samples of queries
// [r * hqpr, (r + 1) * hqpr) on the sparse levels per tile of that head (an
// LDS histogram) and stores the counts as row (b*M + m)*hqr + r of `counts`
// (every tile, zeros included: nothing needs clearing beforehand). The main
// kernel's workgroups sum these rows into their record cursors.
template <int M, int L, int K>
__global__ void __launch_bounds__(kBinThreads)
bin_count_head_kernel(Geometry g, TilePlan tp, const float2 *__restrict__ loc, uint32_t *__restrict__ counts)
{
    extern __shared__ uint32_t s_hist[];  // [tpb]
    __shared__ LevelRec s_lv[L];
    __shared__ TileLevel s_tl[L];
    __shared__ int s_sparse[L];
    const int nkeys = tp.tpb;
    for (int i = threadIdx.x; i < nkeys; i += kBinThreads) s_hist[i] = 0;
    if (threadIdx.x < L) {
        const int l = threadIdx.x;
        s_lv[l] = LevelRec{(float)g.lv.W[l], (float)g.lv.H[l], g.lv.W[l], g.lv.start[l]};
        s_tl[l] = tile_level(tp, l);
    }
    int nsl = 0;
#pragma unroll
    for (int l = 0; l < L; ++l)
        if (!((tp.dense_mask >> l) & 1)) {
            if (threadIdx.x == 0) s_sparse[nsl] = l;
            ++nsl;
        }
    __syncthreads();
    const int w = blockIdx.x;
    const int bm = w / tp.hqr, r = w - (w / tp.hqr) * tp.hqr;
    const int b = bm / M, m = bm - (bm / M) * M;
    const int q0 = r * tp.hqpr, q1 = min(q0 + tp.hqpr, g.Nq);
    const int nblk = (q1 - q0) * nsl;
    // kBinBatch (query, level) blocks per thread at a time, their loads issued
    // together
    for (int i0 = threadIdx.x; i0 < nblk; i0 += kBinThreads * kBinBatch) {
        float2 u[kBinBatch][K];
#pragma unroll
        for (int h = 0; h < kBinBatch; ++h) {
            const int i = min(i0 + h * kBinThreads, nblk - 1);
            const int qi = i / nsl;
            const int l = s_sparse[i - qi * nsl];
            const float2 *src = loc + ((((int64_t)b * g.Nq + q0 + qi) * M + m) * L + l) * K;
#pragma unroll
            for (int k = 0; k < K; ++k) u[h][k] = src[k];
        }
#pragma unroll
        for (int h = 0; h < kBinBatch; ++h) {
            const int i = i0 + h * kBinThreads;
            if (i >= nblk) break;
            const int qi = i / nsl;
            const int l = s_sparse[i - qi * nsl];
            const LevelRec lv = s_lv[l];
            const int H = (int)lv.Hf;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                int cx, cy;
                float fx, fy;
                if (!sample_cell(u[h][k], lv.Wf, lv.Hf, cx, cy, fx, fy)) continue;
                const SampleTiles st = sample_tiles(s_tl[l], lv.W, H, cx, cy);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (st.t[j] >= 0) atomicAdd(&s_hist[st.t[j]], 1u);
            }
        }
    }
    __syncthreads();
    uint32_t *row = counts + (int64_t)w * nkeys;
    for (int i = threadIdx.x; i < nkeys; i += kBinThreads) row[i] = s_hist[i];
}

// The per-head main kernel: grad_attn and grad_loc of head m for a range of
// queries, and the record lists of the sparse levels' tiles. The records of
// head (b, m) fill [(b*M + m) * 4 * Nq * L * K, ...) tile after tile (a sample
// lands in at most four tiles); the workgroup sums its head's count rows into
// tile totals, scans them into its cursors (plus the counts of the head's
// workgroups before it), and the head's first workgroup publishes the totals
// and list bases.
//
// FUSED: the gradients of the fused forward's inputs (as the main kernel's
// fused form): grad_loc becomes the offsets' gradient and grad_attn the
// logits' (the L*K softmax of the head's samples sits in adjacent lanes of
// phase 3). The reference-point gradient sums over heads, which live in other
// workgroups, so each workgroup writes its head's sums over the K points to
// ref_part[b, q, m, l] and ref_grad_sum_kernel adds the heads in order.
template <typename VT, int M, int L, int K, int LS, bool FUSED>
__global__ void __launch_bounds__(kHeadThreads)
backward_head_kernel(Geometry g, TilePlan tp, const VT *__restrict__ value, const float2 *__restrict__ loc,
                     const float *__restrict__ attn, const float4 *__restrict__ grad_out,
                     float2 *__restrict__ grad_loc, float *__restrict__ grad_attn,
                     const uint32_t *__restrict__ counts, uint32_t *__restrict__ totals,
                     uint32_t *__restrict__ bases, uint4 *__restrict__ records, uint32_t stage_bytes,
                     uint32_t grid, const uint8_t *__restrict__ mask, FusedGrads fg, float4 *__restrict__ ref_part)
{
    constexpr int C = 256;
    constexpr int D = C / M;
    constexpr int LPH = D / 4;         // lanes (4 channels each) per query
    constexpr int QPW = kWave / LPH;   // queries side by side in a wave
    constexpr int LK = L * K;
    constexpr int PAD = LK + 1;
    constexpr int NPASS = (QPW * LK + kWave - 1) / kWave;  // samples per lane in phase 1
    constexpr uint32_t RB = C * sizeof(VT);
    static_assert(0 < LS && LS < L, "some levels from memory, some from LDS");
    using Chunk = typename StageChunk<VT>::type;

    extern __shared__ __align__(16) unsigned char s_raw[];
    Chunk *s_stage = reinterpret_cast<Chunk *>(s_raw);                      // [(rows + 1) * LPH]
    uint32_t *s_cursor = reinterpret_cast<uint32_t *>(s_raw + stage_bytes);  // [tpb + kWave]
    uint32_t *s_pre = s_cursor + tp.tpb + kWave;  // [tpb]: counts of the head's workgroups before this one
    __shared__ LevelRec s_lv[L];
    __shared__ float2 s_inv[L];  // (1/W_l, 1/H_l): the offsets' gradient in the fused form
    __shared__ TileLevel s_tl[L];
    __shared__ int4 s_off[kHeadWaves][QPW * PAD];
    // (fx, fy, A*W_l, A*H_l) per sample, overwritten in place by (grad_attn,
    // grad_x, grad_y, -) once the wave has read it
    __shared__ float4 s_geo[kHeadWaves][QPW * PAD];
    __shared__ uint32_t s_wsum[kHeadWaves];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t wg = xcd_tile(blockIdx.x, grid);
    if (wg >= (uint32_t)(g.B * M * tp.hqr)) return;  // whole workgroup: before any barrier
    const int bm = (int)(wg / tp.hqr), r = (int)(wg - (wg / tp.hqr) * tp.hqr);
    const int b = bm / M, m = bm - (bm / M) * M;
    const int q0 = r * tp.hqpr, q1 = min(q0 + tp.hqpr, g.Nq);
    const int nkeys = tp.tpb;
    if (threadIdx.x < L) {
        const int l = threadIdx.x;
        s_lv[l] = LevelRec{(float)g.lv.W[l], (float)g.lv.H[l], g.lv.W[l], g.lv.start[l]};
        s_inv[l] = make_float2(1.0f / (float)g.lv.W[l], 1.0f / (float)g.lv.H[l]);
        s_tl[l] = tile_level(tp, l);
    }
    // head m's rows of the staged levels, then a zero row that off-map
    // corners read; rows at padded positions are staged as zeros
    const int srow0 = g.lv.start[LS];
    const int nrows = g.S - srow0;
    {
        constexpr int kStageBatch = 8;
        const Chunk *src = reinterpret_cast<const Chunk *>(value + ((int64_t)b * g.S + srow0) * C + m * D);
        const int n = nrows * LPH;
        for (int i0 = threadIdx.x; i0 < n; i0 += kHeadThreads * kStageBatch) {
            Chunk v[kStageBatch];
#pragma unroll
            for (int k = 0; k < kStageBatch; ++k) {
                const int i = i0 + k * kHeadThreads;
                const bool keep = i < n && !(mask && mask[(int64_t)b * g.S + srow0 + i / LPH]);
                v[k] = keep ? src[(int64_t)(i / LPH) * (C / 4) + i % LPH] : StageChunk<VT>::zero();
            }
#pragma unroll
            for (int k = 0; k < kStageBatch; ++k) {
                const int i = i0 + k * kHeadThreads;
                if (i < n) s_stage[i] = v[k];
            }
        }
        if (threadIdx.x < LPH) s_stage[nrows * LPH + threadIdx.x] = StageChunk<VT>::zero();
    }
    // the record cursors of head (b, m)'s tiles: region base + exclusive
    // prefix of the tile totals + the counts of the head's workgroups before
    // this one. A tile's total sums the head's hqr count rows; the head's
    // first workgroup publishes the totals and bases for tile_accum.
    const uint32_t *cnt = counts + (int64_t)bm * tp.hqr * nkeys;
    for (int i = threadIdx.x; i < nkeys; i += kHeadThreads) {
        uint32_t t = 0, pre = 0;
        int rr = 0;
        for (; rr + 32 <= tp.hqr; rr += 32) {
            uint32_t c[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) c[k] = cnt[(int64_t)(rr + k) * nkeys + i];
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                pre += rr + k < r ? c[k] : 0u;
                t += c[k];
            }
        }
        for (; rr < tp.hqr; ++rr) {
            const uint32_t c = cnt[(int64_t)rr * nkeys + i];
            pre += rr < r ? c : 0u;
            t += c;
        }
        s_cursor[i] = t;
        s_pre[i] = pre;
        if (r == 0) totals[(int64_t)bm * nkeys + i] = t;
    }
    if (threadIdx.x < kWave) s_cursor[nkeys + threadIdx.x] = 0;  // lanes' idle slots
    __syncthreads();
    {
        const int per = (nkeys + kHeadThreads - 1) / kHeadThreads;
        const int i0 = min((int)threadIdx.x * per, nkeys), i1 = min(i0 + per, nkeys);
        uint32_t sum = 0;
        for (int i = i0; i < i1; ++i) sum += s_cursor[i];
        uint32_t incl = sum;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t t = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += t;
        }
        if (lane == kWave - 1) s_wsum[wave] = incl;
        __syncthreads();
        uint32_t run = (uint32_t)bm * (uint32_t)(g.Nq * tp.rslots) + incl - sum;
        for (int v = 0; v < wave; ++v) run += s_wsum[v];
        for (int i = i0; i < i1; ++i) {
            const uint32_t c = s_cursor[i];
            s_cursor[i] = run;
            run += c;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nkeys; i += kHeadThreads) {
            const uint32_t base = s_cursor[i];
            if (r == 0) bases[(int64_t)bm * nkeys + i] = base;
            s_cursor[i] = base + s_pre[i];
        }
    }
    __syncthreads();

    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(value + (int64_t)b * g.S * C, (uint32_t)g.S * RB);
    const int jq = lane / LPH;
    const int zero_row = nrows * LPH;
    const uint32_t rcap = (uint32_t)g.B * (uint32_t)(g.Nq * M * tp.rslots);  // record slots
    for (int qb = q0 + wave * QPW; qb < q1; qb += kHeadWaves * QPW) {
        // the lane index, opaque to the compiler within each pass (what phase 1
        // derives from it is recomputed per pass, not held across the loop)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        // ---- phase 1: the QPW*L*K samples of this pass, one per lane per step ----
        // Step p takes samples [p*SPS, (p+1)*SPS) of every query of the pass,
        // so that with the levels split evenly over the steps a step's levels
        // are all staged or all from memory, all dense or all sparse, and the
        // branches below are uniform. Record keys (tile, with the sample's
        // cell in that tile in the bits from kKeyBits up) and record weights.
        constexpr int SPS = LK / NPASS;  // samples of a query per step
        static_assert(NPASS * kWave == QPW * LK && LK % NPASS == 0, "whole queries per step");
        int keys[NPASS][4];
        float rfx[NPASS], rfy[NPASS], ra[NPASS];
        float pa[NPASS];  // the samples' A, for phase 3 of the fused form
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            rfx[p] = rfy[p] = ra[p] = pa[p] = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) keys[p][j] = nkeys + ln;
            const int j = ln / SPS;
            {
                const int i = p * SPS + ln % SPS;
                const int l = i / K;
                const bool staged = l >= LS;
                const int q = qb + j;
                int4 o = staged ? make_int4(zero_row, zero_row, zero_row, zero_row)
                                : make_int4((int)kOutOfRange, (int)kOutOfRange, (int)kOutOfRange, (int)kOutOfRange);
                float4 geo = make_float4(0.f, 0.f, 0.f, 0.f);
                if (q < q1) {
                    const int64_t si = (((int64_t)b * g.Nq + q) * M + m) * LK + i;
                    const LevelRec lv = s_lv[l];
                    int cx, cy;
                    float fx, fy;
                    const bool in = sample_cell(loc[si], lv.Wf, lv.Hf, cx, cy, fx, fy);
                    const float a = attn[si];
                    pa[p] = a;
                    const int H = (int)lv.Hf;
                    const bool x0ok = in & (cx >= 0) & (cx < lv.W);
                    const bool x1ok = in & (cx + 1 >= 0) & (cx + 1 < lv.W);
                    const bool y0ok = (cy >= 0) & (cy < H);
                    const bool y1ok = (cy + 1 >= 0) & (cy + 1 < H);
                    const int row = lv.start + __mul24(cy, lv.W) + cx;  // |cy|, W < 2^20
                    bool k00 = y0ok & x0ok, k01 = y0ok & x1ok, k10 = y1ok & x0ok, k11 = y1ok & x1ok;
                    if (staged) {
                        const int r00 = (row - srow0) * LPH, r10 = r00 + lv.W * LPH;
                        o.x = k00 ? r00 : zero_row;
                        o.y = k01 ? r00 + LPH : zero_row;
                        o.z = k10 ? r10 : zero_row;
                        o.w = k11 ? r10 + LPH : zero_row;
                    } else {
                        if (mask) unmask_corners(mask + (int64_t)b * g.S, row, lv.W, k00, k01, k10, k11);
                        const uint32_t o00 = (uint32_t)row * RB, o10 = o00 + (uint32_t)lv.W * RB;
                        o.x = (int)(k00 ? o00 : kOutOfRange);
                        o.y = (int)(k01 ? o00 + RB : kOutOfRange);
                        o.z = (int)(k10 ? o10 : kOutOfRange);
                        o.w = (int)(k11 ? o10 + RB : kOutOfRange);
                    }
                    geo = make_float4(fx, fy, a * lv.Wf, a * lv.Hf);
                    if (in && !((tp.dense_mask >> l) & 1)) {
                        const SampleTiles st = sample_tiles(s_tl[l], lv.W, H, cx, cy);
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            if (st.t[jj] >= 0) keys[p][jj] = st.t[jj] | (st.cell[jj] << kKeyBits);
                        rfx[p] = fx;
                        rfy[p] = fy;
                        ra[p] = a;
                    }
                }
                s_off[wave][j * PAD + i] = o;
                s_geo[wave][j * PAD + i] = geo;
            }
            // the step's records: a position per key from the LDS cursor (all
            // adds in flight at once; a lane without a record adds on a spare
            // slot of its own), unless no lane of the wave has one
            bool has = false;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) has |= (keys[p][jj] & kKeyMask) < nkeys;
            if (__any(has)) {
                const uint32_t bq = (uint32_t)(b * g.Nq + qb + j);
                uint32_t pos[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) pos[jj] = atomicAdd(&s_cursor[keys[p][jj] & kKeyMask], 1u);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if ((keys[p][jj] & kKeyMask) < nkeys && pos[jj] < rcap)
                        records[pos[jj]] = tile_record(bq, keys[p][jj] >> kKeyBits, rfx[p], rfy[p], ra[p]);
            }
        }
        wave_lds_sync();
        // ---- phase 2: a query's samples split over teams of its lanes ----
        // The query's LPH lanes form NT teams of TEAM lanes; a team takes K/NT
        // of each level's samples, and each of its lanes CPL = NT chunks (4
        // channels each) of the row: gathers, dots with G over the lane's
        // channels, sums over the team's lanes (fewer cross-lane sums and
        // per-sample arithmetic per lane than one sample per whole query).
        constexpr int TEAM = kHeadTeam;
        constexpr int NT = LPH / TEAM;   // teams per query
        constexpr int CPL = LPH / TEAM;  // row chunks per lane
        constexpr int KT = K / NT;       // samples of a level per team
        static_assert(LPH % TEAM == 0 && K % NT == 0, "teams divide the row and the points");
        const int lq = lane - (lane / LPH) * LPH;
        const int team = lq / TEAM, tl = lq - (lq / TEAM) * TEAM;
        const int qg = qb + jq;
        float4 G[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k)
            G[k] = qg < q1 ? grad_out[((int64_t)b * g.Nq + qg) * (C / 4) + m * LPH + tl * CPL + k]
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        const uint32_t team_off = (uint32_t)(m * D + tl * CPL * 4) * sizeof(VT);
        const int4 *offs = &s_off[wave][jq * PAD];
        const float4 *geo = &s_geo[wave][jq * PAD];
        float4 *res = &s_geo[wave][jq * PAD];
        auto grad_sample = [&](int i, const float4 (&vv)[4][CPL]) {
            const float4 f = geo[i];
            float d[4];
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                d[cn] = dot4(G[0], vv[cn][0]);
#pragma unroll
                for (int k = 1; k < CPL; ++k) d[cn] += dot4(G[k], vv[cn][k]);
            }
            const float fx = f.x, fy = f.y;
            const float hx = 1.0f - fx, hy = 1.0f - fy;
            float ga = hy * (hx * d[0] + fx * d[1]) + fy * (hx * d[2] + fx * d[3]);
            float gx = hy * (d[1] - d[0]) + fy * (d[3] - d[2]);
            float gy = hx * (d[2] - d[0]) + fx * (d[3] - d[1]);
            ga = group_sum<TEAM>(ga);
            gx = group_sum<TEAM>(gx);
            gy = group_sum<TEAM>(gy);
            res[i] = make_float4(ga, f.z * gx, f.w * gy, 0.0f);  // the team's lanes all write the same
        };
        auto staged_sample = [&](int i) {
            const int4 o = offs[i];
            const int oc[4] = {o.x, o.y, o.z, o.w};
            float4 vv[4][CPL];
#pragma unroll
            for (int cn = 0; cn < 4; ++cn)
#pragma unroll
                for (int k = 0; k < CPL; ++k) vv[cn][k] = StageChunk<VT>::widen(s_stage[oc[cn] + tl * CPL + k]);
            grad_sample(i, vv);
        };
        // level by level: a memory level's gathers are issued, a staged level
        // is done from LDS while they are in flight, then the memory level
#pragma unroll
        for (int l = 0; l < LS; ++l) {
            float4 v[KT][4][CPL];
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) {
                const int4 o = offs[l * K + team * KT + kk];
                const uint32_t oc[4] = {(uint32_t)o.x, (uint32_t)o.y, (uint32_t)o.z, (uint32_t)o.w};
#pragma unroll
                for (int cn = 0; cn < 4; ++cn)
#pragma unroll
                    for (int k = 0; k < CPL; ++k)
                        v[kk][cn][k] = ValueTraits<VT>::load4(rsrc, oc[cn] + team_off + (uint32_t)(k * 4 * sizeof(VT)));
            }
            if (LS + l < L) {
#pragma unroll
                for (int kk = 0; kk < KT; ++kk) staged_sample((LS + l) * K + team * KT + kk);
            }
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) grad_sample(l * K + team * KT + kk, v[kk]);
        }
#pragma unroll
        for (int l = 2 * LS; l < L; ++l)  // staged levels left over
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) staged_sample(l * K + team * KT + kk);
        wave_lds_sync();
        // ---- phase 3: the pass's results ----
        // Each lane takes back its phase-1 samples (step p: sample p*SPS +
        // ln % SPS of query ln / SPS), so the fused form has their A in
        // registers; a query's sum over its L*K samples is the lane's own
        // sum over the steps, then over the query's SPS lanes, and a level's
        // K points sit in K adjacent lanes of a step.
        static_assert((SPS & (SPS - 1)) == 0 && SPS % K == 0, "a query's lanes and a level's points in aligned groups");
        {
            const int j = ln / SPS;
            const int q = qb + j;
            const bool valid = q < q1;  // the same for the SPS lanes of a query
            float4 rr[NPASS];
#pragma unroll
            for (int p = 0; p < NPASS; ++p) rr[p] = s_geo[wave][j * PAD + p * SPS + ln % SPS];
            if constexpr (FUSED) {
                float ts = 0.0f;
#pragma unroll
                for (int p = 0; p < NPASS; ++p) ts += pa[p] * rr[p].x;
                const float tsum = group_sum<SPS>(ts);
#pragma unroll
                for (int p = 0; p < NPASS; ++p) {
                    const int i = p * SPS + ln % SPS;
                    const int l = i / K, k = i - (i / K) * K;
                    const int64_t si = (((int64_t)b * g.Nq + q) * M + m) * LK + i;
                    float4 bx = make_float4(0.f, 0.f, 0.f, 0.f);
                    float2 o = make_float2(0.f, 0.f);
                    if (fg.ref_dims == 4 && valid) {
                        bx = reinterpret_cast<const float4 *>(fg.ref)[((int64_t)b * g.Nq + q) * L + l];
                        o = fg.off[si];
                    }
                    if (valid) {
                        grad_attn[si] = pa[p] * (rr[p].x - tsum);
                        const float2 inv = s_inv[l];
                        grad_loc[si] = fg.ref_dims == 4 ? make_float2(rr[p].y * (bx.z * 0.5f / (float)K),
                                                                      rr[p].z * (bx.w * 0.5f / (float)K))
                                                        : make_float2(rr[p].y * inv.x, rr[p].z * inv.y);
                    }
                    if (fg.grad_ref) {
                        // (x, y) from grad_loc; for boxes (w, h) from grad_loc * offset / (2K); summed
                        // over the K points of the level (adjacent lanes)
                        float4 pr = make_float4(rr[p].y, rr[p].z, 0.f, 0.f);
                        if (fg.ref_dims == 4) {
                            pr.z = rr[p].y * o.x * 0.5f / (float)K;
                            pr.w = rr[p].z * o.y * 0.5f / (float)K;
                        }
                        pr.x = group_sum<K>(pr.x);
                        pr.y = group_sum<K>(pr.y);
                        pr.z = group_sum<K>(pr.z);
                        pr.w = group_sum<K>(pr.w);
                        if (valid && k == 0) ref_part[(((int64_t)b * g.Nq + q) * M + m) * L + l] = pr;
                    }
                }
            } else if (valid) {
#pragma unroll
                for (int p = 0; p < NPASS; ++p) {
                    const int i = p * SPS + ln % SPS;
                    const int64_t si = (((int64_t)b * g.Nq + q) * M + m) * LK + i;
                    grad_attn[si] = rr[p].x;
                    grad_loc[si] = make_float2(rr[p].y, rr[p].z);
                }
            }
        }
        wave_lds_sync();  // the next pass rewrites this wave's records
    }
}

// grad_ref[b, q, l] = the sum over heads m of ref_part[b, q, m, l] (heads in
// order), one thread per (b, q, l).
template <int M, int L>
__global__ void __launch_bounds__(256)
ref_grad_sum_kernel(Geometry g, const float4 *__restrict__ ref_part, FusedGrads fg)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= g.queries() * L) return;
    const int64_t bq = t / L;
    const int l = (int)(t - bq * L);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float4 v = ref_part[(bq * M + m) * L + l];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    if (fg.ref_dims == 4)
        reinterpret_cast<float4 *>(fg.grad_ref)[t] = s;
    else
        reinterpret_cast<float2 *>(fg.grad_ref)[t] = make_float2(s.x, s.y);
}

// --------------------------------------------------------------- 3. tile_accum

// defined with the dense levels below; tile_accum runs it for its extra items
// One workgroup per tile (b, m, level, tile). Its records are counting-sorted
// by cell in LDS; then each lane group (LG lanes, 4 channels each, D = 4*LG)
// takes (cell, split) tasks: it walks the cell's records (every S-th one for
// split s), loads each record's G row once and accumulates A*w_c*G into four
// corner accumulators, kBatch records at a time so that many loads are in
// flight. The corner sums go to single-writer LDS slots (pixel, corner role,
// split); finally every pixel adds its slots and is written once. The
// compiled (M, L, K) make the sample-index division and the level lookups
// compile-time.
template <int M, int L, int K>
__global__ void __launch_bounds__(kBlock)
tile_accum_kernel(Geometry g, TilePlan tp, const float4 *__restrict__ grad_out, float4 *__restrict__ grad_value,
                  const uint4 *__restrict__ records, const uint32_t *__restrict__ bases,
                  const uint32_t *__restrict__ totals, int accumulate, const uint8_t *__restrict__ mask)
{
    constexpr int LG = 256 / M / 4;  // lanes (4 channels each) per head row
    constexpr int NG = kBlock / LG;
    // (pixel, role, split) slots in use: npix*4 when cells >= NG, else at most 4*NG
    constexpr int kPartSlots0 = 4 * (kTilePix > NG ? kTilePix : NG);
    constexpr int kPartSlots = kPartSlots0 > kDirectPix * NG ? kPartSlots0 : kDirectPix * NG;
    __shared__ uint32_t s_start[kTileCells + 1];
    __shared__ uint32_t s_cur[kTileCells];
    // a chunk's records sorted by cell: the four corner weights A*w_c, and
    // the byte offset of the query's grad_output row
    __shared__ float4 s_w[kChunk];
    __shared__ uint32_t s_q[kChunk];
    __shared__ float4 s_part[kPartSlots][LG];

    // work item (b, m, level, tile, chunk); consecutive items (same batch and
    // head, neighbouring tiles) read G rows of neighbouring queries, so each
    // XCD (private L2) gets a contiguous item range
    const int item = (int)xcd_tile(blockIdx.x, gridDim.x);
    if (item >= g.B * g.M * tp.ipb) return;
    const int bm = item / tp.ipb;
    const int b = bm / M, m = bm - (bm / M) * M;
    const int r_in = item - bm * tp.ipb;
    int l = 0;
#pragma unroll
    for (int i = 1; i < L; ++i)
        if (r_in >= tp.ibase[i]) l = i;
    int th = 1, tw = 1, ntw = 1, tb = 0, nch = 1, ib = 0, W = 1, H = 1, lstart = 0;
#pragma unroll
    for (int i = 0; i < L; ++i)
        if (i == l) {
            th = tp.th[i];
            tw = tp.tw[i];
            ntw = tp.ntw[i];
            tb = tp.tbase[i];
            nch = tp.nchunk[i];
            ib = tp.ibase[i];
            W = g.lv.W[i];
            H = g.lv.H[i];
            lstart = g.lv.start[i];
        }
    const int t_in = (r_in - ib) / nch;
    const int chunk = r_in - ib - t_in * nch;
    const int key = bm * tp.tpb + tb + t_in;
    const int ty = t_in / ntw, tx = t_in - ty * ntw;
    const int r0 = ty * th, r1 = min(r0 + th, H);
    const int c0 = tx * tw, c1 = min(c0 + tw, W);
    const int pw = c1 - c0, ph = r1 - r0;   // pixels of this tile
    const int cw = pw + 1;                  // cell columns c0-1 .. c1-1
    const int ncells = (ph + 1) * cw;       // cell rows r0-1 .. r1-1
    const int npix = ph * pw;
    const int S = ncells >= NG ? 1 : NG / ncells;   // lane groups per cell
    const int ntask = ncells * S;
    // divisors of the task and pixel numbering (S <= NG, cw and pw <= kTilePix + 1)
    const float inv_s = 1.0f / (float)S, inv_cw = 1.0f / (float)cw, inv_pw = 1.0f / (float)pw;
    const uint32_t nqueries = (uint32_t)g.queries();
    const int grp = threadIdx.x / LG;
    const int lig = threadIdx.x % LG;
    // grad_output rows through a buffer resource: 32-bit offsets, and an
    // out-of-range offset reads zeros (the host keeps grad_output < 2 GB)
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(grad_out, (uint32_t)((uint64_t)g.queries() * g.M * LG * 16));
    const uint32_t grow_bytes = (uint32_t)g.M * LG * 16;  // one query's row, all heads
    const uint32_t gbase = ((uint32_t)m * LG + lig) * 16;
    uint32_t rbeg = bases[key];
    uint32_t rtot = totals[key];
    {
        // keep the range inside the record array whatever the workspace holds
        const uint32_t rcap = (uint32_t)g.B * (uint32_t)(g.Nq * M * tp.rslots);
        rtot = rbeg < rcap ? min(rtot, rcap - rbeg) : 0u;
    }

    if (npix <= kDirectPix) {
        if (nch > 1) {  // this workgroup's share of the tile's records
            const uint32_t per = (rtot + nch - 1) / nch;
            const uint32_t lo = min(rtot, per * chunk);
            rbeg += lo;
            rtot = min(rtot - lo, per);
        }
        // Direct mode for small (dense) tiles: no sort. Lane groups stride over
        // the records, kBatch at a time, and keep one accumulator per pixel of
        // the tile; a record adds A*w to each pixel it is a corner of.
        float4 acc[kDirectPix];
#pragma unroll
        for (int p = 0; p < kDirectPix; ++p) acc[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (uint32_t i0 = grp; i0 < rtot; i0 += NG * kBatch) {
            uint4 rec[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const uint32_t i = i0 + j * NG;
                rec[j] = i < rtot ? records[rbeg + i] : make_uint4(nqueries << kCellBits, 0u, 0u, 0u);
            }
            float4 gv[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const uint32_t bq = rec[j].x >> kCellBits;
                const bool ok = bq < nqueries;  // see the chunked path below
                gv[j] = ok ? grad_out[((int64_t)bq * g.M + m) * LG + lig] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                // the record's cell (ry, rx) has its top-left corner at tile pixel (ry - 1, rx - 1)
                const int cell = (int)(rec[j].x & ((1u << kCellBits) - 1));
                const int ry = small_div(cell, inv_cw), rx = cell - ry * cw;
                const bool in = (rec[j].x >> kCellBits) < nqueries;
                const float fx = __uint_as_float(rec[j].y);
                const float ay0 = __uint_as_float(rec[j].z), ay1 = __uint_as_float(rec[j].w);
#pragma unroll
                for (int p = 0; p < kDirectPix; ++p) {
                    // pixel (py, px) of the tile is corner (dx, dy) of the cell
                    const int py = p / pw, px = p % pw;
                    const int dx = px - (rx - 1), dy = py - (ry - 1);
                    const bool hit = in && p < npix && (dx == 0 || dx == 1) && (dy == 0 || dy == 1);
                    const float w = hit ? (dy ? ay1 : ay0) * (dx ? fx : 1.0f - fx) : 0.0f;
                    acc[p].x = __builtin_fmaf(w, gv[j].x, acc[p].x);
                    acc[p].y = __builtin_fmaf(w, gv[j].y, acc[p].y);
                    acc[p].z = __builtin_fmaf(w, gv[j].z, acc[p].z);
                    acc[p].w = __builtin_fmaf(w, gv[j].w, acc[p].w);
                }
            }
        }
        // reduce over the lane groups: slots [group * kDirectPix + p]
#pragma unroll
        for (int p = 0; p < kDirectPix; ++p) s_part[grp * kDirectPix + p][lig] = acc[p];
        lds_barrier();
        if (grp < npix) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int q = 0; q < NG; ++q) {
                const float4 t = s_part[q * kDirectPix + grp][lig];
                v.x += t.x;
                v.y += t.y;
                v.z += t.z;
                v.w += t.w;
            }
            const int py = r0 + grp / pw, px = c0 + grp % pw;
            const int64_t pix = (int64_t)b * g.S + lstart + (int64_t)py * W + px;
            if (mask && mask[pix]) v = make_float4(0.f, 0.f, 0.f, 0.f);  // padded: no gradient
            float4 *dst = grad_value + (pix * g.M + m) * LG + lig;
            if (nch > 1) {
                // several workgroups share this tile: add the partial into the
                // row (zeroed beforehand unless accumulating)
                float *d = reinterpret_cast<float *>(dst);
                atomicAdd(d + 0, v.x);
                atomicAdd(d + 1, v.y);
                atomicAdd(d + 2, v.z);
                atomicAdd(d + 3, v.w);
            } else {
                if (accumulate) {
                    const float4 o = *dst;
                    v.x += o.x;
                    v.y += o.y;
                    v.z += o.z;
                    v.w += o.w;
                }
                *dst = v;
            }
        }
        return;
    }

    for (int i = threadIdx.x; i < npix * 4 * S * LG; i += kBlock)
        s_part[i / LG][i % LG] = make_float4(0.f, 0.f, 0.f, 0.f);

    for (uint32_t c0r = 0; c0r < rtot; c0r += kChunk) {
        const int n = (int)min((uint32_t)kChunk, rtot - c0r);
        for (int i = threadIdx.x; i < ncells; i += kBlock) s_cur[i] = 0;
        lds_barrier();
        // this chunk's records: cell, corner weights and G row offset, kept
        // in registers (kChunk / kBlock per thread, loads all in flight)
        // until their sorted slots are known; count per cell
        constexpr int RPT = kChunk / kBlock;
        static_assert(kChunk % kBlock == 0, "a chunk is whole records per thread");
        float4 rw[RPT];
        uint32_t rq[RPT];
        int rc[RPT];
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const int i = threadIdx.x + k * kBlock;
            const uint4 rec = i < n ? records[rbeg + c0r + i] : make_uint4(nqueries << kCellBits, 0u, 0u, 0u);
            // the checks only keep a corrupt record from addressing outside
            // grad_output or the cell table
            const uint32_t bq = rec.x >> kCellBits;
            const int cell = (int)(rec.x & ((1u << kCellBits) - 1));
            const float fx = __uint_as_float(rec.y);
            const float ay0 = __uint_as_float(rec.z), ay1 = __uint_as_float(rec.w);
            rw[k] = make_float4(ay0 * (1.0f - fx), ay0 * fx, ay1 * (1.0f - fx), ay1 * fx);
            rq[k] = bq * grow_bytes;
            rc[k] = (bq < nqueries && cell < ncells) ? cell : -1;
        }
#pragma unroll
        for (int k = 0; k < RPT; ++k)
            if (rc[k] >= 0) atomicAdd(&s_cur[rc[k]], 1u);
        lds_barrier();
        // exclusive scan of the (at most kTileCells = 2 * kWave) cell counts, one wave
        if (threadIdx.x < kWave) {
            const int i0 = 2 * threadIdx.x;
            const uint32_t a = i0 < ncells ? s_cur[i0] : 0u;
            const uint32_t c = i0 + 1 < ncells ? s_cur[i0 + 1] : 0u;
            uint32_t incl = a + c;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const uint32_t t = __shfl_up(incl, o, kWave);
                if ((int)threadIdx.x >= o) incl += t;
            }
            const uint32_t ex = incl - a - c;
            if (i0 < ncells) s_start[i0] = s_cur[i0] = ex;
            if (i0 + 1 < ncells) s_start[i0 + 1] = s_cur[i0 + 1] = ex + a;
            if (threadIdx.x == kWave - 1) s_start[ncells] = incl;
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < RPT; ++k)
            if (rc[k] >= 0) {
                const uint32_t pos = atomicAdd(&s_cur[rc[k]], 1u);
                s_w[pos] = rw[k];
                s_q[pos] = rq[k];
            }
        lds_barrier();
        // (cell, split) tasks; each adds its four corner sums into its own
        // (pixel, role, split) slots, which no other task touches
        for (int t = 0; t < kTaskSlots; ++t) {
            const int task = grp + t * NG;
            if (task >= ntask) break;
            const int cell = small_div(task, inv_s), split = task - cell * S;
            float4 acc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);
            const uint32_t e_end = s_start[cell + 1];
            for (uint32_t e0 = s_start[cell] + split; e0 < e_end; e0 += S * kBatch) {
                // branch-free batch: entries past the cell's end re-read its
                // last entry and load a zero G row (out-of-range offset)
                float4 w[kBatch], gv[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const uint32_t e = min(e0 + j * S, e_end - 1);
                    w[j] = s_w[e];
                    const uint32_t off = s_q[e] + gbase;
                    gv[j] = load_f32x4(grs, e0 + j * S < e_end ? off : kOutOfRange);
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const float wr[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        acc[r].x = __builtin_fmaf(wr[r], gv[j].x, acc[r].x);
                        acc[r].y = __builtin_fmaf(wr[r], gv[j].y, acc[r].y);
                        acc[r].z = __builtin_fmaf(wr[r], gv[j].z, acc[r].z);
                        acc[r].w = __builtin_fmaf(wr[r], gv[j].w, acc[r].w);
                    }
                }
            }
            // role r: 0 top-left, 1 top-right, 2 bottom-left, 3 bottom-right
            // corner of the cell; cell (ry, rx) (relative, halo row/column at
            // 0) has its top-left corner at tile pixel (ry-1, rx-1)
            const int ry = small_div(cell, inv_cw), rx = cell - ry * cw;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int py = ry - 1 + (r >> 1), px = rx - 1 + (r & 1);
                if (py >= 0 && py < ph && px >= 0 && px < pw) {
                    float4 &slot = s_part[((py * pw + px) * 4 + r) * S + split][lig];
                    const float4 o = slot;
                    slot = make_float4(o.x + acc[r].x, o.y + acc[r].y, o.z + acc[r].z, o.w + acc[r].w);
                }
            }
        }
        lds_barrier();  // LDS is reused by the next chunk
    }
    if (rtot == 0) lds_barrier();  // orders the zeroing of s_part before the sums below
    for (int pix = grp; pix < npix; pix += NG) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int i = 0; i < 4 * S; ++i) {
            const float4 t = s_part[pix * 4 * S + i][lig];
            v.x += t.x;
            v.y += t.y;
            v.z += t.z;
            v.w += t.w;
        }
        const int pr = small_div(pix, inv_pw);
        const int py = r0 + pr, px = c0 + (pix - pr * pw);
        const int64_t row = (int64_t)b * g.S + lstart + (int64_t)py * W + px;
        if (mask && mask[row]) v = make_float4(0.f, 0.f, 0.f, 0.f);  // padded: no gradient
        float4 *dst = grad_value + (row * g.M + m) * LG + lig;
        if (accumulate) {
            const float4 o = *dst;
            v.x += o.x;
            v.y += o.y;
            v.z += o.z;
            v.w += o.w;
        }
        *dst = v;
    }
}

// Zero the grad_value rows of the sparse levels whose split tiles add their
// partial sums with atomics. One thread per float4.
__global__ void __launch_bounds__(kBlock)
zero_split_levels_kernel(Geometry g, TilePlan tp, float4 *__restrict__ grad_value)
{
    const int64_t row4 = (int64_t)g.M * g.D / 4;  // float4s per value row
    int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    for (int l = 0; l < g.L; ++l) {
        if (!level_uses_atomics(tp, l)) continue;
        const int64_t n = (int64_t)g.lv.H[l] * g.lv.W[l] * row4;
        if (t < (int64_t)g.B * n) {
            const int64_t b = t / n, r = t - b * n;
            grad_value[((int64_t)b * g.S + g.lv.start[l]) * row4 + r] = make_float4(0.f, 0.f, 0.f, 0.f);
            return;
        }
        t -= (int64_t)g.B * n;
    }
}

// ------------------------------------------------------------- 4. dense_accum

// Dense levels: many samples per pixel, few pixels. Binning them into tiles
// would write each sample's record up to four times; instead one workgroup
// per (b, m, pixel part, query split) reads its queries' samples of every
// dense level directly (adjacent in memory per query when the dense levels
// are adjacent, as the coarsest ones are) together with their grad_output
// rows, and, sub-chunk after sub-chunk:
//  - ranks each (sample, corner) pair whose pixel lies in its part within
//    the pixel's LDS count (integer LDS atomics); the pixels of all dense
//    levels are numbered one after the other (TilePlan::dbase),
//  - scans the counts and writes every pair's weight A*w_c and query slot,
//    sorted by pixel,
//  - lets each lane group sum weight * G over the pairs of the pixels it
//    owns, in registers.
// The next sub-chunk's loads are issued before the current one is sorted and
// stay in flight across the LDS-only barriers. With several query splits each
// item parks its sums in the workspace and dense_reduce_kernel adds them up in
// split order, writing every pixel once.
constexpr int kDensePix = 640;             // pixels per part at most
constexpr int kDenseSub = 1024;            // samples per sub-chunk at most
constexpr int kDenseQ = 128;               // queries per sub-chunk at most
constexpr int kDenseBatch = 4;             // pairs in flight per lane group
constexpr int kDenseThreads = 512;         // threads per dense workgroup
constexpr double kDenseMinPerPix = 24.0;   // samples per pixel (per batch and head) that make a level dense
constexpr int kDenseMaxPix = 2048;         // pixels of a dense level at most
constexpr double kDenseItemSamples = 3072; // samples per dense work item (sets the query splits)
constexpr int kDenseMaxSplit = 64;

template <int M, int L, int K>
__global__ void __launch_bounds__(kDenseThreads)
dense_accum_kernel(Geometry g, TilePlan tp, const float2 *__restrict__ loc, const float *__restrict__ attn,
                   const float4 *__restrict__ grad_out, float4 *__restrict__ grad_value,
                   float4 *__restrict__ partials, int accumulate, const uint8_t *__restrict__ mask)
{
    constexpr int LG = 256 / M / 4;                         // lanes (4 channels each) per head row
    constexpr int NG = kDenseThreads / LG;                  // lane groups
    constexpr int PPG = (kDensePix + NG - 1) / NG;          // pixel slots per lane group
    constexpr int kPer = kDenseSub / kDenseThreads;         // samples per thread per sub-chunk
    constexpr int kGRows = (kDenseQ * LG + kDenseThreads - 1) / kDenseThreads;  // float4 of G staged per thread
    static_assert(kDenseSub % kDenseThreads == 0 && kDensePix % kWave == 0, "dense tiling");
    __shared__ float4 s_g[kDenseQ * LG];       // G rows of the sub-chunk's queries
    __shared__ uint2 s_pair[4 * kDenseSub];    // (bits(A * w_c), query slot), sorted by pixel
    __shared__ uint32_t s_cnt[kDensePix];
    __shared__ uint32_t s_start[kDensePix + 1];
    __shared__ LevelRec s_lv[L];               // the dense levels, in order
    __shared__ int s_dbase[L];                 // their first pixel in the dense numbering

    const int item = (int)xcd_tile(blockIdx.x, gridDim.x);
    if (item >= g.B * g.M * tp.dipb) return;
    const int bm = item / tp.dipb;
    const int b = bm / M, m = bm - (bm / M) * M;
    const int r_in = item - bm * tp.dipb;
    const int part = r_in / tp.dsplits, split = r_in - (r_in / tp.dsplits) * tp.dsplits;
    const int ndl = tp.ndl;
    if (threadIdx.x == 0) {
        int j = 0;
        for (int l = 0; l < L; ++l)
            if ((tp.dense_mask >> l) & 1) {
                s_lv[j] = LevelRec{(float)g.lv.W[l], (float)g.lv.H[l], g.lv.W[l], g.lv.start[l]};
                s_dbase[j] = tp.dbase[l];
                ++j;
            }
    }
    // this part's pixels of the dense numbering, this split's queries
    const int p0 = (int)((int64_t)tp.ndpix * part / tp.dparts);
    const int npix = (int)((int64_t)tp.ndpix * (part + 1) / tp.dparts) - p0;
    const int qa0 = (int)((int64_t)g.Nq * split / tp.dsplits);
    const int qa1 = (int)((int64_t)g.Nq * (split + 1) / tp.dsplits);
    const int spq = ndl * K;                   // dense samples per query
    const int QS = min(kDenseQ, kDenseSub / spq);  // queries per sub-chunk
    const float inv_spq = 1.0f / (float)spq;       // spq <= L*K <= 128, sample numbers < kDenseSub
    constexpr int64_t LKs = (int64_t)L * K;
    const int grp = threadIdx.x / LG;
    const int lig = threadIdx.x % LG;

    for (int i = threadIdx.x; i < kDensePix; i += kDenseThreads) s_cnt[i] = 0;
    __syncthreads();  // s_lv, s_dbase

    // loads of one sub-chunk (starting at query qa), held in registers; the
    // dense levels' samples of a query are taken in level order, then point
    // order, with the dense levels' first index `lfirst` (dense levels are
    // adjacent: checked by the plan)
    int lfirst = 0;
    for (int l = 0; l < L; ++l)
        if ((tp.dense_mask >> l) & 1) {
            lfirst = l;
            break;
        }
    float2 u[kPer];
    float a[kPer];
    float4 gst[kGRows];
    auto fetch_samples = [&](int qa) {
        const int ns = min(QS, qa1 - qa) * spq;
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const int i = threadIdx.x + t * kDenseThreads;
            const int qi = small_div(i, inv_spq), r = i - qi * spq;
            const int64_t sidx = (((int64_t)b * g.Nq + qa + qi) * g.M + m) * LKs + (int64_t)lfirst * K + r;
            u[t] = i < ns ? loc[sidx] : make_float2(-1e30f, -1e30f);
            a[t] = i < ns ? attn[sidx] : 0.0f;
        }
    };
    auto fetch_g = [&](int qa) {
        const int nrow = min(QS, qa1 - qa) * LG;  // float4 of G to stage
#pragma unroll
        for (int t = 0; t < kGRows; ++t) {
            const int i = threadIdx.x + t * kDenseThreads;
            const int qi = i / LG, c = i - (i / LG) * LG;
            gst[t] = i < nrow ? grad_out[(((int64_t)b * g.Nq + qa + qi) * g.M + m) * LG + c]
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };

    float4 acc[PPG];
#pragma unroll
    for (int j = 0; j < PPG; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);

    if (qa0 < qa1) {
        fetch_samples(qa0);
        fetch_g(qa0);
    }
    for (int qa = qa0; qa < qa1; qa += QS) {
        lds_barrier();  // s_cnt cleared; the previous sub-chunk is done with s_g and s_pair
#pragma unroll
        for (int t = 0; t < kGRows; ++t)
            if ((kDenseQ * LG) % kDenseThreads == 0 || threadIdx.x + t * kDenseThreads < kDenseQ * LG)
                s_g[threadIdx.x + t * kDenseThreads] = gst[t];
        // the next sub-chunk's G rows: in flight through this one's ranking
        if (qa + QS < qa1) fetch_g(qa + QS);
        // rank this part's pairs within their pixel's count
        int pix[kPer][4];
        uint32_t rank[kPer][4];
        float wpair[kPer][4];
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const int i = threadIdx.x + t * kDenseThreads;
            const int dl = (i - small_div(i, inv_spq) * spq) / K;
            const LevelRec lv = s_lv[dl < ndl ? dl : 0];
            const int H = (int)lv.Hf, W = lv.W;
            const int pbase = s_dbase[dl < ndl ? dl : 0] - p0;
            int cx, cy;
            float fx, fy;
            const bool in = sample_cell(u[t], lv.Wf, lv.Hf, cx, cy, fx, fy);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int px = cx + (c & 1), py = cy + (c >> 1);
                const int p = pbase + py * W + px;
                wpair[t][c] = a[t] * ((c & 1) ? fx : 1.0f - fx) * ((c & 2) ? fy : 1.0f - fy);
                pix[t][c] = -1;
                if (in && px >= 0 && px < W && py >= 0 && py < H && p >= 0 && p < npix) {
                    pix[t][c] = p;
                    rank[t][c] = atomicAdd(&s_cnt[p], 1u);
                }
            }
        }
        if (qa + QS < qa1) fetch_samples(qa + QS);  // in flight until the next sub-chunk is ranked
        lds_barrier();
        // exclusive scan of the (at most kDensePix) pixel counts, one wave
        if (threadIdx.x < kWave) {
            constexpr int E = kDensePix / kWave;
            uint32_t v[E];
            uint32_t sum = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                v[e] = s_cnt[threadIdx.x * E + e];
                sum += v[e];
            }
            uint32_t incl = sum;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const uint32_t t = __shfl_up(incl, o, kWave);
                if ((int)threadIdx.x >= o) incl += t;
            }
            uint32_t run = incl - sum;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                s_start[threadIdx.x * E + e] = run;
                run += v[e];
            }
            if (threadIdx.x == kWave - 1) s_start[kDensePix] = incl;
        }
        lds_barrier();
#pragma unroll
        for (int t = 0; t < kPer; ++t) {
            const uint32_t qi = (uint32_t)small_div((int)threadIdx.x + t * kDenseThreads, inv_spq);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (pix[t][c] >= 0)
                    s_pair[s_start[pix[t][c]] + rank[t][c]] = make_uint2(__float_as_uint(wpair[t][c]), qi);
        }
        for (int i = threadIdx.x; i < kDensePix; i += kDenseThreads) s_cnt[i] = 0;  // for the next sub-chunk
        lds_barrier();
        // each lane group sums over the pairs of its pixels grp, grp + NG, ...
#pragma unroll
        for (int j = 0; j < PPG; ++j) {
            const int pl = grp + j * NG;
            if (pl >= npix) break;
            const uint32_t e1 = s_start[pl + 1];
            for (uint32_t e0 = s_start[pl]; e0 < e1; e0 += kDenseBatch) {
                uint2 pr[kDenseBatch];
                float4 gv[kDenseBatch];
#pragma unroll
                for (int v = 0; v < kDenseBatch; ++v) pr[v] = e0 + v < e1 ? s_pair[e0 + v] : make_uint2(0u, 0u);
#pragma unroll
                for (int v = 0; v < kDenseBatch; ++v) gv[v] = s_g[pr[v].y * LG + lig];
#pragma unroll
                for (int v = 0; v < kDenseBatch; ++v) {
                    const float w = __uint_as_float(pr[v].x);
                    acc[j].x = __builtin_fmaf(w, gv[v].x, acc[j].x);
                    acc[j].y = __builtin_fmaf(w, gv[v].y, acc[j].y);
                    acc[j].z = __builtin_fmaf(w, gv[v].z, acc[j].z);
                    acc[j].w = __builtin_fmaf(w, gv[v].w, acc[j].w);
                }
            }
        }
    }
    // one query split: write the part's pixels; several: park the sums in the
    // workspace for dense_reduce_kernel
#pragma unroll
    for (int j = 0; j < PPG; ++j) {
        const int pl = grp + j * NG;
        if (pl >= npix) break;
        float4 v = acc[j];
        const int p = p0 + pl;  // in the dense numbering
        if (tp.dsplits > 1) {
            partials[((int64_t)bm * tp.ppb + (int64_t)split * tp.ndpix + p) * LG + lig] = v;
        } else {
            int dl = 0;
            while (dl + 1 < ndl && p >= s_dbase[dl + 1]) ++dl;
            const int64_t row = (int64_t)b * g.S + s_lv[dl].start + (p - s_dbase[dl]);
            if (mask && mask[row]) v = make_float4(0.f, 0.f, 0.f, 0.f);  // padded: no gradient
            float4 *dst = grad_value + (row * g.M + m) * LG + lig;
            if (accumulate) {
                const float4 o = *dst;
                v.x += o.x;
                v.y += o.y;
                v.z += o.z;
                v.w += o.w;
            }
            *dst = v;
        }
    }
}

// Sum the dense levels' query splits, in split order, into grad_value.
// Thread t of (batch, dense pixel, head, float4 of channels).
// Lanes that share one output's query splits: R adjacent groups of LG lanes,
// each adding every R-th split; their sums are then added across the groups
// by lane exchange, in a fixed order.
constexpr int kReduceWays = 4;

template <int LG>
__device__ void dense_reduce_one(const Geometry &g, const TilePlan &tp, const float4 *__restrict__ partials,
                                 float4 *__restrict__ grad_value, int accumulate, const uint8_t *__restrict__ mask,
                                 int64_t t)
{
    constexpr int R = kReduceWays;
    static_assert((LG & (LG - 1)) == 0 && LG * R <= kWave, "an output's lanes within one wave");
    // the thread count is a whole number of outputs, so an output's lanes are
    // all present or all gone
    if (tp.dsplits <= 1 || t >= (int64_t)g.B * tp.ndpix * g.M * LG * R) return;
    constexpr int M = 64 / LG;  // 256 channels: M heads of 4*LG
    const int c = (int)(t % LG);
    const int r = (int)((t / LG) % R);
    const int64_t o = t / (LG * R);  // (b, p, m)
    const int m = (int)(o % M);
    // b * ndpix + p < B * S < 2^31: 32-bit division
    const uint32_t bp = (uint32_t)(o / M);
    const int b = (int)(bp / (uint32_t)tp.ndpix);
    const int p = (int)(bp - (uint32_t)b * (uint32_t)tp.ndpix);
    const int64_t p0 = (int64_t)(b * g.M + m) * tp.ppb + p;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int s = r; s < tp.dsplits; s += R) {
        const float4 x = partials[(p0 + (int64_t)s * tp.ndpix) * LG + c];
        v.x += x.x;
        v.y += x.y;
        v.z += x.z;
        v.w += x.w;
    }
    for (int d = LG; d < LG * R; d <<= 1) {
        v.x += __shfl_xor(v.x, d);
        v.y += __shfl_xor(v.y, d);
        v.z += __shfl_xor(v.z, d);
        v.w += __shfl_xor(v.w, d);
    }
    if (r != 0) return;
    // the dense level holding pixel p
    int l = -1;
    for (int i = 0; i < g.L; ++i)
        if (((tp.dense_mask >> i) & 1) && p >= tp.dbase[i]) l = i;
    const int64_t row = (int64_t)b * g.S + g.lv.start[l] + (p - tp.dbase[l]);
    if (mask && mask[row]) v = make_float4(0.f, 0.f, 0.f, 0.f);  // padded: no gradient
    float4 *dst = grad_value + (row * g.M + m) * LG + c;
    if (accumulate) {
        const float4 o = *dst;
        v.x += o.x;
        v.y += o.y;
        v.z += o.z;
        v.w += o.w;
    }
    *dst = v;
}

// The dense levels' query splits added up: kReduceWays threads per (batch,
// dense pixel, head, float4 of channels).
template <int LG>
__global__ void __launch_bounds__(kBlock)
dense_reduce_kernel(Geometry g, TilePlan tp, const float4 *__restrict__ partials, float4 *__restrict__ grad_value,
                    int accumulate, const uint8_t *__restrict__ mask)
{
    dense_reduce_one<LG>(g, tp, partials, grad_value, accumulate, mask, (int64_t)blockIdx.x * kBlock + threadIdx.x);
}

// ------------------------------------------------------------ generic fallback

template <typename VT>
__device__ __forceinline__ float vload(const VT *p);
template <> __device__ __forceinline__ float vload<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float vload<uint16_t>(const uint16_t *p)
{
    return __uint_as_float((uint32_t)*p << 16);
}

// One thread per (b, q, m), looping over the D channels; grad_value by float
// atomics (must be zeroed first unless accumulating).
template <typename VT>
__global__ void __launch_bounds__(256)
backward_generic_kernel(Geometry g, const VT *__restrict__ value, const float2 *__restrict__ loc,
                        const float *__restrict__ attn, const float *__restrict__ grad_out,
                        float *__restrict__ grad_value, float2 *__restrict__ grad_loc,
                        float *__restrict__ grad_attn, const uint8_t *__restrict__ mask)
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
                        const int64_t pix = g.lv.start[l] + (int64_t)yi * W + xi;
                        if (mask && mask[(int64_t)b * g.S + pix]) continue;  // padded: reads zero, no gradient
                        const float wx = dx ? fx : 1.0f - fx, wy = dy ? fy : 1.0f - fy;
                        const int64_t row = pix * C;
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

// One thread per (b, q, m, 4 channels) where D/4 is a power of two up to 64:
// the D/4 threads of a head are adjacent lanes of one wave. Each corner is one
// 4-channel buffer load (off-map or padded corners read zero and add nothing),
// the grad_value row takes four float atomics per corner (zeroed first unless
// accumulating), and the head's partial sums for the sample's weight and
// location gradients are added across its lanes with lane exchanges.
template <typename VT>
__global__ void __launch_bounds__(256)
backward_generic4_kernel(Geometry g, const VT *__restrict__ value, const float2 *__restrict__ loc,
                         const float *__restrict__ attn, const float4 *__restrict__ grad_out,
                         float *__restrict__ grad_value, float2 *__restrict__ grad_loc,
                         float *__restrict__ grad_attn, const uint8_t *__restrict__ mask)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int D4 = g.D / 4, C = g.M * g.D;
    // the thread count is a whole number of heads, so a head's lanes are all
    // present or all gone
    if (t >= g.queries() * g.M * D4) return;
    const int64_t bqm = t / D4;
    const int c4 = (int)(t - bqm * D4);
    const int64_t bq = bqm / g.M;
    const int m = (int)(bqm - bq * g.M);
    const int b = (int)(bq / g.Nq);
    const uint32_t RB = (uint32_t)C * sizeof(VT);
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(value + (int64_t)b * g.S * C, (uint32_t)g.S * RB);
    const uint32_t lane_off = (uint32_t)(m * g.D + c4 * 4) * sizeof(VT);
    const uint8_t *mask_b = mask ? mask + (int64_t)b * g.S : nullptr;
    float *gvb = grad_value + (int64_t)b * g.S * C + m * g.D + c4 * 4;
    const float4 G = grad_out[t];  // [B, Nq, M*D]: element 4t is (b, q, m, 4*c4)
    for (int l = 0; l < g.L; ++l) {
        const int W = g.lv.W[l], H = g.lv.H[l];
        const float Wf = (float)W, Hf = (float)H;
        for (int k = 0; k < g.K; ++k) {
            const int64_t s = (bqm * g.L + l) * g.K + k;
            float2 u = loc[s];
            const float a = attn[s];
            const bool in = sample_in_range(u.x, u.y, Wf, Hf);
            u.x = in ? u.x : 0.0f;
            u.y = in ? u.y : 0.0f;
            float cx, fx, cy, fy;
            cell_1d(u.x, Wf, cx, fx);
            cell_1d(u.y, Hf, cy, fy);
            const bool x0ok = (cx >= 0.0f) & (cx < Wf);
            const bool x1ok = (cx >= -1.0f) & (cx + 1.0f < Wf);
            const bool y0ok = in & (cy >= 0.0f) & (cy < Hf);
            const bool y1ok = in & (cy >= -1.0f) & (cy + 1.0f < Hf);
            bool k00 = y0ok & x0ok, k01 = y0ok & x1ok, k10 = y1ok & x0ok, k11 = y1ok & x1ok;
            const int row = g.lv.start[l] + (int)cy * W + (int)cx;
            if (mask_b) unmask_corners(mask_b, row, W, k00, k01, k10, k11);
            const uint32_t o00 = (uint32_t)row * RB + lane_off, o10 = o00 + (uint32_t)W * RB;
            const float4 v00 = ValueTraits<VT>::load4(rsrc, k00 ? o00 : kOutOfRange);
            const float4 v01 = ValueTraits<VT>::load4(rsrc, k01 ? o00 + RB : kOutOfRange);
            const float4 v10 = ValueTraits<VT>::load4(rsrc, k10 ? o10 : kOutOfRange);
            const float4 v11 = ValueTraits<VT>::load4(rsrc, k11 ? o10 + RB : kOutOfRange);
            const float d00 = G.x * v00.x + G.y * v00.y + G.z * v00.z + G.w * v00.w;
            const float d01 = G.x * v01.x + G.y * v01.y + G.z * v01.z + G.w * v01.w;
            const float d10 = G.x * v10.x + G.y * v10.y + G.z * v10.z + G.w * v10.w;
            const float d11 = G.x * v11.x + G.y * v11.y + G.z * v11.z + G.w * v11.w;
            const float wy0 = 1.0f - fy, wx0 = 1.0f - fx;
            float ga = wy0 * (wx0 * d00 + fx * d01) + fy * (wx0 * d10 + fx * d11);
            float gx = wy0 * (d01 - d00) + fy * (d11 - d10);
            float gy = wx0 * (d10 - d00) + fx * (d11 - d01);
            const float ay0 = a * wy0, ay1 = a * fy;
            const float w[4] = {ay0 * wx0, ay0 * fx, ay1 * wx0, ay1 * fx};
            const bool kk[4] = {k00, k01, k10, k11};
            const int64_t rows[4] = {row, row + 1, row + W, row + W + 1};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (kk[j]) {
                    float *d = gvb + rows[j] * C;
                    atomicAdd(d + 0, w[j] * G.x);
                    atomicAdd(d + 1, w[j] * G.y);
                    atomicAdd(d + 2, w[j] * G.z);
                    atomicAdd(d + 3, w[j] * G.w);
                }
            for (int o = 1; o < D4; o <<= 1) {
                ga += __shfl_xor(ga, o);
                gx += __shfl_xor(gx, o);
                gy += __shfl_xor(gy, o);
            }
            if (c4 == 0) {
                grad_attn[s] = ga;
                grad_loc[s] = make_float2(a * Wf * gx, a * Hf * gy);
            }
        }
    }
}

// ------------------------------------------------------------------- host side

struct Workspace {
    uint32_t *counts, *totals, *bases;
    uint4 *records;
    float4 *partials;  // the dense levels' query-split sums (TilePlan::pbase)
    float4 *ref_part;  // fused per-head path: [B, Nq, M, L] sums of the reference-point gradient
};

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t layout(const Geometry &g, const TilePlan &tp, char *base, Workspace *ws)
{
    const size_t nkeys = (size_t)g.B * g.M * tp.tpb;
    // per-workgroup counts of the query-range binning or of the per-head one
    const size_t ncount = std::max((size_t)g.B * tp.wpb, (size_t)g.B * tp.hqr) * g.M * tp.tpb;
    const size_t nrec = (size_t)g.queries() * g.M * tp.rslots;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char *p = base ? base + off : nullptr;
        off += align256(bytes);
        return reinterpret_cast<uint32_t *>(p);
    };
    Workspace w;
    w.counts = take(ncount * 4);
    w.totals = take(nkeys * 4);
    w.bases = take(nkeys * 4);
    w.records = reinterpret_cast<uint4 *>(take(nrec * sizeof(uint4)));
    w.partials = reinterpret_cast<float4 *>(take((size_t)g.B * g.M * tp.ppb * g.D * 4));
    w.ref_part = reinterpret_cast<float4 *>(take((size_t)g.queries() * g.M * g.L * 16));
    if (ws) *ws = w;
    return off;
}

// A second stream per device (and host thread) for the dense levels, which
// need neither the binning nor the main kernel and so overlap them, with its
// fork and join events. Created on first use at the default priority and
// kept for the life of the process; thread-local, so host threads never
// share the events. Under graph capture the side stream joins the capture
// through the fork event.
struct SideStream {
    hipStream_t s;
    hipEvent_t fork, join;
};

hipError_t side_stream(SideStream **out)
{
    constexpr int kMaxDevices = 64;
    thread_local SideStream per_device[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    SideStream &ss = per_device[dev];
    if (!ss.s) {
        if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking)) != hipSuccess) return e;
    }
    *out = &ss;
    return hipSuccess;
}

// The binning of the sparse levels' samples into their tiles' record lists
// (it depends on the locations only).
template <int M, int L, int K>
hipError_t launch_binning(const Geometry &g, const TilePlan &tp, const float *loc, const Workspace &ws,
                          hipStream_t st)
{
    const int nkb = M * tp.tpb;
    const int nkeys = g.B * nkb;
    if (nkeys == 0) return hipSuccess;
    {
        KernelScope ks_("clear_totals_kernel", st);
        hipLaunchKernelGGL(clear_totals_kernel, dim3((nkeys + kBlock - 1) / kBlock), dim3(kBlock), 0, st, nkeys,
                           ws.totals);
    }
    {
        KernelScope ks_("bin_count_kernel", st);
        hipLaunchKernelGGL((bin_count_kernel<M, L, K>), dim3(g.B * tp.wpb), dim3(kBinThreads), (size_t)nkb * 4, st,
                           g, tp, reinterpret_cast<const float2 *>(loc), ws.counts, ws.totals);
    }
    return hipGetLastError();
}

// The first level whose rows (with every coarser level's) fit in LDS beside
// the per-head kernel's records and tile cursors, or 0 when the per-head path
// does not apply (other shapes, fewer queries, or nothing fits).
template <typename VT, int M, int L, int K>
int head_stage_level(const Geometry &g, const TilePlan &tp, uint32_t &stage_bytes)
{
    if constexpr (!(M == 8 && L == 4 && K == 4)) {
        return 0;
    } else {
        constexpr int LPH = 256 / M / 4, QPW = kWave / LPH;
        constexpr size_t kStatic = (size_t)kHeadWaves * QPW * (L * K + 1) * 32 + 2 * 16 * L + 4 * kHeadWaves;
        if (g.Nq < kHeadMinQueries) return 0;
        const size_t cursors = (size_t)(2 * tp.tpb + kWave) * 4;  // cursors and prefix counts
        for (int ls = 1; ls < L; ++ls) {
            const int64_t rows = (int64_t)g.S - g.lv.start[ls];
            const size_t bytes = ((size_t)(rows + 1) * LPH * sizeof(typename StageChunk<VT>::type) + 15) & ~(size_t)15;
            if (kStatic + bytes + cursors + 1024 <= kHeadLds) {
                stage_bytes = (uint32_t)bytes;
                return ls;
            }
        }
        return 0;
    }
}

// The per-head path's binning: one row of tile counts per (batch, head, query range).
template <int M, int L, int K>
hipError_t launch_head_binning(const Geometry &g, const TilePlan &tp, const float *loc, const Workspace &ws,
                               hipStream_t st)
{
    const int nwg = g.B * M * tp.hqr;
    {
        KernelScope ks_("bin_count_head_kernel", st);
        hipLaunchKernelGGL((bin_count_head_kernel<M, L, K>), dim3(nwg), dim3(kBinThreads), (size_t)tp.tpb * 4, st, g,
                           tp, reinterpret_cast<const float2 *>(loc), ws.counts);
    }
    return hipGetLastError();
}

// The per-head main kernel (after launch_head_binning on the same stream).
template <typename VT, int M, int L, int K, int LS, bool FUSED>
hipError_t launch_head(const Geometry &g, const TilePlan &tp, const void *value, const float *loc,
                       const float *attn, const float *go, float *gl, float *ga, const Workspace &ws,
                       uint32_t stage_bytes, const uint8_t *mask, const FusedGrads &fg, hipStream_t st)
{
    const int nwg = g.B * M * tp.hqr;
    const uint32_t grid = round_up8((uint32_t)nwg);
    const size_t dyn = (size_t)stage_bytes + (size_t)(2 * tp.tpb + kWave) * 4;
    {
        KernelScope ks_(FUSED ? "backward_fused_head_kernel" : "backward_head_kernel", st);
        hipLaunchKernelGGL((backward_head_kernel<VT, M, L, K, LS, FUSED>), dim3(grid), dim3(kHeadThreads), dyn, st, g,
                           tp, static_cast<const VT *>(value), reinterpret_cast<const float2 *>(loc), attn,
                           reinterpret_cast<const float4 *>(go), reinterpret_cast<float2 *>(gl), ga, ws.counts,
                           ws.totals, ws.bases, ws.records, stage_bytes, grid, mask, fg, ws.ref_part);
    }
    if (FUSED && fg.grad_ref) {
        KernelScope ks_("ref_grad_sum_kernel", st);
        hipLaunchKernelGGL((ref_grad_sum_kernel<M, L>), dim3((unsigned)((g.queries() * L + 255) / 256)), dim3(256),
                           0, st, g, ws.ref_part, fg);
    }
    return hipGetLastError();
}

template <typename VT, int M, int L, int K, bool FUSED>
hipError_t launch_fast(const Geometry &g, const TilePlan &tp, const void *value, const float *loc,
                       const float *attn, const float *go, float *gv, float *gl, float *ga, const FusedGrads &fg,
                       void *wsp, bool accumulate, bool side_ok, const uint8_t *mask, hipStream_t st)
{
    Workspace ws;
    layout(g, tp, static_cast<char *>(wsp), &ws);
    const int nkb = M * tp.tpb;
    const int nwg = g.B * tp.wpb;
    const size_t hist_bytes = (size_t)(nkb + kWave) * 4;  // + a slot per lane for its idle adds
    constexpr int LG = 256 / M / 4;
    // The dense levels (and the sum of their query splits) read only the
    // inputs and write their own grad_value rows and workspace section, so
    // they run on the side stream beside everything else on `st`, which
    // waits for them only at the end. Without the side stream (side_ok
    // false: the caller's stream only; or while the launches are timed, so
    // that each event pair times its kernel alone) they run last on `st`.
    SideStream *side = nullptr;
    auto launch_dense = [&](hipStream_t ds) -> hipError_t {
        const uint32_t ditems = (uint32_t)(g.B * g.M * tp.dipb);
        {
            KernelScope ks_("dense_accum_kernel", ds);
            hipLaunchKernelGGL((dense_accum_kernel<M, L, K>), dim3(round_up8(ditems)), dim3(kDenseThreads), 0, ds, g,
                               tp, reinterpret_cast<const float2 *>(loc), attn, reinterpret_cast<const float4 *>(go),
                               reinterpret_cast<float4 *>(gv), ws.partials, accumulate ? 1 : 0, mask);
        }
        const int64_t nred = tp.dsplits > 1 ? (int64_t)g.B * tp.ndpix * g.M * LG * kReduceWays : 0;
        if (nred > 0) {
            KernelScope ks_("dense_reduce_kernel", ds);
            hipLaunchKernelGGL((dense_reduce_kernel<LG>), dim3((unsigned)((nred + kBlock - 1) / kBlock)), dim3(kBlock),
                               0, ds, g, tp, ws.partials, reinterpret_cast<float4 *>(gv), accumulate ? 1 : 0, mask);
        }
        return hipGetLastError();
    };
    if (tp.dipb > 0 && side_ok && !timing_on(st)) {
        hipError_t e = side_stream(&side);
        if (e == hipSuccess) e = hipEventRecord(side->fork, st);
        if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
        if (e == hipSuccess) e = launch_dense(side->s);
        if (e == hipSuccess) e = hipEventRecord(side->join, side->s);
        if (e != hipSuccess) return e;
    }
    uint32_t stage_bytes = 0;
    const int hls = head_stage_level<VT, M, L, K>(g, tp, stage_bytes);
    if (hls > 0) {
        // the per-head path: binning and main kernel per (batch, head, query range)
        hipError_t e = launch_head_binning<M, L, K>(g, tp, loc, ws, st);
        if (e != hipSuccess) return e;
        e = hipErrorInvalidValue;
        if constexpr (M == 8 && L == 4 && K == 4) {
#define MSDA_HEAD(LS_)                                                                                            \
    if (hls == LS_)                                                                                               \
        e = launch_head<VT, M, L, K, LS_, FUSED>(g, tp, value, loc, attn, go, gl, ga, ws, stage_bytes, mask, fg, st);
            MSDA_HEAD(1)
            MSDA_HEAD(2)
            MSDA_HEAD(3)
#undef MSDA_HEAD
        }
        if (e != hipSuccess) return e;
    } else {
        const hipError_t e = launch_binning<M, L, K>(g, tp, loc, ws, st);
        if (e != hipSuccess) return e;
    }
    const uint32_t grid = round_up8((uint32_t)nwg);
    if (hls == 0) {
        KernelScope ks_(FUSED ? "backward_fused_c256_kernel" : "backward_c256_kernel", st);
        hipLaunchKernelGGL((backward_c256_kernel<VT, M, L, K, FUSED>), dim3(grid),
                           dim3(MainWaves<M, L, K>::kValue * kWave), hist_bytes, st, g, tp,
                           static_cast<const VT *>(value), reinterpret_cast<const float2 *>(loc), attn,
                           reinterpret_cast<const float4 *>(go), reinterpret_cast<float2 *>(gl), ga, ws.counts,
                           ws.totals, ws.bases, ws.records, grid, fg, mask);
    }
    if (!accumulate) {
        int64_t n = 0;
        for (int l = 0; l < g.L; ++l)
            if (level_uses_atomics(tp, l)) n += (int64_t)g.B * g.lv.H[l] * g.lv.W[l] * g.M * g.D / 4;
        if (n > 0) {
            KernelScope ks_("zero_split_levels_kernel", st);
            hipLaunchKernelGGL(zero_split_levels_kernel, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                               st, g, tp, reinterpret_cast<float4 *>(gv));
        }
    }
    // the sparse levels' tiles
    const uint32_t items = (uint32_t)(g.B * g.M * tp.ipb);
    if (items > 0) {
        KernelScope ks_("tile_accum_kernel", st);
        hipLaunchKernelGGL((tile_accum_kernel<M, L, K>), dim3(round_up8(items)), dim3(kBlock), 0, st, g, tp,
                           reinterpret_cast<const float4 *>(go), reinterpret_cast<float4 *>(gv), ws.records, ws.bases,
                           ws.totals, accumulate ? 1 : 0, mask);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (side) return hipStreamWaitEvent(st, side->join, 0);
    if (tp.dipb > 0) return launch_dense(st);
    return hipSuccess;
}

// Which (VT-independent) fast-path instantiation serves g, if any.
enum class Fast { None, M8L4K4, M4L4K4, M16L4K4, M8L1K4, M8L4K8, M8L3K4, M8L4K1, M8L5K4, M8L4K2 };

Fast fast_kind(const Geometry &g)
{
    if (g.M * g.D != 256) return Fast::None;
    if (g.L == 4 && g.K == 4) {
        if (g.M == 8) return Fast::M8L4K4;
        if (g.M == 4) return Fast::M4L4K4;
        if (g.M == 16) return Fast::M16L4K4;
    }
    if (g.M == 8) {
        if (g.L == 1 && g.K == 4) return Fast::M8L1K4;
        if (g.L == 4 && g.K == 8) return Fast::M8L4K8;
        if (g.L == 3 && g.K == 4) return Fast::M8L3K4;
        if (g.L == 4 && g.K == 1) return Fast::M8L4K1;
        if (g.L == 5 && g.K == 4) return Fast::M8L5K4;
        if (g.L == 4 && g.K == 2) return Fast::M8L4K2;
    }
    return Fast::None;
}

// The fused gradients for shapes without an in-kernel form: in place, one
// thread per (b, q): grad_attn -> grad_logits through the L*K softmax,
// grad_loc -> grad_offsets, and grad_ref from the sums of grad_loc over (m, k).
__global__ void __launch_bounds__(256)
fused_grads_kernel(Geometry g, const float *__restrict__ attn, float *__restrict__ grad_attn,
                   float2 *__restrict__ grad_loc, FusedGrads fg)
{
    const int64_t bq = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (bq >= g.queries()) return;
    const int LK = g.L * g.K;
    const float Kf = (float)g.K;
    for (int m = 0; m < g.M; ++m) {
        const int64_t row = (bq * g.M + m) * LK;
        float dot = 0.0f;
        for (int i = 0; i < LK; ++i) dot += attn[row + i] * grad_attn[row + i];
        for (int i = 0; i < LK; ++i) grad_attn[row + i] = attn[row + i] * (grad_attn[row + i] - dot);
    }
    for (int l = 0; l < g.L; ++l) {
        int W = 1, H = 1;
#pragma unroll
        for (int i = 0; i < MSDA_MAX_LEVELS; ++i)
            if (i == l) {
                W = g.lv.W[i];
                H = g.lv.H[i];
            }
        float4 bx = make_float4(0.f, 0.f, 0.f, 0.f);
        if (fg.ref_dims == 4) bx = reinterpret_cast<const float4 *>(fg.ref)[bq * g.L + l];
        float sx = 0.0f, sy = 0.0f, sw = 0.0f, sh = 0.0f;
        for (int m = 0; m < g.M; ++m)
            for (int k = 0; k < g.K; ++k) {
                const int64_t s = ((bq * g.M + m) * g.L + l) * g.K + k;
                const float2 v = grad_loc[s];
                sx += v.x;
                sy += v.y;
                if (fg.ref_dims == 4) {
                    const float2 o = fg.off[s];
                    sw += v.x * o.x * 0.5f / Kf;
                    sh += v.y * o.y * 0.5f / Kf;
                    grad_loc[s] = make_float2(v.x * (bx.z * 0.5f / Kf), v.y * (bx.w * 0.5f / Kf));
                } else {
                    grad_loc[s] = make_float2(v.x / (float)W, v.y / (float)H);
                }
            }
        if (fg.grad_ref) {
            if (fg.ref_dims == 4)
                reinterpret_cast<float4 *>(fg.grad_ref)[bq * g.L + l] = make_float4(sx, sy, sw, sh);
            else
                reinterpret_cast<float2 *>(fg.grad_ref)[bq * g.L + l] = make_float2(sx, sy);
        }
    }
}

template <typename VT>
hipError_t launch_typed(const Geometry &g, const TilePlan *tpp, const void *value, const float *loc,
                        const float *attn, const float *go, float *gv, float *gl, float *ga, const FusedGrads *fg,
                        void *ws, bool accumulate, bool side_ok, const uint8_t *mask, hipStream_t st)
{
    // fused gradients inside the main kernel where the L*K softmax fits the
    // wave's lanes; otherwise the plain gradients, converted afterwards
    const bool fused = fg != nullptr;
    const bool in_kernel = fused && fused_forward_supported(g);
    hipError_t e = hipSuccess;
    bool done = false;
#define MSDA_FAST(M_, L_, K_)                                                                                    \
    e = in_kernel ? launch_fast<VT, M_, L_, K_, true>(g, *tpp, value, loc, attn, go, gv, gl, ga, *fg, ws,        \
                                                      accumulate, side_ok, mask, st)                             \
                  : launch_fast<VT, M_, L_, K_, false>(g, *tpp, value, loc, attn, go, gv, gl, ga, FusedGrads{},  \
                                                       ws, accumulate, side_ok, mask, st);                       \
    done = true;
    switch (tpp ? fast_kind(g) : Fast::None) {
    case Fast::M8L4K4: MSDA_FAST(8, 4, 4) break;
    case Fast::M4L4K4: MSDA_FAST(4, 4, 4) break;
    case Fast::M16L4K4: MSDA_FAST(16, 4, 4) break;
    case Fast::M8L1K4: MSDA_FAST(8, 1, 4) break;
    case Fast::M8L4K8: MSDA_FAST(8, 4, 8) break;
    case Fast::M8L3K4: MSDA_FAST(8, 3, 4) break;
    case Fast::M8L4K1: MSDA_FAST(8, 4, 1) break;
    case Fast::M8L5K4: MSDA_FAST(8, 5, 4) break;
    case Fast::M8L4K2: MSDA_FAST(8, 4, 2) break;
    case Fast::None: break;
    }
#undef MSDA_FAST
    if (e != hipSuccess) return e;
    if (!done) {
        if (!accumulate) {
            e = launch_zero_fill(gv, (int64_t)g.B * g.S * g.M * g.D, st);
            if (e != hipSuccess) return e;
        }
        const int d4 = g.D / 4;
        if (g.D % 4 == 0 && d4 <= kWave && (d4 & (d4 - 1)) == 0 &&
            reinterpret_cast<uintptr_t>(value) % (4 * sizeof(VT)) == 0 && reinterpret_cast<uintptr_t>(go) % 16 == 0) {
            const int64_t n = g.queries() * g.M * d4;
            KernelScope ks_("backward_generic4_kernel", st);
            hipLaunchKernelGGL((backward_generic4_kernel<VT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                               g, static_cast<const VT *>(value), reinterpret_cast<const float2 *>(loc), attn,
                               reinterpret_cast<const float4 *>(go), gv, reinterpret_cast<float2 *>(gl), ga, mask);
        } else {
            const int64_t n = g.queries() * g.M;
            KernelScope ks_("backward_generic_kernel", st);
            hipLaunchKernelGGL((backward_generic_kernel<VT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                               g, static_cast<const VT *>(value), reinterpret_cast<const float2 *>(loc), attn, go,
                               gv, reinterpret_cast<float2 *>(gl), ga, mask);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (fused && !(done && in_kernel)) {
        KernelScope ks_("fused_grads_kernel", st);
        hipLaunchKernelGGL(fused_grads_kernel, dim3((unsigned)((g.queries() + 255) / 256)), dim3(256), 0, st, g,
                           attn, ga, reinterpret_cast<float2 *>(gl), *fg);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

// Tile sizes per level: the largest tile (at most kTilePix pixels and
// kTileCells cells with its halo; squarer wins a tie, since it duplicates
// fewer records) whose expected record count, with samples spread evenly over
// the level, stays within 3/4 of one chunk (a 1x1 tile if none does).
bool make_tile_plan(const Geometry &g, TilePlan &tp)
{
    if (fast_kind(g) == Fast::None) return false;
    const double target = kTileTarget;
    // every (cell, split) task needs a slot: cells <= kTaskSlots * lane groups
    const int max_cells = std::min(kTileCells, kTaskSlots * (kBlock / (g.D / 4)));
    int base = 0, ibase = 0;
    // dense levels (at least kDenseMinPerPix samples per pixel, at most
    // kDenseMaxPix pixels): the last run of adjacent such levels, so that a
    // query's dense samples are adjacent in memory
    tp.dense_mask = 0;
    for (int l = 0; l < g.L; ++l) {
        const int H = g.lv.H[l], W = g.lv.W[l];
        // tile indices come from float reciprocals, exact below 2^20
        if (H >= (1 << 20) || W >= (1 << 20)) return false;
        const double per_cell = (double)g.Nq * g.K / ((double)H * W);
        if (per_cell >= kDenseMinPerPix && H * W <= kDenseMaxPix)
            tp.dense_mask |= 1 << l;
        else if (tp.dense_mask)
            tp.dense_mask = 0;  // a sparse level after dense ones: only a later run counts
    }
    tp.ndl = tp.ndpix = 0;
    for (int l = 0; l < MSDA_MAX_LEVELS; ++l) {
        tp.dbase[l] = tp.ndpix;
        if (l < g.L && ((tp.dense_mask >> l) & 1)) {
            ++tp.ndl;
            tp.ndpix += g.lv.H[l] * g.lv.W[l];
        }
    }
    // (pixel part, query split) work items over all dense levels
    tp.dparts = tp.dsplits = 1;
    if (tp.ndl > 0) {
        tp.dparts = (tp.ndpix + kDensePix - 1) / kDensePix;
        const double s = std::ceil((double)g.Nq * g.K * tp.ndl / kDenseItemSamples);
        tp.dsplits = (int)std::min<double>(kDenseMaxSplit, std::max(1.0, s));
    }
    tp.dipb = tp.ndl > 0 ? tp.dparts * tp.dsplits : 0;
    tp.ppb = tp.ndl > 0 && tp.dsplits > 1 ? tp.dsplits * tp.ndpix : 0;
    for (int l = 0; l < g.L; ++l) {
        const int H = g.lv.H[l], W = g.lv.W[l];
        const double per_cell = (double)g.Nq * g.K / ((double)H * W);
        if ((tp.dense_mask >> l) & 1) {
            // dense level: no tiles
            tp.th[l] = tp.tw[l] = tp.ntw[l] = tp.nchunk[l] = 1;
            tp.tinv_h[l] = tp.tinv_w[l] = 1.0f;
            tp.tbase[l] = base;
            tp.ibase[l] = ibase;
            continue;
        }
        int bt = 1, bw = 1, barea = 0, bcells = 1 << 30;
        for (int th = 1; th <= std::min(H, kTilePix); ++th)
            for (int tw = 1; tw <= std::min(W, kTilePix / th); ++tw) {
                const int cells = (th + 1) * (tw + 1);
                if (cells > max_cells || cells * per_cell > target) continue;
                const int area = th * tw;
                if (area > barea || (area == barea && cells < bcells)) {
                    barea = area;
                    bcells = cells;
                    bt = th;
                    bw = tw;
                }
            }
        if (barea <= kDirectPix) {
            // too dense for the sorted path to pay off: a 2x2 tile in direct
            // mode (no record limit) duplicates fewer records than 1x1
            bt = std::min(H, 2);
            bw = std::min(W, 2);
        }
        tp.th[l] = bt;
        tp.tw[l] = bw;
        tp.tinv_h[l] = 1.0f / (float)bt;
        tp.tinv_w[l] = 1.0f / (float)bw;
        tp.ntw[l] = (W + bw - 1) / bw;
        tp.tbase[l] = base;
        const int ntiles = ((H + bt - 1) / bt) * tp.ntw[l];
        base += ntiles;
        // direct-mode tiles share their records among enough workgroups to
        // give each about kDirectRecords of them
        int nch = 1;
        if (bt * bw <= kDirectPix) {
            const double recs = per_cell * (bt + 1) * (bw + 1);
            nch = (int)std::min<double>(kMaxSplit, std::max(1.0, std::ceil(recs / kDirectRecords)));
        }
        tp.nchunk[l] = nch;
        tp.ibase[l] = ibase;
        ibase += ntiles * nch;
    }
    for (int l = g.L; l < MSDA_MAX_LEVELS; ++l) {
        tp.th[l] = tp.tw[l] = tp.ntw[l] = tp.nchunk[l] = 1, tp.tbase[l] = base, tp.ibase[l] = ibase;
        tp.tinv_h[l] = tp.tinv_w[l] = 1.0f;
    }
    tp.tpb = base;
    tp.ipb = ibase;
    // queries per workgroup of the per-query path: kQueriesPerGroup, halved
    // down to 8 (a workgroup's waves) while the workgroups would not cover
    // the CUs (few queries: the decoder's 300 per image)
    tp.qpw = kQueriesPerGroup;
    while (tp.qpw > 8 && (int64_t)g.B * ((g.Nq + tp.qpw - 1) / tp.qpw) < kMinQueryWGs) tp.qpw /= 2;
    tp.wpb = (g.Nq + tp.qpw - 1) / tp.qpw;
    tp.hqr = std::max(1, (kHeadTargetWGs + g.B * g.M - 1) / (g.B * g.M));
    tp.hqpr = std::max(1, (g.Nq + tp.hqr - 1) / tp.hqr);
    tp.hqr = std::max(1, (g.Nq + tp.hqpr - 1) / tp.hqpr);
    int nsparse = 0;
    for (int l = 0; l < g.L; ++l) nsparse += !((tp.dense_mask >> l) & 1);
    tp.rslots = 4 * g.K * nsparse;
    // the per-workgroup histogram / cursors live in LDS (and their indices
    // below 2^kKeyBits); record positions are 32-bit and a record holds its
    // query index in 32 - kCellBits bits
    if (((size_t)g.M * tp.tpb + kWave) * 4 > 64 * 1024) return false;  // the main kernel's LDS cursors
    static_assert((64 * 1024 / 4) <= (1 << kKeyBits), "cursor indices fit below the key bits");
    if ((uint64_t)g.queries() * g.M * tp.rslots >= (1ull << 32)) return false;
    if ((uint64_t)g.queries() >= (1ull << (32 - kCellBits))) return false;
    // grad_output is read through 32-bit buffer offsets below the out-of-range marker
    if ((uint64_t)g.queries() * g.M * g.D * 4 >= (uint64_t)kOutOfRange) return false;
    return true;
}

size_t backward_workspace_bytes(const Geometry &g)
{
    TilePlan tp;
    if (!make_tile_plan(g, tp)) return 0;
    return layout(g, tp, nullptr, nullptr);
}

bool backward_plan_masks(const Geometry &g, uint32_t &dense, uint32_t &direct, uint32_t &split)
{
    dense = direct = split = 0;
    TilePlan tp;
    if (!make_tile_plan(g, tp)) return false;
    dense = (uint32_t)tp.dense_mask;
    for (int l = 0; l < g.L; ++l) {
        if ((dense >> l) & 1) continue;
        if (tp.th[l] * tp.tw[l] <= kDirectPix) direct |= 1u << l;
        if (level_uses_atomics(tp, l)) split |= 1u << l;
    }
    return true;
}

bool backward_uses_workspace(const Geometry &g, const void *value, msda_dtype vt, const float *go,
                             const float *gv)
{
    TilePlan tp;
    const size_t vb = vt == MSDA_BF16 ? 2 : 4;
    return make_tile_plan(g, tp) && (reinterpret_cast<uintptr_t>(value) % (4 * vb)) == 0 &&
           (reinterpret_cast<uintptr_t>(go) % 16) == 0 && (reinterpret_cast<uintptr_t>(gv) % 16) == 0;
}

hipError_t launch_backward(const Geometry &g, const void *value, msda_dtype vt, const float *loc,
                           const float *attn, const float *go, float *gv, float *gl, float *ga, void *ws,
                           bool accumulate, bool side_ok, hipStream_t st)
{
    TilePlan tp;
    const TilePlan *tpp = backward_uses_workspace(g, value, vt, go, gv) && make_tile_plan(g, tp) ? &tp : nullptr;
    if (vt == MSDA_BF16)
        return launch_typed<uint16_t>(g, tpp, value, loc, attn, go, gv, gl, ga, nullptr, ws, accumulate, side_ok,
                                      nullptr, st);
    return launch_typed<float>(g, tpp, value, loc, attn, go, gv, gl, ga, nullptr, ws, accumulate, side_ok, nullptr,
                               st);
}

hipError_t launch_backward_fused(const Geometry &g, const void *value, msda_dtype vt, const float *loc,
                                 const float *attn, const float *go, float *gv, float *goff, float *glogits,
                                 const FusedGrads &fg, void *ws, bool accumulate, bool side_ok, hipStream_t st)
{
    TilePlan tp;
    const TilePlan *tpp = backward_uses_workspace(g, value, vt, go, gv) && make_tile_plan(g, tp) ? &tp : nullptr;
    if (vt == MSDA_BF16)
        return launch_typed<uint16_t>(g, tpp, value, loc, attn, go, gv, goff, glogits, &fg, ws, accumulate, side_ok,
                                      fg.mask, st);
    return launch_typed<float>(g, tpp, value, loc, attn, go, gv, goff, glogits, &fg, ws, accumulate, side_ok,
                               fg.mask, st);
}

// ---------------------------------------------------- allocation-free scratch

// The workspace of msda_backward_noalloc: a file-scope device array (each GPU
// the library runs on holds its own copy, at its own address, until the
// process ends). Host code never passes `scratch` itself to a kernel (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device, and is used everywhere instead.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace msda
