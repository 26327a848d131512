// trace_quant.hip -- rollout-guided FP4 (E2M1) quantisation and fake-quant
// kernels for MI355X (gfx950), behind the C ABI of include/trace_quant.h.
//
// Method: TRACE (Rollout-Guided Quantization-Aware Training for FP4 RL of MoE
// language models), as described on "Alibaba Qwen Proposes TRACE for 5.4x
// Faster FP4 RL Rollouts": section "Why Does FP4 Rollout 'Break' RL
// Training?" (Figure 1: both sides share the global and block scale, then
// round to E2M1) and section "TRACE Core Concept" (Figure 3: the training side
// picks, of the two adjacent E2M1 points, the one nearer the rollout's code,
// reconstructed from the block scale plus a few low index bits).
//
// Design (one GPU, HBM-bound streaming; nothing here is a contraction, so no
// MFMA):
//   * one 16-element block per lane: each lane issues two 16-byte loads of
//     bf16, so the block amax, the block scale and its reciprocal stay in the
//     lane's registers (no cross-lane traffic at all);
//   * codes, scale bytes and guidance bits are packed in registers and
//     written with one store per lane per plane (8, 1 and 2k bytes), which
//     are contiguous across the wavefront;
//   * the rounding decision of every mode is one fp32 compare against a
//     threshold read from a 1.3 KB LDS table indexed by (mode row, bucket of
//     |v|): chosen index = floor index + (|v| > threshold);
//   * persistent workgroups walk tiles of 256 x kUnroll lane-blocks, loads
//     of all kUnroll blocks first, so each wave keeps 32 x kUnroll bytes per
//     lane in flight.
#include <hip/hip_runtime.h>

#include <bit>
#include <cfloat>
#include <cstdint>

#include "trace_quant.h"

namespace {

constexpr int kThreads = 256;          // 4 wavefronts of 64
constexpr int kUnroll = 2;             // lane-blocks per thread per tile
constexpr int kTile = kThreads * kUnroll;
constexpr int kBuckets = 11;           // buckets of |v| (see bucket_of)
constexpr int kMaxGrid = 256 * 8;      // 8 workgroups per CU

// ---------------------------------------------------------------------------
// Decision table.
//
// |v| is split into 11 buckets by its fp32 exponent and top mantissa bit:
//   [0,.25) [.25,.375) [.375,.5) [.5,.75) [.75,1) [1,1.5) [1.5,2) [2,3)
//   [3,4) [4,6) [6,inf]
// Within a bucket the floor E2M1 index jl is fixed (0 0 0 1 1 2 3 4 5 6 7)
// and the upper neighbour is jl + 1.  For each (row, bucket) the table holds
// a threshold T: the chosen index is jl + (|v| > T).  T >= value(jl), so an
// on-grid |v| keeps jl; T = +inf always keeps jl; T = value(jl) always moves
// up off the grid; a tie at x resolved upward is encoded as the float just
// below x.  The second word holds bf16(value(jl + 1)) << 16 | bf16(value(jl)).
//
// Rows: 0 RTN; 1-2 guided k=1 (gb 0, 1); 3-6 guided k=2 (gb 0..3);
//       7-14 full code (rollout magnitude index 0..7, sign checked apart).
// ---------------------------------------------------------------------------
constexpr int kRowRtn = 0, kRowK1 = 1, kRowK2 = 3, kRowFull = 7, kRows = 15;

constexpr float kGrid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
constexpr int kBucketFloor[kBuckets] = {0, 0, 0, 1, 1, 2, 3, 4, 5, 6, 7};

// One decision for an open bracket (value(jl), value(jl+1)).
struct Rule {
    char kind;      // 'L' keep jl, 'H' take jl + 1, 'T' threshold
    float x;        // threshold for 'T'
    bool tie_up;    // 'T': at |v| == x take jl + 1
};
constexpr Rule L{'L', 0.0f, false};
constexpr Rule H{'H', 0.0f, false};
constexpr Rule Tlo(float x) { return Rule{'T', x, false}; }
constexpr Rule Tup(float x) { return Rule{'T', x, true}; }

// RTN: nearest, ties to the even index (midpoint of each bracket).
constexpr Rule kRtn[7] = {Tlo(0.25f), Tup(0.75f), Tlo(1.25f), Tup(1.75f), Tlo(2.5f), Tup(3.5f), Tlo(5.0f)};

// Guided, derived from the rule of "TRACE Core Concept" with the rollout
// code reconstructed as the nearest code whose low k index bits equal gb:
//   k=1: gb 0 -> {0,1,2,4}, gb 1 -> {0.5,1.5,3,6};
//   k=2: gb 0 -> {0,2}, 1 -> {0.5,3}, 2 -> {1,4}, 3 -> {1.5,6};
// pick the bracket end nearer that code; a tie between two candidate codes
// falls back to RTN, which decides the tie side of each threshold.
constexpr Rule kGuidedK1[7][2] = {
    {L, H}, {H, L}, {L, H}, {H, L}, {L, Tlo(2.25f)}, {H, L}, {L, Tlo(4.5f)},
};
constexpr Rule kGuidedK2[7][4] = {
    {L, H, H, H},
    {L, L, H, H},
    {H, L, L, H},
    {H, Tup(1.75f), L, L},
    {L, H, Tlo(2.5f), L},
    {L, L, H, Tup(3.75f)},
    {L, L, L, H},
};

struct Entry {
    uint32_t thr;
    uint32_t vals;
};

constexpr uint32_t bits_of(float f) { return std::bit_cast<uint32_t>(f); }

constexpr Entry make_entry(Rule r, int jl)
{
    uint32_t lo = bits_of(kGrid[jl]) >> 16;
    uint32_t hi = bits_of(kGrid[jl < 7 ? jl + 1 : 7]) >> 16;
    uint32_t thr = 0x7f800000u;                        // +inf: keep jl
    if (jl < 7) {
        if (r.kind == 'H')
            thr = bits_of(kGrid[jl]);
        else if (r.kind == 'T')
            thr = bits_of(r.x) - (r.tie_up ? 1u : 0u);
    }
    return Entry{thr, (hi << 16) | lo};
}

struct Table {
    Entry e[kRows * kBuckets];
};

constexpr Table build_table()
{
    Table t{};
    for (int f = 0; f < kBuckets; ++f) {
        int jl = kBucketFloor[f];
        int b = jl < 7 ? jl : 0;
        t.e[kRowRtn * kBuckets + f] = make_entry(kRtn[b], jl);
        for (int gb = 0; gb < 2; ++gb)
            t.e[(kRowK1 + gb) * kBuckets + f] = make_entry(kGuidedK1[b][gb], jl);
        for (int gb = 0; gb < 4; ++gb)
            t.e[(kRowK2 + gb) * kBuckets + f] = make_entry(kGuidedK2[b][gb], jl);
        // full code: move up exactly when the rollout magnitude lies above jl
        // (same sign is checked per element)
        for (int r = 0; r < 8; ++r)
            t.e[(kRowFull + r) * kBuckets + f] = make_entry(r > jl ? H : L, jl);
    }
    return t;
}

__constant__ Table kTable = build_table();

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// Words hold two bf16; element 2m is the low half.
__device__ __forceinline__ float bf_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return as_f(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = as_u(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// E4M3 (OCP "FN") encode of t >= 0: nearest, ties to even, saturating at 448,
// subnormals kept.
__device__ __forceinline__ uint32_t e4m3_encode(float t)
{
    if (t >= 448.0f)
        return 0x7eu;
    if (t < 0.015625f)                                   // below 2^-6: step 2^-9
        return (uint32_t)__builtin_rintf(t * 512.0f);     // exact scaling, RNE
    uint32_t u = as_u(t);
    uint32_t r = u + 0x7ffffu + ((u >> 20) & 1u);        // RNE to 3 mantissa bits
    return (r >> 20) - (120u << 3);                      // rebias 127 -> 7
}

__device__ __forceinline__ float e4m3_decode(uint32_t c)
{
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    return e ? as_f(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Reciprocal of the combined scale c = s * g: 0 when c == 0, FLT_MAX when
// 1 / c overflows.  IEEE division (HIP's default correctly rounded path).
__device__ __forceinline__ float inv_combined(float s, float g)
{
    float c = s * g;
    if (!(c > 0.0f))
        return 0.0f;
    return fminf(1.0f / c, FLT_MAX);
}

// Block scale from the block amax and g (t = 0 when g == 0).
__device__ __forceinline__ uint32_t block_scale(float ab, float g)
{
    float t = 0.0f;
    if (g > 0.0f)
        t = ab / (6.0f * g);
    return e4m3_encode(t);
}

__device__ __forceinline__ int bucket_of(uint32_t mag)
{
    int f = (int)(mag >> 22) - 249;
    return min(max(f, 0), kBuckets - 1);
}

__device__ __forceinline__ uint32_t floor_index(int f)
{
    return f < 5 ? (uint32_t)(f >= 3) : (uint32_t)(f - 3);
}

// Unsigned division by an invariant d (Granlund & Montgomery 1994, Fig. 4.1).
struct DivMagic {
    uint32_t m, s1, s2;
};
__device__ __forceinline__ uint32_t div_magic(uint32_t n, DivMagic d)
{
    uint32_t t = __umulhi(d.m, n);
    return (t + ((n - t) >> d.s1)) >> d.s2;
}

struct Block16 {
    uint32_t w[8];
};

__device__ __forceinline__ Block16 load_block(const uint4 *p, uint32_t lb)
{
    uint4 a = p[2 * (size_t)lb];
    uint4 b = p[2 * (size_t)lb + 1];
    return Block16{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}

__device__ __forceinline__ float block_amax(const Block16 &x)
{
    uint32_t m = 0;
    for (int i = 0; i < 8; ++i) {
        uint32_t w = x.w[i] & 0x7fff7fffu;
        m = max(m, max(w & 0xffffu, w >> 16));
    }
    return as_f(m << 16);
}

// k low bits of each of 8 nibbles of w, packed LSB-first (k = 1 or 2).
__device__ __forceinline__ uint32_t compact_k2(uint32_t w)
{
    uint32_t x = w & 0x33333333u;
    x = (x | (x >> 2)) & 0x0f0f0f0fu;
    x = (x | (x >> 4)) & 0x00ff00ffu;
    return (x | (x >> 8)) & 0x0000ffffu;
}
__device__ __forceinline__ uint32_t compact_k1(uint32_t w)
{
    uint32_t x = w & 0x11111111u;
    x = (x | (x >> 3)) & 0x03030303u;
    x = (x | (x >> 6)) & 0x000f000fu;
    return (x | (x >> 12)) & 0x000000ffu;
}

// Per-element decision: returns the chosen nibble and the dequantised value.
// `row` selects the table row (already multiplied by kBuckets).
__device__ __forceinline__ float decide(const Entry *tab, uint32_t row, float v, float s, float g, uint32_t &nib,
                                        bool allow_up = true)
{
    uint32_t vb = as_u(v);
    uint32_t mag = vb & 0x7fffffffu;
    int f = bucket_of(mag);
    Entry e = tab[row + f];
    bool up = allow_up && (as_f(mag) > as_f(e.thr));
    float val = as_f(up ? (e.vals & 0xffff0000u) : (e.vals << 16));
    float y = (val * s) * g;
    nib = (floor_index(f) + (up ? 1u : 0u)) | ((vb >> 28) & 8u);
    return as_f(as_u(y) | (vb & 0x80000000u));
}

__device__ __forceinline__ void load_table(Entry *lds, int rows_lo, int rows_hi)
{
    for (int i = rows_lo * kBuckets + threadIdx.x; i < rows_hi * kBuckets; i += kThreads)
        lds[i] = kTable.e[i];
    __syncthreads();
}

struct OutPtr {
    void *y;
    int f32;
};

__device__ __forceinline__ void store_y(OutPtr o, uint32_t lb, const float (&y)[16])
{
    if (o.f32) {
        float4 *p = reinterpret_cast<float4 *>(o.y) + 4 * (size_t)lb;
        for (int q = 0; q < 4; ++q)
            p[q] = make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
    } else {
        uint32_t w[8];
        for (int i = 0; i < 8; ++i)
            w[i] = f32_to_bf16(y[2 * i]) | (f32_to_bf16(y[2 * i + 1]) << 16);
        uint4 *p = reinterpret_cast<uint4 *>(o.y) + 2 * (size_t)lb;
        p[0] = make_uint4(w[0], w[1], w[2], w[3]);
        p[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
}

// Global scale of the group holding lane-block lb (groups are bpg blocks
// long; the index is clamped to the last group so a read can never leave g).
template <bool kOneGroup>
__device__ __forceinline__ float group_scale(const float *g, uint32_t lb, DivMagic dm, uint32_t last)
{
    if (kOneGroup)
        return g[0];
    return g[min(div_magic(lb, dm), last)];
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

__global__ void k_amax_clear(uint32_t *g_bits, int G)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < G)
        g_bits[i] = 0u;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    for (int off = 32; off > 0; off >>= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

// Group amax as float bits (|bf16| << 16 orders like the float), atomicMax
// per wave on each group change.  Work items are (group, tile) pairs; each
// workgroup takes a contiguous range of items.
__global__ void __launch_bounds__(kThreads) k_amax(const uint4 *__restrict__ x, uint32_t bpg, uint32_t tiles_per_group,
                                                  uint64_t items, uint32_t *g_bits, int *status)
{
    uint64_t per_wg = (items + gridDim.x - 1) / gridDim.x;
    uint64_t w0 = (uint64_t)blockIdx.x * per_wg;
    uint64_t w1 = min(items, w0 + per_wg);
    uint32_t run = 0, bad = 0;
    int64_t cur = -1;
    for (uint64_t w = w0; w < w1; ++w) {
        uint32_t grp = (uint32_t)(w / tiles_per_group);
        uint32_t tile = (uint32_t)(w - (uint64_t)grp * tiles_per_group);
        if ((int64_t)grp != cur) {
            if (cur >= 0) {
                uint32_t m = wave_max(run);
                if ((threadIdx.x & 63) == 0 && m)
                    atomicMax(g_bits + cur, m);
            }
            cur = grp;
            run = 0;
        }
        uint32_t base = grp * bpg;
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t j = tile * kTile + u * kThreads + threadIdx.x;
            if (j < bpg) {
                Block16 b = load_block(x, base + j);
                for (int i = 0; i < 8; ++i) {
                    uint32_t lo = b.w[i] & 0x7fffu, hi = (b.w[i] >> 16) & 0x7fffu;
                    bool flo = lo < 0x7f80u, fhi = hi < 0x7f80u;
                    bad |= (!flo) | (!fhi);
                    run = max(run, max(flo ? lo << 16 : 0u, fhi ? hi << 16 : 0u));
                }
            }
        }
    }
    if (cur >= 0) {
        uint32_t m = wave_max(run);
        if ((threadIdx.x & 63) == 0 && m)
            atomicMax(g_bits + cur, m);
    }
    if (bad && status)
        *status = TRACE_E_NONFINITE;
}

__global__ void k_amax_finalize(float *g, int G)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < G)
        g[i] = g[i] / 2688.0f;                   // g[i] holds the amax bits
}

// Rollout: RTN codes, scale bytes, and (optionally) the guidance stream.
template <int K, bool kOneGroup>
__global__ void __launch_bounds__(kThreads)
    k_quant_rollout(const uint4 *__restrict__ y, uint32_t nblk, const float *__restrict__ g, DivMagic dm,
                    uint32_t last_group,
                    uint2 *__restrict__ codes, uint8_t *__restrict__ scales, uint8_t *__restrict__ gd_scales,
                    uint8_t *__restrict__ gd_bits, uint32_t pad_begin, uint32_t pad_end)
{
    __shared__ Entry tab[kRows * kBuckets];
    load_table(tab, kRowRtn, kRowRtn + 1);
    if (gd_scales && blockIdx.x == 0)
        for (uint32_t p = pad_begin + threadIdx.x; p < pad_end; p += kThreads)
            gd_scales[p] = 0;
    uint32_t ntiles = (nblk + kTile - 1) / kTile;
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        Block16 xb[kUnroll];
        uint32_t lbs[kUnroll];
        for (int u = 0; u < kUnroll; ++u) {
            lbs[u] = t * kTile + u * kThreads + threadIdx.x;
            if (lbs[u] < nblk)
                xb[u] = load_block(y, lbs[u]);
        }
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t lb = lbs[u];
            if (lb >= nblk)
                continue;
            float gg = group_scale<kOneGroup>(g, lb, dm, last_group);
            uint32_t sc = block_scale(block_amax(xb[u]), gg);
            float s = e4m3_decode(sc);
            float inv = inv_combined(s, gg);
            uint32_t nw[2] = {0u, 0u};
            for (int i = 0; i < 16; ++i) {
                uint32_t w = xb[u].w[i >> 1];
                float v = ((i & 1) ? bf_hi(w) : bf_lo(w)) * inv;
                uint32_t nib;
                decide(tab, kRowRtn * kBuckets, v, s, gg, nib);
                nw[i >> 3] |= nib << (4 * (i & 7));
            }
            codes[lb] = make_uint2(nw[0], nw[1]);
            scales[lb] = (uint8_t)sc;
            if (gd_scales) {
                gd_scales[lb] = (uint8_t)sc;
                if (K == 4)
                    reinterpret_cast<uint2 *>(gd_bits)[lb] = make_uint2(nw[0], nw[1]);
                else if (K == 2)
                    reinterpret_cast<uint32_t *>(gd_bits)[lb] = compact_k2(nw[0]) | (compact_k2(nw[1]) << 16);
                else
                    reinterpret_cast<uint16_t *>(gd_bits)[lb] = (uint16_t)(compact_k1(nw[0]) | (compact_k1(nw[1]) << 8));
            }
        }
    }
}

// Guidance stream from codes + scales.
template <int K>
__global__ void __launch_bounds__(kThreads)
    k_guidance_pack(const uint2 *__restrict__ codes, const uint8_t *__restrict__ scales, uint32_t nblk,
                    uint8_t *__restrict__ gd_scales, uint8_t *__restrict__ gd_bits, uint32_t pad_begin,
                    uint32_t pad_end)
{
    if (blockIdx.x == 0)
        for (uint32_t p = pad_begin + threadIdx.x; p < pad_end; p += kThreads)
            gd_scales[p] = 0;
    for (uint32_t lb = blockIdx.x * kThreads + threadIdx.x; lb < nblk; lb += gridDim.x * kThreads) {
        uint2 c = codes[lb];
        gd_scales[lb] = scales[lb];
        if (K == 4)
            reinterpret_cast<uint2 *>(gd_bits)[lb] = c;
        else if (K == 2)
            reinterpret_cast<uint32_t *>(gd_bits)[lb] = compact_k2(c.x) | (compact_k2(c.y) << 16);
        else
            reinterpret_cast<uint16_t *>(gd_bits)[lb] = (uint16_t)(compact_k1(c.x) | (compact_k1(c.y) << 8));
    }
}

// Training side.  MODE: 1, 2 = guided with k bits; 4 = full code;
// 0 = RTN with shared scales (from the scale plane / scales_in);
// 5 = RTN with own scales computed from x.
template <int MODE, bool kOneGroup, bool kCodes>
__global__ void __launch_bounds__(kThreads)
    k_fakequant(const uint4 *x, uint32_t nblk, const float *__restrict__ g, DivMagic dm, uint32_t last_group,
                const uint8_t *__restrict__ scale_plane, const uint8_t *__restrict__ bits, OutPtr out,
                uint2 *__restrict__ codes_out, uint8_t *__restrict__ scales_out)
{
    __shared__ Entry tab[kRows * kBuckets];
    constexpr int lo = MODE == 1 ? kRowK1 : MODE == 2 ? kRowK2 : MODE == 4 ? kRowFull : kRowRtn;
    constexpr int hi = MODE == 1 ? kRowK1 + 2 : MODE == 2 ? kRowK2 + 4 : MODE == 4 ? kRowFull + 8 : kRowRtn + 1;
    load_table(tab, lo, hi);
    uint32_t ntiles = (nblk + kTile - 1) / kTile;
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        Block16 xb[kUnroll];
        uint32_t lbs[kUnroll], sc[kUnroll];
        uint2 gb[kUnroll];
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t lb = t * kTile + u * kThreads + threadIdx.x;
            lbs[u] = lb;
            if (lb < nblk) {
                xb[u] = load_block(x, lb);
                if (MODE != 5)
                    sc[u] = scale_plane[lb];
                if (MODE == 1)
                    gb[u] = make_uint2(reinterpret_cast<const uint16_t *>(bits)[lb], 0u);
                else if (MODE == 2)
                    gb[u] = make_uint2(reinterpret_cast<const uint32_t *>(bits)[lb], 0u);
                else if (MODE == 4)
                    gb[u] = reinterpret_cast<const uint2 *>(bits)[lb];
            }
        }
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t lb = lbs[u];
            if (lb >= nblk)
                continue;
            float gg = group_scale<kOneGroup>(g, lb, dm, last_group);
            uint32_t s8 = MODE == 5 ? block_scale(block_amax(xb[u]), gg) : (sc[u] & 0x7fu);
            float s = e4m3_decode(s8);
            float inv = inv_combined(s, gg);
            float yv[16];
            uint32_t nw[2] = {0u, 0u};
            for (int i = 0; i < 16; ++i) {
                uint32_t w = xb[u].w[i >> 1];
                float v = ((i & 1) ? bf_hi(w) : bf_lo(w)) * inv;
                uint32_t row, nib;
                bool allow = true;
                if (MODE == 1) {
                    row = (kRowK1 + ((gb[u].x >> i) & 1u)) * kBuckets;
                } else if (MODE == 2) {
                    row = (kRowK2 + ((gb[u].x >> (2 * i)) & 3u)) * kBuckets;
                } else if (MODE == 4) {
                    uint32_t r = ((i < 8 ? gb[u].x : gb[u].y) >> (4 * (i & 7))) & 0xfu;
                    row = (kRowFull + (r & 7u)) * kBuckets;
                    allow = ((r >> 3) == (as_u(v) >> 31));
                } else {
                    row = kRowRtn * kBuckets;
                }
                yv[i] = decide(tab, row, v, s, gg, nib, allow);
                nw[i >> 3] |= nib << (4 * (i & 7));
            }
            store_y(out, lb, yv);
            if (kCodes)
                codes_out[lb] = make_uint2(nw[0], nw[1]);
            if (MODE == 5 && scales_out)
                scales_out[lb] = (uint8_t)s8;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int64_t kMaxN = int64_t(1) << 36;

DivMagic make_div_magic(uint32_t d)
{
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < d)
        ++l;
    uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return DivMagic{(uint32_t)m, l < 1 ? l : 1u, l > 0 ? l - 1 : 0u};
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_sizes(int64_t n, int G)
{
    if (n <= 0 || n % 16 != 0 || n >= kMaxN)
        return TRACE_E_SIZE;
    if (G < 1 || n % (16 * (int64_t)G) != 0)
        return TRACE_E_SIZE;
    return TRACE_OK;
}

int grid_for(uint32_t nblk)
{
    uint32_t tiles = (nblk + kTile - 1) / kTile;
    return (int)(tiles < (uint32_t)kMaxGrid ? tiles : (uint32_t)kMaxGrid);
}

int launched()
{
    return hipGetLastError() == hipSuccess ? TRACE_OK : TRACE_E_HIP;
}

int64_t bitplane_offset(int64_t n) { return (n / 16 + 255) / 256 * 256; }

template <int MODE, bool kOneGroup>
void launch_fq(dim3 grid, hipStream_t st, const uint4 *x, uint32_t nblk, const float *g, DivMagic dm,
               uint32_t last, const uint8_t *sp, const uint8_t *bits, OutPtr out, uint2 *codes, uint8_t *scales_out)
{
    if (codes)
        hipLaunchKernelGGL((k_fakequant<MODE, kOneGroup, true>), grid, dim3(kThreads), 0, st, x, nblk, g, dm, last,
                           sp, bits, out, codes, scales_out);
    else
        hipLaunchKernelGGL((k_fakequant<MODE, kOneGroup, false>), grid, dim3(kThreads), 0, st, x, nblk, g, dm, last,
                           sp, bits, out, codes, scales_out);
}

template <int MODE>
int fakequant_any(const void *x, int64_t n, int G, const float *g, const uint8_t *sp, const uint8_t *bits, void *y,
                  int out_dtype, uint8_t *codes, uint8_t *scales_out, void *stream)
{
    uint32_t nblk = (uint32_t)(n / 16);
    DivMagic dm = make_div_magic(nblk / (uint32_t)G);
    dim3 grid(grid_for(nblk));
    hipStream_t st = (hipStream_t)stream;
    OutPtr out{y, out_dtype == TRACE_OUT_F32};
    (void)hipGetLastError();
    if (G == 1)
        launch_fq<MODE, true>(grid, st, (const uint4 *)x, nblk, g, dm, 0u, sp, bits, out, (uint2 *)codes,
                              scales_out);
    else
        launch_fq<MODE, false>(grid, st, (const uint4 *)x, nblk, g, dm, (uint32_t)G - 1u, sp, bits, out,
                               (uint2 *)codes, scales_out);
    return launched();
}

int check_common(const void *x, int64_t n, int G, const float *g, void *y, int out_dtype)
{
    int rc = check_sizes(n, G);
    if (rc)
        return rc;
    if (!x || !g || !y)
        return TRACE_E_NULL;
    if (!aligned16(x) || !aligned16(g) || !aligned16(y))
        return TRACE_E_ALIGN;
    if (out_dtype != TRACE_OUT_BF16 && out_dtype != TRACE_OUT_F32)
        return TRACE_E_DTYPE;
    return TRACE_OK;
}

}  // namespace

extern "C" {

size_t trace_code_bytes(int64_t n) { return check_sizes(n, 1) ? 0 : (size_t)(n / 2); }

size_t trace_scale_bytes(int64_t n) { return check_sizes(n, 1) ? 0 : (size_t)(n / 16); }

size_t trace_guidance_bytes(int64_t n, int k)
{
    if (check_sizes(n, 1) || (k != 1 && k != 2 && k != 4))
        return 0;
    return (size_t)(bitplane_offset(n) + n * k / 8);
}

int trace_amax(const void *x_bf16, int64_t n, int G, float *g_out, int *status_dev, void *stream)
{
    int rc = check_sizes(n, G);
    if (rc)
        return rc;
    if (!x_bf16 || !g_out)
        return TRACE_E_NULL;
    if (!aligned16(x_bf16) || !aligned16(g_out) || (status_dev && !aligned16(status_dev)))
        return TRACE_E_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    uint32_t nblk = (uint32_t)(n / 16), bpg = nblk / (uint32_t)G;
    uint32_t tpg = (bpg + kTile - 1) / kTile;
    uint64_t items = (uint64_t)tpg * (uint64_t)G;
    int grid = (int)(items < (uint64_t)kMaxGrid ? items : (uint64_t)kMaxGrid);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_amax_clear, dim3((G + 255) / 256), dim3(256), 0, st, (uint32_t *)g_out, G);
    hipLaunchKernelGGL(k_amax, dim3(grid), dim3(kThreads), 0, st, (const uint4 *)x_bf16, bpg, tpg, items,
                       (uint32_t *)g_out, status_dev);
    hipLaunchKernelGGL(k_amax_finalize, dim3((G + 255) / 256), dim3(256), 0, st, g_out, G);
    return launched();
}

int trace_quant_rollout(const void *y_bf16, int64_t n, int G, const float *g, int k, uint8_t *codes, uint8_t *scales,
                        uint8_t *guidance, void *stream)
{
    int rc = check_sizes(n, G);
    if (rc)
        return rc;
    if (!y_bf16 || !g || !codes || !scales)
        return TRACE_E_NULL;
    if (!aligned16(y_bf16) || !aligned16(g) || !aligned16(codes) || !aligned16(scales) ||
        (guidance && !aligned16(guidance)))
        return TRACE_E_ALIGN;
    if (k != 1 && k != 2 && k != 4)
        return TRACE_E_K;
    uint32_t nblk = (uint32_t)(n / 16);
    DivMagic dm = make_div_magic(nblk / (uint32_t)G);
    dim3 grid(grid_for(nblk));
    hipStream_t st = (hipStream_t)stream;
    uint8_t *bits = guidance ? guidance + bitplane_offset(n) : nullptr;
    uint32_t pb = nblk, pe = (uint32_t)bitplane_offset(n);
    (void)hipGetLastError();
#define TRACE_LAUNCH_ROLLOUT(KK, ONE)                                                                            \
    hipLaunchKernelGGL((k_quant_rollout<KK, ONE>), grid, dim3(kThreads), 0, st, (const uint4 *)y_bf16, nblk, g, dm, \
                       (uint32_t)G - 1u, (uint2 *)codes, scales, guidance, bits, pb, pe)
    if (G == 1) {
        if (k == 1) TRACE_LAUNCH_ROLLOUT(1, true);
        else if (k == 2) TRACE_LAUNCH_ROLLOUT(2, true);
        else TRACE_LAUNCH_ROLLOUT(4, true);
    } else {
        if (k == 1) TRACE_LAUNCH_ROLLOUT(1, false);
        else if (k == 2) TRACE_LAUNCH_ROLLOUT(2, false);
        else TRACE_LAUNCH_ROLLOUT(4, false);
    }
#undef TRACE_LAUNCH_ROLLOUT
    return launched();
}

int trace_guidance_pack(const uint8_t *codes, const uint8_t *scales, int64_t n, int k, uint8_t *guidance, void *stream)
{
    int rc = check_sizes(n, 1);
    if (rc)
        return rc;
    if (!codes || !scales || !guidance)
        return TRACE_E_NULL;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(guidance))
        return TRACE_E_ALIGN;
    if (k != 1 && k != 2 && k != 4)
        return TRACE_E_K;
    uint32_t nblk = (uint32_t)(n / 16);
    uint32_t wgs = (nblk + kThreads - 1) / kThreads;
    dim3 grid(wgs < (uint32_t)kMaxGrid ? wgs : (uint32_t)kMaxGrid);
    hipStream_t st = (hipStream_t)stream;
    uint8_t *bits = guidance + bitplane_offset(n);
    uint32_t pb = nblk, pe = (uint32_t)bitplane_offset(n);
    (void)hipGetLastError();
    if (k == 1)
        hipLaunchKernelGGL((k_guidance_pack<1>), grid, dim3(kThreads), 0, st, (const uint2 *)codes, scales, nblk,
                           guidance, bits, pb, pe);
    else if (k == 2)
        hipLaunchKernelGGL((k_guidance_pack<2>), grid, dim3(kThreads), 0, st, (const uint2 *)codes, scales, nblk,
                           guidance, bits, pb, pe);
    else
        hipLaunchKernelGGL((k_guidance_pack<4>), grid, dim3(kThreads), 0, st, (const uint2 *)codes, scales, nblk,
                           guidance, bits, pb, pe);
    return launched();
}

int trace_fakequant_guided(const void *x_bf16, int64_t n, int G, const float *g, const uint8_t *guidance, int k,
                           void *y_out, int out_dtype, uint8_t *codes_out, void *stream)
{
    int rc = check_common(x_bf16, n, G, g, y_out, out_dtype);
    if (rc)
        return rc;
    if (!guidance)
        return TRACE_E_NULL;
    if (!aligned16(guidance) || (codes_out && !aligned16(codes_out)))
        return TRACE_E_ALIGN;
    if (k != 1 && k != 2)
        return TRACE_E_K;
    const uint8_t *bits = guidance + bitplane_offset(n);
    if (k == 1)
        return fakequant_any<1>(x_bf16, n, G, g, guidance, bits, y_out, out_dtype, codes_out, nullptr, stream);
    return fakequant_any<2>(x_bf16, n, G, g, guidance, bits, y_out, out_dtype, codes_out, nullptr, stream);
}

int trace_fakequant_fullcode(const void *x_bf16, int64_t n, int G, const float *g, const uint8_t *guidance,
                             void *y_out, int out_dtype, uint8_t *codes_out, void *stream)
{
    int rc = check_common(x_bf16, n, G, g, y_out, out_dtype);
    if (rc)
        return rc;
    if (!guidance)
        return TRACE_E_NULL;
    if (!aligned16(guidance) || (codes_out && !aligned16(codes_out)))
        return TRACE_E_ALIGN;
    const uint8_t *bits = guidance + bitplane_offset(n);
    return fakequant_any<4>(x_bf16, n, G, g, guidance, bits, y_out, out_dtype, codes_out, nullptr, stream);
}

int trace_fakequant_rtn(const void *x_bf16, int64_t n, int G, const float *g, const uint8_t *scales_in, void *y_out,
                        int out_dtype, uint8_t *codes_out, uint8_t *scales_out, void *stream)
{
    int rc = check_common(x_bf16, n, G, g, y_out, out_dtype);
    if (rc)
        return rc;
    if ((scales_in && !aligned16(scales_in)) || (codes_out && !aligned16(codes_out)) ||
        (scales_out && !aligned16(scales_out)))
        return TRACE_E_ALIGN;
    if (scales_in) {
        rc = fakequant_any<0>(x_bf16, n, G, g, scales_in, nullptr, y_out, out_dtype, codes_out, nullptr, stream);
        if (rc == TRACE_OK && scales_out)
            rc = hipMemcpyAsync(scales_out, scales_in, (size_t)(n / 16), hipMemcpyDeviceToDevice,
                                (hipStream_t)stream) == hipSuccess
                     ? TRACE_OK
                     : TRACE_E_HIP;
        return rc;
    }
    return fakequant_any<5>(x_bf16, n, G, g, nullptr, nullptr, y_out, out_dtype, codes_out, scales_out, stream);
}

const char *trace_status_str(int status)
{
    switch (status) {
    case TRACE_OK: return "ok";
    case TRACE_E_NULL: return "a required pointer is NULL";
    case TRACE_E_SIZE: return "n or G violates the size rules (n > 0, n % 16 == 0, n % (16 G) == 0, n < 2^36)";
    case TRACE_E_ALIGN: return "a pointer is not 16-byte aligned";
    case TRACE_E_K: return "unsupported guidance width k";
    case TRACE_E_DTYPE: return "unknown output dtype";
    case TRACE_E_HIP: return "HIP runtime error";
    case TRACE_E_NONFINITE: return "an input was inf or NaN";
    default: return "unknown status";
    }
}

int trace_version(void) { return 100; }

}  // extern "C"
