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
//   * one 8-element chunk per lane: a single 16-byte non-temporal load of bf16
//     per lane, contiguous across the wavefront (a 16-byte-per-lane stream
//     reaches ~6.1 TB/s on MI355X, 32 bytes per lane only ~5.5);
//   * a 16-element block spans a lane pair: the block amax is a packed 16-bit
//     max within the lane plus one DPP swap with the neighbour lane, so both
//     lanes hold the block scale and its reciprocal in registers;
//   * codes, scale bytes and guidance bits are packed in registers and
//     written with one store per lane per plane (4, 1 and k bytes; scale
//     bytes from the even lane), contiguous across the wavefront;
//   * RTN to E2M1 uses gfx950's v_cvt_scalef32_pk_fp4_f32 with scale 1.0
//     (two elements per instruction, nibbles packed in place) and the
//     matching v_cvt_scalef32_pk_f32_fp4 to decode; bf16 outputs use
//     v_cvt_pk_bf16_f32.  With scale 1.0 both conversions equal round to
//     nearest even on every finite fp32 input (checked exhaustively);
//   * the guided decision is one fp32 compare against a threshold read from
//     a small LDS table indexed by (bucket of |v|, guidance value): chosen
//     index = floor index + (|v| > threshold);
//   * streaming kernels launch one tile of 256 x kUnroll chunks per
//     workgroup (many small workgroups balance best across the 8 XCDs).
#include <hip/hip_runtime.h>

#include <bit>
#include <cfloat>
#include <cstdint>

#include "trace_quant.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Launch shape and cache hints (fixed at build time; the values below are the
// measured best on MI355X for the 64x512x2048 activation workload).
#ifndef TRACE_UNROLL
#define TRACE_UNROLL 2
#endif
#ifndef TRACE_WG_PER_CU
#define TRACE_WG_PER_CU 0
#endif
#ifndef TRACE_NT_LOAD
#define TRACE_NT_LOAD 1
#endif
#ifndef TRACE_NT_STORE
#define TRACE_NT_STORE 0
#endif
#ifndef TRACE_PAIR_SPLIT
#define TRACE_PAIR_SPLIT 1
#endif


constexpr int kThreads = 256;          // 4 wavefronts of 64
constexpr int kUnroll = TRACE_UNROLL;  // chunks per thread per tile
constexpr int kTile = kThreads * kUnroll;
constexpr int kMaxGrid = TRACE_WG_PER_CU > 0 ? 256 * TRACE_WG_PER_CU : 0x7fffffff;
#ifndef TRACE_AMAX_THREADS
#define TRACE_AMAX_THREADS 1024
#endif
#ifndef TRACE_AMAX_UNROLL
#define TRACE_AMAX_UNROLL 4
#endif
#ifndef TRACE_AMAX_GRID
#define TRACE_AMAX_GRID 512
#endif
constexpr int kAmaxThreads = TRACE_AMAX_THREADS;   // amax: two 1024-thread workgroups per CU ...
constexpr int kAmaxUnroll = TRACE_AMAX_UNROLL;     // ... chunks in flight per lane ...
constexpr int kAmaxTile = kAmaxThreads * kAmaxUnroll;
constexpr int kAmaxGrid = TRACE_AMAX_GRID;         // ... and persistent grid
constexpr int kBuckets = 11;           // buckets of |v| (see decide)
static_assert(!TRACE_PAIR_SPLIT || kUnroll == 2, "the lane-pair split of the block-scale work needs two chunks per lane");
constexpr int kSlots = 16;             // table slots per row (bucket -> slot)

// ---------------------------------------------------------------------------
// Guided decision tables.
//
// |v| is split into 11 buckets by its fp32 exponent and top mantissa bit:
//   [0,.25) [.25,.375) [.375,.5) [.5,.75) [.75,1) [1,1.5) [1.5,2) [2,3)
//   [3,4) [4,6) [6,inf]
// Within a bucket the floor E2M1 index jl is fixed (0 0 0 1 1 2 3 4 5 6 7)
// and the upper neighbour is jl + 1.  For each (bucket, row) the table holds
// a threshold T: the chosen index is jl + (|v| > T).  T >= value(jl), so an
// on-grid |v| keeps jl; T = +inf always keeps jl; T = value(jl) always moves
// up off the grid; a tie at x resolved upward is encoded as the float just
// below x.  The second word holds bf16(value(jl + 1)) << 16 | bf16(value(jl)).
// Bucket f is found from c = clamp(|v|, 0.2, 6): bits(c) >> 22 runs over
// 249 .. 259, and its low 4 bits, slot = (249 + f) & 15, are distinct, so the
// table has 16 slots (slots 4 .. 8 unused) and the address needs no offset.
// Layout: entry index = slot * rows + row; rows = 2 (k=1: gb), 4 (k=2: gb),
// 8 (full code: rollout magnitude index, the sign is checked apart).
// ---------------------------------------------------------------------------
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

template <int R>
struct Table {
    Entry e[kSlots * R];
};

// mode: 1 = guided k=1, 2 = guided k=2, 4 = full code
template <int MODE, int R>
constexpr Table<R> build_table()
{
    Table<R> t{};
    for (int f = 0; f < kBuckets; ++f) {
        int jl = kBucketFloor[f];
        int b = jl < 7 ? jl : 0;
        for (int r = 0; r < R; ++r) {
            Rule rule = MODE == 1 ? kGuidedK1[b][r] : MODE == 2 ? kGuidedK2[b][r] : (r > jl ? H : L);
            t.e[((249 + f) & 15) * R + r] = make_entry(rule, jl);
        }
    }
    return t;
}

__constant__ Table<2> kTabK1 = build_table<1, 2>();
__constant__ Table<4> kTabK2 = build_table<2, 4>();
__constant__ Table<8> kTabFull = build_table<4, 8>();

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// Words hold two bf16; element 2m is the low half.
__device__ __forceinline__ float bf_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return as_f(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
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

// Unsigned division by an invariant d (Granlund & Montgomery 1994, Fig. 4.1).
struct DivMagic {
    uint32_t m, s1, s2;
};
__device__ __forceinline__ uint32_t div_magic(uint32_t n, DivMagic d)
{
    uint32_t t = __umulhi(d.m, n);
    return (t + ((n - t) >> d.s1)) >> d.s2;
}

// Global scale of the group holding block blk (groups are bpg blocks long;
// the index is clamped to the last group so a read can never leave g).
template <bool kOneGroup>
__device__ __forceinline__ float group_scale(const float *g, uint32_t blk, DivMagic dm, uint32_t last)
{
    if (kOneGroup)
        return g[0];
    return g[min(div_magic(blk, dm), last)];
}

template <class T>
__device__ __forceinline__ T ld_stream(const T *p)
{
#if TRACE_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <class T>
__device__ __forceinline__ void st_stream(T v, T *p)
{
#if TRACE_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// 8 consecutive bf16 elements: element 2m is the low half of w[m].
struct Chunk {
    uint32_t w[4];
};

__device__ __forceinline__ Chunk load_chunk(const u32x4 *p, uint32_t c)
{
    u32x4 a = ld_stream(p + c);
    return Chunk{{a.x, a.y, a.z, a.w}};
}

// max |x| over the chunk, as bf16 magnitude bits (finite inputs).
__device__ __forceinline__ uint32_t chunk_amax_bits(const Chunk &x)
{
    u16x2 m = __builtin_bit_cast(u16x2, x.w[0] & 0x7fff7fffu);
    for (int i = 1; i < 4; ++i)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, x.w[i] & 0x7fff7fffu));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// Combine with the neighbour lane (lane ^ 1) that holds the other half of the
// block: DPP quad_perm [1,0,3,2].  Both lanes of a pair are always active
// together (chunk counts are even and tiles start at even chunks).
__device__ __forceinline__ uint32_t pair_max(uint32_t m)
{
    return max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xb1, 0xf, 0xf, false));
}

// Value of the neighbour lane (lane ^ 1).
__device__ __forceinline__ uint32_t pair_swap(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false);
}

// Per-block scale work of a lane's two chunks (u = 0, 1), split across the
// lane pair that shares their two blocks: the even lane derives block 0, the
// odd lane block 1, and one DPP swap per value hands each lane the other.
struct PairScales {
    uint32_t sc[2];
    float s[2], inv[2];
};

__device__ __forceinline__ PairScales pair_scales_from_amax(uint32_t ab0, uint32_t ab1, float g0, float g1)
{
    bool odd = threadIdx.x & 1u;
    float gm = odd ? g1 : g0;
    uint32_t sc = block_scale(as_f((odd ? ab1 : ab0) << 16), gm);
    float s = e4m3_decode(sc);
    float inv = inv_combined(s, gm);
    uint32_t sc_o = pair_swap(sc), s_o = pair_swap(as_u(s)), inv_o = pair_swap(as_u(inv));
    PairScales r;
    r.sc[0] = odd ? sc_o : sc;
    r.sc[1] = odd ? sc : sc_o;
    r.s[0] = odd ? as_f(s_o) : s;
    r.s[1] = odd ? s : as_f(s_o);
    r.inv[0] = odd ? as_f(inv_o) : inv;
    r.inv[1] = odd ? inv : as_f(inv_o);
    return r;
}

__device__ __forceinline__ PairScales pair_scales_from_bytes(uint32_t sc0, uint32_t sc1, float g0, float g1)
{
    bool odd = threadIdx.x & 1u;
    float gm = odd ? g1 : g0;
    uint32_t sc = (odd ? sc1 : sc0) & 0x7fu;
    float s = e4m3_decode(sc);
    float inv = inv_combined(s, gm);
    uint32_t s_o = pair_swap(as_u(s)), inv_o = pair_swap(as_u(inv));
    PairScales r;
    r.sc[0] = sc0 & 0x7fu;
    r.sc[1] = sc1 & 0x7fu;
    r.s[0] = odd ? as_f(s_o) : s;
    r.s[1] = odd ? s : as_f(s_o);
    r.inv[0] = odd ? as_f(inv_o) : inv;
    r.inv[1] = odd ? inv : as_f(inv_o);
    return r;
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

// RTN of the 8 elements of a chunk times inv into 8 nibbles (element 2m low).
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds to nearest, ties to the
// even E2M1 mantissa, saturates at +-6 and keeps the sign (also of -0).
__device__ __forceinline__ uint32_t rtn8(const Chunk &x, float inv)
{
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf_lo(x.w[0]) * inv, bf_hi(x.w[0]) * inv, 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf_lo(x.w[1]) * inv, bf_hi(x.w[1]) * inv, 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf_lo(x.w[2]) * inv, bf_hi(x.w[2]) * inv, 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf_lo(x.w[3]) * inv, bf_hi(x.w[3]) * inv, 1.0f, 3);
    return r;
}

// Signed E2M1 values of the 8 nibbles of r (v_cvt_scalef32_pk_f32_fp4, scale 1).
__device__ __forceinline__ void decode8(uint32_t r, float *out)
{
    f32x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r, 1.0f, 0);
    f32x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r, 1.0f, 1);
    f32x2 d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r, 1.0f, 2);
    f32x2 d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r, 1.0f, 3);
    out[0] = d0.x; out[1] = d0.y; out[2] = d1.x; out[3] = d1.y;
    out[4] = d2.x; out[5] = d2.y; out[6] = d3.x; out[7] = d3.y;
}

// Floor E2M1 index of bucket f (0 0 0 1 1 2 3 4 5 6 7), from its slot.
__device__ __forceinline__ uint32_t floor_index_of_slot(uint32_t slot)
{
    uint32_t f = (slot - 9u) & 15u;
    return (f >= 3u ? 1u : 0u) + (f > 4u ? f - 4u : 0u);
}

// Bits of the chosen value: the high bf16 of `vals` when up, else the low
// one, moved to the top half (v_perm_b32 byte select).
__device__ __forceinline__ uint32_t pick_half(uint32_t vals, bool up)
{
    return __builtin_amdgcn_perm(0u, vals, up ? 0x03020c0cu : 0x01000c0cu);
}

// Guided / full-code decision for one element.  `row` is the guidance value
// (gb, or the rollout magnitude index for full code); `allow` is false when
// the full-code sign disagrees (then the point nearer zero is kept).
template <int R, bool kCodes>
__device__ __forceinline__ float decide(const Entry *tab, float v, uint32_t row, bool allow, float s, float g,
                                        uint32_t &nib)
{
    float a = fabsf(v);
    float c = __builtin_amdgcn_fmed3f(a, 0.2f, 6.0f);   // bucket clamp
    uint32_t slot = (as_u(c) >> 22) & 15u;
    Entry e = tab[slot * R + row];
    bool up = allow && (a > as_f(e.thr));
    float val = as_f(pick_half(e.vals, up));
    float y = (val * s) * g;
    if (kCodes)
        nib = (floor_index_of_slot(slot) + (up ? 1u : 0u)) | ((as_u(v) >> 28) & 8u);
    return as_f(as_u(y) | (as_u(v) & 0x80000000u));
}

struct OutPtr {
    void *y;
    int f32;
};

__device__ __forceinline__ void store_y(OutPtr o, uint32_t c, const float (&y)[8])
{
    if (o.f32) {
        f32x4 *p = reinterpret_cast<f32x4 *>(o.y) + 2 * (size_t)c;
        st_stream(f32x4{y[0], y[1], y[2], y[3]}, p);
        st_stream(f32x4{y[4], y[5], y[6], y[7]}, p + 1);
    } else {
        u32x4 w = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
        st_stream(w, reinterpret_cast<u32x4 *>(o.y) + c);
    }
}

template <int R>
__device__ __forceinline__ void load_table(Entry *lds, const Entry *src)
{
    for (int i = threadIdx.x; i < kSlots * R; i += kThreads)
        lds[i] = src[i];
    __syncthreads();
}

// Zero the pad between the scale plane and the bit plane of a guidance stream.
__device__ __forceinline__ void zero_pad(uint8_t *gd, uint32_t begin, uint32_t end)
{
    if (blockIdx.x == 0)
        for (uint32_t p = begin + threadIdx.x; p < end; p += kThreads)
            gd[p] = 0;
}

// Guidance bits of one chunk (8 codes in cw): k = 1 -> 1 byte, 2 -> 2 bytes,
// 4 -> the 4 code bytes.
template <int K>
__device__ __forceinline__ void store_bits(uint8_t *gd_bits, uint32_t c, uint32_t cw)
{
    if (K == 4)
        reinterpret_cast<uint32_t *>(gd_bits)[c] = cw;
    else if (K == 2)
        reinterpret_cast<uint16_t *>(gd_bits)[c] = (uint16_t)compact_k2(cw);
    else
        gd_bits[c] = (uint8_t)compact_k1(cw);
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

// Fold the workgroup's running max and raise the group's word with one atomic
// max, skipped when the word already holds a value at least as large.
__device__ __forceinline__ void amax_publish(uint32_t run, uint32_t *wmax, uint32_t *word)
{
    uint32_t m = run;
    for (int off = 32; off > 0; off >>= 1)
        m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    if ((threadIdx.x & 63) == 0)
        wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = 0;
        for (int i = 0; i < kAmaxThreads / 64; ++i)
            b = max(b, wmax[i]);
        b <<= 16;
        if (b > __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMax(word, b);
    }
    __syncthreads();
}

// Group amax as float bits (|bf16| << 16 orders like the float).  Work items
// are (group, tile) pairs walked grid-stride; each thread keeps a running max
// for the current group and the workgroup publishes it when the group changes
// and at the end.  Non-finite inputs are left out and flagged.
__global__ void __launch_bounds__(kAmaxThreads)
    k_amax(const u32x4 *__restrict__ x, uint32_t cpg, uint32_t tiles_per_group, uint32_t items,
           uint32_t *g_bits, int *status)
{
    __shared__ uint32_t wmax[kAmaxThreads / 64];
    uint32_t run = 0;
    uint32_t cur = 0xffffffffu;
    for (uint32_t w = blockIdx.x; w < items; w += gridDim.x) {
        uint32_t grp = w / tiles_per_group;
        uint32_t tile = w - grp * tiles_per_group;
        if (grp != cur) {
            if (cur != 0xffffffffu) {
                amax_publish(run, wmax, g_bits + cur);
                run = 0;
            }
            cur = grp;
        }
        uint32_t base = grp * cpg;
        Chunk b[kAmaxUnroll];
        bool ok[kAmaxUnroll];
        for (int u = 0; u < kAmaxUnroll; ++u) {
            uint32_t j = tile * kAmaxTile + u * kAmaxThreads + threadIdx.x;
            ok[u] = j < cpg;
            if (ok[u])
                b[u] = load_chunk(x, base + j);
        }
        for (int u = 0; u < kAmaxUnroll; ++u) {
            if (!ok[u])
                continue;
            uint32_t m = chunk_amax_bits(b[u]);
            if (m >= 0x7f80u) {                            // rare: an inf or NaN in the chunk
                m = 0;
                for (int i = 0; i < 4; ++i) {
                    uint32_t lo = b[u].w[i] & 0x7fffu, hi = (b[u].w[i] >> 16) & 0x7fffu;
                    m = max(m, max(lo < 0x7f80u ? lo : 0u, hi < 0x7f80u ? hi : 0u));
                }
                if (status)
                    *status = TRACE_E_NONFINITE;
            }
            run = max(run, m);
        }
    }
    if (cur != 0xffffffffu)
        amax_publish(run, wmax, g_bits + cur);
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
    k_quant_rollout(const u32x4 *__restrict__ y, uint32_t nchunk, const float *__restrict__ g, DivMagic dm,
                    uint32_t last_group, uint32_t *__restrict__ codes, uint8_t *__restrict__ scales,
                    uint8_t *__restrict__ gd_scales, uint8_t *__restrict__ gd_bits, uint32_t pad_begin,
                    uint32_t pad_end)
{
    if (gd_scales)
        zero_pad(gd_scales, pad_begin, pad_end);
    uint32_t ntiles = (nchunk + kTile - 1) / kTile;
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        Chunk xc[kUnroll];
        uint32_t cs[kUnroll];
        for (int u = 0; u < kUnroll; ++u) {
            cs[u] = t * kTile + u * kThreads + threadIdx.x;
            xc[u] = cs[u] < nchunk ? load_chunk(y, cs[u]) : Chunk{{0u, 0u, 0u, 0u}};
        }
        if (cs[0] >= nchunk)                       // later chunks of this lane are further out
            continue;
        uint32_t sc[kUnroll];
        float inv[kUnroll];
        float gg[kUnroll];
        for (int u = 0; u < kUnroll; ++u)
            gg[u] = group_scale<kOneGroup>(g, cs[u] >> 1, dm, last_group);
#if TRACE_PAIR_SPLIT
        PairScales ps = pair_scales_from_amax(pair_max(chunk_amax_bits(xc[0])), pair_max(chunk_amax_bits(xc[1])),
                                              gg[0], gg[1]);
        for (int u = 0; u < kUnroll; ++u) {
            sc[u] = ps.sc[u];
            inv[u] = ps.inv[u];
        }
        {   // each lane writes the scale byte of the block it derived
            int mine = threadIdx.x & 1;
            uint32_t c = cs[mine];
            if (c < nchunk) {
                scales[c >> 1] = (uint8_t)sc[mine];
                if (gd_scales)
                    gd_scales[c >> 1] = (uint8_t)sc[mine];
            }
        }
#else
        for (int u = 0; u < kUnroll; ++u) {
            sc[u] = block_scale(as_f(pair_max(chunk_amax_bits(xc[u])) << 16), gg[u]);
            inv[u] = inv_combined(e4m3_decode(sc[u]), gg[u]);
            if (cs[u] < nchunk && (cs[u] & 1u) == 0) {
                scales[cs[u] >> 1] = (uint8_t)sc[u];
                if (gd_scales)
                    gd_scales[cs[u] >> 1] = (uint8_t)sc[u];
            }
        }
#endif
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t c = cs[u];
            if (c >= nchunk)
                continue;
            uint32_t cw = rtn8(xc[u], inv[u]);
            st_stream(cw, codes + c);
            if (gd_scales)
                store_bits<K>(gd_bits, c, cw);
        }
    }
}

// Guidance stream from codes + scales.  Each lane packs four chunks (two
// blocks): one 16-byte code load, one 2-byte scale load, and one store per
// plane; a trailing pair of chunks (n % 32 == 16) takes a narrow path.
template <int K>
__global__ void __launch_bounds__(kThreads)
    k_guidance_pack(const uint32_t *__restrict__ codes, const uint8_t *__restrict__ scales, uint32_t nchunk,
                    uint8_t *__restrict__ gd_scales, uint8_t *__restrict__ gd_bits, uint32_t pad_begin,
                    uint32_t pad_end)
{
    zero_pad(gd_scales, pad_begin, pad_end);
    uint32_t q = blockIdx.x * kThreads + threadIdx.x;     // quad of chunks
    uint32_t c = 4 * q;
    if (c + 4 <= nchunk) {
        u32x4 cw = ld_stream(reinterpret_cast<const u32x4 *>(codes) + q);
        reinterpret_cast<uint16_t *>(gd_scales)[q] = reinterpret_cast<const uint16_t *>(scales)[q];
        if (K == 4) {
            reinterpret_cast<u32x4 *>(gd_bits)[q] = cw;
        } else if (K == 2) {
            u32x2 b = {compact_k2(cw.x) | (compact_k2(cw.y) << 16), compact_k2(cw.z) | (compact_k2(cw.w) << 16)};
            reinterpret_cast<u32x2 *>(gd_bits)[q] = b;
        } else {
            reinterpret_cast<uint32_t *>(gd_bits)[q] = compact_k1(cw.x) | (compact_k1(cw.y) << 8) |
                                                       (compact_k1(cw.z) << 16) | (compact_k1(cw.w) << 24);
        }
    } else if (c < nchunk) {                                 // the last two chunks: one block
        gd_scales[c >> 1] = scales[c >> 1];
        store_bits<K>(gd_bits, c, codes[c]);
        store_bits<K>(gd_bits, c + 1, codes[c + 1]);
    }
}

// Training side, guided (MODE 1, 2: k guidance bits) or full code (MODE 4).
template <int MODE, bool kOneGroup, bool kCodes>
__global__ void __launch_bounds__(kThreads)
    k_fakequant_guided(const u32x4 *x, uint32_t nchunk, const float *__restrict__ g, DivMagic dm,
                       uint32_t last_group, const uint8_t *__restrict__ scale_plane,
                       const uint8_t *__restrict__ bits, OutPtr out, uint32_t *__restrict__ codes_out)
{
    constexpr int R = MODE == 1 ? 2 : MODE == 2 ? 4 : 8;
    __shared__ Entry tab[kSlots * R];
    load_table<R>(tab, MODE == 1 ? kTabK1.e : MODE == 2 ? kTabK2.e : kTabFull.e);
    uint32_t ntiles = (nchunk + kTile - 1) / kTile;
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        Chunk xc[kUnroll];
        uint32_t cs[kUnroll], sc[kUnroll], gb[kUnroll];
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t c = t * kTile + u * kThreads + threadIdx.x;
            cs[u] = c;
            xc[u] = Chunk{{0u, 0u, 0u, 0u}};
            sc[u] = 0u;
            gb[u] = 0u;
            if (c < nchunk) {
                xc[u] = load_chunk(x, c);
                sc[u] = scale_plane[c >> 1];
                if (MODE == 1)
                    gb[u] = bits[c];
                else if (MODE == 2)
                    gb[u] = reinterpret_cast<const uint16_t *>(bits)[c];
                else
                    gb[u] = ld_stream(reinterpret_cast<const uint32_t *>(bits) + c);
            }
        }
        if (cs[0] >= nchunk)
            continue;
        float gg[kUnroll], s[kUnroll], inv[kUnroll];
        for (int u = 0; u < kUnroll; ++u)
            gg[u] = group_scale<kOneGroup>(g, cs[u] >> 1, dm, last_group);
#if TRACE_PAIR_SPLIT
        PairScales ps = pair_scales_from_bytes(sc[0], sc[1], gg[0], gg[1]);
        for (int u = 0; u < kUnroll; ++u) {
            s[u] = ps.s[u];
            inv[u] = ps.inv[u];
        }
#else
        for (int u = 0; u < kUnroll; ++u) {
            s[u] = e4m3_decode(sc[u] & 0x7fu);
            inv[u] = inv_combined(s[u], gg[u]);
        }
#endif
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t c = cs[u];
            if (c >= nchunk)
                continue;
            float yv[8];
            uint32_t nw = 0;
            for (int i = 0; i < 8; ++i) {
                uint32_t w = xc[u].w[i >> 1];
                float v = ((i & 1) ? bf_hi(w) : bf_lo(w)) * inv[u];
                uint32_t row, nib = 0;
                bool allow = true;
                if (MODE == 1) {
                    row = (gb[u] >> i) & 1u;
                } else if (MODE == 2) {
                    row = (gb[u] >> (2 * i)) & 3u;
                } else {
                    uint32_t r = (gb[u] >> (4 * i)) & 0xfu;
                    row = r & 7u;
                    allow = (r >> 3) == (as_u(v) >> 31);
                }
                yv[i] = decide<R, kCodes>(tab, v, row, allow, s[u], gg[u], nib);
                if (kCodes)
                    nw |= nib << (4 * i);
            }
            store_y(out, c, yv);
            if (kCodes)
                st_stream(nw, codes_out + c);
        }
    }
}

// Training side, plain RTN: shared scales from `scales_in` (kOwn = false) or
// block scales computed from x (kOwn = true, optionally written out).
template <bool kOwn, bool kOneGroup, bool kCodes>
__global__ void __launch_bounds__(kThreads)
    k_fakequant_rtn(const u32x4 *x, uint32_t nchunk, const float *__restrict__ g, DivMagic dm, uint32_t last_group,
                    const uint8_t *__restrict__ scales_in, OutPtr out, uint32_t *__restrict__ codes_out,
                    uint8_t *__restrict__ scales_out)
{
    uint32_t ntiles = (nchunk + kTile - 1) / kTile;
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        Chunk xc[kUnroll];
        uint32_t cs[kUnroll], sc[kUnroll];
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t c = t * kTile + u * kThreads + threadIdx.x;
            cs[u] = c;
            xc[u] = Chunk{{0u, 0u, 0u, 0u}};
            sc[u] = 0u;
            if (c < nchunk) {
                xc[u] = load_chunk(x, c);
                if (!kOwn)
                    sc[u] = scales_in[c >> 1];
            }
        }
        if (cs[0] >= nchunk)
            continue;
        float gg[kUnroll], s[kUnroll], inv[kUnroll];
        for (int u = 0; u < kUnroll; ++u)
            gg[u] = group_scale<kOneGroup>(g, cs[u] >> 1, dm, last_group);
#if TRACE_PAIR_SPLIT
        PairScales ps = kOwn ? pair_scales_from_amax(pair_max(chunk_amax_bits(xc[0])),
                                                     pair_max(chunk_amax_bits(xc[1])), gg[0], gg[1])
                             : pair_scales_from_bytes(sc[0], sc[1], gg[0], gg[1]);
        for (int u = 0; u < kUnroll; ++u) {
            sc[u] = ps.sc[u];
            s[u] = ps.s[u];
            inv[u] = ps.inv[u];
        }
        if (kOwn && scales_out) {                  // each lane writes the block it derived
            int mine = threadIdx.x & 1;
            if (cs[mine] < nchunk)
                scales_out[cs[mine] >> 1] = (uint8_t)sc[mine];
        }
#else
        for (int u = 0; u < kUnroll; ++u) {
            sc[u] = kOwn ? block_scale(as_f(pair_max(chunk_amax_bits(xc[u])) << 16), gg[u]) : (sc[u] & 0x7fu);
            s[u] = e4m3_decode(sc[u]);
            inv[u] = inv_combined(s[u], gg[u]);
            if (kOwn && scales_out && cs[u] < nchunk && (cs[u] & 1u) == 0)
                scales_out[cs[u] >> 1] = (uint8_t)sc[u];
        }
#endif
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t c = cs[u];
            if (c >= nchunk)
                continue;
            uint32_t cw = rtn8(xc[u], inv[u]);
            float yv[8];
            decode8(cw, yv);
            for (int i = 0; i < 8; ++i)
                yv[i] = (yv[i] * s[u]) * gg[u];         // signed value: the sign rides along
            store_y(out, c, yv);
            if (kCodes)
                st_stream(cw, codes_out + c);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int64_t kMaxN = int64_t(1) << 35;   // chunk indices (n / 8) fit in 32 bits

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

int grid_for(uint32_t nchunk)
{
    uint32_t tiles = (nchunk + kTile - 1) / kTile;
    return (int)(tiles < (uint32_t)kMaxGrid ? tiles : (uint32_t)kMaxGrid);
}

int launched() { return hipGetLastError() == hipSuccess ? TRACE_OK : TRACE_E_HIP; }

int64_t bitplane_offset(int64_t n) { return (n / 16 + 255) / 256 * 256; }

struct Launch {
    dim3 grid;
    hipStream_t st;
    uint32_t nchunk;
    DivMagic dm;
    uint32_t last;
    bool one;
};

Launch plan(int64_t n, int G, void *stream)
{
    uint32_t nchunk = (uint32_t)(n / 8);
    uint32_t nblk = (uint32_t)(n / 16);
    return Launch{dim3(grid_for(nchunk)), (hipStream_t)stream, nchunk, make_div_magic(nblk / (uint32_t)G),
                  (uint32_t)G - 1u, G == 1};
}

template <int MODE>
int launch_guided(const Launch &L, const void *x, const float *g, const uint8_t *sp, const uint8_t *bits,
                  OutPtr out, uint8_t *codes)
{
    (void)hipGetLastError();
    const u32x4 *xp = (const u32x4 *)x;
    uint32_t *cp = (uint32_t *)codes;
#define TRACE_G(ONE, CODES)                                                                                    \
    hipLaunchKernelGGL((k_fakequant_guided<MODE, ONE, CODES>), L.grid, dim3(kThreads), 0, L.st, xp, L.nchunk, g, \
                       L.dm, L.last, sp, bits, out, cp)
    if (L.one) {
        if (codes) TRACE_G(true, true); else TRACE_G(true, false);
    } else {
        if (codes) TRACE_G(false, true); else TRACE_G(false, false);
    }
#undef TRACE_G
    return launched();
}

template <bool kOwn>
int launch_rtn(const Launch &L, const void *x, const float *g, const uint8_t *scales_in, OutPtr out, uint8_t *codes,
               uint8_t *scales_out)
{
    (void)hipGetLastError();
    const u32x4 *xp = (const u32x4 *)x;
    uint32_t *cp = (uint32_t *)codes;
#define TRACE_R(ONE, CODES)                                                                                   \
    hipLaunchKernelGGL((k_fakequant_rtn<kOwn, ONE, CODES>), L.grid, dim3(kThreads), 0, L.st, xp, L.nchunk, g, \
                       L.dm, L.last, scales_in, out, cp, scales_out)
    if (L.one) {
        if (codes) TRACE_R(true, true); else TRACE_R(true, false);
    } else {
        if (codes) TRACE_R(false, true); else TRACE_R(false, false);
    }
#undef TRACE_R
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
    uint32_t nchunk = (uint32_t)(n / 8), cpg = nchunk / (uint32_t)G;
    uint32_t tpg = (cpg + kAmaxTile - 1) / kAmaxTile;
    uint64_t items = (uint64_t)tpg * (uint64_t)G;         // <= nchunk < 2^32
    int grid = (int)(items < (uint64_t)kAmaxGrid ? items : (uint64_t)kAmaxGrid);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_amax_clear, dim3((G + 255) / 256), dim3(256), 0, st, (uint32_t *)g_out, G);
    hipLaunchKernelGGL(k_amax, dim3(grid), dim3(kAmaxThreads), 0, st, (const u32x4 *)x_bf16, cpg, tpg,
                       (uint32_t)items, (uint32_t *)g_out, status_dev);
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
    Launch L = plan(n, G, stream);
    uint8_t *bits = guidance ? guidance + bitplane_offset(n) : nullptr;
    uint32_t pb = (uint32_t)(n / 16), pe = (uint32_t)bitplane_offset(n);
    (void)hipGetLastError();
#define TRACE_Q(KK, ONE)                                                                                            \
    hipLaunchKernelGGL((k_quant_rollout<KK, ONE>), L.grid, dim3(kThreads), 0, L.st, (const u32x4 *)y_bf16, L.nchunk, \
                       g, L.dm, L.last, (uint32_t *)codes, scales, guidance, bits, pb, pe)
    if (L.one) {
        if (k == 1) TRACE_Q(1, true);
        else if (k == 2) TRACE_Q(2, true);
        else TRACE_Q(4, true);
    } else {
        if (k == 1) TRACE_Q(1, false);
        else if (k == 2) TRACE_Q(2, false);
        else TRACE_Q(4, false);
    }
#undef TRACE_Q
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
    uint32_t nchunk = (uint32_t)(n / 8);
    uint32_t nquad = (nchunk + 3) / 4;
    dim3 grid((nquad + kThreads - 1) / kThreads);
    hipStream_t st = (hipStream_t)stream;
    uint8_t *bits = guidance + bitplane_offset(n);
    uint32_t pb = (uint32_t)(n / 16), pe = (uint32_t)bitplane_offset(n);
    const uint32_t *cp = (const uint32_t *)codes;
    (void)hipGetLastError();
    if (k == 1)
        hipLaunchKernelGGL((k_guidance_pack<1>), grid, dim3(kThreads), 0, st, cp, scales, nchunk, guidance, bits, pb,
                           pe);
    else if (k == 2)
        hipLaunchKernelGGL((k_guidance_pack<2>), grid, dim3(kThreads), 0, st, cp, scales, nchunk, guidance, bits, pb,
                           pe);
    else
        hipLaunchKernelGGL((k_guidance_pack<4>), grid, dim3(kThreads), 0, st, cp, scales, nchunk, guidance, bits, pb,
                           pe);
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
    Launch L = plan(n, G, stream);
    OutPtr out{y_out, out_dtype == TRACE_OUT_F32};
    const uint8_t *bits = guidance + bitplane_offset(n);
    if (k == 1)
        return launch_guided<1>(L, x_bf16, g, guidance, bits, out, codes_out);
    return launch_guided<2>(L, x_bf16, g, guidance, bits, out, codes_out);
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
    Launch L = plan(n, G, stream);
    OutPtr out{y_out, out_dtype == TRACE_OUT_F32};
    return launch_guided<4>(L, x_bf16, g, guidance, guidance + bitplane_offset(n), out, codes_out);
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
    Launch L = plan(n, G, stream);
    OutPtr out{y_out, out_dtype == TRACE_OUT_F32};
    if (scales_in) {
        rc = launch_rtn<false>(L, x_bf16, g, scales_in, out, codes_out, nullptr);
        if (rc == TRACE_OK && scales_out)
            rc = hipMemcpyAsync(scales_out, scales_in, (size_t)(n / 16), hipMemcpyDeviceToDevice, L.st) == hipSuccess
                     ? TRACE_OK
                     : TRACE_E_HIP;
        return rc;
    }
    return launch_rtn<true>(L, x_bf16, g, nullptr, out, codes_out, scales_out);
}

const char *trace_status_str(int status)
{
    switch (status) {
    case TRACE_OK: return "ok";
    case TRACE_E_NULL: return "a required pointer is NULL";
    case TRACE_E_SIZE: return "n or G violates the size rules (n > 0, n % 16 == 0, n % (16 G) == 0, n < 2^35)";
    case TRACE_E_ALIGN: return "a pointer is not 16-byte aligned";
    case TRACE_E_K: return "unsupported guidance width k";
    case TRACE_E_DTYPE: return "unknown output dtype";
    case TRACE_E_HIP: return "HIP runtime error";
    case TRACE_E_NONFINITE: return "an input was inf or NaN";
    case TRACE_E_FORMAT: return "guidance record fails its header or hash check";
    case TRACE_E_IO: return "file could not be opened, written or read";
    default: return "unknown status";
    }
}

int trace_version(void) { return 300; }

}  // extern "C"
