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
//   * streaming kernels launch one tile of 128 x kUnroll chunks per
//     workgroup (many small workgroups balance best across the 8 XCDs);
//   * the one-pass kernels (amax and quantise from one read) run one
//     persistent 512-thread workgroup per compute unit that holds its share
//     of the tensor on chip (registers and LDS) across a bounded grid
//     barrier; many groups beyond the chip's capacity run in teams of
//     workgroups, each team with a barrier of its own per group.
#include <hip/hip_runtime.h>

#include <bit>
#include <cfloat>
#include <cstdint>
#include <cstdlib>
#include <algorithm>
#include <mutex>

#include "trace_quant.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Launch shape and cache hints (fixed at build time; the values below are the
// measured best on MI355X for the 64x512x2048 activations and the batched
// MoE step of 128x1024x4096 activations plus a 2x65536x8x128 KV layer).
#ifndef TRACE_UNROLL
#define TRACE_UNROLL 2
#endif
#ifndef TRACE_WG_PER_CU
#define TRACE_WG_PER_CU 0
#endif
#ifndef TRACE_NT_LOAD
#define TRACE_NT_LOAD 1
#endif
// Store policy per kernel family: 1 = non-temporal stores, 0 = default
// policy.  TRACE_NT_STORE, when given, sets all three.  Timed inside the
// rollout + guided + full-code + RTN sequence on gfx950: non-temporal stores
// take the guided kernel from about 49 to 45 us at 64M bf16 elements and
// leave the rollout quantiser unchanged, while they slow the own-scale RTN
// kernel from about 40 to 43 us, so RTN keeps the default policy.
#ifdef TRACE_NT_STORE
#define TRACE_NT_STORE_QUANT TRACE_NT_STORE
#define TRACE_NT_STORE_GUIDED TRACE_NT_STORE
#define TRACE_NT_STORE_RTN TRACE_NT_STORE
#endif
#ifndef TRACE_NT_STORE_QUANT
#define TRACE_NT_STORE_QUANT 1
#endif
#ifndef TRACE_NT_STORE_GUIDED
#define TRACE_NT_STORE_GUIDED 1
#endif
#ifndef TRACE_NT_STORE_RTN
#define TRACE_NT_STORE_RTN 0
#endif
#ifndef TRACE_PAIR_SPLIT
#define TRACE_PAIR_SPLIT 1
#endif


constexpr int kThreads = 128;          // 2 wavefronts of 64
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
// Both candidates are kept in registers before the select (an empty asm
// that reads them), so the compiler cannot sink either into a branch: the
// per-block code stays one basic block and tiles can be interleaved.
__device__ __forceinline__ void keep(uint32_t a, uint32_t b) { asm volatile("" ::"v"(a), "v"(b)); }

// All cases are computed and one is selected.
__device__ __forceinline__ uint32_t e4m3_encode(float t)
{
    uint32_t sub = (uint32_t)__builtin_rintf(t * 512.0f); // below 2^-6: step 2^-9 (exact scaling, RNE)
    uint32_t u = as_u(t);
    uint32_t r = u + 0x7ffffu + ((u >> 20) & 1u);        // RNE to 3 mantissa bits
    uint32_t nrm = (r >> 20) - (120u << 3);              // rebias 127 -> 7
    keep(sub, nrm);
    return t >= 448.0f ? 0x7eu : (t < 0.015625f ? sub : nrm);
}

__device__ __forceinline__ float e4m3_decode(uint32_t c)
{
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    uint32_t nrm = ((e + 120u) << 23) | (m << 20);
    uint32_t sub = as_u((float)m * 0.001953125f);
    keep(nrm, sub);
    return as_f(e ? nrm : sub);
}

// Reciprocal of the combined scale c = s * g: 0 when c == 0, FLT_MAX when
// 1 / c overflows.  IEEE division (HIP's default correctly rounded path).
__device__ __forceinline__ float inv_combined(float s, float g)
{
    float c = s * g;
    float inv = fminf(1.0f / c, FLT_MAX);                // 1 / 0 = inf is discarded below
    return c > 0.0f ? inv : 0.0f;
}

// Block scale from the block amax and g (t = 0 when g == 0).
__device__ __forceinline__ uint32_t block_scale(float ab, float g)
{
    float q = ab / (6.0f * g);                           // inf or NaN when g == 0, discarded
    return e4m3_encode(g > 0.0f ? q : 0.0f);
}

// Table-driven block scale of one group, equal to block_scale for every
// finite block amax of the group.  A bf16 amax ab is V * 2^(e1 - 127) with
// V = 1 + j/128 (exponent field e >= 1, e1 = e) or V = j/128 (e = 0, e1 = 1).
// With d = fl(6g) = Dm * 2^Xd, Dm in [1, 2): ab / d = (V / Dm) * 2^E,
// E = e1 - 127 - Xd, and because scaling by a power of two commutes with
// rounding to fp32 in the normal range, fl(ab / d) = fl(V / Dm) * 2^E when
// that is normal (when it is not, t < 2^-126 and the code is 0 either way).
// So a 256-entry table indexed by (e > 0, j) holds q = fl(V / Dm) and the
// E4M3 normal-range code of q, rebased so that adding 8 * e1 gives the code
// of t (the RNE carry into the exponent is the same for q and t); 512 t is
// ldexp(q, e1 + K).  A per-code table then gives 1 / (s * g).  Together they
// replace two IEEE divisions and the E4M3 decode per block with two LDS reads
// (the one-pass rollout's phase 2 is VALU-bound: 108 -> 72 VALU instructions
// per register tile).
__device__ __forceinline__ void split_pow2(float d, float &dm, int &xd)   // finite d > 0
{
    uint32_t u = as_u(d), e = u >> 23;
    if (e == 0) {                                        // subnormal: normalise
        int s = __clz(u) - 8;
        u <<= s;
        xd = -126 - s;
    } else {
        xd = (int)e - 127;
    }
    dm = as_f((u & 0x7fffffu) | 0x3f800000u);
}

__device__ __forceinline__ float2 scale_table_entry(uint32_t idx, float g)
{
    if (!(g > 0.0f))
        return make_float2(0.0f, 0.0f);                  // t = 0 for every block: code 0
    float dm;
    int xd;
    split_pow2(6.0f * g, dm, xd);
    float v = idx >= 128u ? 1.0f + (float)(idx - 128u) * 0.0078125f : (float)idx * 0.0078125f;
    float q = v / dm;
    uint32_t u = as_u(q);
    int32_t p = (int32_t)((u + 0x7ffffu + ((u >> 20) & 1u)) >> 20) - 960 - 8 * (127 + xd);
    return make_float2(q, __int_as_float(p));
}

__device__ __forceinline__ int scale_table_k(float g)
{
    if (!(g > 0.0f))
        return 0;
    float dm;
    int xd;
    split_pow2(6.0f * g, dm, xd);
    return -118 - xd;                                    // 9 - 127 - Xd
}

__device__ __forceinline__ uint32_t block_scale_tab(uint32_t hab, const float2 *tab, int k)
{
    uint32_t idx = min(hab, (hab & 127u) | 128u);        // (e > 0) * 128 + j
    uint32_t e1 = max(hab >> 7, 1u);
    float2 ent = tab[idx];
    float tt = __builtin_amdgcn_ldexpf(ent.x, (int)e1 + k);
    uint32_t sub = (uint32_t)__builtin_rintf(tt);
    uint32_t nrm = min((uint32_t)__float_as_int(ent.y) + (e1 << 3), 0x7eu);
    keep(sub, nrm);
    return tt < 8.0f ? sub : nrm;
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

template <bool kNt, class T>
__device__ __forceinline__ void st_stream(T v, T *p)
{
    if constexpr (kNt)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
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
// The 3-bit magnitude indices of 8 nibbles, packed LSB-first into 24 bits.
__device__ __forceinline__ uint32_t compact_k3(uint32_t w)
{
    uint32_t x = w & 0x77777777u;
    uint32_t y = (x & 0x07070707u) | ((x & 0x70707070u) >> 1);   // 6 bits per byte
    uint32_t z = (y & 0x003f003fu) | ((y & 0x3f003f00u) >> 2);   // 12 bits per half
    return (z & 0x00000fffu) | ((z & 0x0fff0000u) >> 4);
}

// compact_k2(c0) | compact_k2(c1) << 16: fold within bytes, then one byte
// permute gathers bytes 0 and 2 of each word.
__device__ __forceinline__ uint32_t compact_k2_pair(uint32_t c0, uint32_t c1)
{
    uint32_t x = c0 & 0x33333333u, y = c1 & 0x33333333u;
    x = (x | (x >> 2)) & 0x0f0f0f0fu;
    y = (y | (y >> 2)) & 0x0f0f0f0fu;
    x |= x >> 4;                                         // bytes 0 and 2 complete
    y |= y >> 4;
    return __builtin_amdgcn_perm(y, x, 0x06040200u);
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
    // One 8-byte LDS read for the whole entry, and no short-circuit: with
    // `allow && ...` the compiler moved the threshold's read into a branch on
    // `allow`, one divergent branch and one waited LDS round trip per element.
    const u32x2 e = reinterpret_cast<const u32x2 *>(tab)[slot * R + row];
    bool up = (a > as_f(e.x)) & allow;
    float val = as_f(pick_half(e.y, up));
    float y = (val * s) * g;
    if (kCodes)
        nib = (floor_index_of_slot(slot) + (up ? 1u : 0u)) | ((as_u(v) >> 28) & 8u);
    return as_f(as_u(y) | (as_u(v) & 0x80000000u));
}

struct OutPtr {
    void *y;
    int f32;
};

template <bool kNt>
__device__ __forceinline__ void store_y(OutPtr o, uint32_t c, const float (&y)[8])
{
    if (o.f32) {
        f32x4 *p = reinterpret_cast<f32x4 *>(o.y) + 2 * (size_t)c;
        st_stream<kNt>(f32x4{y[0], y[1], y[2], y[3]}, p);
        st_stream<kNt>(f32x4{y[4], y[5], y[6], y[7]}, p + 1);
    } else {
        u32x4 w = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
        st_stream<kNt>(w, reinterpret_cast<u32x4 *>(o.y) + c);
    }
}

template <int R>
__device__ __forceinline__ void load_table(Entry *lds, const Entry *src)
{
    for (int i = threadIdx.x; i < kSlots * R; i += kThreads)
        lds[i] = src[i];
    __syncthreads();
}

// Zero the pad between the scale plane and the bit plane of a guidance stream
// (workgroup 0 of a launch of T threads per workgroup).
template <int T>
__device__ __forceinline__ void zero_pad(uint8_t *gd, uint32_t begin, uint32_t end)
{
    if (blockIdx.x == 0)
        for (uint32_t p = begin + threadIdx.x; p < end; p += T)
            gd[p] = 0;
}

// Guidance bits of one chunk (8 codes in cw): k = 1 -> 1 byte, 2 -> 2 bytes,
// 4 -> the 4 code bytes.
template <int K>
__device__ __forceinline__ void store_bits(uint8_t *gd_bits, uint32_t c, uint32_t cw)
{
    if (K == 4) {
        reinterpret_cast<uint32_t *>(gd_bits)[c] = cw;
    } else if (K == 3) {
        // 3 bytes at 3c: a 2-byte store on the even-aligned side and a 1-byte
        // store on the other (offsets chosen per lane, no divergent branch)
        uint32_t b = compact_k3(cw), odd = c & 1u;
        size_t o16 = 3 * (size_t)c + odd, o8 = 3 * (size_t)c + (odd ? 0u : 2u);   // 3c passes 2^32
        *reinterpret_cast<uint16_t *>(gd_bits + o16) = (uint16_t)(odd ? b >> 8 : b);
        gd_bits[o8] = (uint8_t)(odd ? b : b >> 16);
    } else if (K == 2) {
        reinterpret_cast<uint16_t *>(gd_bits)[c] = (uint16_t)compact_k2(cw);
    } else {
        gd_bits[c] = (uint8_t)compact_k1(cw);
    }
}

// The 24 guidance bits of chunk c of a k = 3 stream (the mirror of store_bits<3>).
__device__ __forceinline__ uint32_t load_bits3(const uint8_t *gd_bits, uint32_t c)
{
    uint32_t odd = c & 1u;
    size_t o = 3 * (size_t)c;                     // passes 2^32 for large tensors
    uint32_t h = *reinterpret_cast<const uint16_t *>(gd_bits + o + odd);
    uint32_t b = gd_bits[o + (odd ? 0u : 2u)];
    return odd ? (b | (h << 8)) : (h | (b << 16));
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// max |x| over the finite elements of a chunk (bf16 magnitude bits); an inf
// or NaN is left out and flagged in *status (when given).
__device__ __forceinline__ uint32_t chunk_amax_finite(const Chunk &x, int *status)
{
    uint32_t m = chunk_amax_bits(x);
    if (m >= 0x7f80u) {                                    // rare: an inf or NaN in the chunk
        m = 0;
        for (int i = 0; i < 4; ++i) {
            uint32_t lo = x.w[i] & 0x7fffu, hi = (x.w[i] >> 16) & 0x7fffu;
            m = max(m, max(lo < 0x7f80u ? lo : 0u, hi < 0x7f80u ? hi : 0u));
        }
        if (status)
            *status = TRACE_E_NONFINITE;
    }
    return m;
}

__global__ void k_amax_clear(uint32_t *g_bits, int G)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < G)
        g_bits[i] = 0u;
}

// Fold the workgroup's running max and raise the group's word with one atomic
// max, skipped when the word already holds a value at least as large.
// kPerformed: use the returning form of the atomic and wait for it, so the
// maximum has been performed at the device's coherence point when the
// function returns (the one-pass kernel's barrier arrival depends on it).
// kScale: publish the global scale fl(A / 2688) of the workgroup's maximum A
// instead of A.  x -> fl(x / 2688) is monotonic (IEEE division rounds
// correctly), so the largest published scale is fl(max A / 2688): the group's
// global scale, with no pass after the reduction.  Non-negative floats order
// like their bit patterns, so the integer atomic max serves both forms.
template <int T = kAmaxThreads, bool kPerformed = false, bool kScale = false>
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
        for (int i = 0; i < T / 64; ++i)
            b = max(b, wmax[i]);
        b <<= 16;
        if (kScale)
            b = as_u(as_f(b) / 2688.0f);
        if (b > __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            if (kPerformed) {
                wmax[0] = __hip_atomic_fetch_max(word, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_s_waitcnt(0);
            } else {
                atomicMax(word, b);
            }
        }
    }
    __syncthreads();
}

// Global scale per group, g = fl(amax / 2688), raised by each workgroup with
// an atomic max on the float bits (amax_publish, kScale).  Work items
// are (group, tile) pairs, walked grid-stride (neighbouring workgroups read
// neighbouring tiles at each step) or, with `runs`, as one contiguous run per
// workgroup.  Each thread keeps a running max for the current group and the
// workgroup publishes it when the group changes and at the end; a change
// costs a workgroup reduction and a device-scope round trip.  Grid-stride,
// with many groups a workgroup changes group on every tile (64 groups of 2M
// elements: 3.7 TB/s, against 5.9 TB/s in runs), while with one group it is
// about 6% faster than runs; the host picks.  Non-finite inputs are left out
// and flagged.
__global__ void __launch_bounds__(kAmaxThreads)
    k_amax(const u32x4 *__restrict__ x, uint32_t cpg, uint32_t tiles_per_group, uint32_t items,
           uint32_t *g_bits, int *status, bool runs)
{
    __shared__ uint32_t wmax[kAmaxThreads / 64];
    uint32_t run = 0;
    uint32_t cur = 0xffffffffu;
    const uint32_t w0 = runs ? (uint32_t)((uint64_t)items * blockIdx.x / gridDim.x) : blockIdx.x;
    const uint32_t w1 = runs ? (uint32_t)((uint64_t)items * (blockIdx.x + 1) / gridDim.x) : items;
    const uint32_t step = runs ? 1u : gridDim.x;
    for (uint32_t w = w0; w < w1; w += step) {
        uint32_t grp = w / tiles_per_group;
        uint32_t tile = w - grp * tiles_per_group;
        if (grp != cur) {
            if (cur != 0xffffffffu) {
                amax_publish<kAmaxThreads, false, true>(run, wmax, g_bits + cur);
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
        for (int u = 0; u < kAmaxUnroll; ++u)
            if (ok[u])
                run = max(run, chunk_amax_finite(b[u], status));
    }
    if (cur != 0xffffffffu)
        amax_publish<kAmaxThreads, false, true>(run, wmax, g_bits + cur);
}

// RTN codes, scale bytes and (with gd_scales) guidance bits of one lane's U
// chunks cs[u], which hold x[u]; chunks at or past `lim` are outside the
// tensor (or group) and are skipped (both lanes of a pair always agree).
// gg[u] is the global scale of chunk u.
template <int K, int U>
__device__ __forceinline__ void quant_lane(const Chunk (&xc)[U], const uint32_t (&cs)[U], uint32_t lim,
                                           const float (&gg)[U], uint32_t *__restrict__ codes,
                                           uint8_t *__restrict__ scales, uint8_t *__restrict__ gd_scales,
                                           uint8_t *__restrict__ gd_bits)
{
    uint32_t sc[U];
    float inv[U];
    if constexpr (TRACE_PAIR_SPLIT && U == 2) {
        PairScales ps = pair_scales_from_amax(pair_max(chunk_amax_bits(xc[0])), pair_max(chunk_amax_bits(xc[1])),
                                              gg[0], gg[1]);
        for (int u = 0; u < U; ++u) {
            sc[u] = ps.sc[u];
            inv[u] = ps.inv[u];
        }
        int mine = threadIdx.x & 1;                // each lane writes the scale byte of the block it derived
        uint32_t c = cs[mine];
        if (c < lim) {
            scales[c >> 1] = (uint8_t)sc[mine];
            if (gd_scales)
                gd_scales[c >> 1] = (uint8_t)sc[mine];
        }
    } else {
        for (int u = 0; u < U; ++u) {
            sc[u] = block_scale(as_f(pair_max(chunk_amax_bits(xc[u])) << 16), gg[u]);
            inv[u] = inv_combined(e4m3_decode(sc[u]), gg[u]);
            if (cs[u] < lim && (cs[u] & 1u) == 0) {
                scales[cs[u] >> 1] = (uint8_t)sc[u];
                if (gd_scales)
                    gd_scales[cs[u] >> 1] = (uint8_t)sc[u];
            }
        }
    }
    for (int u = 0; u < U; ++u) {
        if (cs[u] >= lim)
            continue;
        uint32_t cw = rtn8(xc[u], inv[u]);
        st_stream<TRACE_NT_STORE_QUANT>(cw, codes + cs[u]);
        if (gd_scales)
            store_bits<K>(gd_bits, cs[u], cw);
    }
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
        zero_pad<kThreads>(gd_scales, pad_begin, pad_end);
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
        float gg[kUnroll];
        for (int u = 0; u < kUnroll; ++u)
            gg[u] = group_scale<kOneGroup>(g, cs[u] >> 1, dm, last_group);
        quant_lane<K>(xc, cs, nchunk, gg, codes, scales, gd_scales, gd_bits);
    }
}

// ---------------------------------------------------------------------------
// One-pass rollout: group amax, then quantisation, in one kernel.
//
// The two-kernel rollout reads y twice (amax, then quantise), because no block
// can be quantised before its group's global scale is known.  Here every
// workgroup (one per compute unit, all resident at once) reads its share of y
// once, keeps as much of it as fits on chip (kOpRegTiles tiles in VGPRs, a
// runtime number in LDS), folds its maximum into the group's word, and waits
// at a grid-wide barrier; after it, the kept tiles are quantised from
// registers and LDS, and only the tiles that did not fit are read again.
// 512 threads per workgroup: two waves per SIMD leave each lane 256 VGPRs, of
// which 160 hold tiles.  Work items are (group, tile) pairs, so a tile never
// straddles two groups; workgroup w takes a contiguous run of items: first the
// ones it reads twice, then the LDS ones, then the register ones.  Within a
// tile each lane owns one 16-element block (two adjacent chunks), so the
// block maximum needs no exchange between lanes and each output plane takes
// one store per lane.
// ---------------------------------------------------------------------------
#ifndef TRACE_OP_NT_STORE
#define TRACE_OP_NT_STORE 1
#endif
#ifndef TRACE_OP_REG_TILES
#define TRACE_OP_REG_TILES 24
#endif
#ifndef TRACE_OP_THREADS
#define TRACE_OP_THREADS 512
#endif
constexpr int kOpThreads = TRACE_OP_THREADS;
constexpr int kOpTile = 2 * kOpThreads;            // chunks per tile (16 KiB of bf16)
constexpr int kOpRegTiles = TRACE_OP_REG_TILES;
constexpr int kOpStream = 4;                       // tiles in flight per lane when streaming
// Work buffer (words): arrival counters of 16 subgroups of workgroups and
// one top counter, each on its own 256-byte line (a same-address atomic costs
// about 30 ns on MI355X, so 256 arrivals on one word serialise for ~8 us;
// two levels of 16 take ~1 us), then the group amax bits.
// Phase clocks of k_quant_onepass (a measurement build only: the product
// library is built with 0 and carries none of it).  With 1, thread 0 of each
// workgroup writes the wall clock at the kernel's start, at the end of phase
// 1, when the grid barrier has passed and at the end of phase 2 into the
// buffer set by trace_debug_phase_clock (4 values per workgroup).
#ifndef TRACE_OP_PHASE_CLOCK
#define TRACE_OP_PHASE_CLOCK 0
#endif
#ifndef TRACE_OP_LINE_WORDS
#define TRACE_OP_LINE_WORDS 64
#endif
constexpr uint32_t kOpLine = TRACE_OP_LINE_WORDS;
constexpr uint32_t kOpSubgroups = 16;
constexpr uint32_t kOpTopWord = kOpSubgroups * kOpLine;
constexpr uint32_t kOpDoneWord = (kOpSubgroups + 1) * kOpLine;      // the same tree again, for departures
// Arrival counters of the teams of k_quant_onepass_teams, one line each.
constexpr uint32_t kOpMaxTeams = 64;
// Register tiles of k_quant_onepass_teams: its loop over groups keeps a few
// more values live than k_quant_onepass, and 24 tiles spill (23 with f32
// fake-quant output).
constexpr int ot_reg_tiles(int out) { return out == 2 ? 22 : 23; }
constexpr uint32_t kOpTeamWord = 2 * (kOpSubgroups + 1) * kOpLine;
constexpr uint32_t kOpAccWord = kOpTeamWord + kOpMaxTeams * kOpLine;
constexpr int kOpGroupSlots = 128;                 // global scales a workgroup keeps in LDS
constexpr uint32_t kOpTabSlots = 4;                // groups with scale tables, several-group rollout

// Groups the allocation-free one-pass entry point accepts: its work buffer
// (barrier trees and group maxima, the layout above) is the static array
// `scratch` below, one copy per device.
constexpr int kScratchMaxGroups = 4096;
constexpr uint32_t kScratchWords = kOpAccWord + kScratchMaxGroups;   // 41 472 bytes

}  // namespace

static __device__ __align__(256) uint32_t scratch[kScratchWords];

namespace {

struct OnePass {
    const u32x4 *y;         // the input (the rollout's y, or the training tensor x)
    uint32_t cpg;           // chunks per group
    uint32_t tpg;           // tiles per group
    DivMagic tpg_div;       // division by tpg (item -> group), a multiply-high on the scalar unit
    uint32_t items;         // G * tpg
    uint32_t G;
    uint32_t lds_tiles;     // tiles a workgroup keeps in LDS
    uint32_t pad_begin, pad_end;
    uint64_t wait_ticks;    // barrier time limit in wall-clock ticks
    uint32_t *work;
    float *g_out;
    int *status;
    uint32_t *codes;        // rollout codes, or the fake-quant's chosen codes (nullable there)
    uint8_t *scales, *gd_scales, *gd_bits;
    void *out;              // fake-quant output (bf16 or f32), else null
    uint32_t team_size;     // k_quant_onepass_teams: workgroups per team
    uint64_t *clock;        // phase clocks (TRACE_OP_PHASE_CLOCK builds), else null
};

// One phase stamp of k_quant_onepass (see TRACE_OP_PHASE_CLOCK).
__device__ __forceinline__ void phase_stamp(const OnePass &a, uint32_t i)
{
    if constexpr (TRACE_OP_PHASE_CLOCK != 0) {
        if (threadIdx.x == 0 && a.clock)
            a.clock[blockIdx.x * 4u + i] = (uint64_t)wall_clock64();
    }
}

// Where the chunks of item it lie (all uniform): chunk u of thread t is
// first + u * T + t, so each load is 16 bytes per lane, contiguous across the
// wave; valid while u * T + t < count (the group's last tile may be short;
// count is even).
struct Item {
    uint32_t grp, first, count;
};

template <bool kOneGroup>
__device__ __forceinline__ Item item_at(const OnePass &a, uint32_t it)
{
    uint32_t grp = kOneGroup ? 0u : div_magic(it, a.tpg_div);
    uint32_t tile = it - grp * a.tpg;
    uint32_t off = tile * kOpTile;
    return Item{grp, grp * a.cpg + off, min(a.cpg - off, (uint32_t)kOpTile)};
}

// Buffer descriptor over an item's chunks (gfx9 raw buffer, stride 0): loads
// past `count` chunks return zeros, which leave a maximum unchanged and are
// never stored; an item that is not live gets no records at all.  So every
// load of a batch is issued without a branch and stays in flight together,
// and the per-lane offset is a 32-bit register instead of a 64-bit address.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t item_rsrc(const OnePass &a, const Item &w, bool live)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)(a.y + (live ? w.first : 0u)), (short)0,
                                             live ? (int)(w.count * 16u) : 0, 0x00020000);
}

__device__ __forceinline__ void load_item(const OnePass &a, const Item &w, bool live, Chunk (&x)[2])
{
    __amdgpu_buffer_rsrc_t r = item_rsrc(a, w, live);
    for (int u = 0; u < 2; ++u) {
        u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (u * kOpThreads + threadIdx.x) * 16u, 0,
                                                        TRACE_NT_LOAD ? 2 : 0);
        x[u] = Chunk{{v.x, v.y, v.z, v.w}};
    }
}

// Copy this lane's two chunks of an item straight into LDS slot j
// (global_load_lds, 16 bytes: lane i of a wave lands at the wave's base +
// 16 i, so chunk u * T + t sits at (2 j + u) * T + t).  Lanes past the
// item's end load nothing; their slots are masked or never stored.  The
// copies are non-temporal like every other streaming load: with the default
// policy they measured 6 us slower (of 24 for phase 1) when the previous
// kernel had just written its output.
__device__ __forceinline__ void load_item_to_lds(const OnePass &a, const Item &w, u32x4 *lds, uint32_t j)
{
    uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int u = 0; u < 2; ++u) {
        uint32_t o = u * kOpThreads + threadIdx.x;
        u32x4 *dst = lds + ((2 * j + u) * kOpThreads + wave * 64);
        if (o < w.count)
            __builtin_amdgcn_global_load_lds(a.y + w.first + o, (__attribute__((address_space(3))) void *)dst, 16, 0,
                                             TRACE_NT_LOAD ? 2 : 0);
    }
}

// This lane's own two chunks of LDS slot j (chunks past the end as zeros).
__device__ __forceinline__ void read_item_from_lds(const u32x4 *lds, const Item &w, uint32_t j, Chunk (&x)[2])
{
    for (int u = 0; u < 2; ++u) {
        u32x4 v = lds[(2 * j + u) * kOpThreads + threadIdx.x];
        x[u] = u * kOpThreads + threadIdx.x < w.count ? Chunk{{v.x, v.y, v.z, v.w}} : Chunk{{0u, 0u, 0u, 0u}};
    }
}

// One whole 16-element block per lane.  Lanes 2m and 2m + 1 hold chunks
// (2m, T + 2m) and (2m + 1, T + 2m + 1); one DPP swap per word hands the
// even lane chunk 2m + 1 and the odd lane chunk T + 2m, so the even lane
// owns block m of the item and the odd lane block T/2 + m.
struct Blk {
    Chunk lo, hi;
};

__device__ __forceinline__ uint32_t block_of_lane()
{
    uint32_t t = threadIdx.x;
    return (t & 1u) ? kOpThreads / 2 + (t >> 1) : (t >> 1);
}

__device__ __forceinline__ Blk to_block(const Chunk (&x)[2])
{
    bool odd = threadIdx.x & 1u;
    Blk b;
    for (int i = 0; i < 4; ++i) {
        uint32_t recv = pair_swap(odd ? x[0].w[i] : x[1].w[i]);
        b.lo.w[i] = odd ? recv : x[0].w[i];
        b.hi.w[i] = odd ? x[1].w[i] : recv;
    }
    return b;
}

// The same block straight from LDS slot j (no exchange needed: a lane may
// read its neighbour's slot).  Blocks past the item's end hold stale data
// and are never stored.
__device__ __forceinline__ Blk block_from_lds(const u32x4 *lds, uint32_t j)
{
    uint32_t t = threadIdx.x, odd = t & 1u;
    const u32x4 *p = lds + (2 * j + odd) * kOpThreads + t - odd;
    u32x4 a = p[0], b = p[1];
    return Blk{Chunk{{a.x, a.y, a.z, a.w}}, Chunk{{b.x, b.y, b.z, b.w}}};
}

__device__ __forceinline__ uint32_t block_amax_bits(const Blk &b)
{
    return max(chunk_amax_bits(b.lo), chunk_amax_bits(b.hi));
}

__device__ __forceinline__ uint32_t group_amax_bits(const OnePass &a, uint32_t grp)
{
    return __hip_atomic_load(a.work + kOpAccWord + grp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Buffer descriptor over `bytes` bytes at p (gfx9 raw buffer, stride 0);
// accesses past the end are dropped (stores) or read as zero (loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// Output descriptors.  Span form (kSpan): one descriptor per output over this
// workgroup's whole run of chunks [c0, c0 + n), fixed for the whole phase; a
// tile's stores add its offset in the run to the lane offset.  Valid when no
// tile inside the run is short of kOpTile chunks except the run's last (one
// group, or groups of whole tiles), since a short tile's missing chunks would
// otherwise alias the next tile's.  Item form: one descriptor per output over
// the item's own slice, for groups whose last tile is short.  Items that are
// not live get descriptors with no records.
struct Outs {
    __amdgpu_buffer_rsrc_t codes, scales, gds, bits, y;
    uint32_t c0;               // first chunk covered
};

// OUT: 0 = rollout (codes, scales, guidance), 1 / 2 = fake-quant output in
// bf16 / f32 (16 / 32 bytes per chunk) with optional codes and scales.
template <int K, int OUT>
__device__ __forceinline__ Outs outs_over(const OnePass &a, uint32_t c0, uint32_t n)
{
    Outs o;                                            // fields a mode does not use stay unset
    o.c0 = c0;
    if constexpr (OUT == 0) {                          // codes and scales are required here
        const bool gd = a.gd_scales != nullptr;
        o.codes = span_rsrc(a.codes + c0, n * 4u);
        o.scales = span_rsrc(a.scales + c0 / 2, n / 2);
        o.gds = span_rsrc(gd ? a.gd_scales + c0 / 2 : a.scales, gd ? n / 2 : 0u);
        o.bits = span_rsrc(gd ? a.gd_bits + (size_t)c0 * K : a.scales, gd ? n * K : 0u);
    } else {                                           // codes and scales are optional here
        constexpr uint32_t cb = OUT == 2 ? 32u : 16u;
        const void *any = a.out;                       // a valid base for a descriptor with no records
        o.codes = span_rsrc(a.codes ? (const void *)(a.codes + c0) : any, a.codes ? n * 4u : 0u);
        o.scales = span_rsrc(a.scales ? (const void *)(a.scales + c0 / 2) : any, a.scales ? n / 2 : 0u);
        o.y = span_rsrc(static_cast<uint8_t *>(a.out) + (size_t)c0 * cb, n * cb);
    }
    return o;
}

// Codes, scale byte and guidance bits of this lane's block of one item (raw
// amax bits ab): one store per plane per lane (8 code bytes, 2k bit-plane
// bytes, one byte in each scale plane), with no branch.
// Per-group tables (kTab): the block-scale table of block_scale_tab with its
// offset k, and 1 / (s * g) per scale code.
struct GroupTabs {
    const float2 *scale;
    const float *inv;
    int k;
};

// A block's scale code and the reciprocal of its combined scale.
struct ScInv {
    uint32_t sc;
    float inv;
};

template <bool kTab>
__device__ __forceinline__ ScInv block_scale_inv(uint32_t ab, float gv, const GroupTabs &tb)
{
    ScInv r;
    if constexpr (kTab) {
        r.sc = block_scale_tab(ab, tb.scale, tb.k);
        r.inv = tb.inv[r.sc];
    } else {
        r.sc = block_scale(as_f(ab << 16), gv);
        r.inv = inv_combined(e4m3_decode(r.sc), gv);
    }
    return r;
}

// The stores of quant_block, given the block's scale code and reciprocal.
template <int K>
__device__ __forceinline__ void quant_block_with(const Outs &o, const Item &w, const Blk &b, ScInv si);

template <int K, bool kTab>
__device__ __forceinline__ void quant_block(const Outs &o, const Item &w, const Blk &b, uint32_t ab, float gv,
                                            const GroupTabs &tb)
{
    quant_block_with<K>(o, w, b, block_scale_inv<kTab>(ab, gv, tb));
}

template <int K>
__device__ __forceinline__ void quant_block_with(const Outs &o, const Item &w, const Blk &b, ScInv si)
{
    const uint32_t cb = w.first - o.c0 + 2 * block_of_lane();   // the block's first chunk, in o's span
    const uint32_t sc = si.sc;
    const float inv = si.inv;
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, o.scales, cb / 2, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, o.gds, cb / 2, 0, 0);
    const uint32_t c0 = rtn8(b.lo, inv), c1 = rtn8(b.hi, inv);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{c0, c1}, o.codes, cb * 4u, 0, TRACE_OP_NT_STORE ? 2 : 0);
    if (K == 4) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{c0, c1}, o.bits, cb * 4u, 0, 0);
    } else if (K == 3) {                                        // 48 bits at 3 cb (even): three halves
        uint32_t lo = compact_k3(c0), hi = compact_k3(c1);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)lo, o.bits, cb * 3u, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)((lo >> 16) | (hi << 8)), o.bits, cb * 3u + 2u, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(hi >> 8), o.bits, cb * 3u + 4u, 0, 0);
    } else if (K == 2)
        __builtin_amdgcn_raw_buffer_store_b32(compact_k2_pair(c0, c1), o.bits, cb * 2u, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(compact_k1(c0) | (compact_k1(c1) << 8)), o.bits, cb, 0, 0);
}

// Plain RTN fake-quant of this lane's block (own block scale from its raw
// amax bits ab and the group's g): optional codes and scale byte as in
// quant_block, and the dequantised values y = (val * s) * g.  Those are
// handed back to the load layout (one DPP swap per word: the even lane keeps
// its first chunk and takes the odd lane's first, the odd lane keeps its
// second and takes the even lane's second), so each lane stores chunks t and
// T + t of the item: 16 B (bf16) or 32 B (f32) per chunk, contiguous across
// the wave.
// (The scale tables of quant_block are not used here: this phase is bound by
// its 4 bytes of stores per element, and timed on gfx950 the two dependent
// table reads per block cost more than the divisions they replace.)
template <int OUT>
__device__ __forceinline__ void rtn_block(const Outs &o, const Item &w, const Blk &b, uint32_t ab, float gv)
{
    const uint32_t t = threadIdx.x, odd = t & 1u;
    const uint32_t cb = w.first - o.c0 + 2 * block_of_lane();
    const uint32_t sc = block_scale(as_f(ab << 16), gv);
    const float s = e4m3_decode(sc);
    const float inv = inv_combined(s, gv);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, o.scales, cb / 2, 0, 0);
    const uint32_t c0 = rtn8(b.lo, inv), c1 = rtn8(b.hi, inv);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{c0, c1}, o.codes, cb * 4u, 0, 0);
    float ylo[8], yhi[8];
    decode8(c0, ylo);
    decode8(c1, yhi);
    for (int i = 0; i < 8; ++i) {
        ylo[i] = (ylo[i] * s) * gv;                     // signed value: the sign rides along
        yhi[i] = (yhi[i] * s) * gv;
    }
    const uint32_t base = w.first - o.c0 + t;           // chunk of slot u = 0, in o's span
    if (OUT == 1) {
        uint32_t lo[4], hi[4], out0[4], out1[4];
        for (int i = 0; i < 4; ++i) {
            lo[i] = pack_bf16(ylo[2 * i], ylo[2 * i + 1]);
            hi[i] = pack_bf16(yhi[2 * i], yhi[2 * i + 1]);
            uint32_t recv = pair_swap(odd ? lo[i] : hi[i]);
            out0[i] = odd ? recv : lo[i];
            out1[i] = odd ? hi[i] : recv;
        }
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{out0[0], out0[1], out0[2], out0[3]}, o.y, base * 16u, 0,
                                               TRACE_OP_NT_STORE ? 2 : 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{out1[0], out1[1], out1[2], out1[3]}, o.y,
                                               (base + kOpThreads) * 16u, 0, TRACE_OP_NT_STORE ? 2 : 0);
    } else {
        uint32_t out0[8], out1[8];
        for (int i = 0; i < 8; ++i) {
            uint32_t recv = pair_swap(odd ? as_u(ylo[i]) : as_u(yhi[i]));
            out0[i] = odd ? recv : as_u(ylo[i]);
            out1[i] = odd ? as_u(yhi[i]) : recv;
        }
        for (int h = 0; h < 2; ++h) {
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{out0[4 * h], out0[4 * h + 1], out0[4 * h + 2], out0[4 * h + 3]},
                                                   o.y, base * 32u + 16u * h, 0, TRACE_OP_NT_STORE ? 2 : 0);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{out1[4 * h], out1[4 * h + 1], out1[4 * h + 2], out1[4 * h + 3]},
                                                   o.y, (base + kOpThreads) * 32u + 16u * h, 0, TRACE_OP_NT_STORE ? 2 : 0);
        }
    }
}

// Count this workgroup into a two-level tree of counters at `base` (16
// subgroup words and a top word, one line each); true for the caller whose
// count completed the top word.  Thread 0 only.
__device__ __forceinline__ bool tree_count(uint32_t *base, uint32_t P, bool *top_done)
{
    const uint32_t sub = blockIdx.x % kOpSubgroups;
    const uint32_t members = (P - sub + kOpSubgroups - 1) / kOpSubgroups;
    const uint32_t nsub = min(P, kOpSubgroups);
    bool last = false;
    if (__hip_atomic_fetch_add(base + sub * kOpLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1)
        last = __hip_atomic_fetch_add(base + kOpSubgroups * kOpLine, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == nsub - 1;
    if (top_done)
        *top_done = last;
    return last;
}

// kSpan: output descriptors over the workgroup's whole run (see Outs).
// OUT: 0 = rollout (codes, scales, guidance of width K); 1 / 2 = plain RTN
// fake-quant with own block scales, output bf16 / f32 (K unused).
// kTab (rollout only): scale tables per group (block_scale_tab); with
// several groups the host launches it only when no workgroup's run spans
// more than kOpTabSlots groups.
template <int K, bool kOneGroup, bool kSpan, int OUT = 0, bool kTab = kOneGroup && OUT == 0>
__global__ void __launch_bounds__(kOpThreads) k_quant_onepass(OnePass a)
{
    static_assert(!kTab || OUT == 0, "scale tables serve the rollout codes only");
    // Tiles read twice go in batches of kOpStream items (one load per chunk
    // in flight per item); halved without span descriptors, where each item
    // of a batch carries its own output descriptors in scalar registers.
    // Batches of eight spilled some variants' registers to scratch memory.
    constexpr int kBatch = kSpan ? kOpStream : kOpStream / 2;
    constexpr uint32_t kSlots = kTab ? (kOneGroup ? 1u : kOpTabSlots) : 0u;
    extern __shared__ u32x4 lds_tiles[];           // a.lds_tiles * 2 * kOpThreads chunks
    __shared__ uint32_t wmax[kOpThreads / 64];
    __shared__ int passed;
    __shared__ bool leaving_last;
    __shared__ float gslot[kOpGroupSlots];
    __shared__ float2 stab[kTab ? kSlots * 256 : 1];   // block-scale table per group slot
    __shared__ float ctab[kTab ? kSlots * 128 : 1];    // 1 / (s * g) per scale code, per slot
    __shared__ int ktab[kTab ? kSlots : 1];

    phase_stamp(a, 0);
    const uint32_t P = gridDim.x;
    const uint32_t i0 = (uint32_t)((uint64_t)a.items * blockIdx.x / P);
    const uint32_t cnt = (uint32_t)((uint64_t)a.items * (blockIdx.x + 1) / P) - i0;
    const uint32_t nreg = min(cnt, (uint32_t)kOpRegTiles);
    const uint32_t nlds = min(cnt - nreg, a.lds_tiles);
    const uint32_t nstr = cnt - nreg - nlds;
    const uint32_t i_lds = i0 + nstr, i_reg = i_lds + nlds;
    uint32_t *acc = a.work + kOpAccWord;

    // ---- phase 1: read everything once, fold the group maxima ------------
    // The LDS tiles go first, straight from memory into LDS (no VGPRs, and
    // they stay in flight behind the rest); then the tiles read twice, a
    // batch at a time; then the register tiles, all at once.
    for (uint32_t j = 0; j < nlds; ++j)
        load_item_to_lds(a, item_at<kOneGroup>(a, i_lds + j), lds_tiles, j);
    uint32_t run = 0;
    uint32_t cur = kOneGroup ? 0u : i0 / a.tpg;
    auto fold = [&](uint32_t grp, uint32_t m) {
        if (!kOneGroup && grp != cur) {            // uniform: all lanes walk the same items
            amax_publish<kOpThreads, true>(run, wmax, acc + cur);
            run = 0;
            cur = grp;
        }
        run = max(run, m);
    };
    auto chunk_pair_max = [&](const Chunk (&x)[2]) {
        return max(chunk_amax_finite(x[0], a.status), chunk_amax_finite(x[1], a.status));
    };
    for (uint32_t j = 0; j < nstr; j += kBatch) {
        Chunk x[kBatch][2];
        Item w[kBatch];
        for (int q = 0; q < kBatch; ++q) {
            w[q] = item_at<kOneGroup>(a, i0 + j + q);
            load_item(a, w[q], j + q < nstr, x[q]);
        }
        for (int q = 0; q < kBatch; ++q)
            if (j + q < nstr)
                fold(w[q].grp, chunk_pair_max(x[q]));
    }
    // Register tiles: loaded coalesced, then regrouped into one block per lane
    // and the block's raw amax kept, while this phase waits on memory anyway.
    Blk hr[kOpRegTiles];
    uint32_t hab[kOpRegTiles];
#pragma unroll
    for (int h = 0; h < kOpRegTiles; ++h) {
        Chunk x[2];
        load_item(a, item_at<kOneGroup>(a, i_reg + h), (uint32_t)h < nreg, x);
        hr[h].lo = x[0];
        hr[h].hi = x[1];
    }
    __builtin_amdgcn_s_waitcnt(0);                 // the LDS copies have landed (this wave's own)
    for (uint32_t j = 0; j < nlds; ++j) {
        Item w = item_at<kOneGroup>(a, i_lds + j);
        Chunk x[2];
        read_item_from_lds(lds_tiles, w, j, x);
        fold(w.grp, chunk_pair_max(x));
    }
#pragma unroll
    for (int h = 0; h < kOpRegTiles; ++h) {
        Chunk x[2] = {hr[h].lo, hr[h].hi};
        hr[h] = to_block(x);
        hab[h] = block_amax_bits(hr[h]);
        if ((uint32_t)h < nreg) {
            uint32_t m = hab[h] < 0x7f80u ? hab[h]
                                          : max(chunk_amax_finite(hr[h].lo, a.status), chunk_amax_finite(hr[h].hi, a.status));
            fold(item_at<kOneGroup>(a, i_reg + h).grp, m);
        }
    }
    if (cnt > 0)
        amax_publish<kOpThreads, true>(run, wmax, acc + cur);
    phase_stamp(a, 1);

    // ---- grid barrier ------------------------------------------------------
    // Bounded: a launch whose workgroups are not all resident gives up after
    // wait_ticks and reports TRACE_E_BARRIER.  The arrival and the spin are
    // device-scope atomics on one word; every maximum this workgroup published
    // has been performed (returning atomic, waited for) before it arrives, and
    // the group maxima are read back below with device-scope atomic loads.
    // Nothing else crosses workgroups before the outputs, so no cache-wide
    // acquire or release fence is needed (on MI355X each is a pass over the
    // L2 of every XCD, measured at over 10 us for this kernel).
    // Arrival is a two-level tree: workgroup b counts into subgroup b % 16;
    // the last member of a subgroup (all members' maxima performed before
    // their counts) counts into the top word, which everyone watches.
    if (threadIdx.x == 0) {
        const uint32_t nsub = min(P, kOpSubgroups);
        uint32_t *top = a.work + kOpTopWord;
        tree_count(a.work, P, nullptr);
        uint64_t t0 = (uint64_t)wall_clock64();
        int ok = 1;
        while (__hip_atomic_load(top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nsub) {
            __builtin_amdgcn_s_sleep(8);
            if ((uint64_t)wall_clock64() - t0 > a.wait_ticks) {
                ok = 0;
                break;
            }
        }
        passed = ok;
    }
    __syncthreads();
    phase_stamp(a, 2);
    if (!passed) {
        // Outputs are undefined.  This workgroup still counts out below, as
        // every workgroup does (also one that arrives after the others gave
        // up), so the last one out leaves the work buffer zeroed.
        if (threadIdx.x == 0 && a.status)
            *a.status = TRACE_E_BARRIER;
    } else {
        // Global scales of the groups this workgroup touches, into LDS (groups
        // past kOpGroupSlots, possible only for groups of a few tiles, are read
        // per item by one lane of each wave).
        const uint32_t g_first = kOneGroup ? 0u : i0 / a.tpg;
        const uint32_t g_count = kOneGroup ? 1u : min((i0 + cnt - 1) / a.tpg - g_first + 1, (uint32_t)kOpGroupSlots);
        for (uint32_t i = threadIdx.x; i < g_count; i += kOpThreads)
            gslot[i] = as_f(group_amax_bits(a, g_first + i)) / 2688.0f;
        __syncthreads();
        // One group, rollout codes: its scale tables, from the global scale just read.
        if constexpr (kTab) {
            const uint32_t ns = min(g_count, kSlots);
            for (uint32_t i = threadIdx.x; i < ns * 384u; i += kOpThreads) {
                const uint32_t sl = i / 384u, e = i - sl * 384u;
                const float gs = gslot[sl];
                if (e < 256u)
                    stab[sl * 256u + e] = scale_table_entry(e, gs);
                else
                    ctab[sl * 128u + e - 256u] = inv_combined(e4m3_decode(e - 256u), gs);
            }
            if (threadIdx.x < ns)
                ktab[threadIdx.x] = scale_table_k(gslot[threadIdx.x]);
            __syncthreads();
        }
        // The tables of an item's group (slot = group - g_first, below kSlots by
        // the host's choice; clamped so that a slip cannot leave the arrays).
        auto tabs_for = [&](uint32_t grp) {
            const uint32_t sl = kOneGroup ? 0u : min(grp - g_first, kSlots > 0 ? kSlots - 1 : 0u);
            return GroupTabs{stab + sl * 256u, ctab + sl * 128u, kTab ? ktab[sl] : 0};
        };

        // ---- phase 2: quantise ------------------------------------------------
        // Item positions are recomputed from a copy the compiler cannot see
        // through, so the scalar values of phase 1 are not kept alive (in spilled
        // SGPRs) across the barrier.
        uint32_t p2_reg = i_reg, p2_lds = i_lds;
        asm volatile("" : "+s"(p2_reg), "+s"(p2_lds));
        if (blockIdx.x == 0) {
            for (uint32_t i = threadIdx.x; i < a.G; i += kOpThreads)
                a.g_out[i] = as_f(group_amax_bits(a, i)) / 2688.0f;
            if (a.gd_scales)
                zero_pad<kOpThreads>(a.gd_scales, a.pad_begin, a.pad_end);
        }
        auto gscale = [&](uint32_t grp) {
            if (kOneGroup)
                return gslot[0];
            uint32_t i = grp - g_first;
            if (i < (uint32_t)kOpGroupSlots)
                return gslot[i];
            uint32_t bits = 0;
            if (__lane_id() == 0)
                bits = group_amax_bits(a, grp);
            return as_f(__builtin_amdgcn_readfirstlane(bits)) / 2688.0f;
        };
        // register tiles: straight-line code (tiles past nreg store nothing)
        // the run of chunks this workgroup owns (items are consecutive, and with
        // kSpan only the run's last item can be short)
        const Item w_first = item_at<kOneGroup>(a, i0), w_last = item_at<kOneGroup>(a, i0 + cnt - 1);
        const Outs span = outs_over<K, OUT>(a, w_first.first, w_last.first + w_last.count - w_first.first);
        const Outs none = outs_over<K, OUT>(a, 0u, 0u);  // no records: every store dropped
        auto outs_for = [&](const Item &w, bool live) {
            // An item that is not live stores nothing wherever it lies (a batch of
            // read-twice items can run past its last one into the LDS items).
            if (!live)
                return none;
            return kSpan ? span : outs_over<K, OUT>(a, w.first, w.count);
        };
        // (gv: the item's global scale; with scale tables it is not needed, and
        // not fetched, since the fetch past the LDS slots is a device-scope load)
        auto block_out = [&](const Outs &o, const Item &w, const Blk &b, uint32_t ab, float gv) {
            if constexpr (OUT == 0)
                quant_block<K, kTab>(o, w, b, ab, gv, tabs_for(w.grp));
            else
                rtn_block<OUT>(o, w, b, ab, gv);
        };
        // (with span descriptors a register tile that is not live lies past the
        // run's end, outside the records, so it needs no descriptor of its own)
        if constexpr (kTab) {
            // Scale tables (groups of whole tiles, so span descriptors): the two
            // dependent table reads of the next tile are issued before this
            // tile's conversion and stores, so their LDS latency overlaps them
            // instead of stalling each tile (2 waves per SIMD hide little).
            static_assert(!kTab || kSpan, "scale tables come with span descriptors");
            auto tabs_of = [&](int h) {
                GroupTabs t = tabs_for(item_at<kOneGroup>(a, p2_reg + h).grp);
                t.k = __builtin_amdgcn_readfirstlane(t.k);
                return t;
            };
            ScInv nx = block_scale_inv<true>(hab[0], 0.0f, tabs_of(0));
    #pragma unroll
            for (int h = 0; h < kOpRegTiles; ++h) {
                const ScInv cur = nx;
                if (h + 1 < kOpRegTiles)
                    nx = block_scale_inv<true>(hab[h + 1], 0.0f, tabs_of(h + 1));
                quant_block_with<K>(span, item_at<kOneGroup>(a, p2_reg + h), hr[h], cur);
            }
        } else {
    #pragma unroll
            for (int h = 0; h < kOpRegTiles; ++h) {
                Item w = item_at<kOneGroup>(a, p2_reg + h);
                bool live = p2_reg + h < i0 + cnt;
                block_out(kSpan ? span : outs_for(w, live), w, hr[h], hab[h], live && !kTab ? gscale(w.grp) : 0.0f);
            }
        }
        for (uint32_t j = 0; j < nlds; ++j) {
            Item w = item_at<kOneGroup>(a, p2_lds + j);
            Blk b = block_from_lds(lds_tiles, j);
            block_out(outs_for(w, true), w, b, block_amax_bits(b), kTab ? 0.0f : gscale(w.grp));
        }
        for (uint32_t j = 0; j < nstr; j += kBatch) {
            Chunk x[kBatch][2];
            Item w[kBatch];
            for (int q = 0; q < kBatch; ++q) {
                w[q] = item_at<kOneGroup>(a, i0 + j + q);
                load_item(a, w[q], j + q < nstr, x[q]);
            }
            for (int q = 0; q < kBatch; ++q) {
                bool live = j + q < nstr;
                Blk b = to_block(x[q]);
                block_out(outs_for(w[q], live), w[q], b, block_amax_bits(b), live && !kTab ? gscale(w[q].grp) : 0.0f);
            }
        }
    }

    // ---- departure: the last workgroup out leaves the work buffer zeroed ---
    // The barrier first: every wave of this workgroup has finished phase 2,
    // including its reads of the group maxima (the per-item fallback past the
    // LDS slots, and workgroup 0's g_out), before the workgroup counts out.
    // Every workgroup counts out exactly once, after its last read of the
    // work buffer, so nothing reads the words the last one clears; the next
    // call on the stream starts after this kernel has finished.
    __syncthreads();
    phase_stamp(a, 3);
    if (threadIdx.x == 0)
        tree_count(a.work + kOpDoneWord, P, &leaving_last);
    __syncthreads();
    if (leaving_last) {
        for (uint32_t i = threadIdx.x; i < 2 * (kOpSubgroups + 1); i += kOpThreads)
            a.work[i * kOpLine] = 0u;
        for (uint32_t i = threadIdx.x; i < a.G; i += kOpThreads)
            a.work[kOpAccWord + i] = 0u;
    }
}

// ---------------------------------------------------------------------------
// One-pass over many groups in teams of workgroups.
//
// When every group is a whole number of tiles and the tensor exceeds the
// on-chip capacity but a group takes only part of the chip, the grid is cut
// into T teams of S workgroups (S the fewest that hold one group on chip).
// Team t takes groups t, t + T, t + 2T, ... in turn.  For each group the
// team's members split its tiles evenly, hold their share on chip (LDS tiles
// first, register tiles last) as k_quant_onepass holds a run, publish the
// group's maximum, and meet at a barrier of their team alone (one counter
// line per team, counted up over the rounds: round r is complete at
// (r + 1) S arrivals); then they convert and store, and go on to the team's
// next group.  The input is read once; no barrier spans the grid, so the
// teams drift apart: one team's stores overlap another team's reads, and a
// slow workgroup holds up only its own team.  Registers and LDS are free at
// the end of each round.
// After a barrier times out the workgroup stops working, still arrives at
// its team's remaining rounds without waiting, and counts out, so every
// workgroup exits and the last one out leaves the work buffer zeroed.
// ---------------------------------------------------------------------------
template <int K, int OUT, bool kTab>
__global__ void __launch_bounds__(kOpThreads) k_quant_onepass_teams(OnePass a)
{
    static_assert(!kTab || OUT == 0, "scale tables serve the rollout codes only");
    constexpr int kOtRegTiles = ot_reg_tiles(OUT);
    extern __shared__ u32x4 lds_tiles[];               // a.lds_tiles * 2 * kOpThreads chunks
    __shared__ uint32_t wmax[kOpThreads / 64];
    __shared__ int passed;
    __shared__ bool leaving_last;
    __shared__ float gshared;
    __shared__ float2 stab[kTab ? 256 : 1];
    __shared__ float ctab[kTab ? 128 : 1];
    __shared__ int ktab;

    const uint32_t S = a.team_size, T = gridDim.x / S;     // the host launches T * S workgroups
    const uint32_t team = blockIdx.x / S, member = blockIdx.x - team * S;
    uint32_t *counter = a.work + kOpTeamWord + team * kOpLine;
    if (threadIdx.x == 0)
        passed = 1;
    __syncthreads();
    uint32_t round = 0;
    for (uint32_t grp = team; grp < a.G; grp += T, ++round) {
        // this member's share of the group: items [i0, i0 + cnt), at most
        // kOtRegTiles + a.lds_tiles (the host's choice of S)
        const uint32_t base = grp * a.tpg;
        const uint32_t i0 = base + (uint32_t)((uint64_t)a.tpg * member / S);
        const uint32_t cnt = base + (uint32_t)((uint64_t)a.tpg * (member + 1) / S) - i0;
        const uint32_t nreg = min(cnt, (uint32_t)kOtRegTiles);
        const uint32_t nlds = cnt - nreg;
        const uint32_t i_reg = i0 + nlds;
        Blk hr[kOtRegTiles];
        uint32_t hab[kOtRegTiles];
        if (passed) {
            // ---- phase 1: read the share once, fold its maximum -----------------
            for (uint32_t j = 0; j < nlds; ++j)
                load_item_to_lds(a, item_at<false>(a, i0 + j), lds_tiles, j);
#pragma unroll
            for (int h = 0; h < kOtRegTiles; ++h) {
                Chunk x[2];
                load_item(a, item_at<false>(a, i_reg + h), (uint32_t)h < nreg, x);
                hr[h].lo = x[0];
                hr[h].hi = x[1];
            }
            __builtin_amdgcn_s_waitcnt(0);             // the LDS copies have landed (this wave's own)
            uint32_t run = 0;
            for (uint32_t j = 0; j < nlds; ++j) {
                Chunk x[2];
                read_item_from_lds(lds_tiles, item_at<false>(a, i0 + j), j, x);
                run = max(run, max(chunk_amax_finite(x[0], a.status), chunk_amax_finite(x[1], a.status)));
            }
#pragma unroll
            for (int h = 0; h < kOtRegTiles; ++h) {
                Chunk x[2] = {hr[h].lo, hr[h].hi};
                hr[h] = to_block(x);
                hab[h] = block_amax_bits(hr[h]);
                if ((uint32_t)h < nreg)
                    run = max(run, hab[h] < 0x7f80u ? hab[h]
                                                    : max(chunk_amax_finite(hr[h].lo, a.status),
                                                          chunk_amax_finite(hr[h].hi, a.status)));
            }
            if (cnt > 0)
                amax_publish<kOpThreads, true>(run, wmax, a.work + kOpAccWord + grp);
        }

        // ---- the team's barrier for this group (bounded) ----------------------
        // Every maximum this workgroup published has been performed before it
        // arrives; the group maximum is read back with a device-scope load.
        if (threadIdx.x == 0) {
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (passed) {
                const uint32_t target = (round + 1) * S;
                const uint64_t t0 = (uint64_t)wall_clock64();
                while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                    __builtin_amdgcn_s_sleep(8);
                    if ((uint64_t)wall_clock64() - t0 > a.wait_ticks) {
                        passed = 0;                    // outputs undefined from here on
                        if (a.status)
                            *a.status = TRACE_E_BARRIER;
                        break;
                    }
                }
                if (passed)
                    gshared = as_f(group_amax_bits(a, grp)) / 2688.0f;
            }
        }
        __syncthreads();
        if (!passed)
            continue;                                  // arrive at the remaining rounds only

        // ---- phase 2: convert and store the share ------------------------------
        // (item positions from copies the compiler cannot see through, so the
        // scalar values of phase 1 are not kept alive across the barrier)
        uint32_t p2_i0 = i0, p2_reg = i_reg, p2_cnt = cnt;
        asm volatile("" : "+s"(p2_i0), "+s"(p2_reg), "+s"(p2_cnt));
        const float gv = gshared;
        if constexpr (kTab) {
            for (uint32_t e = threadIdx.x; e < 384u; e += kOpThreads) {
                if (e < 256u)
                    stab[e] = scale_table_entry(e, gv);
                else
                    ctab[e - 256u] = inv_combined(e4m3_decode(e - 256u), gv);
            }
            if (threadIdx.x == 0)
                ktab = scale_table_k(gv);
            __syncthreads();
        }
        if (member == 0 && threadIdx.x == 0)
            a.g_out[grp] = gv;
        if (blockIdx.x == 0 && round == 0 && a.gd_scales)
            zero_pad<kOpThreads>(a.gd_scales, a.pad_begin, a.pad_end);
        const GroupTabs tabs{stab, ctab, kTab ? __builtin_amdgcn_readfirstlane(ktab) : 0};
        // one descriptor per output over the share (whole tiles); register
        // tiles past the share lie outside its records and store nothing
        const Outs span = outs_over<K, OUT>(a, item_at<false>(a, p2_i0).first, p2_cnt * (uint32_t)kOpTile);
        if constexpr (kTab) {
            // the next tile's two dependent table reads are issued before this
            // tile's conversion and stores (as in k_quant_onepass)
            ScInv nx = block_scale_inv<true>(hab[0], 0.0f, tabs);
#pragma unroll
            for (int h = 0; h < kOtRegTiles; ++h) {
                const ScInv cur = nx;
                if (h + 1 < kOtRegTiles)
                    nx = block_scale_inv<true>(hab[h + 1], 0.0f, tabs);
                quant_block_with<K>(span, item_at<false>(a, p2_reg + h), hr[h], cur);
            }
        } else {
#pragma unroll
            for (int h = 0; h < kOtRegTiles; ++h) {
                const Item w = item_at<false>(a, p2_reg + h);
                if constexpr (OUT == 0)
                    quant_block<K, false>(span, w, hr[h], hab[h], gv, tabs);
                else
                    rtn_block<OUT>(span, w, hr[h], hab[h], gv);
            }
        }
        for (uint32_t j = 0; j < p2_reg - p2_i0; ++j) {
            const Item w = item_at<false>(a, p2_i0 + j);
            const Blk b = block_from_lds(lds_tiles, j);
            if constexpr (OUT == 0)
                quant_block<K, kTab>(span, w, b, block_amax_bits(b), gv, tabs);
            else
                rtn_block<OUT>(span, w, b, block_amax_bits(b), gv);
        }
    }

    // ---- departure, as in k_quant_onepass (the team lines cleared too) -------
    __syncthreads();
    if (threadIdx.x == 0)
        tree_count(a.work + kOpDoneWord, gridDim.x, &leaving_last);
    __syncthreads();
    if (leaving_last) {
        for (uint32_t i = threadIdx.x; i < 2 * (kOpSubgroups + 1) + kOpMaxTeams; i += kOpThreads)
            a.work[i * kOpLine] = 0u;
        for (uint32_t i = threadIdx.x; i < a.G; i += kOpThreads)
            a.work[kOpAccWord + i] = 0u;
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
    zero_pad<kThreads>(gd_scales, pad_begin, pad_end);
    uint32_t q = blockIdx.x * kThreads + threadIdx.x;     // quad of chunks
    uint32_t c = 4 * q;
    if (c + 4 <= nchunk) {
        u32x4 cw = ld_stream(reinterpret_cast<const u32x4 *>(codes) + q);
        reinterpret_cast<uint16_t *>(gd_scales)[q] = reinterpret_cast<const uint16_t *>(scales)[q];
        if (K == 4) {
            reinterpret_cast<u32x4 *>(gd_bits)[q] = cw;
        } else if (K == 3) {                                 // 4 x 24 bits = 3 words at 12 q
            uint32_t b0 = compact_k3(cw.x), b1 = compact_k3(cw.y), b2 = compact_k3(cw.z), b3 = compact_k3(cw.w);
            uint32_t *p = reinterpret_cast<uint32_t *>(gd_bits) + 3 * q;
            p[0] = b0 | (b1 << 24);
            p[1] = (b1 >> 8) | (b2 << 16);
            p[2] = (b2 >> 16) | (b3 << 8);
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

// Training side, guided (MODE 1, 2, 3: k guidance bits) or full code (MODE 4).
template <int MODE, bool kOneGroup, bool kCodes>
__global__ void __launch_bounds__(kThreads)
    k_fakequant_guided(const u32x4 *x, uint32_t nchunk, const float *__restrict__ g, DivMagic dm,
                       uint32_t last_group, const uint8_t *__restrict__ scale_plane,
                       const uint8_t *__restrict__ bits, OutPtr out, uint32_t *__restrict__ codes_out)
{
    // MODE 3 (the whole magnitude index) decides like the full code with the
    // sign taken from v, so it shares the full-code table
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
                else if (MODE == 3)
                    gb[u] = load_bits3(bits, c);
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
                } else if (MODE == 3) {
                    row = (gb[u] >> (3 * i)) & 7u;
                } else {
                    uint32_t r = (gb[u] >> (4 * i)) & 0xfu;
                    row = r & 7u;
                    allow = (r >> 3) == (as_u(v) >> 31);
                }
                yv[i] = decide<R, kCodes>(tab, v, row, allow, s[u], gg[u], nib);
                if (kCodes)
                    nw |= nib << (4 * i);
            }
            store_y<TRACE_NT_STORE_GUIDED>(out, c, yv);
            if (kCodes)
                st_stream<TRACE_NT_STORE_GUIDED>(nw, codes_out + c);
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
            store_y<TRACE_NT_STORE_RTN>(out, c, yv);
            if (kCodes)
                st_stream<TRACE_NT_STORE_RTN>(cw, codes_out + c);
        }
    }
}

// Straight-through gradient of the fake-quant, clipped at the quantiser's
// range: gx = gy where |v| <= 6 and 0 where |v| > 6 (the forward saturated
// there, so its output does not move with x), v = x * inv with the inv =
// 1 / (s * g) of the scales the forward used (pair_scales_from_bytes, as the
// guided and shared-scale kernels compute it).  kF32: gradients in fp32,
// else bf16.  gx may be gy.
template <bool kOneGroup, bool kF32>
__global__ void __launch_bounds__(kThreads)
    k_ste_grad(const u32x4 *__restrict__ x, uint32_t nchunk, const float *__restrict__ g, DivMagic dm,
               uint32_t last_group, const uint8_t *__restrict__ scales, const u32x4 *gy, u32x4 *gx)
{
    constexpr int W = kF32 ? 2 : 1;                     // 16-byte words of gradient per chunk
    uint32_t ntiles = (nchunk + kTile - 1) / kTile;
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        Chunk xc[kUnroll];
        u32x4 gw[kUnroll][W];
        uint32_t cs[kUnroll], sc[kUnroll];
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t c = t * kTile + u * kThreads + threadIdx.x;
            cs[u] = c;
            xc[u] = Chunk{{0u, 0u, 0u, 0u}};
            sc[u] = 0u;
            for (int h = 0; h < W; ++h)
                gw[u][h] = u32x4{0u, 0u, 0u, 0u};
            if (c < nchunk) {
                xc[u] = load_chunk(x, c);
                sc[u] = scales[c >> 1];
                for (int h = 0; h < W; ++h)
                    gw[u][h] = ld_stream(gy + (size_t)W * c + h);
            }
        }
        if (cs[0] >= nchunk)
            continue;
        float gg[kUnroll];
        for (int u = 0; u < kUnroll; ++u)
            gg[u] = group_scale<kOneGroup>(g, cs[u] >> 1, dm, last_group);
        PairScales ps = pair_scales_from_bytes(sc[0], sc[1], gg[0], gg[1]);
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t c = cs[u];
            if (c >= nchunk)
                continue;
            uint32_t keep = 0;                          // bit i: element i passes its gradient
            for (int i = 0; i < 8; ++i) {
                uint32_t w = xc[u].w[i >> 1];
                float v = ((i & 1) ? bf_hi(w) : bf_lo(w)) * ps.inv[u];
                keep |= (fabsf(v) <= 6.0f ? 1u : 0u) << i;
            }
            for (int h = 0; h < W; ++h) {
                u32x4 o = gw[u][h];
                if constexpr (kF32) {                     // one element per word
                    for (int j = 0; j < 4; ++j)
                        o[j] = ((keep >> (4 * h + j)) & 1u) ? o[j] : 0u;
                } else {                                  // two bf16 per word, element 2m low
                    for (int j = 0; j < 4; ++j) {
                        uint32_t m = (((keep >> (2 * j)) & 1u) ? 0x0000ffffu : 0u) |
                                     (((keep >> (2 * j + 1)) & 1u) ? 0xffff0000u : 0u);
                        o[j] &= m;
                    }
                }
                st_stream<TRACE_NT_STORE_RTN>(o, gx + (size_t)W * c + h);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// MXFP4 variant: blocks of 32 elements with a power-of-two (E8M0) scale and no
// global scale (OCP Microscaling Formats v1.0 conversion; the block format of
// gfx950's scaled FP4 conversions).  Four consecutive lanes hold a block: the
// block maximum is two DPP steps, the scale needs no division (code = bf16
// exponent field - 2, i.e. floor(log2 amax) - 2 + 127, clamped at 0), and
// normalising and dequantising are exact multiplies by powers of two.  RTN,
// the guided tables and the stores are the ones above.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t quad_max(uint32_t m)
{
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xb1, 0xf, 0xf, false));   // lane ^ 1
    return max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4e, 0xf, 0xf, false));  // lane ^ 2
}

// E8M0 code of a block from its amax (bf16 magnitude bits): the exponent
// field e gives floor(log2 amax) = e - 127 for normal values; subnormal,
// tiny and zero blocks clamp to code 0.
__device__ __forceinline__ uint32_t mx_code(uint32_t a16)
{
    uint32_t e = a16 >> 7;
    return e >= 2 ? e - 2 : 0u;
}

__device__ __forceinline__ float mx_scale(uint32_t code) { return __builtin_ldexpf(1.0f, (int)code - 127); }
__device__ __forceinline__ float mx_inv(uint32_t code) { return __builtin_ldexpf(1.0f, 127 - (int)code); }

template <int K>
__global__ void __launch_bounds__(kThreads)
    k_mx_quant_rollout(const u32x4 *__restrict__ y, uint32_t nchunk, uint32_t *__restrict__ codes,
                       uint8_t *__restrict__ scales, uint8_t *__restrict__ gd_scales, uint8_t *__restrict__ gd_bits,
                       uint32_t pad_begin, uint32_t pad_end)
{
    if (gd_scales)
        zero_pad<kThreads>(gd_scales, pad_begin, pad_end);
    uint32_t ntiles = (nchunk + kTile - 1) / kTile;
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        Chunk xc[kUnroll];
        uint32_t cs[kUnroll];
        for (int u = 0; u < kUnroll; ++u) {
            cs[u] = t * kTile + u * kThreads + threadIdx.x;
            xc[u] = cs[u] < nchunk ? load_chunk(y, cs[u]) : Chunk{{0u, 0u, 0u, 0u}};
        }
        if (cs[0] >= nchunk)
            continue;
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t code = mx_code(quad_max(chunk_amax_bits(xc[u])));
            uint32_t c = cs[u];
            if (c >= nchunk)
                continue;
            if ((c & 3u) == 0) {
                scales[c >> 2] = (uint8_t)code;
                if (gd_scales)
                    gd_scales[c >> 2] = (uint8_t)code;
            }
            uint32_t cw = rtn8(xc[u], mx_inv(code));
            st_stream<TRACE_NT_STORE_QUANT>(cw, codes + c);
            if (gd_scales)
                store_bits<K>(gd_bits, c, cw);
        }
    }
}

// Training side with MX scales: guided (MODE 1, 2, 3) or full code (MODE 4).
template <int MODE, bool kCodes>
__global__ void __launch_bounds__(kThreads)
    k_mx_fakequant_guided(const u32x4 *x, uint32_t nchunk, const uint8_t *__restrict__ scale_plane,
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
                sc[u] = scale_plane[c >> 2];
                if (MODE == 1)
                    gb[u] = bits[c];
                else if (MODE == 2)
                    gb[u] = reinterpret_cast<const uint16_t *>(bits)[c];
                else if (MODE == 3)
                    gb[u] = load_bits3(bits, c);
                else
                    gb[u] = ld_stream(reinterpret_cast<const uint32_t *>(bits) + c);
            }
        }
        if (cs[0] >= nchunk)
            continue;
        for (int u = 0; u < kUnroll; ++u) {
            uint32_t c = cs[u];
            if (c >= nchunk)
                continue;
            float s = mx_scale(sc[u]), inv = mx_inv(sc[u]);
            float yv[8];
            uint32_t nw = 0;
            for (int i = 0; i < 8; ++i) {
                uint32_t w = xc[u].w[i >> 1];
                float v = ((i & 1) ? bf_hi(w) : bf_lo(w)) * inv;
                uint32_t row, nib = 0;
                bool allow = true;
                if (MODE == 1) {
                    row = (gb[u] >> i) & 1u;
                } else if (MODE == 2) {
                    row = (gb[u] >> (2 * i)) & 3u;
                } else if (MODE == 3) {
                    row = (gb[u] >> (3 * i)) & 7u;
                } else {
                    uint32_t r = (gb[u] >> (4 * i)) & 0xfu;
                    row = r & 7u;
                    allow = (r >> 3) == (as_u(v) >> 31);
                }
                yv[i] = decide<R, kCodes>(tab, v, row, allow, s, 1.0f, nib);
                if (kCodes)
                    nw |= nib << (4 * i);
            }
            store_y<TRACE_NT_STORE_GUIDED>(out, c, yv);
            if (kCodes)
                st_stream<TRACE_NT_STORE_GUIDED>(nw, codes_out + c);
        }
    }
}

// Plain RTN with MX scales: from scales_in (kOwn = false) or from x.
template <bool kOwn, bool kCodes>
__global__ void __launch_bounds__(kThreads)
    k_mx_fakequant_rtn(const u32x4 *x, uint32_t nchunk, const uint8_t *__restrict__ scales_in, OutPtr out,
                       uint32_t *__restrict__ codes_out, uint8_t *__restrict__ scales_out)
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
                    sc[u] = scales_in[c >> 2];
            }
        }
        if (cs[0] >= nchunk)
            continue;
        for (int u = 0; u < kUnroll; ++u) {
            if (kOwn)
                sc[u] = mx_code(quad_max(chunk_amax_bits(xc[u])));
            uint32_t c = cs[u];
            if (c >= nchunk)
                continue;
            if (kOwn && scales_out && (c & 3u) == 0)
                scales_out[c >> 2] = (uint8_t)sc[u];
            float s = mx_scale(sc[u]);
            uint32_t cw = rtn8(xc[u], mx_inv(sc[u]));
            float yv[8];
            decode8(cw, yv);
            for (int i = 0; i < 8; ++i)
                yv[i] = yv[i] * s;                         // exact: a power of two
            store_y<TRACE_NT_STORE_RTN>(out, c, yv);
            if (kCodes)
                st_stream<TRACE_NT_STORE_RTN>(cw, codes_out + c);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// Chunk counts (n / 8) stay below 2^31, so every 32-bit chunk index, tile
// count and rounded-up sum in the kernels and their launch plans fits.
constexpr int64_t kMaxN = int64_t(1) << 34;

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

// Device facts the one-pass launch depends on, queried once per device.
struct OnePassDevice {
    int cus = 0;               // compute units
    int per_cu = 0;            // resident one-pass workgroups per compute unit
    uint32_t lds_tiles = 0;    // tiles a workgroup keeps in LDS
    int64_t clock_khz = 0;     // wall-clock rate
};

constexpr int kMaxDevices = 64;

int onepass_device(OnePassDevice &out)
{
    static OnePassDevice cache[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TRACE_E_HIP;
    std::call_once(once[dev], [dev] {
        OnePassDevice d;
        int lds = 0, khz = 0, per = 0;
        if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
            return;
        // static LDS of the kernel (under 12 KiB: the group-scale slots and
        // the scale tables of up to kOpTabSlots groups) sits below the
        // dynamic tiles; occupancy is taken for the variant with the most
        d.lds_tiles = lds > 12288 ? (uint32_t)((lds - 12288) / (kOpTile * 16)) : 0u;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_quant_onepass<2, false, true, 0, true>, kOpThreads,
                                                         (size_t)d.lds_tiles * kOpTile * 16) != hipSuccess)
            return;
        d.per_cu = per;
        d.clock_khz = khz;
        cache[dev] = d;
    });
    (void)hipGetLastError();
    out = cache[dev];
    return out.cus > 0 && out.per_cu > 0 && out.clock_khz > 0 ? TRACE_OK : TRACE_E_HIP;
}

uint32_t onepass_work_words(int G) { return kOpAccWord + (uint32_t)G; }

}  // namespace

extern "C" {

size_t trace_onepass_work_bytes(int G)
{
    if (G < 1)
        return 0;
    return ((size_t)onepass_work_words(G) * 4 + 255) / 256 * 256;
}

int64_t trace_onepass_capacity(int max_workgroups)
{
    OnePassDevice d;
    if (max_workgroups < 0 || onepass_device(d) != TRACE_OK)
        return 0;
    int64_t grid = (int64_t)d.cus * d.per_cu;
    if (max_workgroups > 0 && max_workgroups < grid)
        grid = max_workgroups;
    return grid * (int64_t)(kOpRegTiles + d.lds_tiles) * kOpTile * 8;
}

}  // extern "C"

namespace {

// Output descriptors over a workgroup's run of chunks hold 32-bit byte
// counts and offsets: the longest run (items spread over `grid` workgroups)
// times the widest output plane's bytes per chunk (4 for rollout codes and
// guidance bits, 16 / 32 for bf16 / f32 fake-quant outputs) must stay below
// 2^32.  Only a small workgroup cap on a large tensor can exceed it.
bool onepass_run_fits(uint64_t items, int64_t grid, uint32_t bytes_per_chunk)
{
    const uint64_t run = (items + (uint64_t)grid - 1) / (uint64_t)grid * (uint64_t)kOpTile;
    return run * bytes_per_chunk < (uint64_t(1) << 32);
}

// The same test before any device query, for one group under an explicit
// workgroup cap (the grid is at most the cap, so the run is at least this).
bool onepass_cap_fits(int64_t n, int G, int max_workgroups, uint32_t bytes_per_chunk)
{
    if (G != 1 || max_workgroups <= 0)
        return true;
    const uint64_t items = ((uint64_t)n / 8 + kOpTile - 1) / kOpTile;
    return onepass_run_fits(items, max_workgroups, bytes_per_chunk);
}

#if TRACE_OP_PHASE_CLOCK
uint64_t *g_phase_clock = nullptr;   // device buffer of 4 values per workgroup, set by trace_debug_phase_clock
#endif

// The launch parameters shared by both one-pass entry points (arguments
// already checked): the item layout, the barrier limit and the grid.
int onepass_plan(const void *in_bf16, int64_t n, int G, float *g_out, void *work, int max_workgroups,
                 int *status_dev, uint32_t bytes_per_chunk, OnePass &a, int64_t &grid, size_t &lds)
{
    OnePassDevice d;
    int rc = onepass_device(d);
    if (rc != TRACE_OK)
        return rc;
    a = OnePass{};
    uint32_t nchunk = (uint32_t)(n / 8);
    a.y = (const u32x4 *)in_bf16;
    a.cpg = nchunk / (uint32_t)G;
    a.tpg = (a.cpg + kOpTile - 1) / kOpTile;
    a.tpg_div = make_div_magic(a.tpg);
    a.items = a.tpg * (uint32_t)G;                       // <= nchunk / 2 + G < 2^32
    a.G = (uint32_t)G;
    a.lds_tiles = d.lds_tiles;
    a.pad_begin = (uint32_t)(n / 16);
    a.pad_end = (uint32_t)bitplane_offset(n);
    // the longest legitimate wait is one pass over the input; allow 1 s plus
    // the input at 50 GB/s (TRACE_ONEPASS_WAIT_US replaces the limit: a test
    // of the failure path)
    double secs = 1.0 + (double)n * 2.0 / 5.0e10;
    if (const char *env = std::getenv("TRACE_ONEPASS_WAIT_US"))
        secs = std::strtod(env, nullptr) * 1e-6;
    a.wait_ticks = (uint64_t)(secs > 0.0 ? secs * (double)d.clock_khz * 1000.0 : 0.0);
    a.work = (uint32_t *)work;
    a.g_out = g_out;
    a.status = status_dev;
#if TRACE_OP_PHASE_CLOCK
    a.clock = g_phase_clock;
#endif
    grid = (int64_t)d.cus * d.per_cu;
    if (max_workgroups > 0 && max_workgroups < grid)
        grid = max_workgroups;
    if (grid > (int64_t)a.items)
        grid = a.items;
    if (!onepass_run_fits(a.items, grid, bytes_per_chunk))
        return TRACE_E_SIZE;
    lds = (size_t)a.lds_tiles * kOpTile * 16;
    return TRACE_OK;
}

// Groups per launch of the one-pass entry points.  A tensor that fits on chip
// is one launch.  With several groups, when the whole tensor does not fit but
// one group does, the call runs one launch per block of whole groups that
// fits (as few blocks as possible, of equal size but the last): each launch
// reads its part once, and groups share nothing, so the results are those of
// one launch.  Otherwise (one group, or a group larger than the chip) one
// launch reads the excess twice.
int onepass_groups_per_launch(int64_t n, int G, int max_workgroups, int &gpb)
{
    OnePassDevice d;
    int rc = onepass_device(d);
    if (rc != TRACE_OK)
        return rc;
    int64_t grid = (int64_t)d.cus * d.per_cu;
    if (max_workgroups > 0 && max_workgroups < grid)
        grid = max_workgroups;
    const int64_t cap_tiles = grid * (int64_t)(kOpRegTiles + d.lds_tiles);
    const int64_t tpg = (n / 8 / G + kOpTile - 1) / kOpTile;
    gpb = G;
    if (G > 1 && tpg * G > cap_tiles && tpg <= cap_tiles) {
        const int64_t fit = cap_tiles / tpg;
        const int64_t blocks = (G + fit - 1) / fit;
        gpb = (int)((G + blocks - 1) / blocks);
    }
    return TRACE_OK;
}

// One launch of the one-pass rollout over n elements in G groups, with the
// outputs at the given places (a block of groups of a larger tensor writes
// into that tensor's planes); the guidance pad [pad_begin, pad_end) is
// relative to gd_scales.
int rollout_onepass_launch(const void *y_bf16, int64_t n, int G, int k, float *g_out, uint8_t *codes,
                           uint8_t *scales, uint8_t *gd_scales, uint8_t *gd_bits, uint32_t pad_begin,
                           uint32_t pad_end, void *work, int max_workgroups, int *status_dev, hipStream_t st)
{
    OnePass a;
    int64_t grid;
    size_t lds;
    int rc = onepass_plan(y_bf16, n, G, g_out, work, max_workgroups, status_dev, 4u, a, grid, lds);
    if (rc != TRACE_OK)
        return rc;
    a.codes = (uint32_t *)codes;
    a.scales = scales;
    a.gd_scales = gd_scales;
    a.gd_bits = gd_bits;
    a.pad_begin = pad_begin;
    a.pad_end = pad_end;
    (void)hipGetLastError();
#define TRACE_OP(KK, ONE, SPAN) \
    hipLaunchKernelGGL((k_quant_onepass<KK, ONE, SPAN>), dim3((uint32_t)grid), dim3(kOpThreads), lds, st, a)
#define TRACE_OPT(KK) \
    hipLaunchKernelGGL((k_quant_onepass<KK, false, true, 0, true>), dim3((uint32_t)grid), dim3(kOpThreads), lds, st, a)
    // the most groups one workgroup's run of items spans (runs as in the kernel)
    uint32_t span = 0;
    for (int64_t b = 0; b < grid; ++b) {
        uint32_t f = (uint32_t)((uint64_t)a.items * (uint64_t)b / (uint64_t)grid);
        uint32_t l = (uint32_t)((uint64_t)a.items * (uint64_t)(b + 1) / (uint64_t)grid) - 1u;
        span = std::max(span, l / a.tpg - f / a.tpg + 1u);
    }
    if (G == 1) {                                      // one group: only the tensor's last tile can be short
        if (k == 1) TRACE_OP(1, true, true);
        else if (k == 2) TRACE_OP(2, true, true);
        else if (k == 3) TRACE_OP(3, true, true);
        else TRACE_OP(4, true, true);
    } else if (a.cpg % kOpTile == 0 && span <= kOpTabSlots) {   // whole tiles, scale tables for every run
        if (k == 1) TRACE_OPT(1);
        else if (k == 2) TRACE_OPT(2);
        else if (k == 3) TRACE_OPT(3);
        else TRACE_OPT(4);
    } else if (a.cpg % kOpTile == 0) {                 // groups of whole tiles
        if (k == 1) TRACE_OP(1, false, true);
        else if (k == 2) TRACE_OP(2, false, true);
        else if (k == 3) TRACE_OP(3, false, true);
        else TRACE_OP(4, false, true);
    } else {
        if (k == 1) TRACE_OP(1, false, false);
        else if (k == 2) TRACE_OP(2, false, false);
        else if (k == 3) TRACE_OP(3, false, false);
        else TRACE_OP(4, false, false);
    }
#undef TRACE_OP
#undef TRACE_OPT
    return launched();
}

// One launch of the one-pass own-scale RTN fake-quant (as above).
int rtn_onepass_launch(const void *x_bf16, int64_t n, int G, float *g_out, void *y_out, bool f32,
                       uint8_t *codes_out, uint8_t *scales_out, void *work, int max_workgroups, int *status_dev,
                       hipStream_t st)
{
    OnePass a;
    int64_t grid;
    size_t lds;
    int rc = onepass_plan(x_bf16, n, G, g_out, work, max_workgroups, status_dev, f32 ? 32u : 16u, a, grid, lds);
    if (rc != TRACE_OK)
        return rc;
    a.codes = (uint32_t *)codes_out;
    a.scales = scales_out;
    a.out = y_out;
    (void)hipGetLastError();
#define TRACE_OR(ONE, SPAN)                                                                                        \
    do {                                                                                                           \
        if (f32)                                                                                                   \
            hipLaunchKernelGGL((k_quant_onepass<2, ONE, SPAN, 2>), dim3((uint32_t)grid), dim3(kOpThreads), lds, st, a); \
        else                                                                                                       \
            hipLaunchKernelGGL((k_quant_onepass<2, ONE, SPAN, 1>), dim3((uint32_t)grid), dim3(kOpThreads), lds, st, a); \
    } while (0)
    if (G == 1)
        TRACE_OR(true, true);
    else if (a.cpg % kOpTile == 0)
        TRACE_OR(false, true);
    else
        TRACE_OR(false, false);
#undef TRACE_OR
    return launched();
}

// Team shape for k_quant_onepass_teams: S workgroups per team (the fewest
// that hold one group on chip) and the grid T * S, or false when it does not
// apply.  It applies when a call would otherwise take several launches
// (gpb < G), every group is a whole number of tiles, and at least two teams
// fit in the grid (at most kOpMaxTeams, each on its own counter line).
bool onepass_team_shape(int64_t n, int G, int gpb, int max_workgroups, int out, uint32_t &S, int64_t &grid)
{
    OnePassDevice d;
    if (gpb >= G || (n / 8 / G) % kOpTile != 0 || onepass_device(d) != TRACE_OK)
        return false;
    int64_t cap = (int64_t)d.cus * d.per_cu;
    if (max_workgroups > 0 && max_workgroups < cap)
        cap = max_workgroups;
    const int64_t tpg = n / 8 / G / kOpTile;
    const int64_t per_wg = ot_reg_tiles(out) + (int64_t)d.lds_tiles;
    const int64_t size = (tpg + per_wg - 1) / per_wg;
    const int64_t teams = std::min<int64_t>({cap / size, (int64_t)kOpMaxTeams, (int64_t)G});
    if (teams < 2)
        return false;
    S = (uint32_t)size;
    grid = teams * size;
    return true;
}

int rollout_onepass_teams(const void *y_bf16, int64_t n, int G, int k, float *g_out, uint8_t *codes,
                          uint8_t *scales, uint8_t *guidance, void *work, uint32_t S, int64_t grid_teams,
                          int *status_dev, hipStream_t st)
{
    OnePass a;
    int64_t grid;
    size_t lds;
    int rc = onepass_plan(y_bf16, n, G, g_out, work, (int)grid_teams, status_dev, 4u, a, grid, lds);
    if (rc != TRACE_OK)
        return rc;
    if (grid != grid_teams)                            // the plan keeps the grid asked for (it is below the cap)
        return TRACE_E_HIP;
    a.team_size = S;
    a.codes = (uint32_t *)codes;
    a.scales = scales;
    a.gd_scales = guidance;
    a.gd_bits = guidance ? guidance + bitplane_offset(n) : nullptr;
    (void)hipGetLastError();
#define TRACE_OT(KK) \
    hipLaunchKernelGGL((k_quant_onepass_teams<KK, 0, true>), dim3((uint32_t)grid), dim3(kOpThreads), lds, st, a)
    if (k == 1)
        TRACE_OT(1);
    else if (k == 2)
        TRACE_OT(2);
    else if (k == 3)
        TRACE_OT(3);
    else
        TRACE_OT(4);
#undef TRACE_OT
    return launched();
}

int rtn_onepass_teams(const void *x_bf16, int64_t n, int G, float *g_out, void *y_out, bool f32, uint8_t *codes_out,
                      uint8_t *scales_out, void *work, uint32_t S, int64_t grid_teams, int *status_dev,
                      hipStream_t st)
{
    OnePass a;
    int64_t grid;
    size_t lds;
    int rc = onepass_plan(x_bf16, n, G, g_out, work, (int)grid_teams, status_dev, f32 ? 32u : 16u, a, grid, lds);
    if (rc != TRACE_OK)
        return rc;
    if (grid != grid_teams)
        return TRACE_E_HIP;
    a.team_size = S;
    a.codes = (uint32_t *)codes_out;
    a.scales = scales_out;
    a.out = y_out;
    (void)hipGetLastError();
    if (f32)
        hipLaunchKernelGGL((k_quant_onepass_teams<2, 2, false>), dim3((uint32_t)grid), dim3(kOpThreads), lds, st, a);
    else
        hipLaunchKernelGGL((k_quant_onepass_teams<2, 1, false>), dim3((uint32_t)grid), dim3(kOpThreads), lds, st, a);
    return launched();
}

// Argument checks of the one-pass rollout entry points (with or without a
// caller-owned work buffer), before anything touches the device.
int rollout_onepass_check(const void *y_bf16, int64_t n, int G, int k, const float *g_out, const uint8_t *codes,
                          const uint8_t *scales, const uint8_t *guidance, bool need_work, const void *work,
                          int max_workgroups, const int *status_dev)
{
    int rc = check_sizes(n, G);
    if (rc)
        return rc;
    if (!y_bf16 || !g_out || !codes || !scales || (need_work && !work))
        return TRACE_E_NULL;
    if (!aligned16(y_bf16) || !aligned16(g_out) || !aligned16(codes) || !aligned16(scales) ||
        (guidance && !aligned16(guidance)) || (need_work && !aligned16(work)) ||
        (status_dev && !aligned16(status_dev)))
        return TRACE_E_ALIGN;
    if (k < 1 || k > 4)
        return TRACE_E_K;
    if (max_workgroups < 0 || !onepass_cap_fits(n, G, max_workgroups, 4u))
        return TRACE_E_SIZE;
    return TRACE_OK;
}

// The one-pass rollout over checked arguments with the given work buffer.
int rollout_onepass_run(const void *y_bf16, int64_t n, int G, int k, float *g_out, uint8_t *codes, uint8_t *scales,
                        uint8_t *guidance, void *work, int max_workgroups, int *status_dev, hipStream_t st)
{
    int gpb, rc;
    if ((rc = onepass_groups_per_launch(n, G, max_workgroups, gpb)) != TRACE_OK)
        return rc;
    uint32_t S;
    int64_t grid;
    if (onepass_team_shape(n, G, gpb, max_workgroups, 0, S, grid))   // many groups of whole tiles: one launch in teams
        return rollout_onepass_teams(y_bf16, n, G, k, g_out, codes, scales, guidance, work, S, grid, status_dev, st);
    const int64_t per = n / G, bits = bitplane_offset(n);
    for (int g0 = 0; g0 < G; g0 += gpb) {              // blocks of whole groups (one block when it all fits)
        const int gb = std::min(gpb, G - g0);
        const int64_t e0 = (int64_t)g0 * per;          // a multiple of 16: every plane's offset is whole bytes
        rc = rollout_onepass_launch(static_cast<const uint16_t *>(y_bf16) + e0, gb * per, gb, k, g_out + g0,
                                    codes + e0 / 2, scales + e0 / 16, guidance ? guidance + e0 / 16 : nullptr,
                                    guidance ? guidance + bits + e0 * k / 8 : nullptr,
                                    g0 == 0 ? (uint32_t)(n / 16) : 0u, g0 == 0 ? (uint32_t)bits : 0u, work,
                                    max_workgroups, status_dev, st);
        if (rc != TRACE_OK)
            return rc;
    }
    return TRACE_OK;
}

// The device address of this device's copy of `scratch`, looked up once per
// device (with that device current) and cleared once, in stream order before
// the first launch that uses it.  In host code `scratch` names a host-side
// stand-in, so only the looked-up address is ever passed to a kernel.
int scratch_for_device(hipStream_t st, void *&out)
{
    static void *addr[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    static bool cleared[kMaxDevices];
    static std::mutex clear_mu;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TRACE_E_HIP;
    std::call_once(once[dev], [dev] {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess)
            addr[dev] = p;
    });
    (void)hipGetLastError();
    if (!addr[dev])
        return TRACE_E_HIP;
    {
        std::lock_guard<std::mutex> lk(clear_mu);
        if (!cleared[dev]) {
            hipLaunchKernelGGL(k_amax_clear, dim3((kScratchWords + 255) / 256), dim3(256), 0, st,
                               static_cast<uint32_t *>(addr[dev]), (int)kScratchWords);
            if (hipGetLastError() != hipSuccess)
                return TRACE_E_HIP;
            cleared[dev] = true;
        }
    }
    out = addr[dev];
    return TRACE_OK;
}

}  // namespace

extern "C" {

int trace_quant_rollout_onepass(const void *y_bf16, int64_t n, int G, int k, float *g_out, uint8_t *codes,
                                uint8_t *scales, uint8_t *guidance, void *work, int max_workgroups,
                                int *status_dev, void *stream)
{
    int rc = rollout_onepass_check(y_bf16, n, G, k, g_out, codes, scales, guidance, true, work, max_workgroups,
                                   status_dev);
    if (rc != TRACE_OK)
        return rc;
    return rollout_onepass_run(y_bf16, n, G, k, g_out, codes, scales, guidance, work, max_workgroups, status_dev,
                               (hipStream_t)stream);
}

int trace_quant_rollout_onepass_noalloc(const void *y_bf16, int64_t n, int G, int k, float *g_out, uint8_t *codes,
                                        uint8_t *scales, uint8_t *guidance, int max_workgroups, int *status_dev,
                                        void *stream)
{
    int rc = rollout_onepass_check(y_bf16, n, G, k, g_out, codes, scales, guidance, false, nullptr, max_workgroups,
                                   status_dev);
    if (rc != TRACE_OK)
        return rc;
    if (G > kScratchMaxGroups)
        return TRACE_E_SCRATCH;
    void *work = nullptr;
    if ((rc = scratch_for_device((hipStream_t)stream, work)) != TRACE_OK)
        return rc;
    return rollout_onepass_run(y_bf16, n, G, k, g_out, codes, scales, guidance, work, max_workgroups, status_dev,
                               (hipStream_t)stream);
}

int trace_fakequant_rtn_onepass(const void *x_bf16, int64_t n, int G, float *g_out, void *y_out, int out_dtype,
                                uint8_t *codes_out, uint8_t *scales_out, void *work, int max_workgroups,
                                int *status_dev, void *stream)
{
    int rc = check_sizes(n, G);
    if (rc)
        return rc;
    if (!x_bf16 || !g_out || !y_out || !work)
        return TRACE_E_NULL;
    if (!aligned16(x_bf16) || !aligned16(g_out) || !aligned16(y_out) || (codes_out && !aligned16(codes_out)) ||
        (scales_out && !aligned16(scales_out)) || !aligned16(work) || (status_dev && !aligned16(status_dev)))
        return TRACE_E_ALIGN;
    if (out_dtype != TRACE_OUT_BF16 && out_dtype != TRACE_OUT_F32)
        return TRACE_E_DTYPE;
    if (max_workgroups < 0 || !onepass_cap_fits(n, G, max_workgroups, out_dtype == TRACE_OUT_F32 ? 32u : 16u))
        return TRACE_E_SIZE;
    int gpb;
    if ((rc = onepass_groups_per_launch(n, G, max_workgroups, gpb)) != TRACE_OK)
        return rc;
    const bool f32 = out_dtype == TRACE_OUT_F32;
    uint32_t S;
    int64_t grid;
    if (onepass_team_shape(n, G, gpb, max_workgroups, f32 ? 2 : 1, S, grid))   // many groups of whole tiles: teams
        return rtn_onepass_teams(x_bf16, n, G, g_out, y_out, f32, codes_out, scales_out, work, S, grid, status_dev,
                                 (hipStream_t)stream);
    const int64_t per = n / G;
    for (int g0 = 0; g0 < G; g0 += gpb) {              // blocks of whole groups (one block when it all fits)
        const int gb = std::min(gpb, G - g0);
        const int64_t e0 = (int64_t)g0 * per;
        rc = rtn_onepass_launch(static_cast<const uint16_t *>(x_bf16) + e0, gb * per, gb, g_out + g0,
                                static_cast<uint8_t *>(y_out) + e0 * (f32 ? 4 : 2), f32,
                                codes_out ? codes_out + e0 / 2 : nullptr, scales_out ? scales_out + e0 / 16 : nullptr,
                                work, max_workgroups, status_dev, (hipStream_t)stream);
        if (rc != TRACE_OK)
            return rc;
    }
    return TRACE_OK;
}

size_t trace_code_bytes(int64_t n) { return check_sizes(n, 1) ? 0 : (size_t)(n / 2); }

size_t trace_scale_bytes(int64_t n) { return check_sizes(n, 1) ? 0 : (size_t)(n / 16); }

size_t trace_guidance_bytes(int64_t n, int k)
{
    if (check_sizes(n, 1) || (k < 1 || k > 4))
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
    // grid-stride unless a workgroup would change group more than once
    uint64_t steps = (items + (uint64_t)grid - 1) / (uint64_t)grid;
    bool runs = (steps < (uint64_t)G ? steps : (uint64_t)G) > 2;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_amax_clear, dim3((G + 255) / 256), dim3(256), 0, st, (uint32_t *)g_out, G);
    hipLaunchKernelGGL(k_amax, dim3(grid), dim3(kAmaxThreads), 0, st, (const u32x4 *)x_bf16, cpg, tpg,
                       (uint32_t)items, (uint32_t *)g_out, status_dev, runs);
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
    if (k < 1 || k > 4)
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
        else if (k == 3) TRACE_Q(3, true);
        else TRACE_Q(4, true);
    } else {
        if (k == 1) TRACE_Q(1, false);
        else if (k == 2) TRACE_Q(2, false);
        else if (k == 3) TRACE_Q(3, false);
        else TRACE_Q(4, false);
    }
#undef TRACE_Q
    return launched();
}

int trace_quant_weight(const void *w_bf16, int64_t n, int G, float *g_out, uint8_t *codes, uint8_t *scales,
                       int *status_dev, void *stream)
{
    int rc = check_sizes(n, G);
    if (rc)
        return rc;
    if (!w_bf16 || !g_out || !codes || !scales)
        return TRACE_E_NULL;
    if (!aligned16(w_bf16) || !aligned16(g_out) || !aligned16(codes) || !aligned16(scales))
        return TRACE_E_ALIGN;
    if ((rc = trace_amax(w_bf16, n, G, g_out, status_dev, stream)) != TRACE_OK)
        return rc;
    return trace_quant_rollout(w_bf16, n, G, g_out, 2, codes, scales, nullptr, stream);   // k unused without guidance
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
    if (k < 1 || k > 4)
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
    else if (k == 3)
        hipLaunchKernelGGL((k_guidance_pack<3>), grid, dim3(kThreads), 0, st, cp, scales, nchunk, guidance, bits, pb,
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
    if (k != 1 && k != 2 && k != 3)
        return TRACE_E_K;
    Launch L = plan(n, G, stream);
    OutPtr out{y_out, out_dtype == TRACE_OUT_F32};
    const uint8_t *bits = guidance + bitplane_offset(n);
    if (k == 1)
        return launch_guided<1>(L, x_bf16, g, guidance, bits, out, codes_out);
    if (k == 3)
        return launch_guided<3>(L, x_bf16, g, guidance, bits, out, codes_out);
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

int trace_fakequant_ste_grad(const void *x_bf16, int64_t n, int G, const float *g, const uint8_t *scales,
                             const void *gy, void *gx, int grad_dtype, void *stream)
{
    int rc = check_sizes(n, G);
    if (rc)
        return rc;
    if (!x_bf16 || !g || !scales || !gy || !gx)
        return TRACE_E_NULL;
    if (!aligned16(x_bf16) || !aligned16(g) || !aligned16(scales) || !aligned16(gy) || !aligned16(gx))
        return TRACE_E_ALIGN;
    if (grad_dtype != TRACE_OUT_BF16 && grad_dtype != TRACE_OUT_F32)
        return TRACE_E_DTYPE;
    Launch L = plan(n, G, stream);
    const u32x4 *xp = (const u32x4 *)x_bf16, *gyp = (const u32x4 *)gy;
    u32x4 *gxp = (u32x4 *)gx;
    (void)hipGetLastError();
#define TRACE_S(ONE, F32)                                                                                         \
    hipLaunchKernelGGL((k_ste_grad<ONE, F32>), L.grid, dim3(kThreads), 0, L.st, xp, L.nchunk, g, L.dm, L.last,   \
                       scales, gyp, gxp)
    if (L.one) {
        if (grad_dtype == TRACE_OUT_F32) TRACE_S(true, true); else TRACE_S(true, false);
    } else {
        if (grad_dtype == TRACE_OUT_F32) TRACE_S(false, true); else TRACE_S(false, false);
    }
#undef TRACE_S
    return launched();
}

// ---- MXFP4 variant --------------------------------------------------------
static int mx_check_sizes(int64_t n)
{
    return (n <= 0 || n % 32 != 0 || n >= kMaxN) ? TRACE_E_SIZE : TRACE_OK;
}

static int64_t mx_bitplane_offset(int64_t n) { return (n / 32 + 255) / 256 * 256; }

size_t trace_mx_scale_bytes(int64_t n) { return mx_check_sizes(n) ? 0 : (size_t)(n / 32); }

size_t trace_mx_guidance_bytes(int64_t n, int k)
{
    if (mx_check_sizes(n) || k < 1 || k > 4)
        return 0;
    return (size_t)(mx_bitplane_offset(n) + n * k / 8);
}

int trace_mx_quant_rollout(const void *y_bf16, int64_t n, int k, uint8_t *codes, uint8_t *scales, uint8_t *guidance,
                           void *stream)
{
    int rc = mx_check_sizes(n);
    if (rc)
        return rc;
    if (!y_bf16 || !codes || !scales)
        return TRACE_E_NULL;
    if (!aligned16(y_bf16) || !aligned16(codes) || !aligned16(scales) || (guidance && !aligned16(guidance)))
        return TRACE_E_ALIGN;
    if (k < 1 || k > 4)
        return TRACE_E_K;
    uint32_t nchunk = (uint32_t)(n / 8);
    uint8_t *bits = guidance ? guidance + mx_bitplane_offset(n) : nullptr;
    uint32_t pb = (uint32_t)(n / 32), pe = (uint32_t)mx_bitplane_offset(n);
    hipStream_t st = (hipStream_t)stream;
    dim3 grid(grid_for(nchunk));
    (void)hipGetLastError();
#define TRACE_MQ(KK)                                                                                              \
    hipLaunchKernelGGL((k_mx_quant_rollout<KK>), grid, dim3(kThreads), 0, st, (const u32x4 *)y_bf16, nchunk,     \
                       (uint32_t *)codes, scales, guidance, bits, pb, pe)
    if (k == 1) TRACE_MQ(1);
    else if (k == 2) TRACE_MQ(2);
    else if (k == 3) TRACE_MQ(3);
    else TRACE_MQ(4);
#undef TRACE_MQ
    return launched();
}

int trace_mx_fakequant_guided(const void *x_bf16, int64_t n, const uint8_t *guidance, int k, void *y_out,
                              int out_dtype, uint8_t *codes_out, void *stream)
{
    int rc = mx_check_sizes(n);
    if (rc)
        return rc;
    if (!x_bf16 || !guidance || !y_out)
        return TRACE_E_NULL;
    if (!aligned16(x_bf16) || !aligned16(guidance) || !aligned16(y_out) || (codes_out && !aligned16(codes_out)))
        return TRACE_E_ALIGN;
    if (out_dtype != TRACE_OUT_BF16 && out_dtype != TRACE_OUT_F32)
        return TRACE_E_DTYPE;
    if (k < 1 || k > 4)
        return TRACE_E_K;
    uint32_t nchunk = (uint32_t)(n / 8);
    const uint8_t *bits = guidance + mx_bitplane_offset(n);
    OutPtr out{y_out, out_dtype == TRACE_OUT_F32};
    hipStream_t st = (hipStream_t)stream;
    dim3 grid(grid_for(nchunk));
    const u32x4 *xp = (const u32x4 *)x_bf16;
    uint32_t *cp = (uint32_t *)codes_out;
    (void)hipGetLastError();
#define TRACE_MG(MODE)                                                                                             \
    do {                                                                                                           \
        if (cp)                                                                                                    \
            hipLaunchKernelGGL((k_mx_fakequant_guided<MODE, true>), grid, dim3(kThreads), 0, st, xp, nchunk,      \
                               guidance, bits, out, cp);                                                           \
        else                                                                                                       \
            hipLaunchKernelGGL((k_mx_fakequant_guided<MODE, false>), grid, dim3(kThreads), 0, st, xp, nchunk,     \
                               guidance, bits, out, cp);                                                           \
    } while (0)
    if (k == 1) TRACE_MG(1);
    else if (k == 2) TRACE_MG(2);
    else if (k == 3) TRACE_MG(3);
    else TRACE_MG(4);
#undef TRACE_MG
    return launched();
}

int trace_mx_fakequant_rtn(const void *x_bf16, int64_t n, const uint8_t *scales_in, void *y_out, int out_dtype,
                           uint8_t *codes_out, uint8_t *scales_out, void *stream)
{
    int rc = mx_check_sizes(n);
    if (rc)
        return rc;
    if (!x_bf16 || !y_out)
        return TRACE_E_NULL;
    if (!aligned16(x_bf16) || !aligned16(y_out) || (scales_in && !aligned16(scales_in)) ||
        (codes_out && !aligned16(codes_out)) || (scales_out && !aligned16(scales_out)))
        return TRACE_E_ALIGN;
    if (out_dtype != TRACE_OUT_BF16 && out_dtype != TRACE_OUT_F32)
        return TRACE_E_DTYPE;
    uint32_t nchunk = (uint32_t)(n / 8);
    OutPtr out{y_out, out_dtype == TRACE_OUT_F32};
    hipStream_t st = (hipStream_t)stream;
    dim3 grid(grid_for(nchunk));
    const u32x4 *xp = (const u32x4 *)x_bf16;
    uint32_t *cp = (uint32_t *)codes_out;
    (void)hipGetLastError();
#define TRACE_MR(OWN, CODES)                                                                                       \
    hipLaunchKernelGGL((k_mx_fakequant_rtn<OWN, CODES>), grid, dim3(kThreads), 0, st, xp, nchunk, scales_in, out,  \
                       cp, scales_out)
    if (scales_in) {
        if (cp) TRACE_MR(false, true); else TRACE_MR(false, false);
    } else {
        if (cp) TRACE_MR(true, true); else TRACE_MR(true, false);
    }
#undef TRACE_MR
    return launched();
}

const char *trace_status_str(int status)
{
    switch (status) {
    case TRACE_OK: return "ok";
    case TRACE_E_NULL: return "a required pointer is NULL";
    case TRACE_E_SIZE: return "n or G violates the size rules (n > 0, n % 16 == 0, n % (16 G) == 0, n < 2^34)";
    case TRACE_E_ALIGN: return "a pointer is not 16-byte aligned";
    case TRACE_E_K: return "unsupported guidance width k";
    case TRACE_E_DTYPE: return "unknown output dtype";
    case TRACE_E_HIP: return "HIP runtime error";
    case TRACE_E_NONFINITE: return "an input was inf or NaN";
    case TRACE_E_FORMAT: return "guidance record fails its header or hash check";
    case TRACE_E_IO: return "file could not be opened, written or read";
    case TRACE_E_BARRIER: return "one-pass rollout: workgroups were not all resident (grid barrier timed out)";
    case TRACE_E_SCRATCH: return "G exceeds the 4096 groups of the allocation-free one-pass rollout's static scratch";
    default: return "unknown status";
    }
}

int trace_version(void) { return 500; }

#if TRACE_OP_PHASE_CLOCK
// Measurement build only: where k_quant_onepass writes its phase clocks (a
// device buffer of 4 values per workgroup, or null to stop).  Returns the
// wall clock's rate on the current device in kHz (0 on error).  Not part of
// the product library's interface.
int trace_debug_phase_clock(void *dev_buf)
{
    g_phase_clock = static_cast<uint64_t *>(dev_buf);
    OnePassDevice d;
    return onepass_device(d) == TRACE_OK ? d.clock_khz : 0;
}
#endif

}  // extern "C"
