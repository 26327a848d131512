/*
 * trace_oracle.c -- plain, slow CPU oracle for rollout-guided FP4 fake-quant.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, table or constant generator with the
 * HIP library: every rule below is written out from its definition.
 *
 * Sources (web pages about TRACE: Rollout-Guided Quantization-Aware Training
 * for FP4 Reinforcement Learning of MoE Language Models):
 *   [en]  "Alibaba Qwen Proposes TRACE for 5.4x Faster FP4 RL Rollouts"
 *         (todayforai.com), sections "Why Does FP4 Rollout 'Break' RL
 *         Training?" (Figure 1 worked example) and "TRACE Core Concept"
 *         (Figure 3 and the paragraph on compact guidance).
 *   [zh]  the same article in Chinese (yktworld.com), sections
 *         "为什么 FP4 Rollout 会把 RL 训练「搞崩」?" and "TRACE 核心".
 *   [ru]  "Alibaba Qwen представила TRACE: Rollout в FP4 ускоряется до 5,4
 *         раза" (news.hamidun.com), section "Где FP4 ломает обучение".
 *
 * What the pages fix: FP4 E2M1 codes, a global scale and a block scale shared
 * by both sides before rounding ([en] Why, Figure 1 example), standard RTN on
 * the rollout side, and on the training side a choice between the two
 * adjacent E2M1 points that favours the one nearer the rollout's code ([en]
 * TRACE Core Concept); guidance = the scale plus a little mantissa
 * information ([en] TRACE Core Concept, compact-guidance paragraph).
 *
 * What the pages leave open, and the reading taken here (each one is listed
 * with its reasoning in the design notes):
 *   - 16-element blocks along the last dim, one E4M3 block scale per block,
 *     one FP32 global scale per group, g = amax / (6 * 448);
 *   - the scale chain is IEEE fp32 with round-to-nearest-even and no fused
 *     operations: t = a_b / (6 g), s = E4M3(t), c = s * g, inv = 1 / c,
 *     v = y * inv (inv = 0 when c = 0, inv = FLT_MAX when 1/c overflows);
 *     the pages fix no order of these operations, so this order (reciprocal,
 *     then multiply, rather than y / c) is a convention: parity unpinned for
 *     that choice alone (the pins fix everything around it);
 *   - E4M3 rounding is nearest with ties to the even code, saturating at
 *     448, subnormals kept;
 *   - RTN ties go to the even magnitude index (the even E2M1 mantissa);
 *   - guidance bits = the low k bits of the rollout's magnitude index
 *     (k = 1 is the mantissa bit; k = 3 is the whole magnitude index, no
 *     sign), or the whole nibble (k = 4);
 *   - the reconstructed rollout code is the code nearest (in value) to the
 *     training value whose low k bits match; any tie falls back to RTN;
 *   - dequantised output y = sign * fp32(fp32(val * s) * g).
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (float is IEEE single on
 * x86-64 SSE, so every float expression below rounds once, to nearest even).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OR_OK 0
#define OR_E_NONFINITE (-7)

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* E2M1 magnitudes, indexed by the 3-bit magnitude index j = (e1 e0 m):
 * 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit, no inf/NaN
 * (OCP Microscaling Formats v1.0, FP4 E2M1).  The pages name E2M1 ([en]
 * TRACE Core Concept) and count 16 codes ([ru] "Где FP4 ломает обучение"). */
static double e2m1_magnitude(int j)
{
    int e = (j >> 1) & 3, m = j & 1;
    if (e == 0)
        return 0.5 * m;                       /* subnormal: m * 2^(1-1) * 0.5 */
    return ldexp(1.0 + 0.5 * m, e - 1);       /* normal: (1 + m/2) * 2^(e-1)  */
}

double oracle_e2m1_value(int nibble)
{
    double mag = e2m1_magnitude(nibble & 7);
    return (nibble & 8) ? -mag : mag;
}

/* E4M3 ("FN") value of a non-negative code 0..126: bias 7, 3 mantissa
 * bits, subnormals at exponent field 0, 0x7F is NaN (OCP FP8 spec). */
double oracle_e4m3_value(int code)
{
    int e = (code >> 3) & 15, m = code & 7;
    if (e == 0)
        return ldexp((double)m, -9);          /* (m/8) * 2^-6 */
    return ldexp(8.0 + m, e - 10);            /* (1 + m/8) * 2^(e-7) */
}

/* Which of two candidate values a, b lies nearer to x: -1 for a, +1 for b,
 * 0 for equidistant.  |x - a| < |x - b| holds exactly when x lies on a's side
 * of the midpoint (a + b) / 2.  The candidates here (E2M1, E4M3 and bf16
 * values) have few significant bits, so a, b, the midpoint and the fp32 x are
 * all exact in double and the comparison is exact, for any magnitude of x. */
static int nearer(double a, double b, double x)
{
    if (a == b)
        return 0;
    double mid = (a + b) / 2.0;
    if (x == mid)
        return 0;
    if (a < b)
        return x < mid ? -1 : 1;
    return x > mid ? -1 : 1;
}

/* Nearest finite non-negative E4M3 code to t >= 0, ties to the even code,
 * saturating at 448 (values above 448 take the largest finite code).
 * Literal search over all 127 codes. */
uint8_t oracle_e4m3_encode(float t)
{
    if (!(t >= 0.0f))
        return 0;                             /* precondition: t >= 0 */
    if ((double)t >= 448.0)
        return 126;
    int best = 0;
    for (int c = 1; c <= 126; ++c) {
        int w = nearer(oracle_e4m3_value(best), oracle_e4m3_value(c), (double)t);
        if (w > 0 || (w == 0 && (c & 1) == 0))
            best = c;
    }
    return (uint8_t)best;
}

/* Round-to-nearest E2M1 magnitude index of |v| (standard RTN, [en] TRACE Core
 * Concept), ties to the even index, saturating at 6 (index 7). */
int oracle_rtn_index(float v)
{
    double a = fabs((double)v);
    if (a > 6.0)
        a = 6.0;
    int best = 0;
    for (int j = 1; j < 8; ++j) {
        int w = nearer(e2m1_magnitude(best), e2m1_magnitude(j), a);
        if (w > 0 || (w == 0 && (j & 1) == 0))
            best = j;
    }
    return best;
}

/* Signed RTN nibble: sign bit = sign bit of v (so -0 and tiny negatives keep
 * their sign), magnitude = oracle_rtn_index. */
int oracle_rtn_nibble(float v)
{
    return (signbit(v) ? 8 : 0) | oracle_rtn_index(v);
}

float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16, nearest representable value, ties to the even mantissa.
 * Literal: compare the two bf16 neighbours of |f| (truncation and the next
 * value up).  Finite inputs only. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t sign = u & 0x80000000u, mag = u & 0x7fffffffu;
    if (mag > 0x7f800000u)                       /* NaN: a quiet NaN of the same sign */
        return (uint16_t)((sign >> 16) | 0x7fc0u);
    if (mag == 0x7f800000u)                      /* infinity converts to infinity */
        return (uint16_t)((sign >> 16) | 0x7f80u);
    uint32_t lo = mag & 0xffff0000u, hi = lo + 0x10000u;
    float flo, fhi, fa;
    memcpy(&flo, &lo, 4);
    memcpy(&fhi, &hi, 4);
    memcpy(&fa, &mag, 4);
    /* above the largest bf16 value the next candidate is 2^128 (IEEE 754
     * rounding: overflow to infinity from the largest value plus half an ulp) */
    double dhi = (hi == 0x7f800000u) ? ldexp(1.0, 128) : (double)fhi;
    int w = nearer((double)flo, dhi, (double)fa);
    uint32_t pick;
    if (w < 0)
        pick = lo;
    else if (w > 0)
        pick = hi;
    else
        pick = ((lo >> 16) & 1) ? hi : lo;
    return (uint16_t)((sign | pick) >> 16);
}

/* ------------------------------------------------------------------ */
/* Scales                                                              */
/* ------------------------------------------------------------------ */

static int64_t blocks_per_group(int64_t n, int G) { return (n / 16) / G; }

/* Global scale per group: A = max |x| over the group, g = A / 2688 in fp32
 * (2688 = 6 * 448: the largest E2M1 magnitude times the largest E4M3 value,
 * so the block holding A gets block scale 448).  Returns OR_E_NONFINITE if
 * any input is inf or NaN. */
int oracle_amax(const uint16_t *x, int64_t n, int G, float *g_out)
{
    int status = OR_OK;
    int64_t per = n / G;
    for (int gi = 0; gi < G; ++gi) {
        float A = 0.0f;
        for (int64_t i = gi * per; i < (gi + 1) * per; ++i) {
            float f = oracle_bf16_to_f32(x[i]);
            if (!isfinite(f)) {
                status = OR_E_NONFINITE;
                continue;
            }
            float a = fabsf(f);
            if (a > A)
                A = a;
        }
        g_out[gi] = A / 2688.0f;
    }
    return status;
}

/* Block scale and reciprocal of the combined scale for block b (the same
 * global scale and block scale that both sides apply before rounding: [en]
 * Why ..., Figure 1 example). */
static void block_scales(const uint16_t *y, int64_t b, float g, uint8_t *s_out, float *inv_out)
{
    float ab = 0.0f;
    for (int i = 0; i < 16; ++i) {
        float a = fabsf(oracle_bf16_to_f32(y[16 * b + i]));
        if (a > ab)
            ab = a;
    }
    float t = 0.0f;
    if (g > 0.0f) {
        float six_g = 6.0f * g;
        t = ab / six_g;
    }
    uint8_t s = oracle_e4m3_encode(t);
    *s_out = s;
    float c = (float)oracle_e4m3_value(s) * g;
    *inv_out = 0.0f;
    if (c > 0.0f) {
        float inv = 1.0f / c;
        *inv_out = isinf(inv) ? FLT_MAX : inv;
    }
}

/* Reciprocal of the combined scale from a given E4M3 scale byte. */
static float inv_from_scale(uint8_t s, float g)
{
    float c = (float)oracle_e4m3_value(s & 0x7f) * g;
    if (!(c > 0.0f))
        return 0.0f;
    float inv = 1.0f / c;
    return isinf(inv) ? FLT_MAX : inv;
}

/* ------------------------------------------------------------------ */
/* Guidance stream layout                                              */
/*   [scale plane: n/16 bytes | zero pad to a multiple of 256 | bits]  */
/* Element i's k bits sit at bit (i*k) mod 8 of bit-plane byte         */
/* floor(i*k/8), least significant first; k = 4 stores the nibble.     */
/* ------------------------------------------------------------------ */

int64_t oracle_bitplane_offset(int64_t n)
{
    int64_t sp = n / 16;
    return (sp + 255) / 256 * 256;
}

int64_t oracle_guidance_bytes(int64_t n, int k)
{
    return oracle_bitplane_offset(n) + n * k / 8;
}

/* Element i's k bits sit at bit positions i*k .. i*k + k - 1 of the bit
 * plane, least significant first (bit position p = bit p % 8 of byte p / 8);
 * for k = 3 a field can straddle two bytes, so bits are moved one at a time. */
static void put_bits(uint8_t *plane, int64_t i, int k, int value)
{
    for (int j = 0; j < k; ++j) {
        int64_t p = i * k + j;
        uint8_t m = (uint8_t)(1u << (p % 8));
        if ((value >> j) & 1)
            plane[p / 8] = (uint8_t)(plane[p / 8] | m);
        else
            plane[p / 8] = (uint8_t)(plane[p / 8] & ~m);
    }
}

static int get_bits(const uint8_t *plane, int64_t i, int k)
{
    int value = 0;
    for (int j = 0; j < k; ++j) {
        int64_t p = i * k + j;
        value |= ((plane[p / 8] >> (p % 8)) & 1) << j;
    }
    return value;
}

static void put_nibble(uint8_t *codes, int64_t i, int nib)
{
    int sh = (i & 1) ? 4 : 0;
    codes[i / 2] = (uint8_t)((codes[i / 2] & ~(0xf << sh)) | ((nib & 0xf) << sh));
}

static int get_nibble(const uint8_t *codes, int64_t i)
{
    return (codes[i / 2] >> ((i & 1) ? 4 : 0)) & 0xf;
}

/* Zero the pad between the scale plane and the bit plane. */
static void zero_pad(uint8_t *guidance, int64_t n)
{
    for (int64_t p = n / 16; p < oracle_bitplane_offset(n); ++p)
        guidance[p] = 0;
}

/* ------------------------------------------------------------------ */
/* Rollout side                                                        */
/* ------------------------------------------------------------------ */

/* RTN quantisation of the rollout tensor for blocks [b0, b1): packed codes
 * (element 2m in the low nibble), E4M3 scale bytes, and optionally the
 * guidance stream (scale plane + low k bits of each magnitude index, or the
 * whole nibble for k = 4).  [en] TRACE Core Concept: the rollout records its
 * quantisation results and keeps only the scale plus a few mantissa bits. */
void oracle_quant_rollout(const uint16_t *y, int64_t n, int G, const float *g, int k,
                          int64_t b0, int64_t b1, uint8_t *codes, uint8_t *scales, uint8_t *guidance)
{
    int64_t bpg = blocks_per_group(n, G);
    uint8_t *bits = guidance ? guidance + oracle_bitplane_offset(n) : NULL;
    for (int64_t b = b0; b < b1; ++b) {
        float gg = g[b / bpg];
        uint8_t s;
        float inv;
        block_scales(y, b, gg, &s, &inv);
        scales[b] = s;
        if (guidance)
            guidance[b] = s;
        for (int i = 0; i < 16; ++i) {
            int64_t e = 16 * b + i;
            float v = oracle_bf16_to_f32(y[e]) * inv;
            int nib = oracle_rtn_nibble(v);
            put_nibble(codes, e, nib);
            if (bits)
                put_bits(bits, e, k, k == 4 ? nib : (nib & 7));
        }
    }
    if (guidance && b0 == 0)
        zero_pad(guidance, n);
}

/* Guidance stream from existing codes and scales, blocks [b0, b1). */
void oracle_guidance_pack(const uint8_t *codes, const uint8_t *scales, int64_t n, int k,
                          int64_t b0, int64_t b1, uint8_t *guidance)
{
    uint8_t *bits = guidance + oracle_bitplane_offset(n);
    for (int64_t b = b0; b < b1; ++b) {
        guidance[b] = scales[b];
        for (int i = 0; i < 16; ++i) {
            int64_t e = 16 * b + i;
            int nib = get_nibble(codes, e);
            put_bits(bits, e, k, k == 4 ? nib : (nib & 7));
        }
    }
    if (b0 == 0)
        zero_pad(guidance, n);
}

/* ------------------------------------------------------------------ */
/* Training side                                                       */
/* ------------------------------------------------------------------ */

/* Adjacent signed E2M1 points lo <= v <= hi; |v| >= 6 saturates to +-6, and
 * a v on the grid gives lo = hi = v. */
static void bracket(float v, double *lo, double *hi)
{
    double x = v;
    if (x >= 6.0) { *lo = *hi = 6.0; return; }
    if (x <= -6.0) { *lo = *hi = -6.0; return; }
    double L = -6.0, H = 6.0;
    for (int nib = 0; nib < 16; ++nib) {
        double val = oracle_e2m1_value(nib);
        if (val <= x && val > L) L = val;
        if (val >= x && val < H) H = val;
    }
    *lo = L;
    *hi = H;
}

static int magnitude_index_of(double val)
{
    double a = fabs(val);
    for (int j = 0; j < 8; ++j)
        if (e2m1_magnitude(j) == a)
            return j;
    return -1;
}

/* Pick between lo and hi: the one nearer the reconstructed rollout value r;
 * equidistance falls back to RTN. */
static double pick_nearer(double lo, double hi, double r, float v)
{
    int w = nearer(lo, hi, r);
    if (w < 0) return lo;
    if (w > 0) return hi;
    return oracle_e2m1_value(oracle_rtn_nibble(v));
}

/* Guided choice for one normalised training value v with guidance bits gb
 * (k = 1, 2 or 3): returns the chosen nibble (sign bit = sign bit of v).
 * [en] TRACE Core Concept: choose between the two adjacent E2M1 points,
 * favouring the one nearer the rollout's actual code; the rollout code is
 * reconstructed as the code nearest v whose low k index bits equal gb, and
 * any tie falls back to RTN. */
int oracle_guided_nibble(float v, int k, int gb)
{
    double lo, hi, chosen;
    bracket(v, &lo, &hi);
    if (lo == hi) {
        chosen = lo;
    } else {
        int mask = (1 << k) - 1;
        /* argmin over the matching signed codes of |val - v| */
        int have = 0;
        double best = 0.0;
        for (int nib = 0; nib < 16; ++nib) {
            if (((nib & 7) & mask) != gb) continue;
            double val = oracle_e2m1_value(nib);
            if (!have || nearer(best, val, (double)v) > 0) { best = val; have = 1; }
        }
        /* another distinct value at the same distance is a tie (+0 and -0
         * are one value) */
        int distinct = 1;
        for (int nib = 0; nib < 16; ++nib) {
            if (((nib & 7) & mask) != gb) continue;
            double val = oracle_e2m1_value(nib);
            if (val != best && nearer(best, val, (double)v) == 0) distinct = 2;
        }
        double first = best;
        if (distinct > 1)
            chosen = oracle_e2m1_value(oracle_rtn_nibble(v));
        else
            chosen = pick_nearer(lo, hi, first, v);
    }
    return (signbit(v) ? 8 : 0) | magnitude_index_of(chosen);
}

/* Full-code variant: the rollout nibble r itself is the reference. */
int oracle_fullcode_nibble(float v, int r)
{
    double lo, hi, chosen;
    bracket(v, &lo, &hi);
    if (lo == hi)
        chosen = lo;
    else
        chosen = pick_nearer(lo, hi, oracle_e2m1_value(r), v);
    return (signbit(v) ? 8 : 0) | magnitude_index_of(chosen);
}

/* Dequantised value: sign * fp32(fp32(val * s) * g). */
float oracle_dequant(int nib, uint8_t s, float g)
{
    float val = (float)e2m1_magnitude(nib & 7);
    float p = val * (float)oracle_e4m3_value(s & 0x7f);
    float y = p * g;
    return (nib & 8) ? -y : y;
}

static void store_out(void *y_out, int out_f32, int64_t e, float y)
{
    if (out_f32)
        ((float *)y_out)[e] = y;
    else
        ((uint16_t *)y_out)[e] = oracle_f32_to_bf16(y);
}

/* mode 1/2: guided with k bits; mode 4: full code; over blocks [b0, b1). */
static void fakequant_guided_any(const uint16_t *x, int64_t n, int G, const float *g,
                                 const uint8_t *guidance, int k, int64_t b0, int64_t b1,
                                 void *y_out, int out_f32, uint8_t *codes_out)
{
    int64_t bpg = blocks_per_group(n, G);
    const uint8_t *bits = guidance + oracle_bitplane_offset(n);
    for (int64_t b = b0; b < b1; ++b) {
        float gg = g[b / bpg];
        uint8_t s = guidance[b];
        float inv = inv_from_scale(s, gg);
        for (int i = 0; i < 16; ++i) {
            int64_t e = 16 * b + i;
            float v = oracle_bf16_to_f32(x[e]) * inv;
            int gb = get_bits(bits, e, k);
            int nib = (k == 4) ? oracle_fullcode_nibble(v, gb) : oracle_guided_nibble(v, k, gb);
            store_out(y_out, out_f32, e, oracle_dequant(nib, s, gg));
            if (codes_out)
                put_nibble(codes_out, e, nib);
        }
    }
}

void oracle_fakequant_guided(const uint16_t *x, int64_t n, int G, const float *g,
                             const uint8_t *guidance, int k, int64_t b0, int64_t b1,
                             void *y_out, int out_f32, uint8_t *codes_out)
{
    fakequant_guided_any(x, n, G, g, guidance, k, b0, b1, y_out, out_f32, codes_out);
}

void oracle_fakequant_fullcode(const uint16_t *x, int64_t n, int G, const float *g,
                               const uint8_t *guidance, int64_t b0, int64_t b1,
                               void *y_out, int out_f32, uint8_t *codes_out)
{
    fakequant_guided_any(x, n, G, g, guidance, 4, b0, b1, y_out, out_f32, codes_out);
}

/* Plain QAT fake-quant (RTN), the unstable baseline of [en] Experimental
 * Results: own block scales from x (scales_in == NULL) or the given scales. */
void oracle_fakequant_rtn(const uint16_t *x, int64_t n, int G, const float *g,
                          const uint8_t *scales_in, int64_t b0, int64_t b1,
                          void *y_out, int out_f32, uint8_t *codes_out, uint8_t *scales_out)
{
    int64_t bpg = blocks_per_group(n, G);
    for (int64_t b = b0; b < b1; ++b) {
        float gg = g[b / bpg];
        uint8_t s;
        float inv;
        if (scales_in) {
            s = scales_in[b];
            inv = inv_from_scale(s, gg);
        } else {
            block_scales(x, b, gg, &s, &inv);
        }
        if (scales_out)
            scales_out[b] = s;
        for (int i = 0; i < 16; ++i) {
            int64_t e = 16 * b + i;
            float v = oracle_bf16_to_f32(x[e]) * inv;
            int nib = oracle_rtn_nibble(v);
            store_out(y_out, out_f32, e, oracle_dequant(nib, s, gg));
            if (codes_out)
                put_nibble(codes_out, e, nib);
        }
    }
}

/* Gradient mask of the fake-quant for quantisation-aware training, blocks
 * [b0, b1).  The pages say the training side fake-quantises ([en] TRACE Core
 * Concept) and nothing about its gradient.  Reading taken: the
 * straight-through estimator clipped at the quantiser's range.  The forward
 * rounds the normalised value v = x * inv (inv from the scales it used) to a
 * signed E2M1 point; where |v| > 6, the largest E2M1 magnitude, it saturates
 * at +-6, so its output stays put as x moves and the gradient there is zero;
 * everywhere else the incoming gradient passes unchanged.  mask[e] = 1 where
 * it passes.  A NaN v is not within the range. */
void oracle_ste_mask(const uint16_t *x, int64_t n, int G, const float *g, const uint8_t *scales,
                     int64_t b0, int64_t b1, uint8_t *mask)
{
    int64_t bpg = blocks_per_group(n, G);
    for (int64_t b = b0; b < b1; ++b) {
        float inv = inv_from_scale(scales[b], g[b / bpg]);
        for (int i = 0; i < 16; ++i) {
            int64_t e = 16 * b + i;
            float v = oracle_bf16_to_f32(x[e]) * inv;
            mask[e] = fabs((double)v) <= 6.0 ? 1 : 0;
        }
    }
}

/* ------------------------------------------------------------------ */
/* MXFP4 variant: 32-element blocks, E8M0 shared scale, no global scale */
/* ------------------------------------------------------------------ */

/* OCP Microscaling Formats (MX) v1.0: a block of 32 FP4 (E2M1) elements
 * shares one E8M0 scale X = 2^(code - 127).  The shared exponent is
 * floor(log2(max |V|)) - emax, with emax = 2 the exponent of E2M1's largest
 * normal (6 = 1.5 * 2^2); each element is V / X rounded to E2M1 (nearest,
 * ties to even, saturating at 6).  Readings taken where the text leaves a
 * choice: the exponent is clamped to E8M0's finite range [-127, 127]
 * (codes 0 .. 254), and an all-zero block gets code 0.  The pages use the
 * NVFP4-style two-level scale; this variant is the block format of gfx950's
 * scaled FP4 conversions, kept beside it. */
uint8_t oracle_mx_scale(float amax)
{
    if (!(amax > 0.0f))
        return 0;
    int e;
    frexp((double)amax, &e);          /* amax = m * 2^e, m in [0.5, 1): floor(log2) = e - 1 */
    int shared = (e - 1) - 2;
    int code = shared + 127;
    if (code < 0) code = 0;
    if (code > 254) code = 254;
    return (uint8_t)code;
}

double oracle_mx_scale_value(uint8_t code)
{
    return ldexp(1.0, (int)code - 127);
}

int64_t oracle_mx_bitplane_offset(int64_t n)
{
    int64_t sp = n / 32;
    return (sp + 255) / 256 * 256;
}

int64_t oracle_mx_guidance_bytes(int64_t n, int k)
{
    return oracle_mx_bitplane_offset(n) + n * k / 8;
}

/* v = V / X, computed in double (exact: X is a power of two) and rounded
 * once to float (exact too, except where V / X falls below the float normal
 * range, far under the smallest nonzero E2M1 point). */
static float mx_normalise(uint16_t h, uint8_t code)
{
    return (float)((double)oracle_bf16_to_f32(h) / oracle_mx_scale_value(code));
}

/* Rollout side, blocks of 32 [b0, b1): codes, E8M0 scale bytes, optional
 * guidance (scale plane of n/32 bytes, zero pad to 256, then k bits). */
void oracle_mx_quant_rollout(const uint16_t *y, int64_t n, int k, int64_t b0, int64_t b1,
                             uint8_t *codes, uint8_t *scales, uint8_t *guidance)
{
    uint8_t *bits = guidance ? guidance + oracle_mx_bitplane_offset(n) : NULL;
    for (int64_t b = b0; b < b1; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(oracle_bf16_to_f32(y[32 * b + i]));
            if (a > amax) amax = a;
        }
        uint8_t code = oracle_mx_scale(amax);
        scales[b] = code;
        if (guidance)
            guidance[b] = code;
        for (int i = 0; i < 32; ++i) {
            int64_t e = 32 * b + i;
            int nib = oracle_rtn_nibble(mx_normalise(y[e], code));
            put_nibble(codes, e, nib);
            if (bits)
                put_bits(bits, e, k, k == 4 ? nib : (nib & 7));
        }
    }
    if (guidance && b0 == 0)
        for (int64_t p = n / 32; p < oracle_mx_bitplane_offset(n); ++p)
            guidance[p] = 0;
}

/* Dequantised MX value: sign * val * X (exact). */
float oracle_mx_dequant(int nib, uint8_t code)
{
    double y = e2m1_magnitude(nib & 7) * oracle_mx_scale_value(code);
    return (nib & 8) ? -(float)y : (float)y;
}

/* Training side: guided (k = 1, 2, 3) or full code (k = 4) with the
 * rollout's MX scales, over blocks of 32 [b0, b1). */
void oracle_mx_fakequant_guided(const uint16_t *x, int64_t n, const uint8_t *guidance, int k, int64_t b0,
                                int64_t b1, void *y_out, int out_f32, uint8_t *codes_out)
{
    const uint8_t *bits = guidance + oracle_mx_bitplane_offset(n);
    for (int64_t b = b0; b < b1; ++b) {
        uint8_t code = guidance[b];
        for (int i = 0; i < 32; ++i) {
            int64_t e = 32 * b + i;
            float v = mx_normalise(x[e], code);
            int gb = get_bits(bits, e, k);
            int nib = (k == 4) ? oracle_fullcode_nibble(v, gb) : oracle_guided_nibble(v, k, gb);
            store_out(y_out, out_f32, e, oracle_mx_dequant(nib, code));
            if (codes_out)
                put_nibble(codes_out, e, nib);
        }
    }
}

/* Plain RTN with MX scales: own scales from x (scales_in == NULL) or given. */
void oracle_mx_fakequant_rtn(const uint16_t *x, int64_t n, const uint8_t *scales_in, int64_t b0, int64_t b1,
                             void *y_out, int out_f32, uint8_t *codes_out, uint8_t *scales_out)
{
    for (int64_t b = b0; b < b1; ++b) {
        uint8_t code;
        if (scales_in) {
            code = scales_in[b];
        } else {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(oracle_bf16_to_f32(x[32 * b + i]));
                if (a > amax) amax = a;
            }
            code = oracle_mx_scale(amax);
        }
        if (scales_out)
            scales_out[b] = code;
        for (int i = 0; i < 32; ++i) {
            int64_t e = 32 * b + i;
            int nib = oracle_rtn_nibble(mx_normalise(x[e], code));
            store_out(y_out, out_f32, e, oracle_mx_dequant(nib, code));
            if (codes_out)
                put_nibble(codes_out, e, nib);
        }
    }
}

