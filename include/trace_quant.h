/*
 * trace_quant.h -- C ABI of the rollout-guided FP4 (E2M1) fake-quant library
 * for MI355X (gfx950).  Library: libtrace_quant.so.
 *
 * The method (TRACE: Rollout-Guided Quantization-Aware Training for FP4
 * Reinforcement Learning of MoE Language Models) is described on the page
 * "Alibaba Qwen Proposes TRACE for 5.4x Faster FP4 RL Rollouts":
 *   - section "Why Does FP4 Rollout 'Break' RL Training?", Figure 1 and its
 *     worked example: both sides apply the same global scale and block scale,
 *     then round to FP4; a tiny difference across a rounding boundary becomes
 *     one whole codebook step;
 *   - section "TRACE Core Concept", Figure 3: the rollout side records the FP4
 *     results of routed-expert activations and KV states; the training side's
 *     fake quantisation still picks one of the two adjacent E2M1 points, but
 *     the one nearer the rollout's actual code rather than plain RTN; what is
 *     kept is the scale plus a little mantissa information, because nearly
 *     all mismatches are a single adjacent codebook entry.
 *
 * Conventions this library fixes where the pages are silent:
 *   - blocks of 16 consecutive elements; one E4M3 block scale per block
 *     (round to nearest even, saturating at 448, subnormals kept); one FP32
 *     global scale per group of consecutive elements, g = amax / 2688
 *     (2688 = 6 * 448), G groups of equal size (G = 1: one per tensor);
 *   - fp32 scale chain, IEEE round-to-nearest-even, no fused operations:
 *     t = a_b / (6 g); s = E4M3(t); c = s * g; inv = 1 / c (0 if c == 0,
 *     FLT_MAX if 1 / c overflows); v = x * inv;
 *   - RTN ties go to the even magnitude index; |v| > 6 saturates to 6;
 *   - nibble = sign(v) << 3 | j, j = 3-bit magnitude index of
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6}; packed codes: element 2m in the low nibble;
 *   - dequantised value y = sign * fp32(fp32(val * s) * g), stored as bf16
 *     (round to nearest even) or fp32.
 *
 * Guidance stream (a flat byte buffer, trace_guidance_bytes(n, k) long):
 *   [ scale plane: n/16 E4M3 bytes | zero pad up to a multiple of 256 | bits ]
 *   bits: element i's k bits at bit positions i*k .. i*k + k - 1 of the bit
 *   plane (position p = bit p mod 8 of byte p / 8), least significant first.
 *   k = 1: the mantissa bit of the rollout magnitude index; k = 2: its two
 *   low bits; k = 3: the whole magnitude index without the sign (fields
 *   straddle bytes); k = 4: the whole nibble (the bit plane then equals the
 *   packed code array).  The global scales (f32[G]) travel beside the stream.
 *
 * Common rules for every entry point:
 *   - pointers are device pointers unless stated; the caller owns every
 *     buffer; the library never allocates device memory and keeps no state
 *     beyond a read-only kernel table, a host-side cache of device
 *     attributes (compute units, LDS size, clock rate) and the static work
 *     array of trace_quant_rollout_onepass_noalloc; calls are thread-safe
 *     (that entry point's calls must still be ordered per device);
 *   - work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns at once; outputs are valid once the stream has
 *     reached that point;
 *   - argument errors are found before anything is enqueued and returned as
 *     a negative trace_status (nothing is written); TRACE_E_HIP reports a
 *     failed launch; inputs must be finite (trace_amax can flag violations);
 *   - n > 0, n % 16 == 0, n % (16 * G) == 0, n < 2^34, 1 <= G <= n / 16;
 *   - every pointer 16-byte aligned; x / y_out may be the same buffer
 *     (in-place fake-quant); any other overlap is undefined.
 */
#ifndef TRACE_QUANT_H
#define TRACE_QUANT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TRACE_OK = 0,
    TRACE_E_NULL = -1,      /* a required pointer is NULL */
    TRACE_E_SIZE = -2,      /* n or G violates the size rules */
    TRACE_E_ALIGN = -3,     /* a pointer is not 16-byte aligned */
    TRACE_E_K = -4,         /* unsupported guidance width */
    TRACE_E_DTYPE = -5,     /* unknown output dtype */
    TRACE_E_HIP = -6,       /* the HIP runtime reported an error */
    TRACE_E_NONFINITE = -7, /* (device status word) an input was inf/NaN */
    TRACE_E_FORMAT = -8,    /* a guidance record fails its header or hash check */
    TRACE_E_IO = -9,        /* a file could not be opened, written or read */
    TRACE_E_BARRIER = -10,  /* (device status word) the one-pass rollout's workgroups
                               were not all resident at once; outputs undefined */
    TRACE_E_SCRATCH = -11   /* G exceeds the static scratch of the allocation-free
                               one-pass rollout (4096 groups) */
} trace_status;

typedef enum { TRACE_OUT_BF16 = 0, TRACE_OUT_F32 = 1 } trace_out_dtype;

/* ---- sizes (host, pure; 0 for invalid arguments) --------------------- */

/* Bytes of the packed code array: n / 2. */
size_t trace_code_bytes(int64_t n);
/* Bytes of the block-scale array: n / 16. */
size_t trace_scale_bytes(int64_t n);
/* Bytes of the guidance stream for width k in {1, 2, 3, 4}:
 * align256(n / 16) + n * k / 8. */
size_t trace_guidance_bytes(int64_t n, int k);

/* ---- rollout side ------------------------------------------------------ */

/* Global scales.  "the same global scale" of the Figure 1 example.
 * x_bf16: bf16[n].  g_out: f32[G], written with amax(|x| over group) / 2688.
 * status_dev: nullable int*; if given and some input is inf or NaN,
 * TRACE_E_NONFINITE is stored there (never cleared: the caller zeroes it).
 * Enqueues two kernels: a clear of g_out, then the reduction, in which each
 * workgroup raises its group's g with an atomic max of fl(its amax / 2688)
 * (the division rounds monotonically, so the largest is fl(amax / 2688)). */
int trace_amax(const void *x_bf16, int64_t n, int G, float *g_out, int *status_dev, void *stream);

/* FP4 weight quantisation for the rollout's FP4 weight/activation GEMMs (the
 * opening paragraph of the page above, and the key facts of the Russian page
 * "Alibaba Qwen представила TRACE: Rollout в FP4 ускоряется до 5,4 раза":
 * rollout runs with FP4 weights and activations plus an FP4 KV cache).  Weights are not guided (rollout and
 * trainer hold the same weights), so no guidance stream is written.
 * w_bf16: bf16[n], G matrices of n / G contiguous elements each, blocks of 16
 * along the contiguous (GEMM reduction) dimension.  g_out: f32[G], written
 * with amax(|w| over the matrix) / 2688.  codes: u8[n/2]; scales: u8[n/16]
 * (as trace_quant_rollout).  status_dev: as trace_amax.  Enqueues
 * trace_amax's kernels, then the RTN quantiser; on an argument error nothing
 * is enqueued. */
int trace_quant_weight(const void *w_bf16, int64_t n, int G, float *g_out, uint8_t *codes, uint8_t *scales,
                       int *status_dev, void *stream);

/* Rollout quantisation with standard RTN ("TRACE Core Concept": the rollout
 * side's actual FP4 result), fused with the guidance emit.
 * y_bf16: bf16[n]; g: f32[G] from trace_amax; k in {1, 2, 3, 4}.
 * codes: u8[n/2] packed nibbles; scales: u8[n/16] E4M3 block scales;
 * guidance: u8[trace_guidance_bytes(n, k)] or NULL (no guidance written). */
int trace_quant_rollout(const void *y_bf16, int64_t n, int G, const float *g, int k,
                        uint8_t *codes, uint8_t *scales, uint8_t *guidance, void *stream);

/* Bytes of the work buffer of trace_quant_rollout_onepass: 25 088 + 4 G,
 * rounded up to a multiple of 256 (0 if G < 1). */
size_t trace_onepass_work_bytes(int G);

/* Elements the one-pass rollout keeps on chip in one launch on the current
 * device with at most max_workgroups workgroups (0 = one per compute unit):
 * tensors up to this size (with G > 1, each group counted in whole tiles of
 * 8192 elements) are one launch that reads the input once.  A larger tensor
 * with G > 1 whose groups each fit runs one launch per block of whole groups
 * that fits (in one launch, by teams of workgroups, when every group is a
 * whole number of tiles and at least two such teams fit), and is still read
 * once.  Otherwise (G = 1, or a group larger
 * than this) the excess is read twice and the two-kernel path (trace_amax +
 * trace_quant_rollout) is usually faster.  0 on error (no device,
 * max_workgroups < 0). */
int64_t trace_onepass_capacity(int max_workgroups);

/* One-pass rollout: the results of trace_amax followed by trace_quant_rollout
 * (bit for bit), from one read of y where it fits on chip.  The global scale
 * needs the whole group before any block can be quantised ("Why Does FP4
 * Rollout 'Break' RL Training?": both sides share the global scale); instead
 * of reading y twice, one workgroup per compute unit keeps its share in VGPRs
 * and LDS (about 116 MiB of bf16 over 256 CUs), meets the others at a
 * grid-wide barrier once every group maximum is folded, and quantises from
 * chip; the part that does not fit is read a second time.
 * y_bf16: bf16[n]; g_out: f32[G], written; k, codes, scales, guidance: as
 * trace_quant_rollout.  work: device buffer of trace_onepass_work_bytes(G)
 * bytes, 16-byte aligned, owned by the caller, zero-filled before its first
 * use; every call leaves it zeroed again, also one that reports
 * TRACE_E_BARRIER (every workgroup counts out once, after its last use of the
 * buffer, and the last one out clears it), so no fill is needed between calls
 * and the call is one kernel launch (graph-capturable); calls that share a
 * work buffer must be ordered on one stream.  max_workgroups: 0 = one per
 * compute unit; a smaller cap leaves compute units to concurrent work but
 * keeps less on chip; TRACE_E_SIZE when the cap would give one workgroup a run
 * of 2^30 or more chunks of 8 elements (the output spans are 32-bit).
 * status_dev: nullable int*, as trace_amax's
 * (TRACE_E_NONFINITE), and TRACE_E_BARRIER if the workgroups were not all
 * resident within a time limit (1 s plus n * 2 bytes at 50 GB/s; the
 * environment variable TRACE_ONEPASS_WAIT_US, read at each call, replaces it,
 * which lets a test force the failure path); the outputs are then undefined.
 * A launch needs one workgroup resident on every compute unit it uses at
 * once: work on other streams that holds compute units (a device-to-host copy
 * into pinned memory is such work, a blit kernel, on this runtime) delays it
 * until that work ends, and two one-pass launches running at the same time
 * on different streams can starve each other until the time limit.
 * Enqueues one kernel, or one per block of groups when the tensor exceeds
 * trace_onepass_capacity and its groups fit (see there); every launch writes
 * its groups' parts of the same output planes and leaves the work buffer
 * zeroed for the next.  In the launch by teams, each team of workgroups takes
 * its groups in turn and meets at a barrier of its own per group (bounded by
 * the same time limit), so teams do not wait for one another. */
int trace_quant_rollout_onepass(const void *y_bf16, int64_t n, int G, int k, float *g_out, uint8_t *codes,
                                uint8_t *scales, uint8_t *guidance, void *work, int max_workgroups,
                                int *status_dev, void *stream);

/* The same one-pass rollout for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no work-buffer argument; its work buffer is a static array of
 * the library, 41 472 bytes per device (barrier counters and up to 4096
 * group maxima), held by each device the library runs on until the process
 * ends.  The first call on a device looks up that device's copy and enqueues
 * one clear of it on `stream` before its launch; every call leaves it zeroed
 * (as trace_quant_rollout_onepass does its work buffer).  All other arguments,
 * results and status words are those of trace_quant_rollout_onepass.
 * Every call on a device shares that device's array: calls that overlap in
 * time on one device (different streams, or different host threads without
 * ordering) race on it and give undefined results; order them on one stream.
 * Returns TRACE_E_SCRATCH, with nothing enqueued, when G > 4096.  Allocates
 * nothing: no hipMalloc, hipFree or allocating library call. */
int trace_quant_rollout_onepass_noalloc(const void *y_bf16, int64_t n, int G, int k, float *g_out, uint8_t *codes,
                                        uint8_t *scales, uint8_t *guidance, int max_workgroups, int *status_dev,
                                        void *stream);

/* One-pass plain QAT fake-quant with own scales: the results of trace_amax
 * on x followed by trace_fakequant_rtn with scales_in = NULL (bit for bit),
 * from one read of x where it fits on chip (the same kernel design, work
 * buffer, capacity, barrier limit and status words as
 * trace_quant_rollout_onepass).  "Experimental Results": plain QAT is the
 * unstable baseline; "Why Does FP4 Rollout 'Break' RL Training?": RTN with
 * a global and a block scale.  g_out: f32[G], written; y_out: bf16[n] or
 * f32[n] per out_dtype; codes_out (u8[n/2]) and scales_out (u8[n/16]) are
 * nullable.  Enqueues one kernel, or one per block of groups as
 * trace_quant_rollout_onepass does. */
int trace_fakequant_rtn_onepass(const void *x_bf16, int64_t n, int G, float *g_out, void *y_out, int out_dtype,
                                uint8_t *codes_out, uint8_t *scales_out, void *work, int max_workgroups,
                                int *status_dev, void *stream);

/* Guidance stream from existing codes and scales (for example an FP4 KV cache
 * written elsewhere); same layout as trace_quant_rollout's.  "TRACE Core
 * Concept", compact-guidance paragraph.  codes: u8[n/2]; scales: u8[n/16];
 * k in {1, 2, 3, 4}; guidance: u8[trace_guidance_bytes(n, k)]. */
int trace_guidance_pack(const uint8_t *codes, const uint8_t *scales, int64_t n, int k,
                        uint8_t *guidance, void *stream);

/* ---- training side ----------------------------------------------------- */

/* Rollout-guided fake-quant ("TRACE Core Concept"): for each element, the
 * two adjacent E2M1 points around v = x * inv (inv from the rollout's g and
 * block scale); the rollout code is reconstructed as the code nearest v whose
 * low k index bits equal the guidance bits; the adjacent point nearer it is
 * chosen; ties fall back to RTN.
 * x_bf16: bf16[n]; g: f32[G] (the rollout's); guidance: a k-bit stream;
 * k in {1, 2, 3} (k = 3, the whole magnitude index, decides like the full
 * code with v's own sign); y_out: bf16[n] or f32[n] per out_dtype;
 * codes_out: nullable u8[n/2] receiving the chosen nibbles. */
int trace_fakequant_guided(const void *x_bf16, int64_t n, int G, const float *g, const uint8_t *guidance,
                           int k, void *y_out, int out_dtype, uint8_t *codes_out, void *stream);

/* Full-code variant: the guidance carries the whole rollout nibble (k = 4
 * stream), and the adjacent point nearer that code is chosen.  The costly
 * option of "Experimental Results" (full guidance slows rollout). */
int trace_fakequant_fullcode(const void *x_bf16, int64_t n, int G, const float *g, const uint8_t *guidance,
                             void *y_out, int out_dtype, uint8_t *codes_out, void *stream);

/* Plain QAT fake-quant with RTN (the unstable baseline of "Experimental
 * Results").  scales_in: NULL = compute block scales from x with g (then g
 * should come from trace_amax on x); else u8[n/16] rollout scales (shared-
 * scale RTN).  codes_out (u8[n/2]) and scales_out (u8[n/16]) are nullable. */
int trace_fakequant_rtn(const void *x_bf16, int64_t n, int G, const float *g, const uint8_t *scales_in,
                        void *y_out, int out_dtype, uint8_t *codes_out, uint8_t *scales_out, void *stream);

/* Backward pass of every fake-quant above for quantisation-aware training
 * ("TRACE Core Concept": the training side fake-quantises; the pages fix no
 * gradient): the straight-through estimator clipped at the quantiser's
 * range.  gx = gy where |v| <= 6 and +0 where |v| > 6 (there the forward
 * saturated at +-6, so its output does not move with x), v = x * inv with
 * inv = 1 / (s * g) as in the forward (the scale chain of the conventions
 * above; a NaN v counts as beyond the range).
 * x_bf16: bf16[n], the forward's input; g: f32[G] and scales: u8[n/16], the
 * scales the forward used (guided and full code: the rollout's g and the
 * guidance stream's scale plane, i.e. its first n/16 bytes; shared-scale RTN:
 * scales_in; own-scale RTN: its g and scales_out).  gy, gx: bf16[n] or
 * f32[n] per grad_dtype (TRACE_OUT_BF16 / TRACE_OUT_F32); gx may be gy. */
int trace_fakequant_ste_grad(const void *x_bf16, int64_t n, int G, const float *g, const uint8_t *scales,
                             const void *gy, void *gx, int grad_dtype, void *stream);

/* ---- MXFP4 variant -------------------------------------------------------
 * The block format of gfx950's scaled FP4 conversions (OCP Microscaling
 * Formats v1.0): blocks of 32 consecutive elements share one E8M0 scale X =
 * 2^(code - 127); there is no global scale.  code = floor(log2(block amax))
 * - 2 + 127 (2 = the exponent of E2M1's largest value, 6 = 1.5 * 2^2),
 * clamped to 0 .. 254; an all-zero block gets code 0.  Elements are RTN(x / X)
 * on the E2M1 grid (ties to even, saturating at 6); dequantised y = sign *
 * val * X (exact).  The pages use the two-level NVFP4-style scale above; the
 * guided rule of "TRACE Core Concept" is the same on MX-normalised values.
 * Guidance stream: [ scale plane: n/32 E8M0 bytes | zero pad to a multiple of
 * 256 | bits ], bits as above.  Sizes: n > 0, n % 32 == 0, n < 2^34; 16-byte
 * aligned pointers; scale bytes 0 .. 254 (255, E8M0's NaN, is not accepted
 * as input). */

/* Bytes of the MX scale array: n / 32. */
size_t trace_mx_scale_bytes(int64_t n);
/* Bytes of the MX guidance stream, k in {1, 2, 3, 4}: align256(n/32) + n*k/8. */
size_t trace_mx_guidance_bytes(int64_t n, int k);

/* MX rollout quantisation: codes u8[n/2], E8M0 scales u8[n/32], guidance
 * (nullable) u8[trace_mx_guidance_bytes(n, k)], k in {1, 2, 3, 4}. */
int trace_mx_quant_rollout(const void *y_bf16, int64_t n, int k, uint8_t *codes, uint8_t *scales,
                           uint8_t *guidance, void *stream);

/* MX training side: guided (k = 1, 2, 3) or full code (k = 4) with the
 * rollout's MX scales from the guidance stream; outputs as
 * trace_fakequant_guided. */
int trace_mx_fakequant_guided(const void *x_bf16, int64_t n, const uint8_t *guidance, int k, void *y_out,
                              int out_dtype, uint8_t *codes_out, void *stream);

/* MX plain RTN fake-quant: scales_in NULL = own scales from x (written to
 * scales_out if given), else u8[n/32] scales. */
int trace_mx_fakequant_rtn(const void *x_bf16, int64_t n, const uint8_t *scales_in, void *y_out, int out_dtype,
                           uint8_t *codes_out, uint8_t *scales_out, void *stream);

/* ---- guidance records (transport and persistence) ---------------------- */
/*
 * "TRACE Core Concept": the rollout's guidance travels GPU -> CPU memory ->
 * disk -> CPU -> GPU before the training step uses it, and long trajectories,
 * large batches and async RL raise that cost; "Experimental Results": full
 * guidance slows rollout badly, the compact form stays close to plain FP4.
 *
 * A record is one self-describing host buffer:
 *   bytes  0..63   header (little-endian): magic 0x44475254 ("TRGD") (u32),
 *                  version 1 (u32), n (i64), k (i32), G (i32), stream bytes
 *                  (u64), bit-plane offset (u64), payload bytes (u64), XXH64
 *                  of the payload (u64), sealed flag (u32), zero pad to 64
 *   bytes 64..     payload: g (f32[G]) zero-padded to a multiple of 64 bytes,
 *                  then the guidance stream (trace_guidance_bytes(n, k))
 * The hash is XXH64 (seed 0) of the whole payload.  Host pointers below may
 * point to any host memory; for asynchronous copies it should be pinned
 * (hipHostMalloc or a pinned torch tensor).  The caller owns every buffer.
 */

/* Total record size for (n, k, G); 0 for invalid arguments. */
size_t trace_record_bytes(int64_t n, int k, int G);

/* Writes the header (unsealed) into record_host now and enqueues the
 * device-to-host copies of g (device f32[G]) and the guidance stream (device)
 * on `stream`.  Call trace_record_seal once the stream has passed the copies. */
int trace_record_to_host(const uint8_t *guidance, const float *g, int64_t n, int k, int G,
                         void *record_host, size_t record_bytes, void *stream);

/* Host only: hashes the payload into the header and marks it sealed. */
int trace_record_seal(void *record_host, size_t record_bytes);

/* Host only: validates magic, version, sizes, the sealed flag and the hash;
 * returns TRACE_OK and (if not NULL) n, k, G, or TRACE_E_FORMAT. */
int trace_record_check(const void *record_host, size_t record_bytes, int64_t *n, int *k, int *G);

/* Validates the header (not the hash: call trace_record_check for that) and
 * enqueues the host-to-device copies of g and the stream on `stream`. */
int trace_record_from_host(const void *record_host, size_t record_bytes, uint8_t *guidance, float *g,
                           void *stream);

/* Host only: whole-record file write / read (POSIX).  read fills at most
 * `capacity` bytes and reports the record size in *bytes_read; it fails with
 * TRACE_E_FORMAT when the file is not a record or does not fit. */
int trace_record_write(const char *path, const void *record_host, size_t record_bytes);
int trace_record_read(const char *path, void *record_host, size_t capacity, size_t *bytes_read);

/* Host only: XXH64 (seed 0) of a host buffer, the hash records use. */
uint64_t trace_xxh64(const void *data, size_t bytes);

/* ---- misc --------------------------------------------------------------- */

/* Static string for a trace_status value. */
const char *trace_status_str(int status);
/* Library version: major * 10000 + minor * 100 + patch. */
int trace_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TRACE_QUANT_H */
