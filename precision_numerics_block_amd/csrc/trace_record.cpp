// trace_record.cpp -- guidance records: moving the compact guidance stream and
// its global scales GPU -> host memory -> disk -> host memory -> GPU.
//
// "Alibaba Qwen Proposes TRACE for 5.4x Faster FP4 RL Rollouts", section
// "TRACE Core Concept": the rollout's quantisation information passes through
// CPU memory and disk before training loads it back to the GPU, and long
// trajectories, large batches and asynchronous RL amplify that traffic, which
// is why only the scale plus a few mantissa bits are kept.  Section
// "Experimental Results": full guidance slows rollout badly; the compact form
// stays close to plain FP4 rollout.
//
// Layout (little-endian, see include/trace_quant.h): a 64-byte header, then
// g (f32[G]) zero-padded to 64 bytes, then the guidance stream.  Integrity is
// an XXH64 hash of the payload, written from the published XXH64 algorithm
// (Yann Collet, xxHash specification: four 64-bit lanes over 32-byte stripes,
// then 8/4/1-byte tails and the final avalanche).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "trace_quant.h"

namespace {

constexpr uint32_t kMagic = 0x44475254u;   // "TRGD"
constexpr uint32_t kVersion = 1u;
constexpr size_t kHeader = 64;

struct Header {
    uint32_t magic;
    uint32_t version;
    int64_t n;
    int32_t k;
    int32_t G;
    uint64_t stream_bytes;
    uint64_t bitplane_offset;
    uint64_t payload_bytes;
    uint64_t hash;
    uint32_t sealed;
    uint32_t pad;
};
static_assert(sizeof(Header) == kHeader, "record header is 64 bytes");

// ---- XXH64 ----------------------------------------------------------------
constexpr uint64_t P1 = 0x9E3779B185EBCA87ull;
constexpr uint64_t P2 = 0xC2B2AE3D27D4EB4Full;
constexpr uint64_t P3 = 0x165667B19E3779F9ull;
constexpr uint64_t P4 = 0x85EBCA77C2B2AE63ull;
constexpr uint64_t P5 = 0x27D4EB2F165667C5ull;

inline uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
inline uint64_t rd64(const uint8_t *p) { uint64_t v; std::memcpy(&v, p, 8); return v; }
inline uint32_t rd32(const uint8_t *p) { uint32_t v; std::memcpy(&v, p, 4); return v; }
inline uint64_t lane_round(uint64_t acc, uint64_t in) { return rotl(acc + in * P2, 31) * P1; }
inline uint64_t merge(uint64_t acc, uint64_t v) { return (acc ^ lane_round(0, v)) * P1 + P4; }

uint64_t xxh64(const uint8_t *p, size_t len, uint64_t seed)
{
    const uint8_t *end = p + len;
    uint64_t h;
    if (len >= 32) {
        uint64_t v1 = seed + P1 + P2, v2 = seed + P2, v3 = seed, v4 = seed - P1;
        const uint8_t *limit = end - 32;
        do {
            v1 = lane_round(v1, rd64(p));
            v2 = lane_round(v2, rd64(p + 8));
            v3 = lane_round(v3, rd64(p + 16));
            v4 = lane_round(v4, rd64(p + 24));
            p += 32;
        } while (p <= limit);
        h = rotl(v1, 1) + rotl(v2, 7) + rotl(v3, 12) + rotl(v4, 18);
        h = merge(h, v1);
        h = merge(h, v2);
        h = merge(h, v3);
        h = merge(h, v4);
    } else {
        h = seed + P5;
    }
    h += (uint64_t)len;
    while (p + 8 <= end) {
        h ^= lane_round(0, rd64(p));
        h = rotl(h, 27) * P1 + P4;
        p += 8;
    }
    if (p + 4 <= end) {
        h ^= (uint64_t)rd32(p) * P1;
        h = rotl(h, 23) * P2 + P3;
        p += 4;
    }
    while (p < end) {
        h ^= (uint64_t)(*p) * P5;
        h = rotl(h, 11) * P1;
        ++p;
    }
    h ^= h >> 33;
    h *= P2;
    h ^= h >> 29;
    h *= P3;
    h ^= h >> 32;
    return h;
}

// ---- layout -----------------------------------------------------------------
size_t g_area(int G) { return ((size_t)G * 4 + 63) / 64 * 64; }

bool valid_args(int64_t n, int k, int G)
{
    return trace_guidance_bytes(n, k) > 0 && G >= 1 && n % (16 * (int64_t)G) == 0;
}

Header make_header(int64_t n, int k, int G)
{
    Header h{};
    h.magic = kMagic;
    h.version = kVersion;
    h.n = n;
    h.k = k;
    h.G = G;
    h.stream_bytes = trace_guidance_bytes(n, k);
    h.bitplane_offset = (uint64_t)((n / 16 + 255) / 256 * 256);
    h.payload_bytes = g_area(G) + h.stream_bytes;
    return h;
}

// Header consistent with itself and with the buffer size.
bool header_ok(const Header &h, size_t record_bytes)
{
    if (h.magic != kMagic || h.version != kVersion || !valid_args(h.n, h.k, h.G))
        return false;
    Header ref = make_header(h.n, h.k, h.G);
    return h.stream_bytes == ref.stream_bytes && h.bitplane_offset == ref.bitplane_offset &&
           h.payload_bytes == ref.payload_bytes && record_bytes >= kHeader + h.payload_bytes;
}

}  // namespace

extern "C" {

uint64_t trace_xxh64(const void *data, size_t bytes)
{
    return xxh64(static_cast<const uint8_t *>(data), bytes, 0);
}

size_t trace_record_bytes(int64_t n, int k, int G)
{
    if (!valid_args(n, k, G))
        return 0;
    return kHeader + make_header(n, k, G).payload_bytes;
}

int trace_record_to_host(const uint8_t *guidance, const float *g, int64_t n, int k, int G, void *record_host,
                         size_t record_bytes, void *stream)
{
    if (!guidance || !g || !record_host)
        return TRACE_E_NULL;
    if (!valid_args(n, k, G))
        return k < 1 || k > 4 ? TRACE_E_K : TRACE_E_SIZE;
    Header h = make_header(n, k, G);
    if (record_bytes < kHeader + h.payload_bytes)
        return TRACE_E_SIZE;
    uint8_t *rec = static_cast<uint8_t *>(record_host);
    std::memcpy(rec, &h, kHeader);
    std::memset(rec + kHeader + (size_t)G * 4, 0, g_area(G) - (size_t)G * 4);
    hipStream_t st = (hipStream_t)stream;
    if (hipMemcpyAsync(rec + kHeader, g, (size_t)G * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipMemcpyAsync(rec + kHeader + g_area(G), guidance, h.stream_bytes, hipMemcpyDeviceToHost, st) !=
            hipSuccess)
        return TRACE_E_HIP;
    return TRACE_OK;
}

int trace_record_seal(void *record_host, size_t record_bytes)
{
    if (!record_host)
        return TRACE_E_NULL;
    if (record_bytes < kHeader)
        return TRACE_E_FORMAT;
    uint8_t *rec = static_cast<uint8_t *>(record_host);
    Header h;
    std::memcpy(&h, rec, kHeader);
    if (!header_ok(h, record_bytes))
        return TRACE_E_FORMAT;
    h.hash = xxh64(rec + kHeader, h.payload_bytes, 0);
    h.sealed = 1;
    std::memcpy(rec, &h, kHeader);
    return TRACE_OK;
}

int trace_record_check(const void *record_host, size_t record_bytes, int64_t *n, int *k, int *G)
{
    if (!record_host)
        return TRACE_E_NULL;
    if (record_bytes < kHeader)
        return TRACE_E_FORMAT;
    const uint8_t *rec = static_cast<const uint8_t *>(record_host);
    Header h;
    std::memcpy(&h, rec, kHeader);
    if (!header_ok(h, record_bytes) || h.sealed != 1 || h.pad != 0)
        return TRACE_E_FORMAT;
    if (xxh64(rec + kHeader, h.payload_bytes, 0) != h.hash)
        return TRACE_E_FORMAT;
    if (n)
        *n = h.n;
    if (k)
        *k = h.k;
    if (G)
        *G = h.G;
    return TRACE_OK;
}

int trace_record_from_host(const void *record_host, size_t record_bytes, uint8_t *guidance, float *g, void *stream)
{
    if (!record_host || !guidance || !g)
        return TRACE_E_NULL;
    if (record_bytes < kHeader)
        return TRACE_E_FORMAT;
    const uint8_t *rec = static_cast<const uint8_t *>(record_host);
    Header h;
    std::memcpy(&h, rec, kHeader);
    if (!header_ok(h, record_bytes))
        return TRACE_E_FORMAT;
    hipStream_t st = (hipStream_t)stream;
    if (hipMemcpyAsync(g, rec + kHeader, (size_t)h.G * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(guidance, rec + kHeader + g_area(h.G), h.stream_bytes, hipMemcpyHostToDevice, st) !=
            hipSuccess)
        return TRACE_E_HIP;
    return TRACE_OK;
}

int trace_record_write(const char *path, const void *record_host, size_t record_bytes)
{
    if (!path || !record_host)
        return TRACE_E_NULL;
    std::FILE *f = std::fopen(path, "wb");
    if (!f)
        return TRACE_E_IO;
    size_t w = std::fwrite(record_host, 1, record_bytes, f);
    int rc = std::fclose(f);
    return (w == record_bytes && rc == 0) ? TRACE_OK : TRACE_E_IO;
}

int trace_record_read(const char *path, void *record_host, size_t capacity, size_t *bytes_read)
{
    if (!path || !record_host)
        return TRACE_E_NULL;
    std::FILE *f = std::fopen(path, "rb");
    if (!f)
        return TRACE_E_IO;
    Header h;
    int rc = TRACE_OK;
    if (std::fread(&h, 1, kHeader, f) != kHeader || capacity < kHeader) {
        rc = TRACE_E_FORMAT;
    } else {
        size_t total = (size_t)(kHeader + h.payload_bytes);
        if (!header_ok(h, total) || total > capacity) {
            rc = TRACE_E_FORMAT;
        } else {
            std::memcpy(record_host, &h, kHeader);
            size_t body = total - kHeader;
            if (std::fread(static_cast<uint8_t *>(record_host) + kHeader, 1, body, f) != body)
                rc = TRACE_E_FORMAT;                    // truncated file
            else if (bytes_read)
                *bytes_read = total;
        }
    }
    std::fclose(f);
    return rc;
}

}  // extern "C"
