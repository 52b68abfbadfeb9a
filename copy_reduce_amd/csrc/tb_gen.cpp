// tb_gen.cpp -- PrepareReference for libtb: the host reference data of one
// source buffer ("TransferBench data validation", Expected source pattern).
// Host-only code; no HIP calls.
#include <stdint.h>
#include <string.h>

#include "tb.h"

namespace {

// Period of the default pattern in elements.
constexpr uint64_t kPeriod = 383;

// Default pattern: PrepSrcValue(b, i) = (((i % 383) * 517) % 383 + 31) * (b + 1).
// The value depends on i only through i % 383, so one period is evaluated
// exactly in integers (every value < 2^24 converts to float exactly) and then
// replicated; the index is the 64-bit element index inside the slice.
void fill_default(float *out, uint64_t n, int32_t b) {
    float period[kPeriod];
    const uint64_t scale = (uint64_t)b + 1;
    for (uint64_t r = 0; r < kPeriod; r++)
        period[r] = (float)(((r * 517) % kPeriod + 31) * scale);
    uint64_t i = 0;
    while (i < n) {
        const uint64_t phase = i % kPeriod;
        uint64_t len = kPeriod - phase;
        if (len > n - i)
            len = n - i;
        memcpy(out + i, period + phase, len * sizeof(float));
        i += len;
    }
}

// fillPattern: the pattern vector repeated over the buffer.
void fill_pattern(float *out, uint64_t n, const float *pat, uint64_t len) {
    uint64_t i = 0;
    while (i < n) {
        uint64_t c = len < n - i ? len : n - i;
        memcpy(out + i, pat, c * sizeof(float));
        i += c;
    }
}

// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): a Weyl sequence with increment
// 0x9E3779B97F4A7C15 passed through a 64-bit finaliser.  Output j of the
// stream seeded with `key` is mix(key + (j + 1) * increment).
struct SplitMix64 {
    static constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
    static uint64_t mix(uint64_t z) {
        z ^= z >> 30;
        z *= 0xBF58476D1CE4E5B9ull;
        z ^= z >> 27;
        z *= 0x94D049BB133111EBull;
        z ^= z >> 31;
        return z;
    }
    static uint64_t at(uint64_t key, uint64_t j) { return mix(key + (j + 1) * kGamma); }
};

// fillCompress (the page names the categories random, 1B0, 2B0, 4B0, 32B0 per
// 64-byte line with percentages setting the mix; the generator and the byte
// layout are this library's documented reading):
//   category of line L:  SplitMix64(seed ^ (2b+1)) output L, mod 100, against
//                        the cumulative percentages;
//   float i:             top 24 bits of SplitMix64(seed ^ 2b) output i, minus
//                        2^23, times 2^-23  (exact, in [-1, 1));
//   category nB0:        leading n bytes of the line set to zero, clipped at
//                        the end of the buffer.
void fill_compress(float *out, uint64_t n, int32_t b, const uint32_t pct[5], uint64_t seed) {
    static const unsigned kZeroBytes[5] = {0, 1, 2, 4, 32};
    const uint64_t vkey = seed ^ (uint64_t)(2 * (int64_t)b);
    const uint64_t ckey = seed ^ (uint64_t)(2 * (int64_t)b + 1);
    uint32_t bound[5];
    uint32_t acc = 0;
    for (int c = 0; c < 5; c++) {
        acc += pct[c];
        bound[c] = acc;
    }
    const uint64_t nbytes = n * 4;
    for (uint64_t line = 0; line * 16 < n; line++) {
        const uint64_t first = line * 16;
        const uint64_t last = first + 16 < n ? first + 16 : n;
        for (uint64_t i = first; i < last; i++) {
            const uint32_t top = (uint32_t)(SplitMix64::at(vkey, i) >> 40);
            out[i] = (float)((int32_t)top - (1 << 23)) * 0x1p-23f;
        }
        const uint32_t pick = (uint32_t)(SplitMix64::at(ckey, line) % 100);
        int cat = 0;
        while (cat < 4 && pick >= bound[cat])
            cat++;
        uint64_t z = kZeroBytes[cat];
        const uint64_t line_start = line * 64;
        if (line_start + z > nbytes)
            z = nbytes - line_start;
        if (z)
            memset(reinterpret_cast<unsigned char *>(out) + line_start, 0, z);
    }
}

}  // namespace

extern "C" int tb_prep_reference(float *host_out, uint64_t nfloats, int32_t buffer_idx,
                                 const tb_fill_cfg *cfg) {
    // the configuration is checked first, whatever the size
    if (buffer_idx < 0)
        return TB_ERR_INVALID;
    const int32_t kind = cfg ? cfg->kind : TB_FILL_DEFAULT;
    if (kind == TB_FILL_PATTERN && (cfg->pattern == nullptr || cfg->pattern_len == 0))
        return TB_ERR_INVALID;
    if (kind == TB_FILL_COMPRESS) {
        uint64_t sum = 0;
        for (int c = 0; c < 5; c++)
            sum += cfg->compress_pct[c];
        if (sum != 100)
            return TB_ERR_INVALID;
    }
    if (kind != TB_FILL_DEFAULT && kind != TB_FILL_PATTERN && kind != TB_FILL_COMPRESS)
        return TB_ERR_INVALID;
    if (nfloats == 0)
        return TB_OK;
    if (host_out == nullptr || nfloats > UINT64_MAX / 4)
        return TB_ERR_INVALID;
    switch (kind) {
    case TB_FILL_DEFAULT:
        fill_default(host_out, nfloats, buffer_idx);
        break;
    case TB_FILL_PATTERN:
        fill_pattern(host_out, nfloats, cfg->pattern, cfg->pattern_len);
        break;
    default:
        fill_compress(host_out, nfloats, buffer_idx, cfg->compress_pct, cfg->seed);
        break;
    }
    return TB_OK;
}
