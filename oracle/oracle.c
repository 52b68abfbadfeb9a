/*
 * oracle.c -- CPU oracle for the transfer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path loads, links or calls
 * this file: only the test suite, the smoke check and the oracle leg of the
 * benchmark (its CPU baseline and the checks of its GPU results) do.  It shares no code, header, table or helper with the HIP
 * library (copy_reduce_amd/), and it includes no HIP header.
 *
 * Everything here is written to be checked by eye against the pages:
 *   - "TransferBench data validation" (ROCm docs 1.66.02): the expected-value
 *     table (0 / 1 / N sources), "Expected source pattern" (PrepareReference,
 *     PrepSrcValue, fillPattern, fillCompress), "Expected destination
 *     (dstReference)" and "How validation (ValidateAllTransfers) works".
 *   - TransferBench PR #365, "Fix one-sided remote-read bandwidth inflation
 *     via source-slice rotation (SRC_ROTATE_BYTES)": Technical Details (slice
 *     count K, slice selection i mod K, negative warmup indices) and the review
 *     item asking for aligned slices.
 *   - Mooncake RFC #5041, "HipTransport ...", Design of #5040: a batch is a
 *     (src, dst, len) descriptor array and each descriptor is a plain copy.
 *
 * Floating point: the pages fix the precision.  TransferBench keeps its
 * reference buffers as float and builds dstReference[k] from dstReference[k-1]
 * one buffer at a time, so the oracle accumulates in binary32 with one
 * round-to-nearest-even per addition, left to right, starting from source 0.
 * Build with plain gcc (x86-64 SSE scalar float, no -ffast-math, no FMA
 * contraction): see oracle/build.py.
 *
 * Parity status of each function is stated above it.  The fillCompress
 * generator is "parity unpinned" by the pages (they give no generator, no
 * zeroing layout and no printed values); it is pinned only by its own written
 * spec and by published SplitMix64 outputs.
 */
#define _POSIX_C_SOURCE 199309L
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

/* ------------------------------------------------------------------------ */
/* Slice geometry and rotation                                               */
/* ------------------------------------------------------------------------ */

/*
 * Number of identical source slices, PR #365 Technical Details:
 * K = ceil(SRC_ROTATE_BYTES / numBytes), where SRC_ROTATE_BYTES = 0 disables
 * rotation.  Readings where the page is silent: rotation off, numBytes = 0 and
 * numBytes >= SRC_ROTATE_BYTES all give K = 1.
 * Pinned by the page's printed examples (4 MB -> 64, 256 MB -> 1).
 */
uint64_t orc_num_slices(uint64_t num_bytes, uint64_t rotate_bytes)
{
    if (rotate_bytes == 0 || num_bytes == 0)
        return 1;
    uint64_t k = rotate_bytes / num_bytes;
    if (rotate_bytes % num_bytes != 0)
        k += 1;
    if (k == 0)
        k = 1;
    return k;
}

/*
 * Distance in bytes between the starts of consecutive slices.  The PR
 * allocates K * numBytes; its review asks for slices aligned for vector
 * loads.  Reading: round numBytes up to a multiple of 256 bytes (identical to
 * the PR whenever numBytes is already a multiple of 256).
 */
uint64_t orc_slice_stride(uint64_t num_bytes)
{
    return (num_bytes + 255u) / 256u * 256u;
}

/*
 * Slice read by iteration i, PR #365 Technical Details: iteration i reads
 * slice i % K, with the iteration folded into [0, K) so that the negative
 * indices used for warmup iterations work.
 */
uint64_t orc_slice_of(int64_t iteration, uint64_t k)
{
    if (k == 0)
        return 0;
    int64_t kk = (int64_t)k;
    int64_t r = iteration % kk;       /* C: sign follows the dividend */
    if (r < 0)
        r += kk;
    return (uint64_t)r;
}

/* ------------------------------------------------------------------------ */
/* Source patterns ("Expected source pattern", PrepareReference)             */
/* ------------------------------------------------------------------------ */

/*
 * Default pattern: PrepSrcValue(bufferIdx, i) =
 *     (((i % 383) * 517) % 383 + 31) * (bufferIdx + 1).
 * Reading: evaluated in integer arithmetic on the 64-bit element index i
 * within one slice, converted to float once at the end.  Every value is at
 * most 413 * (bufferIdx + 1) < 2^24, so the conversion is exact.
 */
void orc_gen_default(float *out, uint64_t n, int buffer_idx)
{
    for (uint64_t i = 0; i < n; i++) {
        uint64_t v = (((i % 383u) * 517u) % 383u + 31u) * (uint64_t)(buffer_idx + 1);
        out[i] = (float)v;
    }
}

/* fillPattern: the given vector of floats repeated over the buffer. */
void orc_gen_pattern(float *out, uint64_t n, const float *pattern, uint64_t pattern_len)
{
    for (uint64_t i = 0; i < n; i++)
        out[i] = pattern[i % pattern_len];
}

/*
 * SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014).  The state advances by the golden-ratio
 * increment and each output is the state passed through the mixing function.
 * orc_splitmix64(key, j) is the j-th output (from 0) of the generator seeded
 * with `key`.
 */
static uint64_t sm64_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t orc_splitmix64(uint64_t key, uint64_t j)
{
    uint64_t state = key + (j + 1u) * 0x9E3779B97F4A7C15ULL;
    return sm64_mix(state);
}

/*
 * fillCompress: per 64-byte line of each source buffer, a mix of random
 * floats with optional zeroing; category 0 = random, 1 = 1B0, 2 = 2B0,
 * 3 = 4B0, 4 = 32B0, with percentages setting the mix.
 *
 * The page gives neither the generator nor the zeroing layout.  Reading
 * (written spec shared by both sides, each side implementing it on its own):
 *   - line L of buffer b has category c chosen by
 *       d = splitmix64(seed ^ (2b + 1), L) % 100
 *     against the cumulative percentages in the order above;
 *   - float i of buffer b (i = 16 L + k) is
 *       x = (int)(splitmix64(seed ^ 2b, i) >> 40) - 2^23,  value = x * 2^-23,
 *     an exact multiple of 2^-23 in [-1, 1);
 *   - category "nB0" sets the leading n bytes of the line (memory order,
 *     little endian) to 0x00; the last line of a buffer may be partial and is
 *     clipped to the buffer.
 * Returns 0, or -1 if the percentages do not sum to 100.
 */
int orc_gen_compress(float *out, uint64_t n, int buffer_idx,
                     const uint32_t pct[5], uint64_t seed)
{
    static const uint32_t zero_bytes[5] = {0, 1, 2, 4, 32};
    uint32_t total = 0;
    for (int c = 0; c < 5; c++)
        total += pct[c];
    if (total != 100)
        return -1;

    uint64_t value_key = seed ^ (uint64_t)(2 * buffer_idx);
    uint64_t line_key = seed ^ (uint64_t)(2 * buffer_idx + 1);

    for (uint64_t i = 0; i < n; i++) {
        int32_t x = (int32_t)(orc_splitmix64(value_key, i) >> 40) - 8388608;
        out[i] = (float)x * 0x1p-23f;
    }

    uint64_t total_bytes = n * 4u;
    uint64_t nlines = (total_bytes + 63u) / 64u;
    unsigned char *bytes = (unsigned char *)out;
    for (uint64_t line = 0; line < nlines; line++) {
        uint32_t draw = (uint32_t)(orc_splitmix64(line_key, line) % 100u);
        int category = 0;
        uint32_t upper = 0;
        for (int c = 0; c < 5; c++) {
            upper += pct[c];
            if (draw < upper) {
                category = c;
                break;
            }
        }
        uint64_t start = line * 64u;
        uint64_t count = zero_bytes[category];
        if (start + count > total_bytes)
            count = total_bytes - start;
        memset(bytes + start, 0, (size_t)count);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Expected destination                                                      */
/* ------------------------------------------------------------------------ */

/*
 * "Expected destination (dstReference)":
 *   dstReference[0] = memset to MEMSET_CHAR           (no sources)
 *   dstReference[1] = srcReference[0]                 (one source)
 *   dstReference[k] = dstReference[k-1] + srcReference[k-1]
 * and dstReference[numSrcs] is what a transfer with numSrcs sources must
 * produce.  Only the running buffer is kept: `dst` holds dstReference[k]
 * after step k.  Each addition is one binary32 addition.
 */
void orc_ref_reduce(float *dst, const float *const *srcs, int nsrc,
                    uint64_t n, unsigned memset_byte)
{
    if (nsrc == 0) {
        memset(dst, (int)(memset_byte & 0xFFu), (size_t)(n * 4u));
        return;
    }
    memcpy(dst, srcs[0], (size_t)(n * 4u));
    for (int k = 2; k <= nsrc; k++) {
        const float *next = srcs[k - 1];
        for (uint64_t i = 0; i < n; i++)
            dst[i] = dst[i] + next[i];
    }
}

/* ------------------------------------------------------------------------ */
/* Batched copy                                                              */
/* ------------------------------------------------------------------------ */

/*
 * Mooncake RFC #5041, Design of #5040: one launch runs a (src, dst, len)
 * descriptor array, each descriptor being an ordinary copy.  Host images
 * stand in for device memory: desc holds n triples
 * (source offset, destination offset, bytes) into src_image and pool.
 * With disjoint destinations the result does not depend on order.
 */
void orc_ref_batch(unsigned char *pool, const unsigned char *src_image,
                   const uint64_t *desc, uint64_t n)
{
    for (uint64_t d = 0; d < n; d++) {
        uint64_t src_off = desc[3 * d + 0];
        uint64_t dst_off = desc[3 * d + 1];
        uint64_t bytes = desc[3 * d + 2];
        memcpy(pool + dst_off, src_image + src_off, (size_t)bytes);
    }
}

/* ------------------------------------------------------------------------ */
/* Validation                                                                */
/* ------------------------------------------------------------------------ */

/*
 * "How validation (ValidateAllTransfers) works", step 3: memcmp of the output
 * against the expected buffer; on a mismatch, the first differing element.
 * Returns -1 when the buffers are equal, else the index of the first element
 * (of elem_size bytes) that differs.
 */
int64_t orc_first_mismatch(const void *out, const void *expected,
                           uint64_t nbytes, uint64_t elem_size)
{
    if (memcmp(out, expected, (size_t)nbytes) == 0)
        return -1;
    const unsigned char *a = (const unsigned char *)out;
    const unsigned char *b = (const unsigned char *)expected;
    for (uint64_t i = 0; i < nbytes; i++)
        if (a[i] != b[i])
            return (int64_t)(i / elem_size);
    return -1;
}

/*
 * The same validation with the report the page describes for a failure: the
 * first differing element's index together with its expected and actual
 * values (here their bytes, as the low elem_size bytes of a little-endian
 * 64-bit word; elem_size is 1 .. 8).  Returns 0 when the buffers are equal
 * (the outputs are left untouched), else 1.
 */
int orc_mismatch_report(const void *out, const void *expected, uint64_t nbytes, uint64_t elem_size,
                        int64_t *index, uint64_t *expected_bits, uint64_t *actual_bits)
{
    const int64_t i = orc_first_mismatch(out, expected, nbytes, elem_size);
    if (i < 0)
        return 0;
    uint64_t e = 0, a = 0;
    memcpy(&e, (const unsigned char *)expected + (uint64_t)i * elem_size, (size_t)elem_size);
    memcpy(&a, (const unsigned char *)out + (uint64_t)i * elem_size, (size_t)elem_size);
    *index = i;
    *expected_bits = e;
    *actual_bits = a;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* Single-core timing of the oracle (CPU baseline)                           */
/* ------------------------------------------------------------------------ */

static double now_seconds(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

/* Wall seconds for one orc_ref_reduce call, on the calling thread. */
double orc_time_ref_reduce(float *dst, const float *const *srcs, int nsrc,
                           uint64_t n, unsigned memset_byte)
{
    double t0 = now_seconds();
    orc_ref_reduce(dst, srcs, nsrc, n, memset_byte);
    return now_seconds() - t0;
}

/* Wall seconds for one orc_ref_batch call, on the calling thread. */
double orc_time_ref_batch(unsigned char *pool, const unsigned char *src_image,
                          const uint64_t *desc, uint64_t n)
{
    double t0 = now_seconds();
    orc_ref_batch(pool, src_image, desc, n);
    return now_seconds() - t0;
}
