/* Exercises every oracle function over small and edge-case sizes in a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer; any out-of-bounds
 * access, overflow or other undefined behaviour aborts the run.  A few cheap
 * invariants are checked on the way.  Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint64_t orc_num_slices(uint64_t num_bytes, uint64_t rotate_bytes);
uint64_t orc_slice_stride(uint64_t num_bytes);
uint64_t orc_slice_of(int64_t iteration, uint64_t k);
void orc_gen_default(float *out, uint64_t n, int buffer_idx);
void orc_gen_pattern(float *out, uint64_t n, const float *pattern, uint64_t pattern_len);
uint64_t orc_splitmix64(uint64_t key, uint64_t j);
int orc_gen_compress(float *out, uint64_t n, int buffer_idx, const uint32_t pct[5], uint64_t seed);
void orc_ref_reduce(float *dst, const float *const *srcs, int nsrc, uint64_t n, unsigned memset_byte);
void orc_ref_batch(unsigned char *pool, const unsigned char *src_image, const uint64_t *desc, uint64_t n);
int64_t orc_first_mismatch(const void *out, const void *expected, uint64_t nbytes, uint64_t elem_size);

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void)
{
    static const uint64_t sizes[] = {0, 1, 3, 15, 16, 17, 63, 64, 65, 383, 384, 1023, 1025, 4099};
    const uint32_t pcts[3][5] = {{50, 20, 10, 10, 10}, {0, 0, 0, 0, 100}, {100, 0, 0, 0, 0}};
    const float pattern[3] = {1.0f, -0.0f, 2.5f};

    CHECK(orc_num_slices(4u << 20, 256u << 20) == 64);
    CHECK(orc_num_slices(0, 256u << 20) == 1 && orc_num_slices(5, 0) == 1);
    CHECK(orc_num_slices(UINT64_MAX, UINT64_MAX) == 1 && orc_num_slices(1, UINT64_MAX) == UINT64_MAX);
    CHECK(orc_slice_stride(1) == 256 && orc_slice_stride(0) == 0);
    CHECK(orc_slice_of(-3, 64) == 61 && orc_slice_of(INT64_MIN, 7) < 7 && orc_slice_of(INT64_MAX, 1) == 0);
    (void)orc_splitmix64(UINT64_MAX, UINT64_MAX);

    for (size_t si = 0; si < sizeof sizes / sizeof sizes[0]; si++) {
        const uint64_t n = sizes[si];
        float *a = malloc((n + 1) * sizeof(float)), *b = malloc((n + 1) * sizeof(float));
        float *c = malloc((n + 1) * sizeof(float)), *d = malloc((n + 1) * sizeof(float));
        CHECK(a && b && c && d);
        orc_gen_default(a, n, 0);
        orc_gen_default(b, n, 15);
        orc_gen_pattern(c, n, pattern, 3);
        for (int p = 0; p < 3; p++)
            CHECK(orc_gen_compress(d, n, p, pcts[p], 3 + (uint64_t)p) == 0);
        const uint32_t bad[5] = {50, 50, 50, 0, 0};
        CHECK(orc_gen_compress(d, n, 0, bad, 1) == -1);
        const float *srcs[4] = {a, b, c, d};
        for (int nsrc = 0; nsrc <= 4; nsrc++) {
            float *out = malloc((n + 1) * sizeof(float));
            CHECK(out);
            orc_ref_reduce(out, srcs, nsrc, n, 0x5A);
            if (nsrc == 1)
                CHECK(orc_first_mismatch(out, a, n * 4, 4) == -1);
            free(out);
        }
        CHECK(orc_first_mismatch(a, a, n * 4, 4) == -1);
        if (n) {
            memcpy(c, a, n * 4);
            c[n - 1] += 1.0f;
            CHECK(orc_first_mismatch(c, a, n * 4, 4) == (int64_t)(n - 1));
        }
        free(a), free(b), free(c), free(d);
    }

    /* batched copy over random disjoint descriptors, pool exactly as large as needed */
    uint64_t desc[3 * 200], src_bytes = 0, pool_bytes = 0, x = 12345;
    for (int i = 0; i < 200; i++) {
        x = orc_splitmix64(x, (uint64_t)i);
        const uint64_t len = x % 3000;
        desc[3 * i + 0] = src_bytes;
        desc[3 * i + 1] = pool_bytes;
        desc[3 * i + 2] = len;
        src_bytes += len + (x >> 40) % 7;
        pool_bytes += len + (x >> 50) % 13;
    }
    unsigned char *img = malloc(src_bytes + 1), *pool = malloc(pool_bytes + 1);
    CHECK(img && pool);
    for (uint64_t i = 0; i < src_bytes; i++)
        img[i] = (unsigned char)(i * 131u + 7u);
    memset(pool, 0xA5, pool_bytes);
    orc_ref_batch(pool, img, desc, 200);
    orc_ref_batch(pool, img, desc, 0);
    for (int i = 0; i < 200; i++)
        CHECK(orc_first_mismatch(pool + desc[3 * i + 1], img + desc[3 * i], desc[3 * i + 2], 1) == -1);
    free(img), free(pool);
    puts("oracle sanitizer run ok");
    return 0;
}
