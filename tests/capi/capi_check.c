/*
 * capi_check.c -- the library's C ABI (include/tb.h) used from plain C11:
 * device memory from the HIP runtime's C API, no Python, no torch.
 *
 * A consumer-side check of the boundary, not a parity test (those compare
 * against the oracle): a two-source reduce-copy whose sums are exact in
 * binary32, a batched copy of 1,000 copies of 1 B - 4 KiB at arbitrary byte
 * offsets, and the argument checks.  Prints "capi ok" and exits 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tb.h"

#define HIP_OK(x)                                                                         \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));               \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

#define TB_OK_(x)                                                                         \
    do {                                                                                  \
        int rc_ = (x);                                                                    \
        if (rc_ != TB_OK) {                                                               \
            fprintf(stderr, "%s -> %s (%s)\n", #x, tb_status_string(rc_), tb_last_hip_error()); \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

/* xorshift64, for the batch's sizes and offsets */
static uint64_t rnd(uint64_t *s) {
    *s ^= *s << 13;
    *s ^= *s >> 7;
    *s ^= *s << 17;
    return *s;
}

static int check_reduce(hipStream_t s) {
    const uint64_t n = (1u << 20) + 3;
    float *h0 = malloc(n * sizeof(float)), *h1 = malloc(n * sizeof(float)), *out = malloc(n * sizeof(float));
    if (!h0 || !h1 || !out)
        return 1;
    for (uint64_t i = 0; i < n; i++) {   /* multiples of 1/4 below 2^10: every sum is exact */
        h0[i] = (float)(i % 1000) * 0.5f;
        h1[i] = (float)(i % 777) * 0.25f;
    }
    float *d0, *d1, *dd;
    HIP_OK(hipMalloc((void **)&d0, n * sizeof(float)));
    HIP_OK(hipMalloc((void **)&d1, n * sizeof(float)));
    HIP_OK(hipMalloc((void **)&dd, n * sizeof(float) + 4));
    HIP_OK(hipMemcpy(d0, h0, n * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d1, h1, n * sizeof(float), hipMemcpyHostToDevice));
    const float *srcs[2] = {d0, d1};
    /* dst one float past an allocation boundary: the head/tail split runs too */
    TB_OK_(tb_reduce_copy(dd + 1, srcs, 2, n, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(out, dd + 1, n * sizeof(float), hipMemcpyDeviceToHost));
    for (uint64_t i = 0; i < n; i++) {
        if (out[i] != h0[i] + h1[i]) {
            fprintf(stderr, "reduce-copy: element %llu is %g, expected %g\n", (unsigned long long)i, out[i],
                    h0[i] + h1[i]);
            return 1;
        }
    }
    /* argument checks: too many sources, a misaligned pointer */
    if (tb_reduce_copy(dd, srcs, TB_MAX_SRCS + 1, n, s) != TB_ERR_INVALID ||
        tb_reduce_copy((float *)((char *)dd + 2), srcs, 2, 16, s) != TB_ERR_INVALID) {
        fprintf(stderr, "reduce-copy accepted invalid arguments\n");
        return 1;
    }
    HIP_OK(hipFree(d0));
    HIP_OK(hipFree(d1));
    HIP_OK(hipFree(dd));
    free(h0);
    free(h1);
    free(out);
    return 0;
}

static int check_batch(hipStream_t s) {
    enum { NCOPY = 1000, SLOT = 8192 };
    const uint64_t src_bytes = (uint64_t)NCOPY * 4096 + 64, pool_bytes = (uint64_t)NCOPY * SLOT;
    uint8_t *hsrc = malloc(src_bytes), *hpool = malloc(pool_bytes), *expect = malloc(pool_bytes);
    tb_copy_desc *desc = malloc(NCOPY * sizeof(tb_copy_desc));
    if (!hsrc || !hpool || !expect || !desc)
        return 1;
    uint64_t seed = 0x9E3779B97F4A7C15ull;
    for (uint64_t i = 0; i < src_bytes; i++)
        hsrc[i] = (uint8_t)rnd(&seed);
    memset(expect, 0xA5, pool_bytes);
    uint8_t *dsrc, *dpool;
    tb_copy_desc *ddesc;
    HIP_OK(hipMalloc((void **)&dsrc, src_bytes));
    HIP_OK(hipMalloc((void **)&dpool, pool_bytes));
    HIP_OK(hipMalloc((void **)&ddesc, NCOPY * sizeof(tb_copy_desc)));
    HIP_OK(hipMemcpy(dsrc, hsrc, src_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(dpool, 0xA5, pool_bytes));
    uint64_t so = 0;
    for (int k = 0; k < NCOPY; k++) {   /* copy k lands in its own 8 KiB slot, at a byte offset */
        const uint64_t bytes = 1 + rnd(&seed) % 4096, doff = (uint64_t)k * SLOT + rnd(&seed) % 64;
        desc[k].src = (uint64_t)(uintptr_t)(dsrc + so);
        desc[k].dst = (uint64_t)(uintptr_t)(dpool + doff);
        desc[k].bytes = bytes;
        memcpy(expect + doff, hsrc + so, bytes);
        so += bytes;
    }
    HIP_OK(hipMemcpy(ddesc, desc, NCOPY * sizeof(tb_copy_desc), hipMemcpyHostToDevice));
    TB_OK_(tb_batched_copy(ddesc, NCOPY, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(hpool, dpool, pool_bytes, hipMemcpyDeviceToHost));
    if (memcmp(hpool, expect, pool_bytes) != 0) {
        for (uint64_t i = 0; i < pool_bytes; i++)
            if (hpool[i] != expect[i]) {
                fprintf(stderr, "batched copy: pool byte %llu is %u, expected %u\n", (unsigned long long)i,
                        hpool[i], expect[i]);
                break;
            }
        return 1;
    }
    if (tb_batched_copy((const tb_copy_desc *)((char *)ddesc + 4), 1, s) != TB_ERR_INVALID) {
        fprintf(stderr, "batched copy accepted a misaligned descriptor array\n");
        return 1;
    }
    HIP_OK(hipFree(dsrc));
    HIP_OK(hipFree(dpool));
    HIP_OK(hipFree(ddesc));
    free(hsrc);
    free(hpool);
    free(expect);
    free(desc);
    return 0;
}

int main(void) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
        fprintf(stderr, "no GPU\n");
        return 2;
    }
    HIP_OK(hipSetDevice(0));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    if (check_reduce(s) != 0 || check_batch(s) != 0)
        return 1;
    HIP_OK(hipStreamDestroy(s));
    TB_OK_(tb_shutdown());
    printf("capi ok\n");
    return 0;
}
