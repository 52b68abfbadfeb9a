/*
 * capi_check.c -- the library's C ABI (include/tb.h) used from plain C11:
 * device memory from the HIP runtime's C API, no Python, no torch.
 *
 * A consumer-side check of the boundary, not a parity test (those compare
 * against the oracle), calling every entry point of the header: slice
 * geometry, source preparation and rotation; a two-source reduce-copy and a
 * nine-source one with every source 4 bytes off dst, whose sums are exact in
 * binary32; a batched copy of 1,000 copies of 1 B - 4 KiB at arbitrary byte
 * offsets through tb_batched_copy (with and without a workgroup cap),
 * tb_batched_copy_noalloc and both kinds of descriptor-slot ring; the spin
 * gate, the launch-carried timing events, the launch figures, the memset
 * form, the recovery-mode hook, the status strings and the argument checks.
 * Prints "capi ok" and exits 0 on success.
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

/* nsrc sources of n floats, source k at byte offset src_off (multiple of 4)
 * from an allocation, dst one float past one: values are multiples of 1/4
 * below 2^10, so every sum of up to 16 is exact in binary32 and equals the
 * double-precision sum. */
static int check_reduce_n(hipStream_t s, int nsrc, uint64_t n, uint32_t src_off) {
    float *h[TB_MAX_SRCS];
    float *d[TB_MAX_SRCS];
    const float *srcs[TB_MAX_SRCS];
    float *out = malloc(n * sizeof(float));
    if (!out)
        return 1;
    for (int k = 0; k < nsrc; k++) {
        h[k] = malloc(n * sizeof(float));
        if (!h[k])
            return 1;
        for (uint64_t i = 0; i < n; i++)
            h[k][i] = (float)((i * (uint64_t)(k + 3) + (uint64_t)k) % 4093) * 0.25f;
        HIP_OK(hipMalloc((void **)&d[k], n * sizeof(float) + 16));
        HIP_OK(hipMemcpy((char *)d[k] + src_off, h[k], n * sizeof(float), hipMemcpyHostToDevice));
        srcs[k] = (const float *)((const char *)d[k] + src_off);
    }
    float *dd;
    HIP_OK(hipMalloc((void **)&dd, n * sizeof(float) + 4));
    TB_OK_(tb_reduce_copy(dd + 1, srcs, nsrc, n, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(out, dd + 1, n * sizeof(float), hipMemcpyDeviceToHost));
    for (uint64_t i = 0; i < n; i++) {
        double want = 0.0;
        for (int k = 0; k < nsrc; k++)
            want += (double)h[k][i];
        if ((double)out[i] != want) {
            fprintf(stderr, "reduce-copy (%d sources, offset %u): element %llu is %g, expected %g\n", nsrc, src_off,
                    (unsigned long long)i, out[i], want);
            return 1;
        }
    }
    for (int k = 0; k < nsrc; k++) {
        HIP_OK(hipFree(d[k]));
        free(h[k]);
    }
    HIP_OK(hipFree(dd));
    free(out);
    return 0;
}

static int check_reduce(hipStream_t s) {
    if (check_reduce_n(s, 2, (1u << 20) + 3, 0) != 0)   /* the vector path, with a head and a tail */
        return 1;
    if (check_reduce_n(s, 9, 300001, 4) != 0)           /* sources off dst's alignment: staged through LDS */
        return 1;
    /* argument checks: too many sources, a misaligned pointer */
    float *dd;
    HIP_OK(hipMalloc((void **)&dd, 4096));
    const float *srcs[2] = {dd, dd};
    if (tb_reduce_copy(dd, srcs, TB_MAX_SRCS + 1, 16, s) != TB_ERR_INVALID ||
        tb_reduce_copy((float *)((char *)dd + 2), srcs, 2, 16, s) != TB_ERR_INVALID) {
        fprintf(stderr, "reduce-copy accepted invalid arguments\n");
        return 1;
    }
    HIP_OK(hipFree(dd));
    return 0;
}

/* Slice geometry, source preparation and rotation: K slices of a prepared
 * source each hold the host reference, and the rotated pointer of iteration
 * i (warmups negative) is slice ((i mod K) + K) mod K, which a one-source
 * reduce-copy (a bitwise copy) then reads. */
static int check_rotation(hipStream_t s) {
    uint64_t k = 0, stride = 0;
    TB_OK_(tb_num_slices(4u << 20, 256u << 20, &k));
    TB_OK_(tb_slice_stride(4u << 20, &stride));
    if (k != 64 || stride != (4u << 20)) {
        fprintf(stderr, "slice geometry: K %llu stride %llu\n", (unsigned long long)k, (unsigned long long)stride);
        return 1;
    }
    const uint64_t n = 100003;   /* 400,012 bytes: stride rounds up to 400,128 */
    TB_OK_(tb_num_slices(n * 4, 1600000, &k));
    TB_OK_(tb_slice_stride(n * 4, &stride));
    if (k != 4 || stride != 400128) {
        fprintf(stderr, "slice geometry: K %llu stride %llu\n", (unsigned long long)k, (unsigned long long)stride);
        return 1;
    }
    float *ref = malloc(n * sizeof(float)), *back = malloc(n * sizeof(float));
    if (!ref || !back)
        return 1;
    tb_fill_cfg cfg;
    memset(&cfg, 0, sizeof(cfg));
    cfg.kind = TB_FILL_DEFAULT;
    TB_OK_(tb_prep_reference(ref, n, 1, &cfg));
    float *base, *dst;
    HIP_OK(hipMalloc((void **)&base, k * stride));
    HIP_OK(hipMalloc((void **)&dst, n * sizeof(float)));
    TB_OK_(tb_prep_sources(base, stride, k, ref, n, s));
    HIP_OK(hipStreamSynchronize(s));
    for (uint64_t sl = 0; sl < k; sl++) {
        HIP_OK(hipMemcpy(back, (char *)base + sl * stride, n * sizeof(float), hipMemcpyDeviceToHost));
        if (memcmp(back, ref, n * sizeof(float)) != 0) {
            fprintf(stderr, "slice %llu differs from the host reference\n", (unsigned long long)sl);
            return 1;
        }
    }
    const float *b0[1] = {base};
    for (int64_t it = -3; it < 6; it++) {
        const float *rot[1];
        TB_OK_(tb_rotate_sources(b0, 1, stride, k, it, rot));
        const uint64_t want = (uint64_t)(((it % (int64_t)k) + (int64_t)k) % (int64_t)k);
        if ((const char *)rot[0] != (const char *)base + want * stride) {
            fprintf(stderr, "iteration %lld rotated to the wrong slice\n", (long long)it);
            return 1;
        }
        HIP_OK(hipMemset(dst, 0, n * sizeof(float)));
        TB_OK_(tb_reduce_copy(dst, rot, 1, n, s));
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(back, dst, n * sizeof(float), hipMemcpyDeviceToHost));
        if (memcmp(back, ref, n * sizeof(float)) != 0) {
            fprintf(stderr, "copy of iteration %lld differs\n", (long long)it);
            return 1;
        }
    }
    HIP_OK(hipFree(base));
    HIP_OK(hipFree(dst));
    free(ref);
    free(back);
    return 0;
}

/* The memset form (N = 0 with an explicit byte), the recovery-mode hook and
 * the status strings. */
static int check_misc(hipStream_t s) {
    const uint64_t n = 4099;
    uint8_t *d, *h = malloc(n * 4);
    if (!h)
        return 1;
    HIP_OK(hipMalloc((void **)&d, n * 4 + 8));
    HIP_OK(hipMemset(d, 0x11, n * 4 + 8));
    TB_OK_(tb_reduce_copy_ex((float *)(d + 4), NULL, 0, n, 0x5Au, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(h, d + 4, n * 4, hipMemcpyDeviceToHost));
    for (uint64_t i = 0; i < n * 4; i++)
        if (h[i] != 0x5A) {
            fprintf(stderr, "memset: byte %llu is %u\n", (unsigned long long)i, h[i]);
            return 1;
        }
    if (tb_reduce_copy_ex((float *)d, NULL, 0, 16, 256u, s) != TB_ERR_INVALID ||
        tb_batched_set_mode(7) != TB_ERR_INVALID) {
        fprintf(stderr, "accepted an invalid memset byte or mode\n");
        return 1;
    }
    TB_OK_(tb_batched_set_mode(TB_BC_NO_WAIT));
    TB_OK_(tb_batched_set_mode(TB_BC_NORMAL));
    if (tb_status_string(TB_ERR_TIMEOUT)[0] == '\0' || tb_last_hip_error() == NULL) {
        fprintf(stderr, "empty status string\n");
        return 1;
    }
    HIP_OK(hipFree(d));
    free(h);
    return 0;
}

/* The spin gate, launch-carried events and launch figures. */
static int check_gate_and_timing(hipStream_t s) {
    float *a, *b;
    const uint64_t n = 1u << 22;
    HIP_OK(hipMalloc((void **)&a, n * sizeof(float)));
    HIP_OK(hipMalloc((void **)&b, n * sizeof(float)));
    HIP_OK(hipMemset(a, 0, n * sizeof(float)));
    hipEvent_t e0, e1;
    HIP_OK(hipEventCreate(&e0));
    HIP_OK(hipEventCreate(&e1));
    TB_OK_(tb_spin_gate_arm(10000, s));
    TB_OK_(tb_time_next_launch(e0, e1));
    const float *srcs[1] = {a};
    TB_OK_(tb_reduce_copy(b, srcs, 1, n, s));
    if (hipEventQuery(e1) != hipErrorNotReady) {   /* held behind the gate */
        fprintf(stderr, "the launch ran before the gate was released\n");
        return 1;
    }
    TB_OK_(tb_spin_gate_release());
    HIP_OK(hipStreamSynchronize(s));
    if (tb_spin_gate_status() != TB_OK) {
        fprintf(stderr, "spin gate timed out\n");
        return 1;
    }
    float ms = 0.f;
    HIP_OK(hipEventElapsedTime(&ms, e0, e1));
    if (!(ms > 0.f)) {
        fprintf(stderr, "launch-carried events gave %g ms\n", ms);
        return 1;
    }
    int32_t cus = 0, rb = 0, bb = 0;
    TB_OK_(tb_launch_info(n, 1, 47520, &cus, &rb, &bb));
    if (cus <= 0 || rb <= 0 || bb <= 0) {
        fprintf(stderr, "launch info %d %d %d\n", cus, rb, bb);
        return 1;
    }
    HIP_OK(hipEventDestroy(e0));
    HIP_OK(hipEventDestroy(e1));
    HIP_OK(hipFree(a));
    HIP_OK(hipFree(b));
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
    /* path 0: tb_batched_copy; 1: the same capped at 64 workgroups; 2: tb_batched_copy_noalloc;
     * 3 / 4: a staged / direct descriptor-slot ring fed the host descriptors in requests of 100 */
    for (int path = 0; path < 5; path++) {
        HIP_OK(hipMemset(dpool, 0xA5, pool_bytes));
        if (path == 0) {
            TB_OK_(tb_batched_copy(ddesc, NCOPY, s));
        } else if (path == 1) {
            TB_OK_(tb_batched_set_max_workgroups(64));
            TB_OK_(tb_batched_copy(ddesc, NCOPY, s));
            TB_OK_(tb_batched_set_max_workgroups(0));
        } else if (path == 2) {
            TB_OK_(tb_batched_copy_noalloc(ddesc, NCOPY, s));
        } else {
            tb_ring *ring = NULL;
            TB_OK_(tb_ring_create(4, 256, path == 3 ? TB_RING_STAGED : TB_RING_DIRECT, s, &ring));
            uint64_t ticket = 0;
            for (int k0 = 0; k0 < NCOPY; k0 += 100)
                TB_OK_(tb_ring_submit(ring, desc + k0, 100, &ticket));
            TB_OK_(tb_ring_wait(ring, ticket));
            int32_t done = 0;
            TB_OK_(tb_ring_poll(ring, ticket, &done));
            if (!done) {
                fprintf(stderr, "ring: ticket %llu not done after its wait\n", (unsigned long long)ticket);
                return 1;
            }
            TB_OK_(tb_ring_destroy(ring));
        }
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(hpool, dpool, pool_bytes, hipMemcpyDeviceToHost));
        if (memcmp(hpool, expect, pool_bytes) != 0) {
            for (uint64_t i = 0; i < pool_bytes; i++)
                if (hpool[i] != expect[i]) {
                    fprintf(stderr, "batched copy (path %d): pool byte %llu is %u, expected %u\n", path,
                            (unsigned long long)i, hpool[i], expect[i]);
                    break;
                }
            return 1;
        }
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
    if (check_reduce(s) != 0 || check_rotation(s) != 0 || check_misc(s) != 0 || check_gate_and_timing(s) != 0 ||
        check_batch(s) != 0)
        return 1;
    HIP_OK(hipStreamDestroy(s));
    TB_OK_(tb_shutdown());
    printf("capi ok\n");
    return 0;
}
