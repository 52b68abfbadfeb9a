// Exercises libtb's host-only entry points (slice geometry, rotation, the
// PrepareReference generators, status strings) and the argument checks of
// the GPU entry points and of the descriptor-slot ring, which return before
// any HIP call, in a build with
// AddressSanitizer and UndefinedBehaviorSanitizer.  Needs no GPU.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "tb.h"

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main() {
    uint64_t k = 0, stride = 0;
    CHECK(tb_num_slices(4u << 20, 256u << 20, &k) == TB_OK && k == 64);
    CHECK(tb_num_slices(1, UINT64_MAX, &k) == TB_OK && k == UINT64_MAX);
    CHECK(tb_num_slices(0, 0, nullptr) == TB_ERR_INVALID);
    CHECK(tb_slice_stride(UINT64_MAX, &stride) == TB_ERR_INVALID);
    CHECK(tb_slice_stride(UINT64_MAX - 255, &stride) == TB_OK);

    const float *base[TB_MAX_SRCS], *out[TB_MAX_SRCS];
    for (int b = 0; b < TB_MAX_SRCS; b++)
        base[b] = reinterpret_cast<const float *>(uintptr_t(0x100000) * (b + 1));
    for (int64_t it : {INT64_MIN, (int64_t)-3, (int64_t)0, (int64_t)5, INT64_MAX})
        CHECK(tb_rotate_sources(base, TB_MAX_SRCS, 4096, 64, it, out) == TB_OK);
    CHECK(tb_rotate_sources(base, TB_MAX_SRCS, UINT64_MAX, 64, 5, out) == TB_ERR_INVALID);
    CHECK(tb_rotate_sources(base, TB_MAX_SRCS + 1, 4096, 64, 5, out) == TB_ERR_INVALID);

    const uint32_t pct[5] = {50, 20, 10, 10, 10}, bad[5] = {50, 50, 50, 0, 0};
    const float pattern[3] = {1.0f, -0.0f, 2.5f};
    for (uint64_t n : {0ull, 1ull, 15ull, 16ull, 17ull, 383ull, 1025ull, 4099ull}) {
        std::vector<float> v(n + 1);
        tb_fill_cfg c;
        memset(&c, 0, sizeof c);
        CHECK(tb_prep_reference(v.data(), n, 0, nullptr) == TB_OK);
        CHECK(tb_prep_reference(v.data(), n, 15, nullptr) == TB_OK);
        c.kind = TB_FILL_PATTERN;
        c.pattern = pattern;
        c.pattern_len = 3;
        CHECK(tb_prep_reference(v.data(), n, 1, &c) == TB_OK);
        c.kind = TB_FILL_COMPRESS;
        memcpy(c.compress_pct, pct, sizeof pct);
        c.seed = 3;
        CHECK(tb_prep_reference(v.data(), n, 2, &c) == TB_OK);
        memcpy(c.compress_pct, bad, sizeof bad);
        CHECK(tb_prep_reference(v.data(), n, 2, &c) == TB_ERR_INVALID);
    }
    for (int s = -6; s <= 2; s++)
        CHECK(tb_status_string(s) != nullptr);

    // argument checks that return before touching HIP
    const float *srcs[17] = {};
    CHECK(tb_reduce_copy(nullptr, srcs, 17, 16, nullptr) == TB_ERR_INVALID);
    CHECK(tb_reduce_copy(reinterpret_cast<float *>(0x1002), srcs, 1, 16, nullptr) == TB_ERR_INVALID);
    CHECK(tb_reduce_copy_ex(reinterpret_cast<float *>(0x1000), srcs, 0, 16, 256, nullptr) == TB_ERR_INVALID);
    CHECK(tb_reduce_copy(nullptr, nullptr, 3, 0, nullptr) == TB_OK);
    CHECK(tb_batched_copy(nullptr, 5, nullptr) == TB_ERR_INVALID);
    CHECK(tb_batched_copy(nullptr, 0, nullptr) == TB_OK);
    tb_ring *ring = nullptr;
    CHECK(tb_ring_create(0, 8, TB_RING_STAGED, nullptr, &ring) == TB_ERR_INVALID && ring == nullptr);
    CHECK(tb_ring_create(2, 0, TB_RING_DIRECT, nullptr, &ring) == TB_ERR_INVALID);
    CHECK(tb_ring_create(1025, 8, TB_RING_STAGED, nullptr, &ring) == TB_ERR_INVALID);
    CHECK(tb_ring_create(2, (1u << 20) + 1, TB_RING_STAGED, nullptr, &ring) == TB_ERR_INVALID);
    CHECK(tb_ring_create(2, 8, 7, nullptr, &ring) == TB_ERR_INVALID);
    CHECK(tb_ring_create(2, 8, TB_RING_STAGED, nullptr, nullptr) == TB_ERR_INVALID);
    uint64_t ticket = 0;
    int32_t done = 0;
    CHECK(tb_ring_submit(nullptr, nullptr, 0, &ticket) == TB_ERR_INVALID);
    CHECK(tb_ring_poll(nullptr, 0, &done) == TB_ERR_INVALID);
    CHECK(tb_ring_wait(nullptr, 0) == TB_ERR_INVALID);
    CHECK(tb_ring_destroy(nullptr) == TB_OK);
    CHECK(tb_time_next_launch(nullptr, nullptr) == TB_OK);
    CHECK(tb_batched_set_mode(7) == TB_ERR_INVALID && tb_batched_set_mode(TB_BC_NORMAL) == TB_OK);
    CHECK(tb_prep_sources(nullptr, 64, 0, nullptr, 16, nullptr) == TB_ERR_INVALID);
    CHECK(tb_spin_gate_arm(0, nullptr) == TB_ERR_INVALID);
    CHECK(tb_spin_gate_release() == TB_ERR_INVALID);
    puts("host sanitizer run ok");
    return 0;
}
