// tb_internal.h -- declarations shared by the host half (tb_host.cpp) and the
// gfx950 kernels (tb_kernels.hip) of libtb.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tb.h"

namespace tbk {

// ---- reduce-copy -----------------------------------------------------------

// Workgroup size of the reduce-copy kernels (4 wave64s).
constexpr int kRcBlock = 256;
// Grid cap of the reduce-copy (a multiple of 8); below it every tile has its
// own workgroup.
constexpr uint64_t kRcMaxBlocks = 1u << 20;

struct ReduceArgs {
    float *dst;
    const float *src[TB_MAX_SRCS];
    uint64_t n;          // floats
    // Vector split (fast path only): `head` floats before the first 16-byte
    // aligned element of dst, then `nvec` float4s, then `tail` floats.
    uint64_t nvec;
    uint32_t head;
    uint32_t tail;
    uint32_t fill;       // 32-bit memset pattern for nsrc == 0
};

// Workgroups the reduce-copy kernel is launched with.
int reduce_grid(uint64_t nfloats, int nsrc, bool vector_path, int cu_count);

// Enqueue the reduce-copy for nsrc sources.  vector_path: every pointer shares
// dst's address modulo 16 (head/nvec/tail filled in by the caller).
hipError_t launch_reduce_copy(const ReduceArgs &args, int nsrc, bool vector_path,
                              int cu_count, hipStream_t stream);

// ---- batched copy ------------------------------------------------------------

constexpr int kBcBlock = 256;        // 4 wave64s per workgroup
constexpr int kBcBlocksPerCu = 8;    // persistent grid: 32 waves per CU; grid = CUs x 8
// Copies longer than this are split into kBcChunk pieces shared by all waves.
constexpr uint64_t kBcSplitAbove = 64 * 1024;
constexpr uint64_t kBcChunk = 32 * 1024;
// Capacity of the large-copy queue; copies beyond it run on their owner wave.
constexpr uint32_t kBcQueueCap = 16384;

struct BcSlot {
    uint32_t desc_plus1;   // 0 = not yet published
    uint32_t next_chunk;   // next unclaimed chunk
};

struct alignas(256) BcCounter {
    uint32_t count;
    uint32_t pad[63];
};

struct BcScratch {
    uint32_t qtail;        // slots handed out (may exceed kBcQueueCap)
    uint32_t done_all;     // XCD groups finished
    uint32_t pad[62];      // keep these counters on their own 256 bytes
    BcCounter done_xcd[8]; // workgroups finished, per XCD (blockIdx % 8)
    BcSlot slot[kBcQueueCap];
};

constexpr size_t kBcScratchBytes = sizeof(BcScratch);

int batched_grid(int cu_count);

// Enqueue the batched copy.  `scratch` must be kBcScratchBytes of device
// memory that was zeroed once; the kernel leaves it zeroed again.
hipError_t launch_batched_copy(const tb_copy_desc *desc, uint32_t n, BcScratch *scratch,
                               int cu_count, hipStream_t stream);

// ---- spin gate ---------------------------------------------------------------

// One thread waits until *flag != 0, or until timeout_ticks of the device
// wall clock have passed (then *timed_out = 1).  Both live in coherent host memory.
hipError_t launch_spin_gate(const uint32_t *flag, uint32_t *timed_out, uint64_t timeout_ticks,
                            hipStream_t stream);

}  // namespace tbk
