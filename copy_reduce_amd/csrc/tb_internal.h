// tb_internal.h -- declarations shared by the host half (tb_host.cpp) and the
// gfx950 kernels (tb_kernels.hip) of libtb.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tb.h"

namespace tbk {

// ---- reduce-copy -----------------------------------------------------------

// Workgroup size of the reduce-copy's memset (N = 0): 4 wave64s, one 4 KiB
// tile.  The summing kernels size their workgroups by source count.
constexpr int kRcBlock = 256;
// Grid cap of the reduce-copy (a multiple of 64, so a workgroup's XCD and its
// place in a group of 64 stay fixed across the grid-stride loop); below it
// every tile has its own workgroup.
constexpr uint64_t kRcMaxBlocks = 1u << 20;

struct ReduceArgs {
    float *dst;
    const float *src[TB_MAX_SRCS];
    uint64_t n;          // floats
    // Vector split: `head` floats before the first 16-byte aligned element of
    // dst, then `nvec` float4s, then `tail` floats.
    uint64_t nvec;
    uint32_t head;
    uint32_t tail;
    uint32_t fill;       // 32-bit memset pattern for nsrc == 0
};

// Workgroups the reduce-copy kernel is launched with.
int reduce_grid(uint64_t nfloats, int nsrc, bool vector_path, int cu_count);

// Enqueue the reduce-copy for nsrc sources (head/nvec/tail filled in by the
// caller).  vector_path: every source agrees with dst modulo 16; otherwise the
// unaligned kernel runs.
hipError_t launch_reduce_copy(const ReduceArgs &args, int nsrc, bool vector_path,
                              int cu_count, hipStream_t stream);

// ---- batched copy ------------------------------------------------------------

constexpr int kBcBlock = 256;        // 4 wave64s per workgroup
// Occupancy: 7 workgroups (28 waves) per CU is what the kernel reaches at
// 72 VGPRs without spilling; that many waves (the last ones of the grid) share the
// pieces of long copies.
constexpr int kBcBlocksPerCu = 7;
constexpr uint32_t kBcResidentWavesPerCu = kBcBlocksPerCu * (kBcBlock / 64);
// Launched grid: about kBcDescPerWave descriptors per wave, between the
// resident count (kBcBlocksPerCu per CU) and kBcMaxGridPerCu per CU.  More
// workgroups than resident let the dispatcher hand finished CUs new work:
// waves own random-size copies and a workgroup's slot is held until its
// slowest wave is done, so smaller units balance better.  Measured on the
// 47,520-copy batch: 3, 2, 1.5 and 1 descriptors per wave gave 53%, 55%,
// 56% and 57% of HBM peak.  No workgroup waits for another at the end, so
// workgroups past the resident ones cost little.
constexpr int kBcMaxGridPerCu = 64;
constexpr uint32_t kBcDescPerWave = 1;
// Copies longer than this are published in a queue and split into kBcChunk
// pieces dealt over all waves; shorter ones are copied whole by their owner.
constexpr uint64_t kBcSplitAbove = 64 * 1024;
constexpr uint64_t kBcChunk = 8 * 1024;
// Capacity of the long-copy queue; copies beyond it are copied by the
// scanning wave that found them.
constexpr uint32_t kBcQueueCap = 16384;
// Descriptors scanned per scanner workgroup (the first workgroups of the grid).
constexpr uint32_t kBcScanPerBlock = 1024;
// Longest wait for the queue to be sealed, in microseconds of device time.
constexpr uint32_t kBcSealWaitUs = 200;

struct alignas(256) BcWord {
    uint64_t word;
    uint64_t pad[31];
};

// Batched-copy scratch.  Nothing in it is ever cleared after a launch:
//  - launch e uses scan[e & 1] and clears scan[(e + 1) & 1] for launch e + 1
//    (launches on one scratch are ordered by their stream);
//  - a slot carries the epoch e of the launch that wrote it, so a reader tells
//    a stale slot from a current one;
//  - redo holds the epoch of the last launch in which a wave took on the
//    recovery copy.
struct BcScratch {
    BcWord scan[2];         // low 32 bits: queue slots handed out (may exceed
                            // kBcQueueCap); high 32 bits: scanners finished
    BcWord redo;
    uint64_t slot[kBcQueueCap];  // (low 32 bits of epoch << 32) | (descriptor index + 1)
};

constexpr size_t kBcScratchBytes = sizeof(BcScratch);

int batched_grid(uint32_t ncopies, int cu_count);
// Cap every later batched-copy launch at max_wgs workgroups (0: no cap).
void set_batched_max_workgroups(uint32_t max_wgs);
uint32_t batched_scanners(uint32_t ncopies, int grid);

// Enqueue the batched copy.  `scratch` must be kBcScratchBytes of device
// memory that was zeroed once; `epoch` numbers the launches made on it, from
// 1, one more for each launch (their stream orders them).
// wait_ticks: the longest wait for the queue, in ticks of the device wall
// clock (normally kBcSealWaitUs).  no_pieces: no wave takes queue pieces, so
// the recovery copy runs (for tests).  done_event, if not null, fires when the
// kernel completes (it is the launch's stop event, not a separate command).
hipError_t launch_batched_copy(const tb_copy_desc *desc, uint32_t n, BcScratch *scratch, uint64_t epoch,
                               int cu_count, uint64_t wait_ticks, bool no_pieces, hipStream_t stream,
                               hipEvent_t done_event = nullptr);

// As launch_batched_copy, for a batch the caller has checked holds no copy
// longer than kBcSplitAbove: the queue is skipped (no scanner workgroups, no
// piece waves, no wait) and the grid has one descriptor per wave with no
// floor.  The launch still clears the scan word of the next epoch, so any
// launch may follow it on the same scratch.
hipError_t launch_batched_copy_short(const tb_copy_desc *desc, uint32_t n, BcScratch *scratch, uint64_t epoch,
                                     int cu_count, hipStream_t stream, hipEvent_t done_event = nullptr);

// Devices the library keeps per-device state for (ordinals 0 .. kMaxDevices-1).
constexpr int kMaxDevices = 64;

// As launch_batched_copy, on the static per-device scratch of
// tb_batched_copy_noalloc instead of caller-given memory: no allocation.  The
// first call on a device (which must be current) takes the scratch's device
// address and clears it, synchronising `stream` once; epochs are numbered per
// device under a lock.  Returns the first failing HIP status.
hipError_t launch_batched_copy_static(const tb_copy_desc *desc, uint32_t n, int device, int cu_count,
                                      uint64_t wait_ticks, bool no_pieces, hipStream_t stream);

// ---- launch events -------------------------------------------------------------

// The next kernel launched by the calling host thread records `start` when it
// begins and `stop` when it completes, as part of the launch (either may be
// null).  Consumed by that launch.
void set_next_launch_events(hipEvent_t start, hipEvent_t stop);

// ---- spin gate ---------------------------------------------------------------

// One thread waits until *flag != 0, or until timeout_ticks of the device
// wall clock have passed (then *timed_out = 1).  Both live in coherent host memory.
hipError_t launch_spin_gate(const uint32_t *flag, uint32_t *timed_out, uint64_t timeout_ticks,
                            hipStream_t stream);

}  // namespace tbk

// ---- host helpers shared by the host sources (tb_host.cpp defines them) -------

namespace tbh {

// Record `what` and e's text for tb_last_hip_error(); returns TB_ERR_HIP.
int hip_fail(hipError_t e, const char *what);

// The TB_BC_* mode last set by tb_batched_set_mode.
int batched_mode();

// True while `s` is being captured into a HIP graph.  The batched copy's
// launches carry their epoch as a kernel argument, so a replayed capture would
// reuse one epoch on the scratch: such calls are refused instead.
bool capturing(hipStream_t s);

}  // namespace tbh
