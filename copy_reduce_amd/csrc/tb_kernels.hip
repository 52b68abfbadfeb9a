// tb_kernels.hip -- gfx950 kernels of libtb: reduce-copy, batched copy, spin gate.
//
// Written for CDNA4: wave64, 256 CUs in 8 XCDs, HBM3E.  Nothing here is a
// contraction, so there is no MFMA; both copies are HBM-bound streams and the
// design is about keeping enough 16-byte loads in flight per CU.
#include <atomic>
#include <mutex>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tb_internal.h"

namespace tbk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ============================================================================
// Reduce-copy
// ("TransferBench data validation": expected-value table; dstReference[k] =
//  dstReference[k-1] + srcReference[k-1], so the sum starts from source 0 and
//  adds the others one at a time, left to right.)
// ============================================================================

// Global-address-space views: loads and stores become global_* instructions
// (generic pointers would give flat_* ones, which the compiler serialises).
typedef __attribute__((address_space(1))) f32x4 gf32x4;
typedef __attribute__((address_space(1))) float gf32;
typedef __attribute__((address_space(1))) u32x4 gu32x4;
typedef __attribute__((address_space(1))) uint32_t gu32;
typedef __attribute__((address_space(1))) uint8_t gu8;
typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void svoid;

// Cache-policy bits of gfx950 buffer instructions (the aux operand): nt marks
// the line for early eviction (streaming); sc0 / sc1 set the coherence scope
// (sc1 = device, sc0 | sc1 = system), which makes a store write through the
// per-XCD L2 instead of sitting there dirty until the end of the kernel.
constexpr int kPolNt = 2;
constexpr int kPolSc0 = 1;
constexpr int kPolSc1 = 16;

// Raw buffer resource over [base, base + bytes): accesses outside the range
// read as zero and are not written (the hardware checks every access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(uint64_t base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Tile shape of the reduce-copy, by number of sources: one float4 per thread
// and source, one tile per workgroup, tiles dealt in address order (workgroup
// b takes tile b), so at any moment the whole chip works on one compact
// window of each buffer.  Workgroups are one wave for up to two sources (a
// 1 KiB tile per buffer) and two waves from three up (2 KiB).  Measured on
// MI355X with every launch writing a destination no recent launch wrote
// (rotated over 1 GiB), 3 warmups + 10 launches, 2-4 runs: a 512 MiB copy
// 85-86% of HBM peak against 83% with four-wave workgroups whose tiles each
// XCD walked in its own contiguous eighth; two sources of 256 MiB 84-85%
// against 82%; three sources 77% against 74% (four-wave tiles of two float4
// per thread); four to sixteen sources within a point of one-wave tiles of
// two float4 per thread.  Larger tiles per wave were slower at every source
// count: two, four, eight and sixteen float4 per thread cost a copy 5-10
// points, and keeping only two or three sources' loads in flight at once
// (a rolling order) changed eight and sixteen sources by under a point.
constexpr int rc_block_of(int nsrc) { return nsrc <= 2 ? 64 : 128; }
// How the vector path reads a tile: through one buffer resource per source on
// the tile's scalar base (the thread's byte offset the only vector operand),
// or with global loads of 64-bit per-thread addresses.  Measured on MI355X
// (64 MiB per source, 3 runs each): buffer loads are 0.6-4 points faster
// from two to eight sources (three: 78% against 75%, four: 80% against 76%)
// and 0.3-1.3 points slower for one, twelve and sixteen.
constexpr bool rc_buffer_loads(int nsrc) { return nsrc >= 2 && nsrc <= 8; }
// Workgroup size of the unaligned path (some source off dst's 16-byte
// alignment): two waves, one float4 per thread and source, whatever the
// source count.  Measured with sources 4 or 8 bytes off: 81% for a 512 MiB
// copy and two sources of 256 MiB against 79% and 76% with one-wave
// workgroups.
constexpr int kRcUnalignedBlock = 128;
// From eight sources up the unaligned path stages every source's aligned
// 16-byte blocks in LDS and reads each thread's four floats back at the
// source's own 4-byte offset (rc_unaligned_lds_kernel): one-wave workgroups,
// all eight sources staged at once at N = 8, four at a time above.
constexpr bool rc_unaligned_lds(int nsrc) { return nsrc >= 8; }
constexpr int kRcLdsBlock = 64;
constexpr int rc_lds_group(int nsrc) { return nsrc <= 8 ? nsrc : 4; }

// Sources are streamed once per launch: nontemporal loads (without them, or
// with device-scope loads, two sources of 256 MiB ran at 77% instead of 85%).
// Results are written with nontemporal stores, which do not allocate in the
// 256 MB memory-side cache (MALL): the kernel's rate is then the same whether
// or not the destination was written recently.  Device-scope stores (sc1)
// allocate there, and a fixed destination rewritten launch after launch (the
// pages' timing) then reads 92-93% for two sources of 256 MiB, against 81-82%
// once the destination rotates over 1 GiB, where nontemporal stores reach
// 84-85% under either timing.  Stores that allocate in the MALL also leave
// dirty lines that a following kernel pays for: behind such batched-copy
// stores the next 256 MiB reduce-copy fell from 81% to 67%.  Up to two
// sources the stores also carry system scope (nt sc0 sc1: written through the
// per-XCD L2): a 512 MiB copy 84.3% against 82.8% with nt alone, and the
// bench's two-source step 85.1% against 84.5%.  From three sources up nt
// alone is faster: four sources of 64 MiB 82-83% against 79-81%, the same
// with a rotated destination (no cache help either way).
constexpr int rc_store_pol(int nsrc) { return nsrc <= 2 ? (kPolNt | kPolSc0 | kPolSc1) : kPolNt; }
__device__ __forceinline__ f32x4 rc_load(const gf32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float rc_load(const gf32 *p) { return __builtin_nontemporal_load(p); }

// Fixed-order scalar sum of element j (used for the unaligned head and tail).
template <int N>
__device__ __forceinline__ float rc_sum_scalar(const ReduceArgs &a, uint64_t j) {
    float acc = rc_load((const gf32 *)(a.src[0]) + j);
#pragma unroll
    for (int k = 1; k < N; k++)
        acc = acc + rc_load((const gf32 *)(a.src[k]) + j);
    return acc;
}

// Vector path: every pointer is congruent to dst modulo 16.  Tile t is the
// BS float4s t * BS .. t * BS + BS - 1 of every buffer, one per thread; each
// thread loads its float4 from every source before the first addition, so N
// 16-byte loads per thread are in flight.
template <int N>
__global__ __launch_bounds__(rc_block_of(N)) void rc_vec_kernel(ReduceArgs a) {
    constexpr int BS = rc_block_of(N);
    const uint64_t nvec = a.nvec;
    const uint64_t ntiles = (nvec + BS - 1) / BS;
    const gf32x4 *src[N];
#pragma unroll
    for (int k = 0; k < N; k++)
        src[k] = (const gf32x4 *)(a.src[k] + a.head);

    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t base = t * BS;
        // dst blocks in this tile: BS, or fewer in the last, partial tile,
        // where threads past nvec do nothing (a wave-uniform branch)
        const uint32_t nblk = (uint32_t)(nvec - base < (uint64_t)BS ? nvec - base : (uint64_t)BS);
        if (threadIdx.x < nblk) {
            f32x4 val[N];
#pragma unroll
            for (int k = 0; k < N; k++) {
                if constexpr (rc_buffer_loads(N))
                    val[k] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   buffer_over(reinterpret_cast<uint64_t>(src[k]) + base * 16, nblk * 16u),
                                   threadIdx.x * 16, 0, kPolNt));
                else
                    val[k] = rc_load(src[k] + base + threadIdx.x);
            }
            f32x4 acc = val[0];
#pragma unroll
            for (int k = 1; k < N; k++)
                acc = acc + val[k];
            const __amdgpu_buffer_rsrc_t out =
                buffer_over(reinterpret_cast<uint64_t>(a.dst + a.head) + base * 16, nblk * 16u);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), out, threadIdx.x * 16, 0,
                                                   rc_store_pol(N));
        }
    }

    // Up to 3 floats before the aligned body (threads 0-2) and 3 after it
    // (threads 32-34): every block size here has at least 64 threads.
    static_assert(BS >= 64, "head and tail threads");
    if (blockIdx.x == 0) {
        gf32 *d = (gf32 *)(a.dst);
        if (threadIdx.x < a.head) {
            const uint64_t j = threadIdx.x;
            d[j] = rc_sum_scalar<N>(a, j);
        } else if (threadIdx.x >= 32 && threadIdx.x < 32 + a.tail) {
            const uint64_t j = a.head + 4 * nvec + (threadIdx.x - 32);
            d[j] = rc_sum_scalar<N>(a, j);
        }
    }
}

// Lane i's copy of lane i + 1's x (DPP wave shift left by one lane); lane 63
// gets `last`.
__device__ __forceinline__ u32x4 shl1_lane(u32x4 x, u32x4 last) {
    constexpr int kWaveShl1 = 0x130;
    u32x4 y;
    y.x = (uint32_t)__builtin_amdgcn_update_dpp((int)last.x, (int)x.x, kWaveShl1, 0xF, 0xF, false);
    y.y = (uint32_t)__builtin_amdgcn_update_dpp((int)last.y, (int)x.y, kWaveShl1, 0xF, 0xF, false);
    y.z = (uint32_t)__builtin_amdgcn_update_dpp((int)last.z, (int)x.z, kWaveShl1, 0xF, 0xF, false);
    y.w = (uint32_t)__builtin_amdgcn_update_dpp((int)last.w, (int)x.w, kWaveShl1, 0xF, 0xF, false);
    return y;
}

// Lane i's copy of lane i + 1's x, and lane 63's of lane 0's (DPP wave
// rotate left by one lane).
__device__ __forceinline__ u32x4 rol1_lane(u32x4 x) {
    constexpr int kWaveRol1 = 0x134;
    u32x4 y;
    y.x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.x, kWaveRol1, 0xF, 0xF, false);
    y.y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.y, kWaveRol1, 0xF, 0xF, false);
    y.z = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.z, kWaveRol1, 0xF, 0xF, false);
    y.w = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.w, kWaveRol1, 0xF, 0xF, false);
    return y;
}

// A float4 at 4-byte alignment: loads through it are single 16-byte loads at
// any 4-byte-aligned address (gfx950 supports unaligned global accesses; the
// memory system splits a lane's access where it crosses a cache line).
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef __attribute__((address_space(1))) f32x4u gf32x4u;

// Unaligned path up to seven sources: every pointer is 4-byte aligned and
// some source disagrees with dst modulo 16.  dst is cut as on the vector path (head floats, float4
// body, tail floats); the thread that writes dst body block i reads, from
// every source, the 16 bytes holding that source's four elements for it, with
// one 16-byte load at the elements' own (4-byte) alignment.  Every load reads
// only the source's own elements, so nothing outside the source is touched.
// Measured at 256 MiB per buffer against an earlier form that loaded aligned
// 16-byte blocks and realigned them in registers (DPP lane shifts; two
// 64-block sub-tiles per wave): one source 81% against 78%, two 81% against
// 76%, and 2-4 points more from four to sixteen sources.
//
// Tiles are dealt in blocks of eight per XCD: workgroup b runs on XCD b mod 8,
// and within every 64 consecutive workgroups XCD x takes the eight
// consecutive tiles 8x .. 8x + 7, so the 128-byte line that straddles two
// tiles of a source is mostly read by one XCD's L2 while the chip still works
// on one compact window.  In plain order neighbouring tiles run on different
// XCDs and both fetch that line from HBM: with four to sixteen sources 4
// bytes off dst, 6.6-7.7% more bytes read than the sources hold (one or two
// sources, dealt: 0.8-0.9%).  Measured at 256 MiB per buffer, sources 4 or 8
// bytes off dst: four sources 78.7-79.4% of HBM peak against 75.9-76.3% in
// plain order, eight 72.5-72.8% against 71.2-71.7%, sixteen 69.9-70.5%
// against 69.5-70.0%; two sources 83% against 81%.  Blocks of sixteen tiles
// per XCD gained nothing more.  (On the vector path, with buffers on line
// boundaries so that no tiles share a line, the same deal cost 2-5 points.)
//
// Tile of workgroup b under that deal: a bijection on [0, ntiles) that
// permutes each complete group of 64 and leaves the last, partial group in
// order (gridDim.x is the whole grid or the cap, a multiple of 64, so b mod 8
// stays the XCD across the grid-stride loop).
__device__ __forceinline__ uint64_t xcd_block_tile(uint64_t b, uint64_t ntiles) {
    if ((b | 63u) >= ntiles)
        return b;
    return (b & ~(uint64_t)63) + (b & 7) * 8 + ((b >> 3) & 7);
}

template <int N>
__global__ __launch_bounds__(kRcUnalignedBlock) void rc_unaligned_kernel(ReduceArgs a) {
    constexpr int BS = kRcUnalignedBlock;
    const uint64_t nvec = a.nvec;
    const uint64_t ntiles = (nvec + BS - 1) / BS;
    const gf32x4u *src[N];
#pragma unroll
    for (int k = 0; k < N; k++)
        src[k] = (const gf32x4u *)(a.src[k] + a.head);

    for (uint64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        const uint64_t t = xcd_block_tile(b, ntiles);
        const uint64_t base = t * BS;
        const uint32_t nblk = (uint32_t)(nvec - base < (uint64_t)BS ? nvec - base : (uint64_t)BS);
        if (threadIdx.x < nblk) {
            const uint64_t i = base + threadIdx.x;
            f32x4 val[N];
#pragma unroll
            for (int k = 0; k < N; k++)
                val[k] = __builtin_nontemporal_load(src[k] + i);
            f32x4 acc = val[0];
#pragma unroll
            for (int k = 1; k < N; k++)
                acc = acc + val[k];
            const __amdgpu_buffer_rsrc_t out =
                buffer_over(reinterpret_cast<uint64_t>(a.dst + a.head) + base * 16, nblk * 16u);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), out, threadIdx.x * 16, 0,
                                                   rc_store_pol(N));
        }
    }

    // Up to 3 floats before the aligned body (threads 0-2) and 3 after it
    // (threads 32-34).
    static_assert(BS >= 64, "head and tail threads");
    if (blockIdx.x == 0) {
        gf32 *d = (gf32 *)(a.dst);
        if (threadIdx.x < a.head) {
            const uint64_t j = threadIdx.x;
            d[j] = rc_sum_scalar<N>(a, j);
        } else if (threadIdx.x >= 32 && threadIdx.x < 32 + a.tail) {
            const uint64_t j = a.head + 4 * nvec + (threadIdx.x - 32);
            d[j] = rc_sum_scalar<N>(a, j);
        }
    }
}

// Unaligned path from eight sources up, staged through LDS.  Every source is
// read with aligned 16-byte loads straight into LDS (global_load_lds_dwordx4:
// lane l's block lands 16 l bytes past the wave's LDS base), and the thread
// that writes dst block i reads its source's four floats back from LDS at the
// source's 4-byte offset s (0..3 floats): they lie in aligned blocks i and
// i + 1 of the source's 16-byte-aligned view A = src + head - s.  A wave's
// tile is 64 dst blocks, so it loads A's blocks i0 .. i0 + 63 plus the first
// dwords of block i0 + 64.  That last load is made by the whole wave, one
// dword per lane (lanes 3..63 all take dword 3): a load for lane 0 alone,
// under an exec mask, was merged by the compiler with the next source's
// full-wave load into one instruction whose LDS address came from lane 0.
// Every load reads an aligned 16-byte block holding at least one of the
// source's elements (indexes are clamped to the last such block), so no load
// leaves the pages the source lies in.  Sources are staged G = rc_lds_group(N)
// at a time and added in order as each group lands.
// Measured on MI355X with sources 4 or 8 bytes off dst, at 256 MiB per
// buffer: eight sources 72.5-73.9% of HBM peak against 70.0-70.4% with the
// 4-byte-aligned loads, sixteen 74.0-74.5% against 69.8-70.0%, level with the
// aligned path (74.1%); at 64 MiB per buffer 1.5-5.6 points ahead from nine to
// sixteen sources, and 1-3 points behind below eight (four sources 76%
// against 78%).  It reads 3.6-4.9% more bytes than the sources hold, as the
// other form does (the line shared by two tiles): the gain is the loads that
// no longer straddle two 16-byte blocks.
template <int N>
__global__ __launch_bounds__(kRcLdsBlock) void rc_unaligned_lds_kernel(ReduceArgs a) {
    constexpr int G = rc_lds_group(N);
    constexpr uint32_t kRegion = 64 * 4 + 64;   // dwords per staged source: 64 blocks, then block 64's dwords
    __shared__ __attribute__((aligned(16))) uint32_t lds[G][kRegion];
    typedef float f32x4l __attribute__((ext_vector_type(4), aligned(4)));
    const uint32_t lane = threadIdx.x;
    const uint32_t xdw = 4 * (lane < 3 ? lane : 3);   // this lane's dword of block i0 + 64
    const uint64_t nvec = a.nvec;
    const uint64_t ntiles = (nvec + kRcLdsBlock - 1) / kRcLdsBlock;
    // Per source: the 16-byte-aligned view A, the offset s in floats, and the
    // last block of A holding one of the source's elements (block nvec holds
    // the body's last s floats when s > 0).  The compiler keeps these across
    // the tile loop, in vector registers from nine sources up (83-147 VGPRs);
    // a form that recomputed them per tile in scalar registers (42-70 VGPRs)
    // ran 3-6 points slower.
    uint64_t abase[N];
    uint32_t sh[N];
    uint64_t last[N];
#pragma unroll
    for (int k = 0; k < N; k++) {
        const uint64_t p = reinterpret_cast<uint64_t>(a.src[k] + a.head);
        sh[k] = (uint32_t)(p & 15) >> 2;
        abase[k] = p - (p & 15);
        last[k] = sh[k] != 0 ? nvec : nvec - 1;
    }
    for (uint64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        const uint64_t i0 = xcd_block_tile(b, ntiles) * kRcLdsBlock;
        const uint32_t nblk = (uint32_t)(nvec - i0 < (uint64_t)kRcLdsBlock ? nvec - i0 : (uint64_t)kRcLdsBlock);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g0 = 0; g0 < N; g0 += G) {
#pragma unroll
            for (int j = 0; j < G; j++) {
                const int k = g0 + j;
                if (k < N) {
                    const uint64_t bl = i0 + lane < last[k] ? i0 + lane : last[k];
                    const uint64_t bx = i0 + 64 < last[k] ? i0 + 64 : last[k];
                    __builtin_amdgcn_global_load_lds((const gvoid *)(abase[k] + bl * 16), (svoid *)&lds[j][0], 16, 0,
                                                     kPolNt);
                    __builtin_amdgcn_global_load_lds((const gvoid *)(abase[k] + bx * 16 + xdw),
                                                     (svoid *)&lds[j][64 * 4], 4, 0, kPolNt);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);   // the group's blocks are in LDS
#pragma unroll
            for (int j = 0; j < G; j++) {
                const int k = g0 + j;
                if (k < N) {
                    const f32x4 v = *(const f32x4l *)((const float *)&lds[j][0] + lane * 4 + sh[k]);
                    acc = k == 0 ? v : acc + v;
                }
            }
            __builtin_amdgcn_s_waitcnt(0);   // LDS read before the next group overwrites it
        }
        if (lane < nblk) {
            const __amdgpu_buffer_rsrc_t out =
                buffer_over(reinterpret_cast<uint64_t>(a.dst + a.head) + i0 * 16, nblk * 16u);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), out, lane * 16, 0,
                                                   rc_store_pol(N));
        }
    }

    // Up to 3 floats before the aligned body (threads 0-2) and 3 after it
    // (threads 32-34).
    if (blockIdx.x == 0) {
        gf32 *d = (gf32 *)(a.dst);
        if (threadIdx.x < a.head) {
            const uint64_t j = threadIdx.x;
            d[j] = rc_sum_scalar<N>(a, j);
        } else if (threadIdx.x >= 32 && threadIdx.x < 32 + a.tail) {
            const uint64_t j = a.head + 4 * nvec + (threadIdx.x - 32);
            d[j] = rc_sum_scalar<N>(a, j);
        }
    }
}

// nsrc == 0: dstReference[0] is a memset.  dst is 4-byte aligned; `fill` is
// the memset byte replicated into 32 bits.  One 4 KiB tile per workgroup and
// one 16-byte store per thread: on MI355X this shape writes 1 GiB at 89-90%
// of HBM peak, where four stores per thread (16 KiB per workgroup) reach only
// 75%.  Stores as for one or two sources (nt sc0 sc1, not allocating in the
// memory-side cache).
__global__ __launch_bounds__(kRcBlock) void rc_memset_kernel(ReduceArgs a) {
    const uint64_t nvec = a.nvec;
    const u32x4 fill4 = {a.fill, a.fill, a.fill, a.fill};
    const uint64_t ntiles = (nvec + kRcBlock - 1) / kRcBlock;
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t base = t * kRcBlock;
        const uint64_t left = nvec - base;   // > 0
        const uint64_t n16 = left < (uint64_t)kRcBlock ? left : (uint64_t)kRcBlock;
        const __amdgpu_buffer_rsrc_t out =
            buffer_over(reinterpret_cast<uint64_t>(a.dst + a.head) + base * 16, (uint32_t)(n16 * 16));
        if (threadIdx.x < n16)
            __builtin_amdgcn_raw_buffer_store_b128(fill4, out, threadIdx.x * 16, 0, rc_store_pol(0));
    }
    if (blockIdx.x == 0) {
        gu32 *d32 = (gu32 *)(a.dst);
        if (threadIdx.x < a.head)
            d32[threadIdx.x] = a.fill;
        else if (threadIdx.x >= 64 && threadIdx.x < 64 + a.tail)
            d32[a.head + 4 * nvec + (threadIdx.x - 64)] = a.fill;
    }
}

int reduce_grid(uint64_t nfloats, int nsrc, bool vector_path, int cu_count) {
    (void)cu_count;
    uint64_t per_block;
    if (nsrc == 0)
        per_block = (uint64_t)kRcBlock * 4;
    else if (vector_path)
        per_block = (uint64_t)rc_block_of(nsrc) * 4;
    else if (rc_unaligned_lds(nsrc))
        per_block = (uint64_t)kRcLdsBlock * 4;
    else
        per_block = (uint64_t)kRcUnalignedBlock * 4;
    // one workgroup per tile, capped; the kernels loop when the cap binds
    uint64_t g = (nfloats + per_block - 1) / per_block;
    if (g > kRcMaxBlocks)
        g = kRcMaxBlocks;
    return (int)(g > 0 ? g : 1);
}

// Events the next launch made by this host thread records as part of the
// launch itself (set by tb_time_next_launch; consumed by that launch).
static thread_local hipEvent_t t_next_start = nullptr;
static thread_local hipEvent_t t_next_stop = nullptr;

void set_next_launch_events(hipEvent_t start, hipEvent_t stop) {
    t_next_start = start;
    t_next_stop = stop;
}

// Every kernel of the library is launched here.  With events (the timing hook,
// or `done` from the caller), the launch carries them as its own start / stop
// events, so no separate event command sits between kernels.  A launch has
// one stop event: when `done` takes it (a ring slot's completion event) and
// the timing hook also set one, the hook's is recorded right after the launch
// as a command of its own, so it too fires when the kernel has completed.
template <typename... KArgs, typename... Args>
static hipError_t launch(void (*kernel)(KArgs...), int grid, int block, hipStream_t s, hipEvent_t done,
                         Args... args) {
    const hipEvent_t start = t_next_start;
    const hipEvent_t hook_stop = t_next_stop;
    const hipEvent_t stop = done != nullptr ? done : hook_stop;
    t_next_start = t_next_stop = nullptr;
    if (start != nullptr || stop != nullptr)
        hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, s, start, stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, s, args...);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && done != nullptr && hook_stop != nullptr)
        e = hipEventRecord(hook_stop, s);
    return e;
}

template <int N>
static hipError_t launch_n(const ReduceArgs &a, bool vector_path, int grid, hipStream_t s) {
    if (vector_path)
        return launch(rc_vec_kernel<N>, grid, rc_block_of(N), s, nullptr, a);
    if constexpr (rc_unaligned_lds(N))
        return launch(rc_unaligned_lds_kernel<N>, grid, kRcLdsBlock, s, nullptr, a);
    else
        return launch(rc_unaligned_kernel<N>, grid, kRcUnalignedBlock, s, nullptr, a);
}

hipError_t launch_reduce_copy(const ReduceArgs &a, int nsrc, bool vector_path, int cu_count,
                              hipStream_t s) {
    const int grid = reduce_grid(a.n, nsrc, vector_path, cu_count);
    switch (nsrc) {
    case 0:
        return launch(rc_memset_kernel, grid, kRcBlock, s, nullptr, a);
    case 1: return launch_n<1>(a, vector_path, grid, s);
    case 2: return launch_n<2>(a, vector_path, grid, s);
    case 3: return launch_n<3>(a, vector_path, grid, s);
    case 4: return launch_n<4>(a, vector_path, grid, s);
    case 5: return launch_n<5>(a, vector_path, grid, s);
    case 6: return launch_n<6>(a, vector_path, grid, s);
    case 7: return launch_n<7>(a, vector_path, grid, s);
    case 8: return launch_n<8>(a, vector_path, grid, s);
    case 9: return launch_n<9>(a, vector_path, grid, s);
    case 10: return launch_n<10>(a, vector_path, grid, s);
    case 11: return launch_n<11>(a, vector_path, grid, s);
    case 12: return launch_n<12>(a, vector_path, grid, s);
    case 13: return launch_n<13>(a, vector_path, grid, s);
    case 14: return launch_n<14>(a, vector_path, grid, s);
    case 15: return launch_n<15>(a, vector_path, grid, s);
    case 16: return launch_n<16>(a, vector_path, grid, s);
    default: return hipErrorInvalidValue;
    }
}

// ============================================================================
// Batched copy
// (Mooncake RFC #5041, Design of #5040: one launch over a (src, dst, len)
//  descriptor array; 16-byte vectors where the ranges allow.)
//
// Grid of about one descriptor per wave (between 7 and 64 workgroups per CU);
// the unit of work is a wave64.  Wave w owns descriptors w, w + W, w + 2W, ...
// (W waves in all) and fetches up to 64 of them with one load per lane.  It
// broadcasts each to the whole wave (readlane, so addresses and lengths are
// scalar) and copies it with 16-byte lanes, 8 loads in flight per lane before
// the matching stores.  Copies longer than kBcSplitAbove instead go through a
// queue: the first workgroups scan the descriptors and publish them, and once
// every scanner has finished the queue is cut into kBcChunk pieces dealt
// round-robin to the last waves of the grid, without atomics.  Every
// wait is bounded: a wave that cannot see the finished queue in time leaves
// its pieces, and the first such wave copies every long copy whole.  No
// workgroup waits for any other at the end, and nothing in the scratch is
// cleared after a launch (scan words alternate by launch; slots carry the
// launch's epoch).
// ============================================================================

constexpr int kBcUnroll = 8;   // 8 x 16 B x 64 lanes = 8 KiB per wave step

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readfirstlane_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Raw buffer load / store of one E-byte element with a cache policy.
template <int E>
struct BufElem;
template <>
struct BufElem<1> {
    typedef uint8_t T;
    template <int Pol>
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        return __builtin_amdgcn_raw_buffer_load_b8(r, vo, so, Pol);
    }
    template <int Pol>
    static __device__ __forceinline__ void store(T v, __amdgpu_buffer_rsrc_t r, int vo, int so) {
        __builtin_amdgcn_raw_buffer_store_b8(v, r, vo, so, Pol);
    }
};
template <>
struct BufElem<16> {
    typedef u32x4 T;
    template <int Pol>
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, Pol);
    }
    template <int Pol>
    static __device__ __forceinline__ void store(T v, __amdgpu_buffer_rsrc_t r, int vo, int so) {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, vo, so, Pol);
    }
};

// Cache policies of the batched copy.  Every source byte is read once per
// launch: nontemporal loads.  Stores are nontemporal with system scope
// (nt sc0 sc1): they go out to HBM without leaving scattered dirty lines in
// the caches for the next kernel to drain.  Measured on MI355X in the bench
// step (reduce-copy then batched copy): this beat plain and device-scope
// stores by 15-35 us per step.
constexpr int kBcLoadPol = kPolNt;
constexpr int kBcStorePol = kPolNt | kPolSc0 | kPolSc1;

// Copy n elements of E bytes from s to d with the whole wave (s, d, n
// wave-uniform; s and d E-byte aligned).  Each step covers kBcUnroll slots of
// 64 elements and issues all its loads back to back before its stores, through
// one raw buffer resource per direction: the lane offset is the only VGPR
// operand and the slot offset goes in the scalar soffset.  Full steps touch
// only bytes inside the copy; in the last, partial step each lane is
// predicated on its element lying inside the copy, so no access ever leaves
// [s, s + nE) or [d, d + nE) (the resource bounds are a second guard).
template <int E>
__device__ __forceinline__ void wave_copy_buf(uint64_t s, uint64_t d, uint64_t n, int lane) {
    typedef typename BufElem<E>::T T;
    constexpr uint32_t kSlot = 64 * E;                 // bytes per slot
    constexpr uint64_t kStepBytes = (uint64_t)kSlot * kBcUnroll;
    const uint64_t total = n * E;
    uint64_t b0 = 0;
    for (; b0 + kStepBytes <= total; b0 += kStepBytes) {
        const __amdgpu_buffer_rsrc_t in = buffer_over(s + b0, (uint32_t)kStepBytes);
        const __amdgpu_buffer_rsrc_t out = buffer_over(d + b0, (uint32_t)kStepBytes);
        T r[kBcUnroll];
#pragma unroll
        for (int u = 0; u < kBcUnroll; u++)
            r[u] = BufElem<E>::template load<kBcLoadPol>(in, lane * E, u * kSlot);
#pragma unroll
        for (int u = 0; u < kBcUnroll; u++)
            BufElem<E>::template store<kBcStorePol>(r[u], out, lane * E, u * kSlot);
    }
    if (b0 < total) {
        const uint32_t left = (uint32_t)(total - b0);
        const __amdgpu_buffer_rsrc_t in = buffer_over(s + b0, left);
        const __amdgpu_buffer_rsrc_t out = buffer_over(d + b0, left);
        T r[kBcUnroll];
#pragma unroll
        for (int u = 0; u < kBcUnroll; u++)
            if (u * kSlot + (uint32_t)lane * E < left)
                r[u] = BufElem<E>::template load<kBcLoadPol>(in, lane * E, u * kSlot);
#pragma unroll
        for (int u = 0; u < kBcUnroll; u++)
            if (u * kSlot + (uint32_t)lane * E < left)
                BufElem<E>::template store<kBcStorePol>(r[u], out, lane * E, u * kSlot);
    }
}

// Up to 15 single bytes, one per lane (lanes at or past n do nothing).
__device__ __forceinline__ void wave_copy_few_bytes(uint64_t s, uint64_t d, uint64_t n, int lane) {
    if ((uint64_t)lane >= n)
        return;
    const __amdgpu_buffer_rsrc_t in = buffer_over(s, (uint32_t)n);
    const __amdgpu_buffer_rsrc_t out = buffer_over(d, (uint32_t)n);
    BufElem<1>::store<kBcStorePol>(BufElem<1>::load<kBcLoadPol>(in, lane, 0), out, lane, 0);
}

// The 16 bytes starting `m` bytes into the 32 bytes (x, y), m in 1..15 and
// wave-uniform: output dword k is bytes 4k + m .. 4k + m + 3.
__device__ __forceinline__ u32x4 bytes_at(u32x4 x, u32x4 y, uint32_t m) {
    const uint32_t q = m >> 2, r = m & 3;
    const uint32_t w0 = q == 0 ? x.x : (q == 1 ? x.y : (q == 2 ? x.z : x.w));
    const uint32_t w1 = q == 0 ? x.y : (q == 1 ? x.z : (q == 2 ? x.w : y.x));
    const uint32_t w2 = q == 0 ? x.z : (q == 1 ? x.w : (q == 2 ? y.x : y.y));
    const uint32_t w3 = q == 0 ? x.w : (q == 1 ? y.x : (q == 2 ? y.y : y.z));
    const uint32_t w4 = q == 0 ? y.x : (q == 1 ? y.y : (q == 2 ? y.z : y.w));
    u32x4 o;
    o.x = __builtin_amdgcn_alignbyte(w1, w0, r);
    o.y = __builtin_amdgcn_alignbyte(w2, w1, r);
    o.z = __builtin_amdgcn_alignbyte(w3, w2, r);
    o.w = __builtin_amdgcn_alignbyte(w4, w3, r);
    return o;
}


// Slots per step of the realigning copy: with 3 KiB steps the routine needs
// 66 VGPRs, which leaves the kernel, calling it, room to keep its own values
// in registers (with 4 KiB steps, 72 VGPRs, the kernel spilled one VGPR to
// scratch around the call in the long-copy piece phase: 1.8 MB of extra HBM
// writes per launch on a batch with long copies).
constexpr int kBcShiftSlots = 3;

// Copy nblk 16-byte blocks to d (16-byte aligned) from s, which lies m = s mod
// 16 (1..15) bytes past a 16-byte boundary, with the whole wave.  Source
// block i of the aligned view A = s - m holds the first 16 - m bytes of
// destination block i, block i + 1 the rest.  Steps of kBcShiftSlots slots of
// 64 blocks: each lane loads A's block for its destination block and takes the
// next one from lane + 1 by DPP; lane 63's next block is lane 0's block of the
// following slot (rotated in), and only the step's last slot loads it for
// lane 63.  Block indexes are clamped to the step's last block b0 + nstep
// (at most nblk, the last block of A that holds a source byte), so every load
// reads a 16-byte block holding a copied byte; stores are predicated on lying
// inside the destination.
__device__ __forceinline__ void wave_copy_shifted(uint64_t s, uint64_t d, uint64_t nblk, int lane) {
    constexpr int kSlots = kBcShiftSlots;
    const uint32_t m = (uint32_t)(s & 15);
    const uint64_t a = s - m;
    for (uint64_t b0 = 0; b0 < nblk; b0 += (uint64_t)kSlots * 64) {
        const uint64_t left = nblk - b0;
        const uint32_t nstep = (uint32_t)(left < (uint64_t)kSlots * 64 ? left : (uint64_t)kSlots * 64);
        // blocks b0 .. b0 + nstep of A: every one holds a source byte
        const __amdgpu_buffer_rsrc_t in = buffer_over(a + b0 * 16, (nstep + 1) * 16u);
        u32x4 x[kSlots];
#pragma unroll
        for (int u = 0; u < kSlots; u++) {
            const uint32_t q = (uint32_t)u * 64 + (uint32_t)lane;
            x[u] = BufElem<16>::load<kBcLoadPol>(in, (q < nstep ? q : nstep) * 16, 0);
        }
        u32x4 z = {0u, 0u, 0u, 0u};
        if (lane == 63)
            z = BufElem<16>::load<kBcLoadPol>(in, nstep * 16, 0);   // block b0 + 64 kSlots, clamped
        const __amdgpu_buffer_rsrc_t out = buffer_over(d + b0 * 16, nstep * 16u);
#pragma unroll
        for (int u = 0; u < kSlots; u++) {
            const u32x4 next = u + 1 < kSlots ? rol1_lane(x[u + 1 < kSlots ? u + 1 : u]) : z;
            const u32x4 y = shl1_lane(x[u], next);
            const uint32_t q = (uint32_t)u * 64 + (uint32_t)lane;
            if (q < nstep)
                BufElem<16>::store<kBcStorePol>(bytes_at(x[u], y, m), out, q * 16, 0);
        }
    }
}

// Copy b bytes from s to d with the whole wave; s, d, b are wave-uniform, any
// alignment.  The bytes before d's first 16-byte boundary and after its last
// one go one per lane; the 16-byte blocks between are copied directly when s
// is then aligned too, and realigned in registers otherwise
// (wave_copy_shifted).  Not inlined: it serves the rare cases, and keeping it
// out of the kernel body keeps the hot path's register allocation small.
__device__ __noinline__ void wave_copy_any(uint64_t s, uint64_t d, uint64_t b, int lane) {
    uint64_t head = (16 - (d & 15)) & 15;
    if (head > b)
        head = b;
    wave_copy_few_bytes(s, d, head, lane);
    s += head;
    d += head;
    b -= head;
    const uint64_t nblk = b >> 4;
    if (nblk != 0) {
        if ((s & 15) == 0)
            wave_copy_buf<16>(s, d, nblk, lane);
        else
            wave_copy_shifted(s, d, nblk, lane);
    }
    const uint64_t body = nblk << 4;
    wave_copy_few_bytes(s + body, d + body, b - body, lane);
}

// Hot path: both ends 16-byte aligned (every copy of the KV-transfer shapes);
// anything else goes to wave_copy_any.
__device__ __forceinline__ void wave_copy(uint64_t s, uint64_t d, uint64_t b, int lane) {
    if (((s | d) & 15) == 0) {
        const uint64_t body = b & ~(uint64_t)15;
        wave_copy_buf<16>(s, d, body >> 4, lane);
        wave_copy_few_bytes(s + body, d + body, b - body, lane);
    } else {
        wave_copy_any(s, d, b, lane);
    }
}

__device__ __forceinline__ uint32_t atomic_load_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void atomic_store_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t atomic_load_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void atomic_store_agent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t atomic_add_agent(uint64_t *p, uint64_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o)
            x += y;
    }
    return x;
}

// A queue slot holds (low 32 bits of the epoch << 32) | (descriptor index + 1).
// It is current when its epoch is this launch's and the index lies in the
// batch; anything else (not yet visible, or left by an earlier launch) counts
// as missing.
__device__ __forceinline__ bool slot_current(uint64_t v, uint64_t epoch, uint32_t n) {
    const uint32_t idx1 = (uint32_t)v;
    return (uint32_t)(v >> 32) == (uint32_t)epoch && idx1 != 0 && idx1 <= n;
}

// Recovery copy: every long copy of the batch, found in the descriptor array
// itself (not through the queue), copied whole by one wave.  It writes the
// same bytes as the pieces, so it may overlap them in time.
__device__ __forceinline__ void copy_all_long(const tb_copy_desc *__restrict__ desc, uint32_t n, int lane) {
    for (uint64_t b0 = 0; b0 < n; b0 += 64) {
        const uint64_t i = b0 + lane;
        const bool is_long = i < n && desc[i].bytes > kBcSplitAbove;
        uint64_t todo = __ballot(is_long);
        while (todo) {
            const int j = __builtin_ctzll(todo);
            todo &= todo - 1;
            const uint64_t di = readlane_u64(i, j);
            wave_copy_any(readfirstlane_u64(desc[di].src), readfirstlane_u64(desc[di].dst),
                          readfirstlane_u64(desc[di].bytes), lane);
        }
    }
}

__global__ __launch_bounds__(kBcBlock, kBcBlocksPerCu) void bc_kernel(const tb_copy_desc *__restrict__ desc,
                                                                      uint32_t n, BcScratch *scr, uint64_t epoch,
                                                                      uint32_t scanners, uint64_t wait_ticks,
                                                                      uint32_t piece_waves, uint32_t no_pieces) {
    const int lane = threadIdx.x & 63;
    // wave-uniform values kept in scalar registers (readfirstlane tells the
    // compiler so; otherwise their arithmetic would run per lane)
    const uint32_t wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t W = gridDim.x * (kBcBlock / 64);
    const uint32_t wave = blockIdx.x * (kBcBlock / 64) + wave_in_block;
    uint64_t *scan = &scr->scan[epoch & 1].word;

    // The word the next launch on this scratch will use (this launch's was
    // cleared by the previous one).
    if (blockIdx.x == 0 && threadIdx.x == 0)
        atomic_store_agent(&scr->scan[(epoch + 1) & 1].word, 0ull);

    // ---- 1. The first `scanners` workgroups (dispatched first) find the long
    // copies and publish them.  Slots are claimed on the low half of the scan
    // word; a copy that no longer fits the queue is copied here, by the wave
    // that found it.  A finished scanner adds 1 to the high half once its
    // slot stores have completed. ----
    if (blockIdx.x < scanners) {
        const uint64_t per = ((uint64_t)n + scanners - 1) / scanners;
        const uint64_t lo = (uint64_t)blockIdx.x * per;
        const uint64_t hi = lo + per < n ? lo + per : n;
        for (uint64_t b0 = lo + (uint64_t)wave_in_block * 64; b0 < hi; b0 += kBcBlock) {
            const uint64_t i = b0 + lane;
            bool here = false;
            if (i < hi && desc[i].bytes > kBcSplitAbove) {
                // n < 2^32 claims in all, so the low half never carries
                const uint32_t slot = (uint32_t)atomic_add_agent(scan, 1ull);
                if (slot < kBcQueueCap)
                    atomic_store_agent(&scr->slot[slot], (epoch << 32) | (uint32_t)(i + 1));
                else
                    here = true;
            }
            uint64_t todo = __ballot(here);
            while (todo) {
                const int j = __builtin_ctzll(todo);
                todo &= todo - 1;
                const uint64_t di = readlane_u64(i, j);
                wave_copy_any(readfirstlane_u64(desc[di].src), readfirstlane_u64(desc[di].dst),
                              readfirstlane_u64(desc[di].bytes), lane);
            }
        }
        // Each wave waits until its slot stores have completed (they are
        // device-coherent atomic stores) before the barrier, so before thread
        // 0 counts this workgroup as finished.  A release fence would do the
        // same but also write back the whole L2 of the XCD.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0)
            atomic_add_agent(scan, 1ull << 32);
    }

    // ---- 2. Own descriptors w, w + W, ...: copy the short ones whole (the
    // long ones belong to the queue).  Up to 64 fetched with one load per
    // lane, then broadcast to the whole wave. ----
    for (uint64_t k0 = 0; wave + k0 * W < n; k0 += 64) {
        const uint64_t i = wave + (k0 + lane) * (uint64_t)W;
        uint64_t s = 0, d = 0, b = 0;
        if (i < n) {
            s = desc[i].src;
            d = desc[i].dst;
            b = desc[i].bytes;
        }
        uint64_t todo = __ballot(b != 0 && b <= kBcSplitAbove);
        while (todo) {
            const int j = __builtin_ctzll(todo);
            todo &= todo - 1;
            wave_copy(readlane_u64(s, j), readlane_u64(d, j), readlane_u64(b, j), lane);
        }
    }

    // ---- 3. The last P waves of the grid share the queue's kBcChunk
    // pieces; the others are done.  The last ones, not the first: they are
    // dispatched after the scanners have finished (the first waves would sit
    // waiting for them, holding their slots, which measured 6 us slower on a
    // 47,520-copy batch), and P = the waves that fit on the chip at once, so
    // all of them can run together.  A piece wave waits (bounded) until every
    // scanner has finished: the queue length is then final, and it comes in
    // the same word as the count of finished scanners, so every wave sees the
    // same length.  The pieces are numbered across all entries and piece g
    // goes to piece wave g mod P, so no atomics are needed to share them. ----
    const uint32_t P = piece_waves < W ? piece_waves : W;
    if (wave < W - P)
        return;
    const uint32_t pw = wave - (W - P);   // piece wave index, in [0, P)
    bool sealed = false;
    uint32_t q = 0;
    if (!no_pieces) {
        const uint64_t t0 = wall_clock64();
        for (;;) {
            const uint64_t sw = readfirstlane_u64(atomic_load_agent(scan));
            if ((uint32_t)(sw >> 32) >= scanners) {
                sealed = true;
                q = (uint32_t)sw < kBcQueueCap ? (uint32_t)sw : kBcQueueCap;
                break;
            }
            if (wall_clock64() - t0 > wait_ticks)
                break;
            __builtin_amdgcn_s_sleep(4);
        }
    }
    if (sealed) {
        uint32_t base_mod = 0;   // (number of the first piece of this group) mod P
        for (uint32_t g0 = 0; g0 < q; g0 += 64) {
            // lane l holds entry g0 + l: its descriptor index and piece count
            const uint32_t e = g0 + lane;
            uint64_t v = 0;
            uint32_t npieces = 0;
            bool missing = false;
            if (e < q) {
                v = atomic_load_agent(&scr->slot[e]);
                if (!slot_current(v, epoch, n))
                    missing = true;
                else
                    npieces = (uint32_t)((desc[(uint32_t)v - 1].bytes + kBcChunk - 1) / kBcChunk);
            }
            if (__ballot(missing)) {
                sealed = false;
                break;
            }
            const uint32_t incl = wave_inclusive_sum(npieces, lane);
            const uint32_t excl = incl - npieces;
            const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
            // this wave's pieces: g = base + r with g = pw (mod P)
            for (uint32_t r = (pw + P - base_mod) % P; r < total; r += P) {
                const uint64_t owners = __ballot(e < q && excl <= r);
                const int j = 63 - __builtin_clzll(owners);
                const uint64_t c = r - (uint32_t)__builtin_amdgcn_readlane(excl, j);   // piece within entry j
                const uint64_t di = (uint32_t)__builtin_amdgcn_readlane((uint32_t)v, j) - 1u;
                const uint64_t bj = readfirstlane_u64(desc[di].bytes);
                const uint64_t off = c * kBcChunk;
                wave_copy(readfirstlane_u64(desc[di].src) + off, readfirstlane_u64(desc[di].dst) + off,
                          bj - off < kBcChunk ? bj - off : kBcChunk, lane);
            }
            base_mod = (uint32_t)(((uint64_t)base_mod + total) % P);
        }
    }

    // ---- 4. A wave that gave up waiting, or met a slot it could not see,
    // may have left pieces undone.  The first such wave of this launch (the
    // epoch exchange elects it) copies every long copy of the batch whole,
    // straight from the descriptor array; the others leave theirs to it. ----
    if (!sealed) {
        uint64_t prev = 0;
        if (lane == 0)
            prev = __hip_atomic_exchange(&scr->redo.word, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (readfirstlane_u64(prev) != epoch)
            copy_all_long(desc, n, lane);
    }
}

// Cap on the batched copy's workgroups set by tb_batched_set_max_workgroups
// (0: none).  Process-wide; read at each launch.
static std::atomic<uint32_t> g_bc_max_wgs{0};

void set_batched_max_workgroups(uint32_t max_wgs) { g_bc_max_wgs.store(max_wgs, std::memory_order_relaxed); }

// A grid of g workgroups, capped, as a multiple of 8 (workgroups are dealt to
// the 8 XCDs in turn), at least 8.
static int capped_grid(uint64_t g) {
    const uint32_t cap = g_bc_max_wgs.load(std::memory_order_relaxed);
    if (cap != 0 && g > cap)
        g = cap & ~7u;
    if (g < 8)
        g = 8;
    return (int)((g + 7) & ~(uint64_t)7);
}

int batched_grid(uint32_t ncopies, int cu_count) {
    const uint64_t cus = (uint64_t)(cu_count > 0 ? cu_count : 1);
    uint64_t g = ((uint64_t)ncopies + kBcDescPerWave * 4 - 1) / (kBcDescPerWave * 4);
    if (g < cus * kBcBlocksPerCu)
        g = cus * kBcBlocksPerCu;
    if (g > cus * kBcMaxGridPerCu)
        g = cus * kBcMaxGridPerCu;
    return capped_grid(g);
}

uint32_t batched_scanners(uint32_t ncopies, int grid) {
    uint32_t s = (ncopies + kBcScanPerBlock - 1) / kBcScanPerBlock;
    if (s < 1)
        s = 1;
    if (s > (uint32_t)grid)
        s = (uint32_t)grid;
    return s;
}

// One launch of bc_kernel; with done_event, the event is the launch's own stop
// event (fired when the kernel completes), which costs no separate command.
static hipError_t launch_bc(int grid, hipStream_t s, hipEvent_t done_event, const tb_copy_desc *desc, uint32_t n,
                            BcScratch *scratch, uint64_t epoch, uint32_t scanners, uint64_t wait_ticks,
                            uint32_t piece_waves, uint32_t no_pieces) {
    return launch(bc_kernel, grid, kBcBlock, s, done_event, desc, n, scratch, epoch, scanners, wait_ticks,
                  piece_waves, no_pieces);
}

hipError_t launch_batched_copy(const tb_copy_desc *desc, uint32_t n, BcScratch *scratch, uint64_t epoch,
                               int cu_count, uint64_t wait_ticks, bool no_pieces, hipStream_t s,
                               hipEvent_t done_event) {
    const int grid = batched_grid(n, cu_count);
    // pieces of long copies go to as many waves as fit on the chip at once
    const uint32_t resident = (uint32_t)(cu_count > 0 ? cu_count : 1) * kBcResidentWavesPerCu;
    return launch_bc(grid, s, done_event, desc, n, scratch, epoch, batched_scanners(n, grid), wait_ticks, resident,
                     no_pieces ? 1u : 0u);
}

hipError_t launch_batched_copy_short(const tb_copy_desc *desc, uint32_t n, BcScratch *scratch, uint64_t epoch,
                                     int cu_count, hipStream_t s, hipEvent_t done_event) {
    // no scanners and no piece waves: every wave copies its own descriptors
    // and is done; one descriptor per wave, no floor on the grid
    const uint64_t cus = (uint64_t)(cu_count > 0 ? cu_count : 1);
    uint64_t g = ((uint64_t)n + kBcDescPerWave * 4 - 1) / (kBcDescPerWave * 4);
    if (g > cus * kBcMaxGridPerCu)
        g = cus * kBcMaxGridPerCu;
    return launch_bc(capped_grid(g), s, done_event, desc, n, scratch, epoch, 0u, 0u, 0u, 0u);
}

// ---- the batched copy over a static scratch (no allocation) --------------------
//
// tb_batched_copy_noalloc's scratch: one BcScratch per device, in the code
// object's static device memory, so that no call allocates.  Its size does not
// depend on the batch (long copies past the queue's capacity are copied by the
// wave that found them), so any batch fits.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is taken once per
// device with hipGetSymbolAddress (with that device current) and only that
// address is used afterwards, for kernel arguments and the clear.
static __device__ __align__(256) unsigned char scratch[kBcScratchBytes];

// Plain stores of zero over n16 16-byte words.
__global__ __launch_bounds__(256) void bc_scratch_clear_kernel(u32x4 *p, uint32_t n16) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i < n16)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

namespace {
struct StaticScratch {
    std::mutex mu;           // orders epoch numbering and the launch it numbers
    void *ptr = nullptr;     // device address of `scratch` on this device, once set up
    uint64_t epoch = 0;      // epoch of the last launch enqueued on it
};
StaticScratch g_static_scratch[kMaxDevices];
}  // namespace

hipError_t launch_batched_copy_static(const tb_copy_desc *desc, uint32_t n, int device, int cu_count,
                                      uint64_t wait_ticks, bool no_pieces, hipStream_t s) {
    if (device < 0 || device >= kMaxDevices)
        return hipErrorInvalidDevice;
    StaticScratch &st = g_static_scratch[device];
    std::lock_guard<std::mutex> lk(st.mu);
    if (st.ptr == nullptr) {
        // Set-up, once per device (the caller made `device` current): the
        // array's address, then a clear, finished before any launch uses it,
        // so that launches on any stream find it zeroed.
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
            return hipErrorInvalidSymbol;
        constexpr uint32_t n16 = (uint32_t)(kBcScratchBytes / 16);
        hipLaunchKernelGGL(bc_scratch_clear_kernel, dim3((n16 + 255) / 256), dim3(256), 0, s,
                           static_cast<u32x4 *>(p), n16);
        e = hipGetLastError();
        if (e == hipSuccess)
            e = hipStreamSynchronize(s);
        if (e != hipSuccess)
            return e;
        st.ptr = p;
    }
    const uint64_t epoch = st.epoch + 1;
    const int grid = batched_grid(n, cu_count);
    const uint32_t resident = (uint32_t)(cu_count > 0 ? cu_count : 1) * kBcResidentWavesPerCu;
    const hipError_t e = launch_bc(grid, s, nullptr, desc, n, static_cast<BcScratch *>(st.ptr), epoch,
                                   batched_scanners(n, grid), wait_ticks, resident, no_pieces ? 1u : 0u);
    if (e == hipSuccess)
        st.epoch = epoch;   // a failed launch does not use up its epoch
    return e;
}

// ============================================================================
// Spin gate ("nvbandwidth deep dive" §3.3.1): hold the stream until the host
// releases it, so queued launches and events then run back to back.  Bounded:
// gives up after timeout_ticks of the constant-rate device clock.
// ============================================================================

__global__ void spin_gate_kernel(const uint32_t *flag, uint32_t *timed_out, uint64_t timeout_ticks) {
    if (threadIdx.x != 0)
        return;
    const uint64_t t0 = wall_clock64();
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == 0u) {
        if (wall_clock64() - t0 > timeout_ticks) {
            __hip_atomic_store(timed_out, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            break;
        }
        __builtin_amdgcn_s_sleep(8);
    }
}

hipError_t launch_spin_gate(const uint32_t *flag, uint32_t *timed_out, uint64_t timeout_ticks,
                            hipStream_t s) {
    return launch(spin_gate_kernel, 1, 64, s, nullptr, flag, timed_out, timeout_ticks);
}

}  // namespace tbk
