// tb_kernels.hip -- gfx950 kernels of libtb: reduce-copy, batched copy, spin gate.
//
// Written for CDNA4: wave64, 256 CUs in 8 XCDs, HBM3E.  Nothing here is a
// contraction, so there is no MFMA; both copies are HBM-bound streams and the
// design is about keeping enough 16-byte loads in flight per CU.
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

// float4s per thread per tile: enough loads in flight without spilling.
template <int N>
constexpr int rc_unroll() {
    return N <= 2 ? 4 : (N <= 4 ? 2 : 1);
}

template <typename T>
__device__ __forceinline__ T rc_load(const T *p) {
    return __builtin_nontemporal_load(p);
}

template <typename T>
__device__ __forceinline__ void rc_store(T *p, T v) {
    __builtin_nontemporal_store(v, p);
}

// Fixed-order scalar sum of element j (used for the unaligned head and tail).
template <int N>
__device__ __forceinline__ float rc_sum_scalar(const ReduceArgs &a, uint64_t j) {
    float acc = a.src[0][j];
#pragma unroll
    for (int k = 1; k < N; k++)
        acc = acc + a.src[k][j];
    return acc;
}

// Vector path: every pointer is congruent to dst modulo 16.  Tiles of
// kRcBlock * U float4s are dealt to workgroups round-robin; each thread loads
// U float4s from every source before the first addition, so N * U 16-byte
// loads per thread are in flight.
template <int N>
__global__ __launch_bounds__(kRcBlock) void rc_vec_kernel(ReduceArgs a) {
    constexpr int U = rc_unroll<N>();
    constexpr uint64_t kTile = (uint64_t)kRcBlock * U;
    const uint64_t nvec = a.nvec;
    f32x4 *dst = reinterpret_cast<f32x4 *>(a.dst + a.head);
    const f32x4 *src[N];
#pragma unroll
    for (int k = 0; k < N; k++)
        src[k] = reinterpret_cast<const f32x4 *>(a.src[k] + a.head);

    for (uint64_t base = (uint64_t)blockIdx.x * kTile; base < nvec;
         base += (uint64_t)gridDim.x * kTile) {
        const uint64_t i0 = base + threadIdx.x;
        if (base + kTile <= nvec) {
            f32x4 v[N][U];
#pragma unroll
            for (int k = 0; k < N; k++)
#pragma unroll
                for (int u = 0; u < U; u++)
                    v[k][u] = rc_load(src[k] + i0 + (uint64_t)u * kRcBlock);
#pragma unroll
            for (int u = 0; u < U; u++) {
                f32x4 acc = v[0][u];
#pragma unroll
                for (int k = 1; k < N; k++)
                    acc = acc + v[k][u];
                rc_store(dst + i0 + (uint64_t)u * kRcBlock, acc);
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const uint64_t i = i0 + (uint64_t)u * kRcBlock;
                if (i < nvec) {
                    f32x4 acc = rc_load(src[0] + i);
#pragma unroll
                    for (int k = 1; k < N; k++)
                        acc = acc + rc_load(src[k] + i);
                    rc_store(dst + i, acc);
                }
            }
        }
    }

    // Up to 3 floats before the aligned body and 3 after it.
    if (blockIdx.x == 0) {
        if (threadIdx.x < a.head) {
            const uint64_t j = threadIdx.x;
            a.dst[j] = rc_sum_scalar<N>(a, j);
        } else if (threadIdx.x >= 64 && threadIdx.x < 64 + a.tail) {
            const uint64_t j = a.head + 4 * nvec + (threadIdx.x - 64);
            a.dst[j] = rc_sum_scalar<N>(a, j);
        }
    }
}

// Scalar path for pointers that disagree modulo 16: one float per load.
template <int N>
__global__ __launch_bounds__(kRcBlock) void rc_scalar_kernel(ReduceArgs a) {
    constexpr int U = 4;
    constexpr uint64_t kTile = (uint64_t)kRcBlock * U;
    const uint64_t n = a.n;
    for (uint64_t base = (uint64_t)blockIdx.x * kTile; base < n;
         base += (uint64_t)gridDim.x * kTile) {
        const uint64_t i0 = base + threadIdx.x;
        float v[N][U];
#pragma unroll
        for (int k = 0; k < N; k++)
#pragma unroll
            for (int u = 0; u < U; u++) {
                const uint64_t i = i0 + (uint64_t)u * kRcBlock;
                v[k][u] = i < n ? a.src[k][i] : 0.0f;
            }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t i = i0 + (uint64_t)u * kRcBlock;
            if (i < n) {
                float acc = v[0][u];
#pragma unroll
                for (int k = 1; k < N; k++)
                    acc = acc + v[k][u];
                a.dst[i] = acc;
            }
        }
    }
}

// nsrc == 0: dstReference[0] is a memset.  dst is 4-byte aligned; `fill` is
// the memset byte replicated into 32 bits.
__global__ __launch_bounds__(kRcBlock) void rc_memset_kernel(ReduceArgs a) {
    constexpr int U = 4;
    constexpr uint64_t kTile = (uint64_t)kRcBlock * U;
    const uint64_t nvec = a.nvec;
    const u32x4 fill4 = {a.fill, a.fill, a.fill, a.fill};
    u32x4 *dst = reinterpret_cast<u32x4 *>(a.dst + a.head);
    for (uint64_t base = (uint64_t)blockIdx.x * kTile; base < nvec;
         base += (uint64_t)gridDim.x * kTile) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t i = base + threadIdx.x + (uint64_t)u * kRcBlock;
            if (i < nvec)
                rc_store(dst + i, fill4);
        }
    }
    if (blockIdx.x == 0) {
        uint32_t *d32 = reinterpret_cast<uint32_t *>(a.dst);
        if (threadIdx.x < a.head)
            d32[threadIdx.x] = a.fill;
        else if (threadIdx.x >= 64 && threadIdx.x < 64 + a.tail)
            d32[a.head + 4 * nvec + (threadIdx.x - 64)] = a.fill;
    }
}

int reduce_grid(uint64_t nfloats, int nsrc, bool vector_path, int cu_count) {
    uint64_t per_tile;
    if (nsrc == 0)
        per_tile = (uint64_t)kRcBlock * 4 * 4;
    else if (vector_path)
        per_tile = (uint64_t)kRcBlock * 4 *
                   (nsrc <= 2 ? 4 : (nsrc <= 4 ? 2 : 1));
    else
        per_tile = (uint64_t)kRcBlock * 4;
    uint64_t tiles = (nfloats + per_tile - 1) / per_tile;
    uint64_t cap = (uint64_t)(cu_count > 0 ? cu_count : 1) * kRcBlocksPerCu;
    uint64_t g = tiles < cap ? tiles : cap;
    return (int)(g > 0 ? g : 1);
}

template <int N>
static hipError_t launch_n(const ReduceArgs &a, bool vector_path, int grid, hipStream_t s) {
    if (vector_path)
        hipLaunchKernelGGL(rc_vec_kernel<N>, dim3(grid), dim3(kRcBlock), 0, s, a);
    else
        hipLaunchKernelGGL(rc_scalar_kernel<N>, dim3(grid), dim3(kRcBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_reduce_copy(const ReduceArgs &a, int nsrc, bool vector_path, int cu_count,
                              hipStream_t s) {
    const int grid = reduce_grid(a.n, nsrc, vector_path, cu_count);
    switch (nsrc) {
    case 0:
        hipLaunchKernelGGL(rc_memset_kernel, dim3(grid), dim3(kRcBlock), 0, s, a);
        return hipGetLastError();
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
// Persistent grid of kBcBlocksPerCu workgroups per CU; the unit of work is a
// wave64.  Wave w owns descriptors w, w + W, w + 2W, ... (W waves in all) and
// fetches up to 64 of them with one load per lane.  It broadcasts each to the
// whole wave (readlane, so addresses and lengths are scalar) and copies it
// with 16-byte lanes, U loads in flight per lane before the matching stores.
// Copies longer than kBcSplitAbove are published in a queue instead; after
// its own small copies every wave claims kBcChunk pieces of queued copies
// with one atomic per piece.  No wave ever waits for another: a queued copy
// is always finished by the wave that published it, helpers only speed it
// up.  The last workgroup to finish clears the queue for the next launch.
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

// Copy b bytes from s to d with the whole wave; s, d, b are wave-uniform.
__device__ __forceinline__ void wave_copy(uint64_t s, uint64_t d, uint64_t b, int lane) {
    if (((s ^ d) & 15) == 0) {
        // bytes up to dst's next 16-byte boundary, one per lane
        uint64_t head = (16 - (d & 15)) & 15;
        if (head > b)
            head = b;
        if ((uint64_t)lane < head)
            reinterpret_cast<uint8_t *>(d)[lane] = reinterpret_cast<const uint8_t *>(s)[lane];
        s += head;
        d += head;
        b -= head;
        const uint64_t nv = b >> 4;
        const u32x4 *sv = reinterpret_cast<const u32x4 *>(s);
        u32x4 *dv = reinterpret_cast<u32x4 *>(d);
        for (uint64_t v0 = 0; v0 < nv; v0 += 64 * kBcUnroll) {
            u32x4 r[kBcUnroll];
#pragma unroll
            for (int u = 0; u < kBcUnroll; u++) {
                const uint64_t i = v0 + (uint64_t)u * 64 + lane;
                if (i < nv)
                    r[u] = sv[i];
            }
#pragma unroll
            for (int u = 0; u < kBcUnroll; u++) {
                const uint64_t i = v0 + (uint64_t)u * 64 + lane;
                if (i < nv)
                    dv[i] = r[u];
            }
        }
        const uint64_t tail = b & 15;
        if ((uint64_t)lane < tail)
            reinterpret_cast<uint8_t *>(d)[nv * 16 + lane] =
                reinterpret_cast<const uint8_t *>(s)[nv * 16 + lane];
    } else if (((s ^ d) & 3) == 0) {
        uint64_t head = (4 - (d & 3)) & 3;
        if (head > b)
            head = b;
        if ((uint64_t)lane < head)
            reinterpret_cast<uint8_t *>(d)[lane] = reinterpret_cast<const uint8_t *>(s)[lane];
        s += head;
        d += head;
        b -= head;
        const uint64_t nw = b >> 2;
        const uint32_t *sw = reinterpret_cast<const uint32_t *>(s);
        uint32_t *dw = reinterpret_cast<uint32_t *>(d);
        for (uint64_t w0 = 0; w0 < nw; w0 += 64 * kBcUnroll) {
            uint32_t r[kBcUnroll];
#pragma unroll
            for (int u = 0; u < kBcUnroll; u++) {
                const uint64_t i = w0 + (uint64_t)u * 64 + lane;
                if (i < nw)
                    r[u] = sw[i];
            }
#pragma unroll
            for (int u = 0; u < kBcUnroll; u++) {
                const uint64_t i = w0 + (uint64_t)u * 64 + lane;
                if (i < nw)
                    dw[i] = r[u];
            }
        }
        const uint64_t tail = b & 3;
        if ((uint64_t)lane < tail)
            reinterpret_cast<uint8_t *>(d)[nw * 4 + lane] =
                reinterpret_cast<const uint8_t *>(s)[nw * 4 + lane];
    } else {
        const uint8_t *sb = reinterpret_cast<const uint8_t *>(s);
        uint8_t *db = reinterpret_cast<uint8_t *>(d);
        for (uint64_t o0 = 0; o0 < b; o0 += 64 * kBcUnroll) {
            uint8_t r[kBcUnroll];
#pragma unroll
            for (int u = 0; u < kBcUnroll; u++) {
                const uint64_t o = o0 + (uint64_t)u * 64 + lane;
                if (o < b)
                    r[u] = sb[o];
            }
#pragma unroll
            for (int u = 0; u < kBcUnroll; u++) {
                const uint64_t o = o0 + (uint64_t)u * 64 + lane;
                if (o < b)
                    db[o] = r[u];
            }
        }
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

__global__ __launch_bounds__(kBcBlock) void bc_kernel(const tb_copy_desc *__restrict__ desc,
                                                      uint32_t n, BcScratch *scr) {
    const int lane = threadIdx.x & 63;
    const uint64_t W = (uint64_t)gridDim.x * (kBcBlock / 64);
    const uint64_t wave = (uint64_t)blockIdx.x * (kBcBlock / 64) + (threadIdx.x >> 6);

    // ---- own descriptors: publish the long ones, copy the rest ----
    for (uint64_t k0 = 0; wave + k0 * W < n; k0 += 64) {
        const uint64_t i = wave + (k0 + lane) * W;
        const bool valid = i < n;
        uint64_t s = 0, d = 0, b = 0;
        if (valid) {
            s = desc[i].src;
            d = desc[i].dst;
            b = desc[i].bytes;
        }
        bool run_here = valid && b != 0;
        if (valid && b > kBcSplitAbove) {
            const uint32_t slot = atomic_add_agent(&scr->qtail, 1u);
            if (slot < kBcQueueCap) {
                atomic_store_agent(&scr->slot[slot].desc_plus1, (uint32_t)i + 1u);
                run_here = false;
            }
        }
        uint64_t todo = __ballot(run_here);
        while (todo) {
            const int j = __builtin_ctzll(todo);
            todo &= todo - 1;
            wave_copy(readlane_u64(s, j), readlane_u64(d, j), readlane_u64(b, j), lane);
        }
    }

    // ---- help with the published long copies ----
    uint32_t seen = 0;
    for (;;) {
        uint32_t q = atomic_load_agent(&scr->qtail);
        q = __builtin_amdgcn_readfirstlane(q < kBcQueueCap ? q : kBcQueueCap);
        if (q <= seen)
            break;
        const uint32_t span = q - seen;
        for (uint32_t r = 0; r < span; r++) {
            const uint32_t e = seen + (uint32_t)((r + wave) % span);
            const uint32_t v = __builtin_amdgcn_readfirstlane(atomic_load_agent(&scr->slot[e].desc_plus1));
            if (v == 0)
                continue;   // not published yet: its owner will copy it
            const uint64_t di = v - 1u;
            const uint64_t s = readfirstlane_u64(desc[di].src);
            const uint64_t d = readfirstlane_u64(desc[di].dst);
            const uint64_t b = readfirstlane_u64(desc[di].bytes);
            const uint64_t nchunks = (b + kBcChunk - 1) / kBcChunk;
            for (;;) {
                uint32_t c = 0;
                if (lane == 0)
                    c = atomic_add_agent(&scr->slot[e].next_chunk, 1u);
                c = __builtin_amdgcn_readfirstlane(c);
                if (c >= nchunks)
                    break;
                const uint64_t off = (uint64_t)c * kBcChunk;
                const uint64_t len = b - off < kBcChunk ? b - off : kBcChunk;
                wave_copy(s + off, d + off, len, lane);
            }
        }
        seen = q;
    }

    // ---- the last workgroup out clears the queue for the next launch ----
    __shared__ uint32_t last_block;
    __syncthreads();
    if (threadIdx.x == 0)
        last_block = (atomic_add_agent(&scr->done, 1u) == gridDim.x - 1) ? 1u : 0u;
    __syncthreads();
    if (last_block) {
        uint32_t q = atomic_load_agent(&scr->qtail);
        if (q > kBcQueueCap)
            q = kBcQueueCap;
        for (uint32_t e = threadIdx.x; e < q; e += kBcBlock) {
            atomic_store_agent(&scr->slot[e].desc_plus1, 0u);
            atomic_store_agent(&scr->slot[e].next_chunk, 0u);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            atomic_store_agent(&scr->qtail, 0u);
            atomic_store_agent(&scr->done, 0u);
        }
    }
}

int batched_grid(int cu_count) {
    return (cu_count > 0 ? cu_count : 1) * kBcBlocksPerCu;
}

hipError_t launch_batched_copy(const tb_copy_desc *desc, uint32_t n, BcScratch *scratch,
                               int cu_count, hipStream_t s) {
    hipLaunchKernelGGL(bc_kernel, dim3(batched_grid(cu_count)), dim3(kBcBlock), 0, s, desc, n,
                       scratch);
    return hipGetLastError();
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
    hipLaunchKernelGGL(spin_gate_kernel, dim3(1), dim3(64), 0, s, flag, timed_out, timeout_ticks);
    return hipGetLastError();
}

}  // namespace tbk
