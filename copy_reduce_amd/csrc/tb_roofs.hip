// tb_roofs.hip -- libtb_roofs: the measuring instruments of bench.py --roofs.
//
// Plain streams for gfx950: every thread makes one 16-byte access per buffer
// and tile, a tile is 4 KiB (256 threads), workgroup t takes tile t.  Partial
// tiles rely on the buffer resource's range check: accesses past the range
// are not made (loads return 0, stores are dropped).  Nothing here is shared
// with libtb's kernels; these only measure what an access pattern allows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "tb_roofs.h"

namespace tbr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;                  // threads per workgroup
constexpr uint64_t kTile = 16 * kBlock;      // bytes per tile and buffer
constexpr uint64_t kMaxGrid = 1u << 20;      // workgroups; tiles beyond are looped over
constexpr uint32_t kMagic = 0x9E3779B9u;     // checksum value that writes the sink
constexpr int kNt = 2, kSc0 = 1, kSc1 = 16;  // cache-policy bits of buffer accesses

}  // namespace tbr

// Written only when a read checksum equals kMagic, which keeps the loads
// live.  External linkage on purpose: a variable no code can read would let
// the compiler drop its stores, and with them the loads.
__device__ uint32_t tbr_sink[64];

namespace tbr {

struct Bufs {
    uint64_t p[TBR_MAX_BUFS];
};

struct Tile {
    uint64_t src;
    uint64_t dst;
    uint32_t bytes;
    uint32_t reserved;
};
static_assert(sizeof(Tile) == sizeof(tbr_tile), "tile layout");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(uint64_t base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <int K>
__global__ __launch_bounds__(kBlock) void read_kernel(Bufs b, uint64_t bytes) {
    const uint64_t ntiles = (bytes + kTile - 1) / kTile;
    uint32_t x = 0;
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t off = t * kTile;
        const uint32_t len = (uint32_t)(bytes - off < kTile ? bytes - off : kTile);
        u32x4 v[K];
#pragma unroll
        for (int k = 0; k < K; k++)
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc(b.p[k] + off, len), threadIdx.x * 16, 0, kNt);
#pragma unroll
        for (int k = 0; k < K; k++)
            x ^= fold(v[k]);
    }
    if (x == kMagic)
        tbr_sink[blockIdx.x & 63] = x;
}

template <int K, int POL>
__global__ __launch_bounds__(kBlock) void write_kernel(Bufs b, uint64_t bytes, uint32_t word) {
    const uint64_t ntiles = (bytes + kTile - 1) / kTile;
    const u32x4 w = {word, word, word, word};
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t off = t * kTile;
        const uint32_t len = (uint32_t)(bytes - off < kTile ? bytes - off : kTile);
#pragma unroll
        for (int k = 0; k < K; k++)
            __builtin_amdgcn_raw_buffer_store_b128(w, rsrc(b.p[k] + off, len), threadIdx.x * 16, 0, POL);
    }
}

template <int POL>
__global__ __launch_bounds__(kBlock) void copy_kernel(uint64_t dst, uint64_t src, uint64_t bytes) {
    const uint64_t ntiles = (bytes + kTile - 1) / kTile;
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t off = t * kTile;
        const uint32_t len = (uint32_t)(bytes - off < kTile ? bytes - off : kTile);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc(src + off, len), threadIdx.x * 16, 0, kNt);
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(dst + off, len), threadIdx.x * 16, 0, POL);
    }
}

// dst = the XOR of K sources, 16 bytes per thread and buffer: the
// reduce-copy's access pattern (K streams read, one written) with integer
// work only.
template <int K, int POL>
__global__ __launch_bounds__(kBlock) void combine_kernel(Bufs b, uint64_t dst, uint64_t bytes) {
    const uint64_t ntiles = (bytes + kTile - 1) / kTile;
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint64_t off = t * kTile;
        const uint32_t len = (uint32_t)(bytes - off < kTile ? bytes - off : kTile);
        u32x4 v[K];
#pragma unroll
        for (int k = 0; k < K; k++)
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc(b.p[k] + off, len), threadIdx.x * 16, 0, kNt);
        u32x4 x = v[0];
#pragma unroll
        for (int k = 1; k < K; k++)
            x ^= v[k];
        __builtin_amdgcn_raw_buffer_store_b128(x, rsrc(dst + off, len), threadIdx.x * 16, 0, POL);
    }
}

__device__ __forceinline__ bool tile_ok(uint64_t src, uint64_t dst, uint32_t bytes) {
    return bytes >= 16 && bytes <= kTile && (bytes & 15u) == 0 && ((src | dst) & 15u) == 0;
}

// mode 0: copy, 1: write `word` over the destination, 2: read the source
// Lane 0's v in scalar registers.  readfirstlane returns an int: each half
// goes through uint32_t, so the low word is not sign-extended into the high.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// The tile record is the same for the whole workgroup: read it once and keep
// it in scalar registers (the array is read-only here, so scalar loads may
// read it).
template <int MODE, int POL>
__global__ __launch_bounds__(kBlock) void tiles_kernel(const Tile *__restrict__ tiles, uint32_t n, uint32_t word) {
    uint32_t x = 0;
    const u32x4 w = {word, word, word, word};
    for (uint32_t i = blockIdx.x; i < n; i += gridDim.x) {
        const uint64_t src = uniform64(tiles[i].src), dst = uniform64(tiles[i].dst);
        const uint32_t bytes = (uint32_t)__builtin_amdgcn_readfirstlane(tiles[i].bytes);
        if (!tile_ok(src, dst, bytes))
            continue;
        if (MODE == 0) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc(src, bytes), threadIdx.x * 16, 0, kNt);
            __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(dst, bytes), threadIdx.x * 16, 0, POL);
        } else if (MODE == 1) {
            __builtin_amdgcn_raw_buffer_store_b128(w, rsrc(dst, bytes), threadIdx.x * 16, 0, POL);
        } else {
            x ^= fold(__builtin_amdgcn_raw_buffer_load_b128(rsrc(src, bytes), threadIdx.x * 16, 0, kNt));
        }
    }
    if (MODE == 2 && x == kMagic)
        tbr_sink[blockIdx.x & 63] = x;
}

thread_local std::string g_err;

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess)
        return TBR_OK;
    g_err = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
    return TBR_ERR_HIP;
}

unsigned grid_for(uint64_t units) {
    const uint64_t g = units < kMaxGrid ? units : kMaxGrid;
    return (unsigned)(g > 0 ? g : 1);
}

bool gather(const void *const *bufs, int32_t nbufs, Bufs *out) {
    if (bufs == nullptr || nbufs < 1 || nbufs > TBR_MAX_BUFS)
        return false;
    for (int32_t k = 0; k < nbufs; k++) {
        const uint64_t p = reinterpret_cast<uint64_t>(bufs[k]);
        if (p == 0 || (p & 15u) != 0)
            return false;
        out->p[k] = p;
    }
    for (int32_t k = nbufs; k < TBR_MAX_BUFS; k++)
        out->p[k] = 0;
    return true;
}

template <int K>
void launch_read(const Bufs &b, uint64_t bytes, hipStream_t s) {
    hipLaunchKernelGGL(read_kernel<K>, dim3(grid_for((bytes + kTile - 1) / kTile)), dim3(kBlock), 0, s, b, bytes);
}

template <int K, int POL>
void launch_write(const Bufs &b, uint64_t bytes, uint32_t word, hipStream_t s) {
    hipLaunchKernelGGL((write_kernel<K, POL>), dim3(grid_for((bytes + kTile - 1) / kTile)), dim3(kBlock), 0, s, b,
                       bytes, word);
}

template <int K>
void launch_write_pol(const Bufs &b, uint64_t bytes, uint32_t word, uint32_t policy, hipStream_t s) {
    if (policy == TBR_STORE_DEVICE)
        launch_write<K, kSc1>(b, bytes, word, s);
    else if (policy == TBR_STORE_NT)
        launch_write<K, kNt>(b, bytes, word, s);
    else
        launch_write<K, kNt | kSc0 | kSc1>(b, bytes, word, s);
}

template <int K>
void launch_combine(const Bufs &b, uint64_t dst, uint64_t bytes, uint32_t policy, hipStream_t s) {
    const dim3 grid(grid_for((bytes + kTile - 1) / kTile)), block(kBlock);
    if (policy == TBR_STORE_DEVICE)
        hipLaunchKernelGGL((combine_kernel<K, kSc1>), grid, block, 0, s, b, dst, bytes);
    else if (policy == TBR_STORE_NT)
        hipLaunchKernelGGL((combine_kernel<K, kNt>), grid, block, 0, s, b, dst, bytes);
    else
        hipLaunchKernelGGL((combine_kernel<K, kNt | kSc0 | kSc1>), grid, block, 0, s, b, dst, bytes);
}

// K in [1, TBR_MAX_BUFS - 1] by a compile-time table
template <int K>
void dispatch_combine(int32_t nsrcs, const Bufs &b, uint64_t dst, uint64_t bytes, uint32_t policy, hipStream_t s) {
    if constexpr (K < TBR_MAX_BUFS) {
        if (nsrcs == K) {
            launch_combine<K>(b, dst, bytes, policy, s);
            return;
        }
        dispatch_combine<K + 1>(nsrcs, b, dst, bytes, policy, s);
    }
}

// K in [1, TBR_MAX_BUFS] by a compile-time table
template <int K>
void dispatch(int32_t nbufs, const Bufs &b, uint64_t bytes, bool write, uint32_t word, uint32_t policy,
              hipStream_t s) {
    if constexpr (K <= TBR_MAX_BUFS) {
        if (nbufs == K) {
            if (write)
                launch_write_pol<K>(b, bytes, word, policy, s);
            else
                launch_read<K>(b, bytes, s);
            return;
        }
        dispatch<K + 1>(nbufs, b, bytes, write, word, policy, s);
    }
}

}  // namespace tbr

extern "C" {

const char *tbr_last_hip_error(void) { return tbr::g_err.c_str(); }

int tbr_read(const void *const *bufs, int32_t nbufs, uint64_t bytes_each, void *stream) {
    tbr::Bufs b;
    if (!tbr::gather(bufs, nbufs, &b) || (bytes_each & 15u) != 0)
        return TBR_ERR_INVALID;
    if (bytes_each == 0)
        return TBR_OK;
    tbr::dispatch<1>(nbufs, b, bytes_each, false, 0u, 0u, static_cast<hipStream_t>(stream));
    return tbr::hip_status(hipGetLastError(), "read launch");
}

int tbr_write(void *const *bufs, int32_t nbufs, uint64_t bytes_each, uint32_t word, uint32_t policy,
              void *stream) {
    tbr::Bufs b;
    if (!tbr::gather(const_cast<const void *const *>(bufs), nbufs, &b) || (bytes_each & 15u) != 0 ||
        policy > TBR_STORE_NT)
        return TBR_ERR_INVALID;
    if (bytes_each == 0)
        return TBR_OK;
    tbr::dispatch<1>(nbufs, b, bytes_each, true, word, policy, static_cast<hipStream_t>(stream));
    return tbr::hip_status(hipGetLastError(), "write launch");
}

int tbr_copy(void *dst, const void *src, uint64_t bytes, uint32_t policy, void *stream) {
    const uint64_t d = reinterpret_cast<uint64_t>(dst), sa = reinterpret_cast<uint64_t>(src);
    if (policy > TBR_STORE_NT || (bytes & 15u) != 0)
        return TBR_ERR_INVALID;
    if (bytes == 0)
        return TBR_OK;
    if (d == 0 || sa == 0 || ((d | sa) & 15u) != 0 || (sa < d + bytes && d < sa + bytes))
        return TBR_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(tbr::grid_for((bytes + tbr::kTile - 1) / tbr::kTile));
    if (policy == TBR_STORE_DEVICE)
        hipLaunchKernelGGL(tbr::copy_kernel<tbr::kSc1>, grid, dim3(tbr::kBlock), 0, s, d, sa, bytes);
    else if (policy == TBR_STORE_NT)
        hipLaunchKernelGGL(tbr::copy_kernel<tbr::kNt>, grid, dim3(tbr::kBlock), 0, s, d, sa, bytes);
    else
        hipLaunchKernelGGL(tbr::copy_kernel<tbr::kNt | tbr::kSc0 | tbr::kSc1>, grid, dim3(tbr::kBlock), 0, s, d, sa,
                           bytes);
    return tbr::hip_status(hipGetLastError(), "copy launch");
}

int tbr_combine(const void *const *srcs, int32_t nsrcs, void *dst, uint64_t bytes_each, uint32_t policy,
                void *stream) {
    tbr::Bufs b;
    const uint64_t d = reinterpret_cast<uint64_t>(dst);
    if (nsrcs < 1 || nsrcs >= TBR_MAX_BUFS || !tbr::gather(srcs, nsrcs, &b) || (bytes_each & 15u) != 0 ||
        policy > TBR_STORE_NT || d == 0 || (d & 15u) != 0)
        return TBR_ERR_INVALID;
    if (bytes_each == 0)
        return TBR_OK;
    for (int32_t k = 0; k < nsrcs; k++)
        if (b.p[k] < d + bytes_each && d < b.p[k] + bytes_each)
            return TBR_ERR_INVALID;
    tbr::dispatch_combine<1>(nsrcs, b, d, bytes_each, policy, static_cast<hipStream_t>(stream));
    return tbr::hip_status(hipGetLastError(), "combine launch");
}

static int tiles_launch(int mode, const tbr_tile *tiles_dev, uint32_t ntiles, uint32_t word, uint32_t policy,
                        void *stream) {
    if (policy > TBR_STORE_NT)
        return TBR_ERR_INVALID;
    if (ntiles == 0)
        return TBR_OK;
    if (tiles_dev == nullptr || (reinterpret_cast<uint64_t>(tiles_dev) & 7u) != 0)
        return TBR_ERR_INVALID;
    const tbr::Tile *t = reinterpret_cast<const tbr::Tile *>(tiles_dev);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(tbr::grid_for(ntiles)), block(tbr::kBlock);
    constexpr int kDev = tbr::kSc1, kStr = tbr::kNt | tbr::kSc0 | tbr::kSc1, kNtOnly = tbr::kNt;
    void (*kernel)(const tbr::Tile *, uint32_t, uint32_t);
    if (mode == 0)
        kernel = policy == TBR_STORE_DEVICE ? tbr::tiles_kernel<0, kDev>
                 : policy == TBR_STORE_NT   ? tbr::tiles_kernel<0, kNtOnly>
                                            : tbr::tiles_kernel<0, kStr>;
    else if (mode == 1)
        kernel = policy == TBR_STORE_DEVICE ? tbr::tiles_kernel<1, kDev>
                 : policy == TBR_STORE_NT   ? tbr::tiles_kernel<1, kNtOnly>
                                            : tbr::tiles_kernel<1, kStr>;
    else
        kernel = tbr::tiles_kernel<2, kStr>;
    hipLaunchKernelGGL(kernel, grid, block, 0, s, t, ntiles, word);
    return tbr::hip_status(hipGetLastError(), "tiles launch");
}

int tbr_tiles_copy(const tbr_tile *tiles_dev, uint32_t ntiles, uint32_t policy, void *stream) {
    return tiles_launch(0, tiles_dev, ntiles, 0u, policy, stream);
}

int tbr_tiles_write(const tbr_tile *tiles_dev, uint32_t ntiles, uint32_t word, uint32_t policy, void *stream) {
    return tiles_launch(1, tiles_dev, ntiles, word, policy, stream);
}

int tbr_tiles_read(const tbr_tile *tiles_dev, uint32_t ntiles, void *stream) {
    return tiles_launch(2, tiles_dev, ntiles, 0u, TBR_STORE_STREAMING, stream);
}

}  // extern "C"
