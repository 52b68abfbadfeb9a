// tb_host.cpp -- host half of libtb: argument checks, slice geometry and
// rotation, source preparation, launch dispatch, scratch and gate ownership.
#include <atomic>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <utility>

#include "tb.h"
#include "tb_internal.h"

namespace {
thread_local std::string g_last_hip_error;
// How the batched copy shares its long copies (TB_BC_*): process-wide.
std::atomic<int> g_batched_mode{TB_BC_NORMAL};
}  // namespace

namespace tbh {

int hip_fail(hipError_t e, const char *what) {
    g_last_hip_error = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
    return TB_ERR_HIP;
}

int batched_mode() { return g_batched_mode.load(std::memory_order_relaxed); }

bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

}  // namespace tbh

namespace {

using tbh::hip_fail;

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Per-device facts queried once.
struct DeviceInfo {
    bool valid = false;
    int cu_count = 0;
    uint64_t wall_clock_khz = 0;
};

std::mutex g_mu;
DeviceInfo g_dev[tbk::kMaxDevices];

int device_info(DeviceInfo *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= tbk::kMaxDevices)
        return TB_ERR_INVALID;
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceInfo &d = g_dev[dev];
    if (!d.valid) {
        int cus = 0, khz = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
        e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
        if (e != hipSuccess)
            return hip_fail(e, "hipDeviceGetAttribute(WallClockRate)");
        d.cu_count = cus;
        d.wall_clock_khz = khz > 0 ? (uint64_t)khz : 100000u;
        d.valid = true;
    }
    *out = d;
    return TB_OK;
}

// Batched-copy scratch, one per (device, stream), zeroed once at allocation,
// with the epoch of the last launch made on it.  Launches on one scratch must
// reach their stream in epoch order (each clears what the next one uses), so
// the epoch is taken and the launch enqueued under the scratch's own lock:
// threads sharing a stream (the legacy default stream, say) stay in order.
struct Scratch {
    void *mem = nullptr;
    uint64_t epoch = 0;
    std::mutex launch_mu;
};
std::map<std::pair<int, hipStream_t>, std::unique_ptr<Scratch>> g_scratch;

// The scratch for `stream` on the current device, created on first use.
int scratch_for(hipStream_t stream, Scratch **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_mu);
    auto key = std::make_pair(dev, stream);
    auto it = g_scratch.find(key);
    if (it != g_scratch.end()) {
        *out = it->second.get();
        return TB_OK;
    }
    void *p = nullptr;
    e = hipMalloc(&p, tbk::kBcScratchBytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        hip_fail(e, "hipMalloc(batched-copy scratch)");
        return TB_ERR_NOMEM;
    }
    // Synchronous clear: the scratch is then ready for any stream.
    e = hipMemset(p, 0, tbk::kBcScratchBytes);
    if (e != hipSuccess) {
        (void)hipFree(p);
        return hip_fail(e, "hipMemset(batched-copy scratch)");
    }
    std::unique_ptr<Scratch> sc(new (std::nothrow) Scratch);
    if (!sc) {
        (void)hipFree(p);
        return TB_ERR_NOMEM;
    }
    sc->mem = p;
    *out = sc.get();
    g_scratch[key] = std::move(sc);
    return TB_OK;
}

// Spin gate: flag and timeout marker in coherent (fine-grained) host memory.
uint32_t *g_gate = nullptr;   // [0] = release flag, [1] = timed-out marker

}  // namespace

extern "C" {

const char *tb_status_string(int status) {
    switch (status) {
    case TB_OK: return "ok";
    case TB_ERR_INVALID: return "invalid argument";
    case TB_ERR_HIP: return "HIP runtime error";
    case TB_ERR_NOMEM: return "out of device memory for library scratch";
    case TB_ERR_TIMEOUT: return "spin gate timed out";
    default: return "unknown status";
    }
}

const char *tb_last_hip_error(void) { return g_last_hip_error.c_str(); }

// K = ceil(R / numBytes), 1 when R == 0 or numBytes == 0.
int tb_num_slices(uint64_t num_bytes, uint64_t rotate_bytes, uint64_t *k_out) {
    if (k_out == nullptr)
        return TB_ERR_INVALID;
    if (rotate_bytes == 0 || num_bytes == 0 || num_bytes >= rotate_bytes) {
        *k_out = 1;
        return TB_OK;
    }
    // rotate_bytes - 1 cannot underflow here and the quotient cannot overflow
    *k_out = (rotate_bytes - 1) / num_bytes + 1;
    return TB_OK;
}

int tb_slice_stride(uint64_t num_bytes, uint64_t *stride_out) {
    if (stride_out == nullptr || num_bytes > UINT64_MAX - 255)
        return TB_ERR_INVALID;
    *stride_out = (num_bytes + 255) & ~(uint64_t)255;
    return TB_OK;
}

int tb_rotate_sources(const float *const *base, int32_t nsrc, uint64_t slice_stride_bytes,
                      uint64_t k, int64_t iteration, const float **out) {
    if (nsrc < 0 || nsrc > TB_MAX_SRCS || k == 0 || k > (uint64_t)INT64_MAX)
        return TB_ERR_INVALID;
    if (nsrc > 0 && (base == nullptr || out == nullptr))
        return TB_ERR_INVALID;
    // fold the (possibly negative) iteration into [0, k)
    const int64_t kk = (int64_t)k;
    int64_t slice = iteration % kk;
    if (slice < 0)
        slice += kk;
    const uint64_t s = (uint64_t)slice;
    if (s != 0 && slice_stride_bytes > UINT64_MAX / s)
        return TB_ERR_INVALID;
    const uint64_t offset = s * slice_stride_bytes;
    const float *tmp[TB_MAX_SRCS];
    for (int32_t b = 0; b < nsrc; b++) {
        const uintptr_t p = reinterpret_cast<uintptr_t>(base[b]);
        if (p > UINTPTR_MAX - offset)
            return TB_ERR_INVALID;
        tmp[b] = reinterpret_cast<const float *>(p + offset);
    }
    for (int32_t b = 0; b < nsrc; b++)
        out[b] = tmp[b];
    return TB_OK;
}

int tb_prep_sources(float *dev_base, uint64_t slice_stride_bytes, uint64_t k, const float *host_ref,
                    uint64_t nfloats, void *stream) {
    if (k == 0 || nfloats > UINT64_MAX / 4)
        return TB_ERR_INVALID;
    if (nfloats == 0)
        return TB_OK;
    const uint64_t nbytes = nfloats * 4;
    if (dev_base == nullptr || host_ref == nullptr || slice_stride_bytes < nbytes ||
        k > UINT64_MAX / slice_stride_bytes)
        return TB_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *base = reinterpret_cast<char *>(dev_base);
    hipError_t e = hipMemcpyAsync(base, host_ref, nbytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess)
        return hip_fail(e, "hipMemcpyAsync(slice 0)");
    // Replicate by doubling: slices [0, m) -> [m, 2m), so K slices take
    // ceil(log2 K) device-to-device copies.
    uint64_t have = 1;
    while (have < k) {
        const uint64_t count = have < k - have ? have : k - have;
        const uint64_t bytes = (count - 1) * slice_stride_bytes + nbytes;
        e = hipMemcpyAsync(base + have * slice_stride_bytes, base, bytes, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess)
            return hip_fail(e, "hipMemcpyAsync(slice replicas)");
        have += count;
    }
    return TB_OK;
}

int tb_reduce_copy_ex(float *dst, const float *const *srcs, int32_t nsrc, uint64_t nfloats,
                      uint32_t memset_byte, void *stream) {
    if (nsrc < 0 || nsrc > TB_MAX_SRCS || memset_byte > 255u)
        return TB_ERR_INVALID;
    if (nfloats == 0)
        return TB_OK;
    if (nfloats > UINT64_MAX / 4 || dst == nullptr || !aligned4(dst) || (nsrc > 0 && srcs == nullptr))
        return TB_ERR_INVALID;
    const uint64_t nbytes = nfloats * 4;
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst);
    if (d0 > UINTPTR_MAX - nbytes)
        return TB_ERR_INVALID;

    tbk::ReduceArgs a;
    memset(&a, 0, sizeof(a));
    a.dst = dst;
    a.n = nfloats;
    a.fill = memset_byte * 0x01010101u;
    for (int32_t k = 0; k < nsrc; k++) {
        const float *p = srcs[k];
        if (p == nullptr || !aligned4(p))
            return TB_ERR_INVALID;
        const uintptr_t s0 = reinterpret_cast<uintptr_t>(p);
        if (s0 > UINTPTR_MAX - nbytes)
            return TB_ERR_INVALID;
        // dst may be exactly a source (each element is read before it is
        // written by the same thread), never partly overlap one.
        if (s0 != d0 && s0 < d0 + nbytes && d0 < s0 + nbytes)
            return TB_ERR_INVALID;
        a.src[k] = p;
    }
    // Vector split: floats before dst's first 16-byte boundary, float4 body, rest.
    uint64_t head = ((16u - (d0 & 15u)) & 15u) / 4u;
    if (head > nfloats)
        head = nfloats;
    a.head = (uint32_t)head;
    a.nvec = (nfloats - head) / 4;
    a.tail = (uint32_t)((nfloats - head) % 4);
    // The vector path needs every source to agree with dst modulo 16 (its
    // element `head` then starts a 16-byte block); otherwise the unaligned
    // kernel reads each source at its own 4-byte alignment.
    bool vector_path = true;
    for (int32_t k = 0; k < nsrc; k++) {
        const uintptr_t body = reinterpret_cast<uintptr_t>(a.src[k]) + 4u * head;
        if ((body & 15u) != 0)
            vector_path = false;
    }

    DeviceInfo info;
    int rc = device_info(&info);
    if (rc != TB_OK)
        return rc;
    hipError_t e = tbk::launch_reduce_copy(a, nsrc, vector_path, info.cu_count,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "reduce-copy launch");
    return TB_OK;
}

int tb_reduce_copy(float *dst, const float *const *srcs, int32_t nsrc, uint64_t nfloats, void *stream) {
    return tb_reduce_copy_ex(dst, srcs, nsrc, nfloats, 0u, stream);
}

int tb_batched_set_mode(int32_t mode) {
    if (mode != TB_BC_NORMAL && mode != TB_BC_NO_WAIT && mode != TB_BC_NO_PIECES)
        return TB_ERR_INVALID;
    g_batched_mode.store(mode, std::memory_order_relaxed);
    return TB_OK;
}

int tb_batched_set_max_workgroups(uint32_t max_workgroups) {
    tbk::set_batched_max_workgroups(max_workgroups);
    return TB_OK;
}

int tb_batched_copy(const tb_copy_desc *desc_dev, uint32_t ncopies, void *stream) {
    if (ncopies == 0)
        return TB_OK;
    if (desc_dev == nullptr || (reinterpret_cast<uintptr_t>(desc_dev) & 7u) != 0)
        return TB_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (tbh::capturing(s))
        return TB_ERR_INVALID;
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc != TB_OK)
        return rc;
    Scratch *sc = nullptr;
    rc = scratch_for(s, &sc);
    if (rc != TB_OK)
        return rc;
    const int mode = g_batched_mode.load(std::memory_order_relaxed);
    const uint64_t wait_ticks =
        mode == TB_BC_NORMAL ? (uint64_t)tbk::kBcSealWaitUs * info.wall_clock_khz / 1000u : 0u;
    std::lock_guard<std::mutex> lk(sc->launch_mu);
    const uint64_t epoch = sc->epoch + 1;    // from 1; 64 bits never wrap in practice
    hipError_t e = tbk::launch_batched_copy(desc_dev, ncopies, static_cast<tbk::BcScratch *>(sc->mem), epoch,
                                            info.cu_count, wait_ticks, mode == TB_BC_NO_PIECES, s);
    if (e != hipSuccess)
        return hip_fail(e, "batched-copy launch");   // the epoch is not used up
    sc->epoch = epoch;
    return TB_OK;
}

int tb_batched_copy_noalloc(const tb_copy_desc *desc_dev, uint32_t ncopies, void *stream) {
    if (ncopies == 0)
        return TB_OK;
    if (desc_dev == nullptr || (reinterpret_cast<uintptr_t>(desc_dev) & 7u) != 0)
        return TB_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (tbh::capturing(s))
        return TB_ERR_INVALID;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= tbk::kMaxDevices)
        return TB_ERR_INVALID;
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc != TB_OK)
        return rc;
    const int mode = g_batched_mode.load(std::memory_order_relaxed);
    const uint64_t wait_ticks =
        mode == TB_BC_NORMAL ? (uint64_t)tbk::kBcSealWaitUs * info.wall_clock_khz / 1000u : 0u;
    e = tbk::launch_batched_copy_static(desc_dev, ncopies, dev, info.cu_count, wait_ticks, mode == TB_BC_NO_PIECES,
                                        s);
    if (e != hipSuccess)
        return hip_fail(e, "batched-copy launch on the static scratch");
    return TB_OK;
}

int tb_time_next_launch(void *start_event, void *stop_event) {
    tbk::set_next_launch_events(static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
    return TB_OK;
}

int tb_spin_gate_arm(uint32_t timeout_ms, void *stream) {
    if (timeout_ms == 0 || timeout_ms > 60000)
        return TB_ERR_INVALID;
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc != TB_OK)
        return rc;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (g_gate == nullptr) {
            void *p = nullptr;
            hipError_t e = hipHostMalloc(&p, 256, hipHostMallocCoherent);
            if (e != hipSuccess)
                return hip_fail(e, "hipHostMalloc(spin gate)");
            g_gate = static_cast<uint32_t *>(p);
        }
        __atomic_store_n(&g_gate[0], 0u, __ATOMIC_SEQ_CST);
        __atomic_store_n(&g_gate[1], 0u, __ATOMIC_SEQ_CST);
    }
    const uint64_t ticks = (uint64_t)timeout_ms * info.wall_clock_khz;
    hipError_t e = tbk::launch_spin_gate(g_gate, g_gate + 1, ticks, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "spin-gate launch");
    return TB_OK;
}

int tb_spin_gate_release(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_gate == nullptr)
        return TB_ERR_INVALID;
    __atomic_store_n(&g_gate[0], 1u, __ATOMIC_SEQ_CST);
    return TB_OK;
}

int tb_spin_gate_status(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_gate == nullptr)
        return TB_ERR_INVALID;
    return __atomic_load_n(&g_gate[1], __ATOMIC_SEQ_CST) ? TB_ERR_TIMEOUT : TB_OK;
}

int tb_launch_info(uint64_t nfloats, int32_t nsrc, uint32_t ncopies, int32_t *cu_count,
                   int32_t *reduce_blocks, int32_t *batched_blocks) {
    if (nsrc < 0 || nsrc > TB_MAX_SRCS)
        return TB_ERR_INVALID;
    DeviceInfo info;
    int rc = device_info(&info);
    if (rc != TB_OK)
        return rc;
    if (cu_count)
        *cu_count = info.cu_count;
    if (reduce_blocks)
        *reduce_blocks = tbk::reduce_grid(nfloats, nsrc, true, info.cu_count);
    if (batched_blocks)
        *batched_blocks = tbk::batched_grid(ncopies, info.cu_count);
    return TB_OK;
}

int tb_shutdown(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_scratch.empty() && g_gate == nullptr)
        return TB_OK;
    int current = 0;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    // every device that holds scratch finishes its work before the scratch
    // goes; an entry leaves the table as its memory is freed, so a failure
    // part-way leaves only live scratch behind
    for (auto it = g_scratch.begin(); it != g_scratch.end();) {
        e = hipSetDevice(it->first.first);
        if (e == hipSuccess)
            e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            (void)hipSetDevice(current);
            return hip_fail(e, "hipDeviceSynchronize");
        }
        (void)hipFree(it->second->mem);
        it = g_scratch.erase(it);
    }
    e = hipSetDevice(current);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();   // the spin gate's device
    if (e != hipSuccess)
        return hip_fail(e, "hipDeviceSynchronize");
    if (g_gate != nullptr) {
        (void)hipHostFree(g_gate);
        g_gate = nullptr;
    }
    return TB_OK;
}

}  // extern "C"
