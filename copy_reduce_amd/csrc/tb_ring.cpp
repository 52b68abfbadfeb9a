// tb_ring.cpp -- descriptor-slot ring: batched copies submitted from host
// descriptor lists, with slots held until their launch's event fires
// (Mooncake RFC #5041, Design of #5040, "Descriptor slots" and "Host trims").
//
// Everything a submit needs is resolved once, at creation: the device's CU
// count and wall-clock rate, the ring's own batched-copy scratch and its
// launch counter, pinned slots and events.  A submit then does no lookups,
// takes no locks and sets no device: it checks and copies the descriptors,
// enqueues (copy,) kernel and event, and returns.  Because the ring sees every
// length on the host, a slot whose copies are all short is launched without
// the long-copy queue and with a grid sized to its descriptors.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>

#include "tb.h"
#include "tb_internal.h"

struct tb_ring {
    int device = 0;
    hipStream_t stream = nullptr;
    uint32_t nslots = 0;
    uint32_t slot_descs = 0;
    uint32_t flags = 0;
    int cu_count = 0;
    uint64_t wait_ticks = 0;              // longest queue wait of the batched copy, device ticks
    tb_copy_desc *host = nullptr;         // nslots * slot_descs, pinned
    tb_copy_desc *host_dev = nullptr;     // the device's address of `host` (direct rings)
    tb_copy_desc *dev = nullptr;          // device copy of every slot (staged rings only)
    hipEvent_t *event = nullptr;          // one per slot
    uint64_t *held_by = nullptr;          // ticket of the launch holding each slot (0: none yet)
    tbk::BcScratch *scratch = nullptr;    // this ring's batched-copy scratch
    uint64_t next_ticket = 1;             // also the epoch of the next launch on `scratch`
    uint64_t done_upto = 0;               // every ticket <= this one has finished
};

namespace {

constexpr uint32_t kMaxSlots = 1024;
constexpr uint32_t kMaxSlotDescs = 1u << 20;

// Release whatever `r` holds (after its launches have finished).
void release(tb_ring *r) {
    if (r->event != nullptr) {
        for (uint32_t k = 0; k < r->nslots; k++)
            if (r->event[k] != nullptr)
                (void)hipEventDestroy(r->event[k]);
        delete[] r->event;
    }
    delete[] r->held_by;
    if (r->host != nullptr)
        (void)hipHostFree(r->host);
    if (r->dev != nullptr)
        (void)hipFree(r->dev);
    if (r->scratch != nullptr)
        (void)hipFree(r->scratch);
    delete r;
}

bool range_ok(uint64_t base, uint64_t bytes) { return base != 0 && base <= UINT64_MAX - bytes; }

// Wait until the launch holding slot k (if any) has finished.
int free_slot(tb_ring *r, uint32_t k) {
    const uint64_t t = r->held_by[k];
    if (t == 0 || t <= r->done_upto)
        return TB_OK;
    hipError_t e = hipEventSynchronize(r->event[k]);
    if (e != hipSuccess)
        return tbh::hip_fail(e, "hipEventSynchronize(ring slot)");
    r->done_upto = t;
    return TB_OK;
}

}  // namespace

extern "C" {

int tb_ring_create(uint32_t nslots, uint32_t slot_descs, uint32_t flags, void *stream, tb_ring **out) {
    if (out == nullptr || nslots == 0 || nslots > kMaxSlots || slot_descs == 0 || slot_descs > kMaxSlotDescs ||
        (flags != TB_RING_STAGED && flags != TB_RING_DIRECT))
        return TB_ERR_INVALID;
    *out = nullptr;
    tb_ring *r = new (std::nothrow) tb_ring;
    if (r == nullptr)
        return TB_ERR_NOMEM;
    r->stream = static_cast<hipStream_t>(stream);
    r->nslots = nslots;
    r->slot_descs = slot_descs;
    r->flags = flags;
    hipError_t e = hipGetDevice(&r->device);
    int khz = 0;
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&r->cu_count, hipDeviceAttributeMultiprocessorCount, r->device);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, r->device);
    if (e != hipSuccess) {
        release(r);
        return tbh::hip_fail(e, "device query (ring)");
    }
    r->wait_ticks = (uint64_t)tbk::kBcSealWaitUs * (uint64_t)(khz > 0 ? khz : 100000) / 1000u;

    r->event = new (std::nothrow) hipEvent_t[nslots]();
    r->held_by = new (std::nothrow) uint64_t[nslots]();
    if (r->event == nullptr || r->held_by == nullptr) {
        release(r);
        return TB_ERR_NOMEM;
    }
    const size_t bytes = (size_t)nslots * slot_descs * sizeof(tb_copy_desc);
    // A direct ring's slots are read by the kernel while it runs: coherent
    // (fine-grained) host memory.  A staged ring's are read by a copy only.
    e = hipHostMalloc(reinterpret_cast<void **>(&r->host), bytes,
                      flags == TB_RING_DIRECT ? hipHostMallocCoherent : hipHostMallocDefault);
    if (e != hipSuccess) {
        r->host = nullptr;
        release(r);
        tbh::hip_fail(e, "hipHostMalloc(ring slots)");
        return TB_ERR_NOMEM;
    }
    if (flags == TB_RING_DIRECT) {
        e = hipHostGetDevicePointer(reinterpret_cast<void **>(&r->host_dev), r->host, 0);
        if (e != hipSuccess) {
            release(r);
            return tbh::hip_fail(e, "hipHostGetDevicePointer(ring slots)");
        }
    } else {
        e = hipMalloc(reinterpret_cast<void **>(&r->dev), bytes);
        if (e != hipSuccess) {
            r->dev = nullptr;
            release(r);
            tbh::hip_fail(e, "hipMalloc(ring slots)");
            return TB_ERR_NOMEM;
        }
    }
    e = hipMalloc(reinterpret_cast<void **>(&r->scratch), tbk::kBcScratchBytes);
    if (e != hipSuccess) {
        r->scratch = nullptr;
        release(r);
        tbh::hip_fail(e, "hipMalloc(ring scratch)");
        return TB_ERR_NOMEM;
    }
    // synchronous clear: the scratch is ready before the first launch
    e = hipMemset(r->scratch, 0, tbk::kBcScratchBytes);
    for (uint32_t k = 0; e == hipSuccess && k < nslots; k++)
        e = hipEventCreateWithFlags(&r->event[k], hipEventDisableTiming);
    if (e != hipSuccess) {
        release(r);
        return tbh::hip_fail(e, "ring set-up");
    }
    *out = r;
    return TB_OK;
}

int tb_ring_submit(tb_ring *r, const tb_copy_desc *host_desc, uint64_t n, uint64_t *ticket) {
    if (r == nullptr || ticket == nullptr || (n > 0 && host_desc == nullptr))
        return TB_ERR_INVALID;
    if (n > 0 && tbh::capturing(r->stream))
        return TB_ERR_INVALID;
    // the whole request is checked before any part of it is enqueued
    for (uint64_t i = 0; i < n; i++) {
        const tb_copy_desc &d = host_desc[i];
        if (d.bytes != 0 && !(range_ok(d.src, d.bytes) && range_ok(d.dst, d.bytes)))
            return TB_ERR_INVALID;
    }
    const int mode = tbh::batched_mode();
    const uint64_t wait_ticks = mode == TB_BC_NORMAL ? r->wait_ticks : 0u;
    for (uint64_t i0 = 0; i0 < n; i0 += r->slot_descs) {
        const uint32_t m = (uint32_t)(n - i0 < r->slot_descs ? n - i0 : r->slot_descs);
        const uint64_t t = r->next_ticket;
        const uint32_t k = (uint32_t)((t - 1) % r->nslots);
        int rc = free_slot(r, k);
        if (rc != TB_OK) {
            *ticket = r->next_ticket - 1;
            return rc;
        }
        tb_copy_desc *slot = r->host + (size_t)k * r->slot_descs;
        bool any_long = false;
        for (uint32_t i = 0; i < m; i++) {
            slot[i] = host_desc[i0 + i];
            any_long |= slot[i].bytes > tbk::kBcSplitAbove;
        }
        const tb_copy_desc *read_from = nullptr;
        hipError_t e = hipSuccess;
        if (r->flags == TB_RING_STAGED) {
            tb_copy_desc *dslot = r->dev + (size_t)k * r->slot_descs;
            e = hipMemcpyAsync(dslot, slot, (size_t)m * sizeof(tb_copy_desc), hipMemcpyHostToDevice, r->stream);
            if (e != hipSuccess) {
                *ticket = r->next_ticket - 1;
                return tbh::hip_fail(e, "hipMemcpyAsync(ring slot)");
            }
            read_from = dslot;
        } else {
            read_from = r->host_dev + (size_t)k * r->slot_descs;
        }
        // The ring sees every length: a slot without long copies skips the
        // queue.  The slot's event is the launch's own stop event, which saves
        // the separate record command (about half the host cost of a submit).
        if (any_long)
            e = tbk::launch_batched_copy(read_from, m, r->scratch, t, r->cu_count, wait_ticks,
                                         mode == TB_BC_NO_PIECES, r->stream, r->event[k]);
        else
            e = tbk::launch_batched_copy_short(read_from, m, r->scratch, t, r->cu_count, r->stream, r->event[k]);
        if (e != hipSuccess) {
            *ticket = r->next_ticket - 1;
            return tbh::hip_fail(e, "batched-copy launch (ring)");
        }
        r->held_by[k] = t;
        r->next_ticket = t + 1;
    }
    *ticket = r->next_ticket - 1;
    return TB_OK;
}

int tb_ring_poll(tb_ring *r, uint64_t ticket, int32_t *done) {
    if (r == nullptr || done == nullptr || ticket >= r->next_ticket)
        return TB_ERR_INVALID;
    if (ticket <= r->done_upto) {
        *done = 1;
        return TB_OK;
    }
    // ticket > done_upto: its slot has not been handed out again since
    const uint32_t k = (uint32_t)((ticket - 1) % r->nslots);
    hipError_t e = hipEventQuery(r->event[k]);
    if (e == hipSuccess) {
        r->done_upto = ticket;
        *done = 1;
        return TB_OK;
    }
    if (e == hipErrorNotReady) {
        *done = 0;
        return TB_OK;
    }
    return tbh::hip_fail(e, "hipEventQuery(ring slot)");
}

int tb_ring_wait(tb_ring *r, uint64_t ticket) {
    if (r == nullptr || ticket >= r->next_ticket)
        return TB_ERR_INVALID;
    if (ticket == 0)
        return TB_OK;
    return free_slot(r, (uint32_t)((ticket - 1) % r->nslots));
}

int tb_ring_destroy(tb_ring *r) {
    if (r == nullptr)
        return TB_OK;
    int rc = TB_OK;
    // the last launch finishing means every earlier one has
    if (r->next_ticket > 1)
        rc = tb_ring_wait(r, r->next_ticket - 1);
    release(r);
    return rc;
}

}  // extern "C"
