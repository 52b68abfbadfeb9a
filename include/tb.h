/*
 * tb.h -- C ABI of libtb, the MI355X (gfx950) transfer hot path.
 *
 * Two operations run on the GPU:
 *   - a multi-source fp32 reduce-copy, dst = src0 + src1 + ... + srcN-1 in a
 *     fixed left-to-right order (a copy for N = 1, a memset for N = 0), read
 *     through rotated source slices so that repeated launches cannot be served
 *     from cache;
 *   - a batched copy that runs a whole (src, dst, bytes) descriptor array in
 *     one launch, also submitted from host descriptor lists through a ring of
 *     descriptor slots.
 *
 * Conventions for every entry point:
 *   - Calls return a tb_status and never throw; the library prints nothing.
 *   - "device pointer" means memory of the current HIP device (hipMalloc or a
 *     torch CUDA tensor); "host pointer" means ordinary process memory.
 *   - `stream` is a hipStream_t of the current device passed as void*; NULL
 *     is the legacy default stream.  GPU work is only enqueued: no call below synchronises unless it
 *     says so, and the library never touches a stream it was not given.
 *   - The caller owns every buffer it passes.  The library owns only the
 *     batched-copy scratch and the spin-gate flag (freed by tb_shutdown) and
 *     what a descriptor-slot ring holds (freed by tb_ring_destroy).
 *   - TB_ERR_HIP means a HIP runtime call failed; tb_last_hip_error() gives
 *     its text.  Faults inside a kernel surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - There is no fallback path: if a kernel cannot be launched the call fails.
 */
#ifndef TB_H
#define TB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tb_status {
    TB_OK = 0,
    TB_ERR_INVALID = -1,   /* bad argument; nothing was enqueued          */
    TB_ERR_HIP = -2,       /* a HIP runtime call failed                   */
    TB_ERR_NOMEM = -3,     /* library scratch could not be allocated      */
    TB_ERR_TIMEOUT = -4    /* the spin gate gave up before it was released */
} tb_status;

/* Most sources one reduce-copy takes. */
#define TB_MAX_SRCS 16

/*
 * One copy of a batch, Mooncake RFC #5041 "HipTransport", Design of #5040:
 * a launch runs an array of (src, dst, len) descriptors.  src and dst are
 * device addresses, bytes the length; 24 bytes, 8-byte aligned.
 */
typedef struct tb_copy_desc {
    uint64_t src;
    uint64_t dst;
    uint64_t bytes;
} tb_copy_desc;

/* Source pattern kinds, "TransferBench data validation", Expected source pattern. */
enum {
    TB_FILL_DEFAULT = 0,   /* PrepSrcValue closed form                         */
    TB_FILL_PATTERN = 1,   /* fillPattern: a float vector repeated             */
    TB_FILL_COMPRESS = 2   /* fillCompress: random floats, per-line zeroing mix */
};

typedef struct tb_fill_cfg {
    int32_t kind;               /* TB_FILL_*                                       */
    uint32_t compress_pct[5];   /* % of 64-byte lines: random, 1B0, 2B0, 4B0, 32B0 */
    const float *pattern;       /* host array for TB_FILL_PATTERN                  */
    uint64_t pattern_len;       /* its length in floats, > 0                       */
    uint64_t seed;              /* TB_FILL_COMPRESS seed                           */
} tb_fill_cfg;

/* ------------------------------------------------------------------------ */
/* Host-only calls (no GPU needed)                                           */
/* ------------------------------------------------------------------------ */

/*
 * Number of identical source slices K for a transfer of num_bytes with
 * SRC_ROTATE_BYTES = rotate_bytes: K = ceil(rotate_bytes / num_bytes), and 1
 * when rotate_bytes is 0 (rotation off) or num_bytes is 0.
 * TransferBench PR #365 "Fix one-sided remote-read bandwidth inflation via
 * source-slice rotation (SRC_ROTATE_BYTES)", Technical Details.
 * Errors: TB_ERR_INVALID if k_out is NULL.
 */
int tb_num_slices(uint64_t num_bytes, uint64_t rotate_bytes, uint64_t *k_out);

/*
 * Byte distance between consecutive slices of one source: num_bytes rounded up
 * to a multiple of 256, so every slice starts aligned for 16-byte vector loads
 * (PR #365 review, "Align replicated source slices for vector loads").  A
 * source with K slices needs K * stride bytes.
 * Errors: TB_ERR_INVALID if stride_out is NULL or the rounding overflows.
 */
int tb_slice_stride(uint64_t num_bytes, uint64_t *stride_out);

/*
 * PrepareReference: fill host_out[0 .. nfloats) with the reference data of
 * source buffer buffer_idx ("TransferBench data validation", Expected source
 * pattern).  cfg may be NULL for the default pattern
 *   PrepSrcValue(b, i) = (((i % 383) * 517) % 383 + 31) * (b + 1)
 * evaluated on the integer index i.  TB_FILL_PATTERN repeats cfg->pattern.
 * TB_FILL_COMPRESS draws, per 64-byte line, a category (random, 1B0, 2B0, 4B0,
 * 32B0) by cfg->compress_pct; each float is a multiple of 2^-23 in [-1, 1)
 * from a SplitMix64 stream, and category nB0 zeroes the line's leading n bytes.
 * host_out: host memory of nfloats floats, written only.
 * Errors: TB_ERR_INVALID for NULL host_out with nfloats > 0, buffer_idx < 0,
 * an unknown kind, an empty pattern, or percentages not summing to 100.
 */
int tb_prep_reference(float *host_out, uint64_t nfloats, int32_t buffer_idx,
                      const tb_fill_cfg *cfg);

/*
 * Source-slice rotation for one iteration (PR #365, Technical Details:
 * RotateSourceSlices; iteration i reads slice i mod K, folded into [0, K) so
 * that negative warmup indices work):
 *   out[b] = base[b] + ((iteration mod k + k) mod k) * slice_stride_bytes.
 * base and out: host arrays of nsrc device addresses (out may equal base).
 * Pure host arithmetic, meant to run outside any timed region.
 * Errors: TB_ERR_INVALID for NULL arrays with nsrc > 0, nsrc outside
 * [0, TB_MAX_SRCS], k == 0, or an address that would overflow.
 */
int tb_rotate_sources(const float *const *base, int32_t nsrc,
                      uint64_t slice_stride_bytes, uint64_t k, int64_t iteration,
                      const float **out);

/* Text for a tb_status value (static storage). */
const char *tb_status_string(int status);

/* Text of the last failing HIP call on this thread, or "" (thread-local). */
const char *tb_last_hip_error(void);

/* ------------------------------------------------------------------------ */
/* GPU calls                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * Initialise the K slices of one source (PR #365, Technical Details, "Prep
 * fill"): copy host_ref (nfloats floats, host memory) into slice 0 of dev_base,
 * then replicate slice 0 device-to-device into slices 1 .. K-1, so the
 * host-to-device traffic stays at one slice.  dev_base must hold
 * k * slice_stride_bytes bytes.  Enqueued on `stream`; host_ref must stay
 * valid until the stream has passed the copy (pageable memory is copied
 * before the call returns).
 * Errors: TB_ERR_INVALID for NULL pointers with nfloats > 0, k == 0,
 * slice_stride_bytes < 4 * nfloats, or size overflow; TB_ERR_HIP.
 */
int tb_prep_sources(float *dev_base, uint64_t slice_stride_bytes, uint64_t k,
                    const float *host_ref, uint64_t nfloats, void *stream);

/*
 * Reduce-copy ("TransferBench data validation", expected-value table and
 * Expected destination): for every j < nfloats
 *   nsrc == 0: dst bytes set to 0x00;
 *   nsrc == 1: dst[j] = srcs[0][j], a bitwise copy;
 *   nsrc >= 2: dst[j] = (...((srcs[0][j] + srcs[1][j]) + srcs[2][j]) ...)
 *              + srcs[nsrc-1][j], binary32 additions rounded to nearest-even,
 *              in exactly this order (subnormals kept).
 * dst: device pointer to nfloats floats; srcs: HOST array of nsrc device
 * pointers (read during the call only).  All pointers 4-byte aligned.  When
 * every source shares dst's address modulo 16 the sources are read as aligned
 * 16-byte vectors; otherwise, up to seven sources, each is read with 16-byte
 * loads at its own 4-byte alignment, and from eight up with aligned 16-byte
 * loads staged through LDS and read back at its offset (0-6 points of HBM peak
 * slower than aligned at 256 MiB per buffer).
 * dst may be exactly equal to a source; any other overlap between dst and a
 * source is rejected.  Enqueues one kernel on `stream`.  nfloats == 0 is a
 * no-op.
 * Errors: TB_ERR_INVALID for NULL pointers with nfloats > 0, nsrc outside
 * [0, TB_MAX_SRCS], misaligned pointers, partial overlap, or size overflow;
 * TB_ERR_HIP if the launch failed.
 */
int tb_reduce_copy(float *dst, const float *const *srcs, int32_t nsrc,
                   uint64_t nfloats, void *stream);

/* As tb_reduce_copy, with the byte written for nsrc == 0 given explicitly
 * (the MEMSET_CHAR of dstReference[0]); memset_byte must be <= 255. */
int tb_reduce_copy_ex(float *dst, const float *const *srcs, int32_t nsrc,
                      uint64_t nfloats, uint32_t memset_byte, void *stream);

/*
 * Batched copy (Mooncake RFC #5041, Design of #5040): for every descriptor d
 * of desc_dev[0 .. ncopies), copy d.bytes bytes from d.src to d.dst, all in one
 * kernel launch.  desc_dev is a DEVICE array that must stay valid and
 * unchanged until the stream has passed the kernel.  Any alignment and any
 * length work: 16-byte vectors where src and dst agree modulo 16, otherwise
 * aligned 16-byte blocks realigned in registers (about 5% slower on C4's
 * copies); zero-length descriptors are skipped; ncopies == 0 is a no-op.
 * Destinations must be pairwise disjoint and disjoint from every source;
 * overlapping descriptors give unspecified bytes in the overlap (not checked:
 * the descriptors are in device memory).
 * The kernel uses a small library-owned scratch area per (device, stream),
 * allocated on the first call for that pair; calls on one stream are ordered,
 * calls on different streams use different scratch (each launch relies on the
 * previous launch on its scratch having finished).  The scratch is found by
 * the stream's handle: synchronise a stream before destroying it if a new
 * stream could be created with the same handle while its copy still runs.
 * Several host threads may call this on one stream: launches are numbered and
 * enqueued under the scratch's lock, so they reach the stream in order.
 * Not for HIP graph capture: each launch is numbered on its scratch when it
 * is enqueued, and a replayed capture would repeat the number, so a call on a
 * capturing stream is refused (the reduce-copy has no such state and may be
 * captured).
 * Errors: TB_ERR_INVALID for a NULL or misaligned desc_dev with ncopies > 0,
 * or a stream under capture; TB_ERR_NOMEM if the scratch cannot be
 * allocated; TB_ERR_HIP.
 */
int tb_batched_copy(const tb_copy_desc *desc_dev, uint32_t ncopies, void *stream);

/*
 * tb_batched_copy without allocation, for callers that cannot allocate device
 * memory (tight serving loops, harnesses that forbid hipMalloc): the same
 * kernel and the same result as tb_batched_copy, with its scratch in a static
 * device array of the library (131,840 bytes per device, held until the
 * process ends) instead of memory allocated per (device, stream).  No call
 * allocates: the first call on a device takes the array's address and clears
 * it, synchronising `stream` once; later calls only enqueue the kernel.  The
 * scratch's size does not depend on the batch (long copies beyond its queue
 * are copied by the wave that finds them), so every ncopies that
 * tb_batched_copy takes is taken here.
 * Every call on one device shares that device's array: calls whose kernels can
 * overlap in time on one device (different streams not ordered by the caller,
 * or this call beside itself on another thread's unordered stream) race and
 * give unspecified bytes.  Calls on one stream are ordered and safe, from any
 * number of host threads.  Launches are numbered per device, and the array
 * keeps the last launch's state, which the next launch expects: nothing needs
 * clearing between calls.  Refused on a stream under graph capture, as
 * tb_batched_copy.
 * Errors: as tb_batched_copy (TB_ERR_INVALID for a NULL or misaligned
 * desc_dev with ncopies > 0, a stream under capture, or a device ordinal of 64
 * or more; TB_ERR_HIP if the array's address, its clear or the launch fails);
 * never TB_ERR_NOMEM.
 */
int tb_batched_copy_noalloc(const tb_copy_desc *desc_dev, uint32_t ncopies, void *stream);

/*
 * Test hook for the batched copy's recovery path (process-wide; affects
 * launches made after the call).  Long copies go through a queue whose pieces
 * the waves share once every scanning workgroup has published; the wait for
 * that is bounded, and a wave that gives up leaves its pieces to the first
 * wave of the launch that gave up, which copies every long copy of the batch
 * whole.  Modes:
 *   TB_BC_NORMAL     waves wait up to 200 us of device time (the default);
 *   TB_BC_NO_WAIT    waves do not wait: any that find the queue unfinished
 *                    give up;
 *   TB_BC_NO_PIECES  no wave takes pieces: one wave copies every long copy.
 * The bytes written are identical in every mode; only the speed differs.
 * Errors: TB_ERR_INVALID for an unknown mode.
 */
enum { TB_BC_NORMAL = 0, TB_BC_NO_WAIT = 1, TB_BC_NO_PIECES = 2 };
int tb_batched_set_mode(int32_t mode);

/*
 * Compute-unit budget of the batched copy (Mooncake RFC #5041, Design of
 * #5040, "Interference with compute", and open question 4 on CU controls):
 * every later batched-copy launch, through tb_batched_copy or a ring, uses at
 * most max_workgroups workgroups of 256 threads (rounded down to a multiple
 * of 8, at least 8); 0 removes the cap (the default).  Fewer workgroups leave
 * compute units to concurrent kernels; each wave then copies more
 * descriptors.  The bytes written do not depend on the cap.  Process-wide.
 * Always TB_OK.
 */
int tb_batched_set_max_workgroups(uint32_t max_workgroups);

/*
 * Descriptor-slot ring (Mooncake RFC #5041, Design of #5040, "Descriptor
 * slots" and "Host trims"): batched copies whose descriptors the caller holds
 * in HOST memory, submitted without blocking and polled for completion.
 *
 * A ring is bound at creation to the current device and to `stream`, and
 * owns: nslots slots of slot_descs descriptors each in pinned host memory;
 * unless TB_RING_DIRECT, a device copy of every slot; one completion event
 * per slot; and its own batched-copy scratch.  tb_ring_submit takes the
 * caller's descriptors into the next slot, enqueues on the ring's stream
 *   TB_RING_STAGED: a host-to-device copy of the slot, then the batched copy
 *                   reading the device copy;
 *   TB_RING_DIRECT: the batched copy reading the pinned slot over the bus,
 * records the slot's event, and returns a ticket.  A slot stays held until
 * its event has fired.  Slots are used in turn, so when the next one is still
 * held, submit blocks until the launch holding it (the oldest in flight) has
 * finished: the wait depends only on the GPU's progress, never on the caller
 * polling.  A request of more than slot_descs descriptors takes several slots
 * (one launch each, in order) and its ticket is that of the last.
 *
 * Tickets count launches on the ring from 1.  Launches on one stream finish
 * in order, so ticket t done means every ticket <= t is done; the ring keeps
 * the highest ticket seen done and answers polls at or below it without
 * asking the runtime again.  Ticket 0 (what an empty first submit returns)
 * is always done.
 *
 * Descriptors have the meaning, and the disjointness rules, of
 * tb_batched_copy.  The caller's array is read during tb_ring_submit only and
 * may be reused on return; the memory the descriptors point at must stay
 * valid until the ticket is done.  A ring is used by one thread at a time;
 * tb_ring_submit must be called with the ring's device current.
 *
 * tb_ring_create: nslots in [1, 1024], slot_descs in [1, 2^20], flags one of
 *   TB_RING_STAGED or TB_RING_DIRECT.  *out receives the ring.  Errors:
 *   TB_ERR_INVALID for a bad argument (checked before any HIP call);
 *   TB_ERR_NOMEM / TB_ERR_HIP if memory, events or the scratch cannot be had.
 * tb_ring_submit: n may be 0 (nothing is enqueued; the ticket is that of the
 *   last launch, or 0).  Every descriptor with bytes > 0 must have non-NULL
 *   src and dst and neither range may wrap the address space, and the
 *   ring's stream must not be under graph capture, else TB_ERR_INVALID and
 *   nothing of the request is enqueued.  TB_ERR_HIP if a
 *   wait, copy or launch fails; launches of the request made before the
 *   failure stay enqueued, and *ticket then receives the ring's last ticket
 *   (that of the last launch that was enqueued), so the caller can wait for
 *   them.
 * tb_ring_poll: *done = 1 if the ticket's launch has finished, else 0.
 *   TB_ERR_INVALID for a ticket not yet handed out; TB_ERR_HIP if the
 *   runtime reports an error for the launch.
 * tb_ring_wait: blocks until the ticket's launch has finished.  Errors as
 *   tb_ring_poll.
 * tb_ring_destroy: waits for every launch in flight, then frees the ring.
 *   NULL is a no-op.  If the wait fails (the runtime reports a device error)
 *   the ring is freed all the same and the error is returned.
 */
typedef struct tb_ring tb_ring;
enum { TB_RING_STAGED = 0, TB_RING_DIRECT = 1 };
int tb_ring_create(uint32_t nslots, uint32_t slot_descs, uint32_t flags, void *stream, tb_ring **out);
int tb_ring_submit(tb_ring *ring, const tb_copy_desc *host_desc, uint64_t n, uint64_t *ticket);
int tb_ring_poll(tb_ring *ring, uint64_t ticket, int32_t *done);
int tb_ring_wait(tb_ring *ring, uint64_t ticket);
int tb_ring_destroy(tb_ring *ring);

/*
 * Timing hook: the next kernel the calling thread launches through this
 * library (any entry point, the spin gate included) records start_event when
 * it begins and stop_event when it completes.  The events travel with the
 * launch (hipExtLaunchKernel's launch events) instead of being separate
 * commands between kernels, which on MI355X add about 3 us per launch to a
 * back-to-back sequence.  Either event may be NULL (a hipEvent_t created by
 * the caller, with timing enabled to read elapsed times).  A ring launch's
 * own stop event is its slot's completion event: the hook's stop event is
 * then recorded by a separate command right after that launch (it still
 * fires when the kernel has completed).  One launch only; a call that fails
 * before launching leaves the hook set for the next.
 * Always TB_OK.
 */
int tb_time_next_launch(void *start_event, void *stop_event);

/*
 * Timing gate (nvbandwidth's spin kernel, "nvbandwidth deep dive" §3.3.1):
 * tb_spin_gate_arm enqueues on `stream` a one-thread kernel that waits until
 * tb_spin_gate_release() is called, so that work queued behind it starts back
 * to back once released.  The wait is bounded: after timeout_ms (1 .. 60000)
 * the kernel exits by itself and tb_spin_gate_status() then returns
 * TB_ERR_TIMEOUT.  One gate per process; arming again re-uses it.
 * tb_spin_gate_status must be called after the stream has been synchronised.
 */
int tb_spin_gate_arm(uint32_t timeout_ms, void *stream);
int tb_spin_gate_release(void);
int tb_spin_gate_status(void);

/*
 * Launch geometry the library uses on the current device: compute units, the
 * workgroup count of the reduce-copy for nfloats floats and nsrc sources, and
 * that of the batched copy for ncopies descriptors (for reports; no GPU work
 * is enqueued).  Any out pointer may be NULL.
 * Errors: TB_ERR_INVALID for nsrc outside [0, TB_MAX_SRCS]; TB_ERR_HIP if the
 * device cannot be queried.
 */
int tb_launch_info(uint64_t nfloats, int32_t nsrc, uint32_t ncopies, int32_t *cu_count,
                   int32_t *reduce_blocks, int32_t *batched_blocks);

/* Free the library's scratch and gate memory (waits for the device first).
 * Safe to call more than once; later calls re-allocate lazily.  Must not run
 * concurrently with other calls of the library. */
int tb_shutdown(void);

#ifdef __cplusplus
}
#endif

#endif /* TB_H */
