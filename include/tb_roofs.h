/*
 * tb_roofs.h -- C ABI of libtb_roofs, the measuring instruments of bench.py
 * --roofs (not part of the transfer path).
 *
 * The pages time a transfer against what the memory system allows
 * ("nvbandwidth deep dive" §3.3: the measurement method; TransferBench PR
 * #365, Motivation: a rate above what the links or memory allow means some
 * bytes came from a cache).  These kernels give that allowance for the access
 * patterns libtb's kernels run, so a kernel's rate can be read against the
 * rate of its pattern rather than against the HBM peak alone:
 *   - read-only and write-only streams over 1 .. 17 buffers at once, and
 *     N streams read with their XOR written to one more (the reduce-copy with
 *     N sources reads N streams and writes one);
 *   - copies, writes and reads of a list of tiles of at most 4 KiB whose
 *     addresses the host computed beforehand (a batch of scattered copies cut
 *     into tiles: the batched copy's exact bytes and destinations, with none
 *     of its descriptor handling).
 * Every kernel is a plain stream: one 16-byte access per thread, one tile of
 * 256 threads per workgroup, tiles dealt in order.  They share no code with
 * libtb.
 *
 * Conventions: calls return 0 (TBR_OK) or a negative status, never throw and
 * print nothing; pointers are device addresses of the current device unless
 * stated; `stream` is a hipStream_t passed as void* (NULL is the legacy
 * default stream); the calls only enqueue work.
 */
#ifndef TB_ROOFS_H
#define TB_ROOFS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    TBR_OK = 0,
    TBR_ERR_INVALID = -1,   /* bad argument; nothing was enqueued */
    TBR_ERR_HIP = -2        /* a HIP runtime call failed          */
};

/* Store cache policy of the write and copy instruments. */
enum {
    TBR_STORE_DEVICE = 0,      /* device scope (sc1): allocates in the memory-side cache */
    TBR_STORE_STREAMING = 1,   /* nontemporal, system scope (nt sc0 sc1): does not       */
    TBR_STORE_NT = 2           /* nontemporal (nt): does not                             */
};

/* Most buffers one read or write instrument takes. */
#define TBR_MAX_BUFS 17

/*
 * One tile: `bytes` bytes from src to dst (device addresses).  bytes is a
 * multiple of 16 in [16, 4096]; src and dst are 16-byte aligned.  24 bytes.
 */
typedef struct tbr_tile {
    uint64_t src;
    uint64_t dst;
    uint32_t bytes;
    uint32_t reserved;   /* 0 */
} tbr_tile;

/*
 * Read every byte of nbufs buffers of bytes_each bytes, all at once: tile t
 * of every buffer (4 KiB) is read by workgroup t, with nontemporal 16-byte
 * loads.  Nothing is written except, when a checksum of the bytes read equals
 * one fixed value, one word of library memory (that keeps the loads live).
 * bufs: HOST array of nbufs device pointers, each 16-byte aligned.
 * Errors: TBR_ERR_INVALID for nbufs outside [1, TBR_MAX_BUFS], a NULL or
 * misaligned pointer, or bytes_each not a multiple of 16; TBR_ERR_HIP.
 * bytes_each == 0 is a no-op.
 */
int tbr_read(const void *const *bufs, int32_t nbufs, uint64_t bytes_each, void *stream);

/*
 * Write `word` to every 32-bit word of nbufs buffers of bytes_each bytes,
 * all at once (tile t of every buffer by workgroup t), with the store policy
 * `policy` (TBR_STORE_*).  Errors as tbr_read, and TBR_ERR_INVALID for an
 * unknown policy.
 */
int tbr_write(void *const *bufs, int32_t nbufs, uint64_t bytes_each, uint32_t word, uint32_t policy,
              void *stream);

/*
 * Copy `bytes` bytes from src to dst (both 16-byte aligned, bytes a multiple
 * of 16, not overlapping): 4 KiB tiles, nontemporal loads, stores with
 * `policy`.  Errors as tbr_write.
 */
int tbr_copy(void *dst, const void *src, uint64_t bytes, uint32_t policy, void *stream);

/*
 * dst = the XOR of nsrcs buffers of bytes_each bytes, all at once: tile t of
 * every source (4 KiB) read by workgroup t with nontemporal 16-byte loads,
 * and tile t of dst written with `policy` stores.  The reduce-copy's access
 * pattern (nsrcs streams read, one written) with integer work only.
 * srcs: HOST array of nsrcs device pointers; nsrcs in [1, TBR_MAX_BUFS - 1];
 * every pointer 16-byte aligned and bytes_each a multiple of 16; dst must not
 * overlap a source.  Errors: TBR_ERR_INVALID for any of that or an unknown
 * policy; TBR_ERR_HIP.  bytes_each == 0 is a no-op.
 */
int tbr_combine(const void *const *srcs, int32_t nsrcs, void *dst, uint64_t bytes_each, uint32_t policy,
                void *stream);

/*
 * Over a DEVICE array of ntiles tiles (each as tbr_tile states; tiles whose
 * length or alignment breaks that are skipped, so a bad tile cannot send an
 * access elsewhere), workgroup t handles tile t:
 *   tbr_tiles_copy   copies it (nontemporal loads, stores with `policy`);
 *   tbr_tiles_write  writes `word` over its destination only;
 *   tbr_tiles_read   reads its source only (checksum as tbr_read).
 * Destinations must not overlap for the copy and the write.  tiles_dev must
 * stay valid until the stream has passed the kernel.
 * Errors: TBR_ERR_INVALID for a NULL or misaligned tiles_dev with ntiles > 0
 * or an unknown policy; TBR_ERR_HIP.  ntiles == 0 is a no-op.
 */
int tbr_tiles_copy(const tbr_tile *tiles_dev, uint32_t ntiles, uint32_t policy, void *stream);
int tbr_tiles_write(const tbr_tile *tiles_dev, uint32_t ntiles, uint32_t word, uint32_t policy, void *stream);
int tbr_tiles_read(const tbr_tile *tiles_dev, uint32_t ntiles, void *stream);

/* Text of the last failing HIP call on this thread, or "". */
const char *tbr_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TB_ROOFS_H */
