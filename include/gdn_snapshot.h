/*
 * gdn_snapshot.h -- state snapshots of one slot on disk (C ABI, libgdn.so).
 *
 * What it implements ("Kapitsa 源码拆解 05：前缀缓存与模型状态恢复", sections on
 * writing and reading the SSD prefix cache and on file integrity): a disk copy
 * of a slot's recurrent state (the window and the state of every GDN layer)
 * that outlives the slot; it is written to a temporary file with the CRC-32C
 * of its header and of its payload and renamed to its final name only when
 * complete (the temporary file is removed on failure); reading checks the
 * file's identity, the header and the payload checksums, and a damaged file
 * can be dropped.  Snapshots are bound to a restore point (a key, e.g. the
 * prefix hash, and a token position), and are only readable into a pool
 * with the same state layout (compatibility: same bytes, same meaning).
 *
 * File format (little-endian; the header is 128 bytes):
 *   offset  0  char[8]  magic "GDNSTAT1"
 *           8  uint32   format version (1)
 *          12  uint32   header bytes (128)
 *          16  uint64   key
 *          24  int64    position (tokens the state has absorbed)
 *          32  int32    number of GDN (non attention-only) layers
 *          36  int32    conv channels C      40 int32 conv width W
 *          44  int32    k heads Hk           48 int32 v heads Hv
 *          52  int32    head k dim dk        56 int32 head v dim dv
 *          60  int32    state dtype (1 = fp32), 64 int32 window dtype (2 = bf16)
 *          68  uint32   0
 *          72  int64    window bytes per layer (W-1)*C*2
 *          80  int64    state bytes per layer Hv*dk*dv*4
 *          88  int64    payload bytes = layers * (window + state bytes)
 *          96  uint32   CRC-32C of the payload
 *         100  uint32   CRC-32C of header bytes [0, 100)
 *         104  24 zero bytes
 *   payload: for each GDN layer in layer order, its window bytes then its
 *            state bytes, exactly as they sit in the page.
 * CRC-32C: the Castagnoli polynomial 0x1EDC6F41, reflected, initial value
 * and final xor 0xFFFFFFFF.
 *
 * Unlike the step calls, the snapshot calls wait for their own copies: they
 * enqueue device<->host copies on `stream` and synchronise it before
 * returning.  Host memory for the payload is allocated and freed inside the
 * call; no device memory is allocated.
 *
 * Reading takes the 128-byte header first: a file that is not a snapshot,
 * whose header checksum fails, or whose size is not the header's plus the
 * payload the header states is rejected before any payload is read or
 * memory for it is allocated.  Writing syncs the file, renames it, then
 * syncs its directory.
 *
 * Errors: GDN_EINVAL (NULL / bad argument, or a pool whose layout differs
 * from the file's), GDN_ERANGE (slot out of range), GDN_EIO (the file could
 * not be written / read / made durable), GDN_ECORRUPT (identity or checksum
 * mismatch, truncated file, a payload size that does not fit the layout),
 * GDN_EHIP (a copy failed), GDN_ENOMEM (host memory for the payload).
 */
#ifndef GDN_SNAPSHOT_H
#define GDN_SNAPSHOT_H

#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GDN_EIO = -9,       /* file system error */
    GDN_ECORRUPT = -10  /* damaged or foreign snapshot file */
};

typedef struct {
    uint64_t key;
    int64_t position;
    int32_t num_linear_layers;
    int32_t conv_channels, conv_width;
    int32_t num_k_heads, num_v_heads, head_k_dim, head_v_dim;
    int64_t window_bytes, state_bytes, payload_bytes;
    uint32_t payload_crc;
} gdn_snapshot_info;

/* CRC-32C of `len` bytes, continuing from `crc` (0 to start). */
uint32_t gdn_crc32c(uint32_t crc, const void* data, size_t len);

/* Write the window and state of `slot` on every GDN layer of the pool to
 * `path` (through `path` + ".tmp" and a rename). */
int gdn_snapshot_save(const gdn_pool* pool, int32_t slot, uint64_t key, int64_t position,
                      const char* path, gdn_stream_t stream);

/* Check `path` (identity, layout against the pool, key, both checksums) and
 * copy its payload into `slot` (payload regions only; padding untouched).
 * *position receives the stored position.  On a checksum or identity
 * failure nothing is written to the device, and the file is deleted when
 * drop_damaged is non-zero. */
int gdn_snapshot_load(const gdn_pool* pool, int32_t slot, const char* path, uint64_t key,
                      int64_t* position, int32_t drop_damaged, gdn_stream_t stream);

/* Check `path` without a pool (identity and both checksums) and return its
 * header fields. */
int gdn_snapshot_read_info(const char* path, gdn_snapshot_info* out);

#ifdef __cplusplus
}
#endif
#endif /* GDN_SNAPSHOT_H */
