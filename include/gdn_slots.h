/*
 * gdn_slots.h -- host-side slot manager of the linear-state prefix cache
 * (C ABI, part of libgdn.so).  Pure host code: no device memory, no GPU call.
 *
 * What it implements ("Linear-State Prefix Cache 内部机制", xLLM notes):
 *   - §1, §2: one manager per data-parallel rank owns every physical slot
 *     [0, num_slots) of the state pool; a slot is free, live (the private,
 *     overwritten-in-place state of one running sequence) or a checkpoint
 *     (public, frozen, restorable, reclaimable in LRU order), all in one id
 *     space.
 *   - §3, §3.1, §3.2: saving is a zero-copy promotion done in two phases:
 *     resolve (before the forward) reserves a replacement slot and records
 *     the promotion without touching the sequence; commit (after the forward,
 *     when the live slot holds the block-aligned state) moves the live slot
 *     out of the sequence without freeing it, inserts it as the checkpoint of
 *     the prefix hash, and hands the sequence the replacement, marked cold.
 *   - §3.3: resolve skips a save when another row of the batch saves the same
 *     hash (the first row wins), when the hash is already cached, when the
 *     promotion condition fails, or when no free replacement slot exists (no
 *     checkpoint is evicted for it).
 *   - §4, §4.1: a restore is requested for a row whose live slot holds no
 *     valid state and whose KV prefix is block aligned; the hash is matched
 *     against the checkpoints (a hit pins the checkpoint until commit) and the
 *     worker copies src -> live slot with gdn_restore_slots.
 *   - §5: linear_state_initialized, the per-sequence "slot content valid"
 *     bit, and needs_restore = !initialized && n_kv > 0 && n_kv % block == 0.
 *   - §6, §6.1, §6.2, §7: the per-row op (live slot, restore hash + src slot,
 *     save hash + dst slot) with the zero-value conventions: hash 0 = not
 *     requested, slot -1 = none; save_dst_slot_id >= 0 only when resolve
 *     confirmed the promotion.
 *
 * Readings where the page is silent:
 *   - the promotion condition (§3.3 names it without defining it): the row's
 *     tokens after this step end on a block boundary (n_tokens_after_step > 0
 *     and a multiple of block_size), so that the forward leaves the
 *     block-aligned state in the live slot;
 *   - checkpoints are reclaimed (least recently inserted or matched first,
 *     pinned ones never) only when a new sequence needs a live slot and no
 *     slot is free; resolve never evicts;
 *   - after commit every row of the batch has a valid live slot (the forward
 *     wrote it), except the promoted rows, which now hold a cold replacement.
 *
 * Errors: 0 (GDN_OK) or a negative GDN_E* code from gdn.h; GDN_ENOSLOT when
 * no slot can be found for a new sequence; GDN_ESTATE for a call out of
 * order (commit without resolve, resolve while a batch is pending).  A
 * call that fails a check changes nothing.  When host memory runs out
 * (GDN_ENOMEM; no C++ exception leaves the library) a resolve is rolled
 * back like an abort, while a commit may have applied part of the batch.
 * gdn_last_error() gives the message.
 * The manager is not thread-safe: one scheduler thread drives it.
 */
#ifndef GDN_SLOTS_H
#define GDN_SLOTS_H

#include <stdint.h>

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GDN_ENOSLOT = -7, /* no free slot and no reclaimable checkpoint */
    GDN_ESTATE = -8   /* call out of order */
};

typedef uint64_t gdn_prefix_hash; /* content fingerprint of a token prefix; 0 = none */

typedef struct gdn_slot_manager gdn_slot_manager;

/* num_slots >= 1, block_size >= 1. */
int gdn_slots_create(int32_t num_slots, int32_t block_size, gdn_slot_manager** out);
void gdn_slots_destroy(gdn_slot_manager* m);

/* A new sequence gets a free slot as its live slot, cold (not initialized).
 * With no free slot, the least recently used unpinned checkpoint is
 * reclaimed for it; GDN_ENOSLOT if there is none.  GDN_EINVAL for a
 * sequence id already present. */
int gdn_slots_add_sequence(gdn_slot_manager* m, int64_t seq_id, int32_t* live_slot);

/* A finished sequence returns its live slot to the free list.  Not allowed
 * while a resolved batch is pending (GDN_ESTATE). */
int gdn_slots_remove_sequence(gdn_slot_manager* m, int64_t seq_id);

/* One batch row as the build stage knows it. */
typedef struct {
    int64_t seq_id;
    int64_t n_kv_cache_tokens;           /* tokens already cached before this step */
    int64_t n_tokens_after_step;         /* n_kv_cache_tokens + tokens this step computes */
    gdn_prefix_hash restore_prefix_hash; /* hash of the cached (block-aligned) prefix, or 0 */
    gdn_prefix_hash save_prefix_hash;    /* hash of the prefix ending this step, or 0 */
} gdn_slot_request;

/* The per-row op sent to the worker. */
typedef struct {
    int32_t linear_state_id;             /* the row's live slot (overwritten by this step) */
    int32_t restore_src_slot_id;         /* checkpoint to copy from, -1 = none / miss */
    int32_t save_dst_slot_id;            /* == linear_state_id when a promotion is reserved, else -1 */
    int32_t has_initial_state;           /* default warm/cold bit for the row */
    gdn_prefix_hash restore_prefix_hash; /* != 0: a restore was requested */
    gdn_prefix_hash save_prefix_hash;    /* copied from the request */
} gdn_linear_state_op;

/* Resolve a batch of n rows (distinct sequences, each added before) into
 * ops[n].  has_initial_state is the row's default before any restore: 1 when
 * its live slot already holds valid state, else 0 (a restore hit then turns
 * it to 1 on the device, gdn_restore_slots).  Reserves the replacement slots
 * and pins the matched checkpoints until gdn_slots_commit / _abort. */
int gdn_slots_resolve(gdn_slot_manager* m, const gdn_slot_request* rows, int32_t n,
                      gdn_linear_state_op* ops);

/* After the forward of the resolved batch: every row's live slot becomes
 * valid, the reserved promotions take place, pins are released. */
int gdn_slots_commit(gdn_slot_manager* m);

/* The forward of the resolved batch did not run: reservations and pins are
 * released, nothing else changes. */
int gdn_slots_abort(gdn_slot_manager* m);

/* The restore ops of a resolved batch for gdn_restore_slots: op i =
 * (linear_state_id, restore_src_slot_id, restore_prefix_hash != 0). */
int gdn_slots_restore_ops(const gdn_linear_state_op* ops, int32_t n, gdn_restore_op* out);

/* ---- inspection (tests, debugging) ------------------------------------ */
enum { GDN_SLOT_FREE = 0, GDN_SLOT_LIVE = 1, GDN_SLOT_CHECKPOINT = 2, GDN_SLOT_RESERVED = 3 };

/* Kind of `slot`; for a live slot *owner = its sequence id, for a checkpoint
 * *hash = its prefix hash and *pins = the pin count (other outputs 0). */
int gdn_slots_slot_info(const gdn_slot_manager* m, int32_t slot, int32_t* kind, int64_t* owner,
                        gdn_prefix_hash* hash, int32_t* pins);

/* Live slot and initialized bit of a sequence (GDN_EINVAL if unknown). */
int gdn_slots_sequence_info(const gdn_slot_manager* m, int64_t seq_id, int32_t* live_slot,
                            int32_t* initialized);

/* Checkpoint slot of a hash, or -1; does not pin or touch the LRU order. */
int32_t gdn_slots_lookup(const gdn_slot_manager* m, gdn_prefix_hash hash);

/* Slots per kind: counts[4] indexed by GDN_SLOT_*. */
int gdn_slots_counts(const gdn_slot_manager* m, int32_t counts[4]);

#ifdef __cplusplus
}
#endif
#endif /* GDN_SLOTS_H */
