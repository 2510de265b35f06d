"""Plain reference model of the linear-state prefix cache's slot bookkeeping.

TEST INFRASTRUCTURE ONLY (imported by tests/, never by the product package);
it shares no code with the C++ slot manager of the library.

Follows "Linear-State Prefix Cache 内部机制" (xLLM notes):
  §1-§2   one id space of physical slots; a slot is free, live (private to
          one running sequence, overwritten in place) or a checkpoint
          (public, frozen, restorable, reclaimable least-recently-used first);
  §3.1    saving is split: resolve (before the forward) only reserves,
          commit (after the forward) hands over;
  §3.2    the hand-over: the live slot leaves the sequence without being
          freed, becomes the checkpoint of the hash, and the sequence takes
          the reserved replacement, marked cold;
  §3.3    resolve skips a save on a duplicate hash in the batch, an already
          cached hash, a failed promotion condition, or no free replacement
          (nothing is evicted for it);
  §4.1    a row's warm/cold bit; §5: needs_restore = not initialized and
          n_kv > 0 and n_kv % block_size == 0;
  §6-§7   the per-row op: live slot, restore hash + src slot (-1 = none),
          save hash + dst slot (= the live slot when the promotion is real).

Where the page is silent the same readings as the library are taken (they
are choices, not derivations): the promotion condition is "the step ends on
a block boundary"; a new sequence gets the lowest free slot, or else the
least recently used unpinned checkpoint; the LRU clock ticks on each
checkpoint insert and each restore match; the warm bit of a row is whether
its live slot holds valid state.
"""
from __future__ import annotations

FREE, LIVE, CHECKPOINT, RESERVED = 0, 1, 2, 3


class SlotManagerModel:
    def __init__(self, num_slots: int, block_size: int):
        assert num_slots >= 1 and block_size >= 1
        self.block = block_size
        self.kind = [FREE] * num_slots
        self.owner = [0] * num_slots        # live slots: sequence id
        self.ckpt_hash = [0] * num_slots    # checkpoints: prefix hash
        self.pins = [0] * num_slots         # checkpoints: restores in flight
        self.last_use = [0] * num_slots     # checkpoints: LRU clock value
        self.clock = 0
        self.seq_slot = {}                  # sequence id -> live slot
        self.seq_init = {}                  # sequence id -> slot content valid
        self.cache = {}                     # prefix hash -> checkpoint slot
        self.pending = None                 # (batch sequence ids, promotions, pinned slots)

    # -- helpers -----------------------------------------------------------
    def _lowest_free(self):
        for s, k in enumerate(self.kind):
            if k == FREE:
                return s
        return None

    def _stamp(self, s):
        self.clock += 1
        self.last_use[s] = self.clock

    # -- sequences -----------------------------------------------------------
    def add_sequence(self, seq):
        """allocate_live_slot; returns the slot or raises LookupError."""
        if seq in self.seq_slot:
            raise ValueError("sequence already present")
        s = self._lowest_free()
        if s is None:
            victims = [c for c in range(len(self.kind))
                       if self.kind[c] == CHECKPOINT and self.pins[c] == 0]
            if not victims:
                raise LookupError("no slot")
            s = min(victims, key=lambda c: self.last_use[c])
            del self.cache[self.ckpt_hash[s]]
        self.kind[s] = LIVE
        self.owner[s] = seq
        self.ckpt_hash[s] = 0
        self.pins[s] = 0
        self.last_use[s] = 0
        self.seq_slot[seq] = s
        self.seq_init[seq] = False
        return s

    def remove_sequence(self, seq):
        if self.pending is not None:
            raise RuntimeError("batch pending")
        if seq not in self.seq_slot:
            raise ValueError("unknown sequence")
        s = self.seq_slot.pop(seq)
        del self.seq_init[seq]
        self.kind[s] = FREE
        self.owner[s] = 0

    # -- one step: resolve, (forward), commit or abort ----------------------
    def resolve(self, rows):
        """rows: (seq, n_kv, n_after, restore_hash, save_hash) tuples."""
        if self.pending is not None:
            raise RuntimeError("batch pending")
        seqs = [r[0] for r in rows]
        if len(set(seqs)) != len(seqs) or any(q not in self.seq_slot for q in seqs):
            raise ValueError("bad batch")
        if any(r[1] < 0 or r[2] < r[1] for r in rows):
            raise ValueError("bad token counts")
        ops, promotions, pinned, promoted_hashes = [], [], [], set()
        for seq, n_kv, n_after, restore_hash, save_hash in rows:
            live = self.seq_slot[seq]
            op = dict(linear_state_id=live, restore_src_slot_id=-1, save_dst_slot_id=-1,
                      has_initial_state=1 if self.seq_init[seq] else 0,
                      restore_prefix_hash=0, save_prefix_hash=save_hash)
            needs_restore = (not self.seq_init[seq]) and n_kv > 0 and n_kv % self.block == 0
            if needs_restore and restore_hash != 0:
                op["restore_prefix_hash"] = restore_hash
                if restore_hash in self.cache:
                    src = self.cache[restore_hash]
                    op["restore_src_slot_id"] = src
                    self.pins[src] += 1
                    pinned.append(src)
                    self._stamp(src)
            if save_hash != 0:
                duplicate = save_hash in promoted_hashes
                cached = save_hash in self.cache
                can_promote = n_after > 0 and n_after % self.block == 0
                replacement = None
                if not duplicate and not cached and can_promote:
                    replacement = self._lowest_free()
                if replacement is not None:
                    self.kind[replacement] = RESERVED
                    promotions.append((save_hash, seq, live, replacement))
                    promoted_hashes.add(save_hash)
                    op["save_dst_slot_id"] = live
            ops.append(op)
        self.pending = (seqs, promotions, pinned)
        return ops

    def commit(self):
        if self.pending is None:
            raise RuntimeError("nothing to commit")
        seqs, promotions, pinned = self.pending
        for seq in seqs:
            self.seq_init[seq] = True
        for save_hash, seq, live, replacement in promotions:
            # 1. move the slot out of the sequence, do not free it
            # 2. it becomes the checkpoint of the prefix
            self.kind[live] = CHECKPOINT
            self.owner[live] = 0
            self.ckpt_hash[live] = save_hash
            self.pins[live] = 0
            self.cache[save_hash] = live
            self._stamp(live)
            # 3. the sequence takes the replacement, cold
            self.kind[replacement] = LIVE
            self.owner[replacement] = seq
            self.seq_slot[seq] = replacement
            self.seq_init[seq] = False
        for s in pinned:
            self.pins[s] -= 1
        self.pending = None

    def abort(self):
        if self.pending is None:
            raise RuntimeError("nothing to abort")
        _, promotions, pinned = self.pending
        for _, _, _, replacement in promotions:
            self.kind[replacement] = FREE
        for s in pinned:
            self.pins[s] -= 1
        self.pending = None

    # -- views -----------------------------------------------------------------
    def slot_info(self, s):
        k = self.kind[s]
        return (k, self.owner[s] if k == LIVE else 0, self.ckpt_hash[s] if k == CHECKPOINT else 0,
                self.pins[s] if k == CHECKPOINT else 0)

    def counts(self):
        return [self.kind.count(k) for k in (FREE, LIVE, CHECKPOINT, RESERVED)]


def restore_ops(ops):
    """(dst, src, requested) per row for the worker's cross-layer copy."""
    return [(o["linear_state_id"], o["restore_src_slot_id"], 1 if o["restore_prefix_hash"] else 0)
            for o in ops]
