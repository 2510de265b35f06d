// Host-side slot manager of the linear-state prefix cache (gdn_slots.h).
//
// "Linear-State Prefix Cache 内部机制" §1-§3: one id space of physical slots,
// each free, live (one sequence's private state), reserved (a promotion's
// replacement between resolve and commit) or a checkpoint (public, frozen,
// reclaimable in LRU order); saving is a two-phase zero-copy promotion.
// §4-§5: a cold-start restore is requested when the live slot holds no valid
// state and the KV prefix is block aligned.  §6-§7: the per-row op.
//
// Choices the page leaves open, applied identically everywhere: a free slot
// is always the lowest-numbered one; the LRU order is a counter stamped on a
// checkpoint when it is inserted and when a restore matches it.
#include <stdint.h>

#include <map>
#include <memory>
#include <set>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "gdn_internal.h"
#include "gdn_slots.h"

using gdn::fail;

struct gdn_slot_manager {
    struct Slot {
        int32_t kind = GDN_SLOT_FREE;
        int64_t owner = 0;        // live: sequence id
        gdn_prefix_hash hash = 0; // checkpoint: prefix hash
        int32_t pins = 0;         // checkpoint: pending restores
        uint64_t stamp = 0;       // checkpoint: last insert / match
    };
    struct Seq {
        int32_t slot = -1;
        bool initialized = false;
    };
    struct Promotion {
        gdn_prefix_hash hash;
        int64_t seq;
        int32_t live;
        int32_t replacement;
    };

    int32_t block = 1;
    std::vector<Slot> slots;
    std::set<int32_t> free_slots;
    std::unordered_map<int64_t, Seq> seqs;
    std::unordered_map<gdn_prefix_hash, int32_t> table; // checkpoint hash -> slot
    std::map<uint64_t, int32_t> lru;                    // stamp -> checkpoint slot
    uint64_t clock = 0;

    bool pending = false; // a resolved batch awaits commit / abort
    std::vector<int64_t> batch;
    std::vector<Promotion> promotions;
    std::vector<int32_t> pinned; // one entry per matched restore

    int32_t take_free()
    {
        const int32_t s = *free_slots.begin();
        free_slots.erase(free_slots.begin());
        return s;
    }
    void release(int32_t s)
    {
        slots[s] = Slot{};
        free_slots.insert(s);
    }
    void touch(int32_t s)
    {
        lru.erase(slots[s].stamp);
        slots[s].stamp = ++clock;
        lru.emplace(slots[s].stamp, s);
    }
    void drop_pins()
    {
        for (int32_t s : pinned)
            --slots[s].pins;
        pinned.clear();
    }
    // undo a resolve (its reservations and pins); allocates nothing
    void rollback()
    {
        for (const auto& p : promotions)
            release(p.replacement);
        drop_pins();
        promotions.clear();
        batch.clear();
        pending = false;
    }
};

namespace {

int add_sequence(gdn_slot_manager* m, int64_t seq_id, int32_t* live_slot)
{
    // the map entry first: if it cannot be allocated, nothing has changed
    gdn_slot_manager::Seq& q = m->seqs[seq_id];
    int32_t s = -1;
    if (!m->free_slots.empty()) {
        s = m->take_free();
    } else {
        // reclaim the least recently used checkpoint nobody is about to restore
        for (const auto& e : m->lru) {
            if (m->slots[e.second].pins == 0) {
                s = e.second;
                break;
            }
        }
        if (s < 0) {
            m->seqs.erase(seq_id);
            return fail(GDN_ENOSLOT, "slots: no free slot and no reclaimable checkpoint");
        }
        m->table.erase(m->slots[s].hash);
        m->lru.erase(m->slots[s].stamp);
    }
    m->slots[s] = gdn_slot_manager::Slot{};
    m->slots[s].kind = GDN_SLOT_LIVE;
    m->slots[s].owner = seq_id;
    q = gdn_slot_manager::Seq{s, false};
    *live_slot = s;
    return GDN_OK;
}

int resolve(gdn_slot_manager* m, const gdn_slot_request* rows, int32_t n, gdn_linear_state_op* ops)
{
    std::unordered_set<int64_t> seen;
    for (int32_t i = 0; i < n; ++i) {
        if (!m->seqs.count(rows[i].seq_id))
            return fail(GDN_EINVAL, "slots: row %d names unknown sequence %lld", i,
                        (long long)rows[i].seq_id);
        if (!seen.insert(rows[i].seq_id).second)
            return fail(GDN_EINVAL, "slots: sequence %lld appears twice in the batch",
                        (long long)rows[i].seq_id);
        if (rows[i].n_kv_cache_tokens < 0 || rows[i].n_tokens_after_step < rows[i].n_kv_cache_tokens)
            return fail(GDN_EINVAL, "slots: row %d has inconsistent token counts", i);
    }
    const int64_t B = m->block;
    std::unordered_set<gdn_prefix_hash> saving; // hashes promoted by earlier rows
    for (int32_t i = 0; i < n; ++i) {
        const gdn_slot_request& r = rows[i];
        const gdn_slot_manager::Seq& q = m->seqs[r.seq_id];
        gdn_linear_state_op& op = ops[i];
        op.linear_state_id = q.slot;
        op.has_initial_state = q.initialized ? 1 : 0;
        op.save_prefix_hash = r.save_prefix_hash;
        op.restore_prefix_hash = 0;
        op.restore_src_slot_id = -1;
        op.save_dst_slot_id = -1;
        // restore: once, into a live slot without valid state, at a block-aligned prefix
        const bool needs_restore =
            !q.initialized && r.n_kv_cache_tokens > 0 && r.n_kv_cache_tokens % B == 0;
        if (needs_restore && r.restore_prefix_hash != 0) {
            op.restore_prefix_hash = r.restore_prefix_hash;
            auto hit = m->table.find(r.restore_prefix_hash);
            if (hit != m->table.end()) {
                const int32_t s = hit->second;
                op.restore_src_slot_id = s;
                ++m->slots[s].pins;
                m->pinned.push_back(s);
                m->touch(s);
            }
        }
        // save: the four skip rules, then reserve the replacement
        if (r.save_prefix_hash == 0)
            continue;
        if (saving.count(r.save_prefix_hash))
            continue; // another row of this batch promotes the same prefix
        if (m->table.count(r.save_prefix_hash))
            continue; // already cached
        if (!(r.n_tokens_after_step > 0 && r.n_tokens_after_step % B == 0))
            continue; // the step does not end on a block boundary
        if (m->free_slots.empty())
            continue; // no replacement: keep the cache sparse, evict nothing
        const int32_t rep = m->take_free();
        m->slots[rep].kind = GDN_SLOT_RESERVED;
        m->promotions.push_back({r.save_prefix_hash, r.seq_id, q.slot, rep});
        saving.insert(r.save_prefix_hash);
        op.save_dst_slot_id = q.slot;
    }
    m->batch.clear();
    for (int32_t i = 0; i < n; ++i)
        m->batch.push_back(rows[i].seq_id);
    m->pending = true;
    return GDN_OK;
}

int commit(gdn_slot_manager* m)
{
    for (int64_t s : m->batch)
        m->seqs[s].initialized = true; // the forward wrote every row's live slot
    for (const auto& p : m->promotions) {
        // 1. the live slot leaves the sequence without being freed,
        // 2. becomes the checkpoint of the prefix,
        // 3. the sequence takes the replacement, cold
        gdn_slot_manager::Slot& c = m->slots[p.live];
        c = gdn_slot_manager::Slot{};
        c.kind = GDN_SLOT_CHECKPOINT;
        c.hash = p.hash;
        m->table[p.hash] = p.live;
        m->touch(p.live);
        gdn_slot_manager::Slot& r = m->slots[p.replacement];
        r = gdn_slot_manager::Slot{};
        r.kind = GDN_SLOT_LIVE;
        r.owner = p.seq;
        m->seqs[p.seq] = gdn_slot_manager::Seq{p.replacement, false};
    }
    m->drop_pins();
    m->promotions.clear();
    m->batch.clear();
    m->pending = false;
    return GDN_OK;
}

} // namespace

extern "C" {

int gdn_slots_create(int32_t num_slots, int32_t block_size, gdn_slot_manager** out)
{
    gdn::clear_error();
    if (!out || num_slots < 1 || block_size < 1)
        return fail(GDN_EINVAL, "slots: num_slots and block_size must be >= 1, out non-NULL");
    return gdn::guarded([&] {
        std::unique_ptr<gdn_slot_manager> m(new gdn_slot_manager());
        m->block = block_size;
        m->slots.resize(size_t(num_slots));
        for (int32_t s = 0; s < num_slots; ++s)
            m->free_slots.insert(s);
        *out = m.release();
        return int(GDN_OK);
    });
}

void gdn_slots_destroy(gdn_slot_manager* m) { delete m; }

int gdn_slots_add_sequence(gdn_slot_manager* m, int64_t seq_id, int32_t* live_slot)
{
    gdn::clear_error();
    if (!m || !live_slot)
        return fail(GDN_EINVAL, "slots: NULL argument");
    if (m->seqs.count(seq_id))
        return fail(GDN_EINVAL, "slots: sequence %lld already has a live slot", (long long)seq_id);
    return gdn::guarded([&] { return add_sequence(m, seq_id, live_slot); });
}

int gdn_slots_remove_sequence(gdn_slot_manager* m, int64_t seq_id)
{
    gdn::clear_error();
    if (!m)
        return fail(GDN_EINVAL, "slots: NULL manager");
    if (m->pending)
        return fail(GDN_ESTATE, "slots: a resolved batch is pending");
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end())
        return fail(GDN_EINVAL, "slots: unknown sequence %lld", (long long)seq_id);
    return gdn::guarded([&] {
        m->release(it->second.slot); // the set insert may allocate
        m->seqs.erase(it);
        return int(GDN_OK);
    });
}

int gdn_slots_resolve(gdn_slot_manager* m, const gdn_slot_request* rows, int32_t n,
                      gdn_linear_state_op* ops)
{
    gdn::clear_error();
    if (!m || n < 0 || (n > 0 && (!rows || !ops)))
        return fail(GDN_EINVAL, "slots: bad resolve arguments");
    if (m->pending)
        return fail(GDN_ESTATE, "slots: the previous batch was neither committed nor aborted");
    return gdn::guarded([&] {
        try {
            return resolve(m, rows, n, ops);
        } catch (...) {
            m->rollback();
            throw;
        }
    });
}

int gdn_slots_commit(gdn_slot_manager* m)
{
    gdn::clear_error();
    if (!m)
        return fail(GDN_EINVAL, "slots: NULL manager");
    if (!m->pending)
        return fail(GDN_ESTATE, "slots: commit without a resolved batch");
    return gdn::guarded([&] { return commit(m); });
}

int gdn_slots_abort(gdn_slot_manager* m)
{
    gdn::clear_error();
    if (!m)
        return fail(GDN_EINVAL, "slots: NULL manager");
    if (!m->pending)
        return fail(GDN_ESTATE, "slots: abort without a resolved batch");
    return gdn::guarded([&] {
        m->rollback(); // the set inserts may allocate
        return int(GDN_OK);
    });
}

int gdn_slots_restore_ops(const gdn_linear_state_op* ops, int32_t n, gdn_restore_op* out)
{
    gdn::clear_error();
    if (n < 0 || (n > 0 && (!ops || !out)))
        return fail(GDN_EINVAL, "slots: bad restore_ops arguments");
    for (int32_t i = 0; i < n; ++i) {
        out[i].dst_slot = ops[i].linear_state_id;
        out[i].src_slot = ops[i].restore_src_slot_id;
        out[i].requested = ops[i].restore_prefix_hash != 0 ? 1 : 0;
    }
    return GDN_OK;
}

int gdn_slots_slot_info(const gdn_slot_manager* m, int32_t slot, int32_t* kind, int64_t* owner,
                        gdn_prefix_hash* hash, int32_t* pins)
{
    gdn::clear_error();
    if (!m || !kind || !owner || !hash || !pins)
        return fail(GDN_EINVAL, "slots: NULL argument");
    if (slot < 0 || slot >= int32_t(m->slots.size()))
        return fail(GDN_ERANGE, "slots: slot %d out of range", slot);
    const auto& s = m->slots[slot];
    *kind = s.kind;
    *owner = s.kind == GDN_SLOT_LIVE ? s.owner : 0;
    *hash = s.kind == GDN_SLOT_CHECKPOINT ? s.hash : 0;
    *pins = s.kind == GDN_SLOT_CHECKPOINT ? s.pins : 0;
    return GDN_OK;
}

int gdn_slots_sequence_info(const gdn_slot_manager* m, int64_t seq_id, int32_t* live_slot,
                            int32_t* initialized)
{
    gdn::clear_error();
    if (!m || !live_slot || !initialized)
        return fail(GDN_EINVAL, "slots: NULL argument");
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end())
        return fail(GDN_EINVAL, "slots: unknown sequence %lld", (long long)seq_id);
    *live_slot = it->second.slot;
    *initialized = it->second.initialized ? 1 : 0;
    return GDN_OK;
}

int32_t gdn_slots_lookup(const gdn_slot_manager* m, gdn_prefix_hash hash)
{
    if (!m || hash == 0)
        return -1;
    auto it = m->table.find(hash);
    return it == m->table.end() ? -1 : it->second;
}

int gdn_slots_counts(const gdn_slot_manager* m, int32_t counts[4])
{
    gdn::clear_error();
    if (!m || !counts)
        return fail(GDN_EINVAL, "slots: NULL argument");
    for (int k = 0; k < 4; ++k)
        counts[k] = 0;
    for (const auto& s : m->slots)
        ++counts[s.kind];
    return GDN_OK;
}

} // extern "C"
