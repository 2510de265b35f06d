// C-ABI entry points of the GDN state library: pool descriptor, validation,
// error reporting, and dispatch to the gfx950 kernels.  Everything here runs
// on the host and never synchronises with the device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <memory>
#include <new>
#include <string>
#include <unordered_set>

#include "gdn_internal.h"

namespace gdn {

namespace {
thread_local char g_last_error[512];
}

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_last_error[0] = '\0'; }

int check_launch(const char* what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(GDN_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return GDN_OK;
}

} // namespace gdn

using gdn::fail;

namespace {

bool aligned16(int64_t v) { return (v & 15) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) intersect (empty ranges never do).
bool overlaps(int64_t a, int64_t na, int64_t b, int64_t nb)
{
    if (na == 0 || nb == 0)
        return false;
    return a < b + nb && b < a + na;
}

int check_layer(const gdn_pool* pool, int32_t layer)
{
    if (layer < 0 || layer >= pool->desc.num_layers)
        return fail(GDN_ERANGE, "layer %d outside [0, %d)", layer, pool->desc.num_layers);
    if (pool->bases[layer] == nullptr)
        return fail(GDN_ERANGE, "layer %d is attention-only (no state pool)", layer);
    return GDN_OK;
}

// `work` is false for a call that reads and writes nothing (no rows, or no
// tokens): its buffers may then be NULL, as empty tensors are.
int check_step_args(const gdn_pool* pool, int32_t layer, const gdn_step_args* a, bool work)
{
    int rc = check_layer(pool, layer);
    if (rc != GDN_OK)
        return rc;
    if (a == nullptr)
        return fail(GDN_EINVAL, "args is NULL");
    if (work && (!a->x || !a->conv_w || !a->alpha || !a->beta || !a->state_indices ||
                 !a->has_initial_state || !a->out))
        return fail(GDN_EINVAL, "a required device pointer in args is NULL");
    if (pool->desc.num_v_heads == 0)
        return fail(GDN_EUNSUPPORTED, "conv-window-only pool has no recurrent state");
    if (!(a->l2_eps >= 0.0f))
        return fail(GDN_EINVAL, "l2_eps must be >= 0");
    return GDN_OK;
}

int describe(const gdn_pool* pool, char* buf, size_t len)
{
    const gdn_pool_desc& d = pool->desc;
    std::string s;
    char line[512];
    const int64_t payload_end =
        std::max(d.conv_offset_bytes + pool->conv_bytes, d.ssm_offset_bytes + pool->ssm_bytes);
    snprintf(line, sizeof line,
             "[gdn-pool] layers=%d (linear=%zu, attention-only=%zu) slots=%lld "
             "page_stride=%lldB padding_after_payload=%lldB\n",
             d.num_layers, pool->linear.size(), d.num_layers - pool->linear.size(),
             (long long)d.num_slots, (long long)d.page_stride_bytes,
             (long long)(d.page_stride_bytes - payload_end));
    s += line;
    snprintf(line, sizeof line,
             "[gdn-pool] ssm: fp32 [Hv=%d][dk=%d][dv=%d] = %lldB at offset %lld, "
             "slot stride %lld elements\n",
             d.num_v_heads, d.head_k_dim, d.head_v_dim, (long long)pool->ssm_bytes,
             (long long)d.ssm_offset_bytes, (long long)(d.page_stride_bytes / 4));
    s += line;
    snprintf(line, sizeof line,
             "[gdn-pool] conv: bf16 [W-1=%d][C=%d] = %lldB at offset %lld, "
             "slot stride %lld elements (Hk=%d)\n",
             d.conv_width - 1, d.conv_channels, (long long)pool->conv_bytes,
             (long long)d.conv_offset_bytes, (long long)(d.page_stride_bytes / 2),
             d.num_k_heads);
    s += line;
    s += "[gdn-pool] attention-only layers:";
    for (int32_t l = 0; l < d.num_layers; ++l)
        if (!pool->bases[l]) {
            snprintf(line, sizeof line, " %d", l);
            s += line;
        }
    s += "\n";
    if (buf && len > 0) {
        size_t n = std::min(len - 1, s.size());
        memcpy(buf, s.data(), n);
        buf[n] = '\0';
    }
    return (int)s.size();
}

int restore(const gdn_pool* pool, const gdn_restore_op* ops, int32_t n_ops, uint8_t* hs_dev,
            gdn_stream_t stream)
{
    const int64_t ns = pool->desc.num_slots;
    std::vector<gdn::HitPair> pairs;
    std::vector<gdn::HsWrite> hs;
    std::unordered_set<int32_t> dsts;
    for (int32_t i = 0; i < n_ops; ++i) {
        const gdn_restore_op& op = ops[i];
        if (!op.requested)
            continue;
        if (op.src_slot < 0) {
            hs.push_back({i, 0});
            continue;
        }
        if (op.src_slot >= ns || op.dst_slot < 0 || op.dst_slot >= ns)
            return fail(GDN_ERANGE, "op %d: dst %d / src %d outside [0, %lld)", i, op.dst_slot,
                        op.src_slot, (long long)ns);
        if (!dsts.insert(op.dst_slot).second)
            return fail(GDN_EOVERLAP, "op %d: dst slot %d is named twice", i, op.dst_slot);
        pairs.push_back({op.dst_slot, op.src_slot});
        hs.push_back({i, pool->linear.empty() ? 0 : 1});
    }
    for (const gdn::HitPair& p : pairs)
        if (dsts.count(p.src))
            return fail(GDN_EOVERLAP, "src slot %d is also a dst slot", p.src);
    const bool soft_failure = !pairs.empty() && pool->linear.empty();
    if (pool->linear.empty())
        pairs.clear();
    int rc = gdn::launch_restore(pool, pairs, hs, hs_dev, reinterpret_cast<hipStream_t>(stream));
    if (rc != GDN_OK)
        return rc;
    if (soft_failure)
        return fail(GDN_WARN_COLD_FALLBACK,
                    "no layer has a state pool: restored rows fall back to a cold start");
    return GDN_OK;
}

} // namespace

extern "C" {

const char* gdn_last_error(void) { return gdn::g_last_error; }

int gdn_pool_create(const gdn_pool_desc* d, gdn_pool** out)
{
    gdn::clear_error();
    if (!d || !out)
        return fail(GDN_EINVAL, "desc and out must not be NULL");
    if (d->num_layers <= 0 || !d->layer_base)
        return fail(GDN_EINVAL, "num_layers must be > 0 and layer_base non-NULL");
    if (d->num_slots <= 0 || d->num_slots > INT32_MAX)
        return fail(GDN_ERANGE, "num_slots %lld outside [1, 2^31)", (long long)d->num_slots);
    if (d->conv_width < 2 || d->conv_width > 8)
        return fail(GDN_EINVAL, "conv_width %d outside [2, 8]", d->conv_width);
    if (d->conv_channels <= 0 || (d->conv_channels & 1))
        return fail(GDN_EINVAL, "conv_channels %d must be positive and even", d->conv_channels);
    if (d->num_v_heads < 0 || d->num_k_heads < 0 || d->head_k_dim < 0 || d->head_v_dim < 0)
        return fail(GDN_EINVAL, "negative head count or head dim");
    if (d->num_v_heads > 0) {
        if (d->num_k_heads <= 0 || d->num_v_heads % d->num_k_heads != 0)
            return fail(GDN_EINVAL, "num_v_heads %d must be a positive multiple of num_k_heads %d",
                        d->num_v_heads, d->num_k_heads);
        if (d->head_k_dim <= 0 || d->head_v_dim <= 0 || (d->head_k_dim & 3) || (d->head_v_dim & 3))
            return fail(GDN_EINVAL, "head dims must be positive multiples of 4");
        const int64_t c = 2LL * d->num_k_heads * d->head_k_dim +
                          (int64_t)d->num_v_heads * d->head_v_dim;
        if (c != d->conv_channels)
            return fail(GDN_EINVAL, "conv_channels %d != 2*Hk*dk + Hv*dv = %lld",
                        d->conv_channels, (long long)c);
    }
    if (!aligned16(d->page_stride_bytes) || !aligned16(d->conv_offset_bytes) ||
        !aligned16(d->ssm_offset_bytes))
        return fail(GDN_EALIGN, "page stride and region offsets must be multiples of 16 bytes");
    const int64_t ssm = (int64_t)d->num_v_heads * d->head_k_dim * d->head_v_dim * 4;
    const int64_t conv = (int64_t)(d->conv_width - 1) * d->conv_channels * 2;
    if (d->conv_offset_bytes < 0 || d->ssm_offset_bytes < 0 ||
        d->conv_offset_bytes + conv > d->page_stride_bytes ||
        d->ssm_offset_bytes + ssm > d->page_stride_bytes)
        return fail(GDN_ERANGE, "a region does not fit in the %lld-byte page",
                    (long long)d->page_stride_bytes);
    if (overlaps(d->conv_offset_bytes, conv, d->ssm_offset_bytes, ssm))
        return fail(GDN_EOVERLAP, "window and state regions overlap");
    for (int32_t l = 0; l < d->num_layers; ++l)
        if (d->layer_base[l] != nullptr && !aligned16(d->layer_base[l]))
            return fail(GDN_EALIGN, "layer_base[%d] is not 16-byte aligned", l);
    return gdn::guarded([&] {
        std::unique_ptr<gdn_pool> p(new gdn_pool());
        p->desc = *d;
        p->bases.assign(d->layer_base, d->layer_base + d->num_layers);
        p->desc.layer_base = p->bases.data();
        for (int32_t l = 0; l < d->num_layers; ++l)
            if (p->bases[l])
                p->linear.push_back(l);
        p->ssm_bytes = ssm;
        p->conv_bytes = conv;
        *out = p.release();
        return int(GDN_OK);
    });
}

void gdn_pool_destroy(gdn_pool* pool) { delete pool; }

int gdn_pool_region_bytes(const gdn_pool* pool, int64_t* ssm_bytes, int64_t* conv_bytes)
{
    if (!pool)
        return fail(GDN_EINVAL, "pool is NULL");
    if (ssm_bytes)
        *ssm_bytes = pool->ssm_bytes;
    if (conv_bytes)
        *conv_bytes = pool->conv_bytes;
    return GDN_OK;
}

int gdn_pool_step_support(const gdn_pool* pool)
{
    if (!pool)
        return fail(GDN_EINVAL, "pool is NULL");
    const gdn_pool_desc& d = pool->desc;
    if (d.num_v_heads <= 0)
        return 0;
    int mask = 0;
    if (gdn::decode_supported(d.head_k_dim, d.head_v_dim, d.conv_width))
        mask |= GDN_STEP_DECODE;
    if (gdn::prefill_supported(d.head_k_dim, d.head_v_dim, d.conv_width))
        mask |= GDN_STEP_PREFILL;
    return mask;
}

int gdn_pool_describe(const gdn_pool* pool, char* buf, size_t len)
{
    if (!pool)
        return fail(GDN_EINVAL, "pool is NULL");
    return gdn::guarded([&] { return describe(pool, buf, len); });
}

int gdn_restore_slots(const gdn_pool* pool, const gdn_restore_op* ops, int32_t n_ops,
                      uint8_t* hs_dev, gdn_stream_t stream)
{
    gdn::clear_error();
    if (!pool)
        return fail(GDN_EINVAL, "pool is NULL");
    if (n_ops < 0)
        return fail(GDN_EINVAL, "n_ops < 0");
    if (n_ops == 0)
        return GDN_OK;
    if (!ops || !hs_dev)
        return fail(GDN_EINVAL, "ops and has_initial_state must not be NULL");
    return gdn::guarded([&] { return restore(pool, ops, n_ops, hs_dev, stream); });
}

// The dense buffers: bf16 window rows, fp32 state rows.
static int check_dense(const gdn_pool* pool, const int32_t* idx, const void* conv_dense,
                       const void* ssm_dense)
{
    if (!idx || (pool->ssm_bytes > 0 && !ssm_dense) || !conv_dense)
        return fail(GDN_EINVAL, "idx / dense buffers must not be NULL");
    if ((reinterpret_cast<uintptr_t>(conv_dense) & 1u) != 0 ||
        (reinterpret_cast<uintptr_t>(ssm_dense) & 3u) != 0)
        return fail(GDN_EALIGN, "conv_dense must be 2-byte and ssm_dense 4-byte aligned");
    return GDN_OK;
}

int gdn_gather_states(const gdn_pool* pool, int32_t layer, const int32_t* idx, int32_t n,
                      void* conv_dense, float* ssm_dense, gdn_stream_t stream)
{
    gdn::clear_error();
    if (!pool)
        return fail(GDN_EINVAL, "pool is NULL");
    int rc = check_layer(pool, layer);
    if (rc != GDN_OK)
        return rc;
    if (n < 0)
        return fail(GDN_EINVAL, "n < 0");
    if (n == 0)
        return GDN_OK;
    rc = check_dense(pool, idx, conv_dense, ssm_dense);
    if (rc != GDN_OK)
        return rc;
    return gdn::launch_gather(pool, layer, idx, n, ssm_dense, conv_dense,
                              reinterpret_cast<hipStream_t>(stream));
}

int gdn_scatter_states(const gdn_pool* pool, int32_t layer, const int32_t* idx, int32_t n,
                       const void* conv_dense, const float* ssm_dense, gdn_stream_t stream)
{
    gdn::clear_error();
    if (!pool)
        return fail(GDN_EINVAL, "pool is NULL");
    int rc = check_layer(pool, layer);
    if (rc != GDN_OK)
        return rc;
    if (n < 0)
        return fail(GDN_EINVAL, "n < 0");
    if (n == 0)
        return GDN_OK;
    rc = check_dense(pool, idx, conv_dense, ssm_dense);
    if (rc != GDN_OK)
        return rc;
    return gdn::launch_scatter(pool, layer, idx, n, ssm_dense, conv_dense,
                               reinterpret_cast<hipStream_t>(stream));
}

int gdn_decode_step(const gdn_pool* pool, int32_t layer, int32_t rows, const gdn_step_args* a,
                    gdn_stream_t stream)
{
    gdn::clear_error();
    if (!pool)
        return fail(GDN_EINVAL, "pool is NULL");
    if (rows < 0)
        return fail(GDN_EINVAL, "rows < 0");
    int rc = check_step_args(pool, layer, a, rows > 0);
    if (rc != GDN_OK)
        return rc;
    const gdn_pool_desc& d = pool->desc;
    if (!gdn::decode_supported(d.head_k_dim, d.head_v_dim, d.conv_width))
        return fail(GDN_EUNSUPPORTED, "no decode kernel for dk=%d dv=%d W=%d", d.head_k_dim,
                    d.head_v_dim, d.conv_width);
    if (rows == 0)
        return GDN_OK;
    if ((reinterpret_cast<uintptr_t>(a->out) & 7u) != 0)
        return fail(GDN_EALIGN, "out must be 8-byte aligned");
    if ((reinterpret_cast<uintptr_t>(a->x) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(a->conv_w) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(a->conv_b) & 3u) != 0)
        return fail(GDN_EALIGN, "x, conv_w and conv_b must be 4-byte aligned");
    return gdn::launch_decode(pool, layer, rows, a, reinterpret_cast<hipStream_t>(stream));
}

namespace {
int prefill_common(const gdn_pool* pool, int32_t layer, int32_t num_seqs,
                   const int32_t* cu_seqlens, int32_t max_seqlen, int64_t total_tokens,
                   const gdn_step_args* a, const int32_t* ckpt_slot, const int32_t* ckpt_len,
                   gdn_stream_t stream)
{
    if (!pool)
        return fail(GDN_EINVAL, "pool is NULL");
    if (num_seqs < 0 || max_seqlen < 0 || total_tokens < 0)
        return fail(GDN_EINVAL, "negative num_seqs / max_seqlen / total_tokens");
    const bool work = num_seqs > 0 && total_tokens > 0 && max_seqlen > 0;
    int rc = check_step_args(pool, layer, a, work);
    if (rc != GDN_OK)
        return rc;
    if (work && !cu_seqlens)
        return fail(GDN_EINVAL, "cu_seqlens is NULL");
    const gdn_pool_desc& d = pool->desc;
    if (!gdn::prefill_supported(d.head_k_dim, d.head_v_dim, d.conv_width))
        return fail(GDN_EUNSUPPORTED, "no prefill kernel for dk=%d dv=%d W=%d", d.head_k_dim,
                    d.head_v_dim, d.conv_width);
    if (!work)
        return GDN_OK;
    if ((reinterpret_cast<uintptr_t>(a->out) & 7u) != 0)
        return fail(GDN_EALIGN, "out must be 8-byte aligned");
    if ((reinterpret_cast<uintptr_t>(a->x) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(a->conv_w) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(a->conv_b) & 3u) != 0)
        return fail(GDN_EALIGN, "x, conv_w and conv_b must be 4-byte aligned");
    return gdn::launch_prefill(pool, layer, num_seqs, total_tokens, cu_seqlens, a, ckpt_slot,
                               ckpt_len, reinterpret_cast<hipStream_t>(stream));
}
} // namespace

int gdn_prefill_varlen(const gdn_pool* pool, int32_t layer, int32_t num_seqs,
                       const int32_t* cu_seqlens, int32_t max_seqlen, int64_t total_tokens,
                       const gdn_step_args* a, gdn_stream_t stream)
{
    gdn::clear_error();
    return prefill_common(pool, layer, num_seqs, cu_seqlens, max_seqlen, total_tokens, a,
                          nullptr, nullptr, stream);
}

int gdn_prefill_varlen_checkpoint(const gdn_pool* pool, int32_t layer, int32_t num_seqs,
                                  const int32_t* cu_seqlens, int32_t max_seqlen,
                                  int64_t total_tokens, const gdn_step_args* a,
                                  const int32_t* ckpt_slot_dev, const int32_t* ckpt_len_dev,
                                  gdn_stream_t stream)
{
    gdn::clear_error();
    if ((!ckpt_slot_dev || !ckpt_len_dev) && num_seqs > 0 && total_tokens > 0 && max_seqlen > 0)
        return fail(GDN_EINVAL, "ckpt_slot and ckpt_len must not be NULL");
    return prefill_common(pool, layer, num_seqs, cu_seqlens, max_seqlen, total_tokens, a,
                          ckpt_slot_dev, ckpt_len_dev, stream);
}

} // extern "C"
