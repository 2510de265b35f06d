/*
 * gdn.h -- C ABI of the slot-indexed Gated DeltaNet state library (MI355X,
 * gfx950).
 *
 * What it computes, with the passages that define it:
 *   - "Linear-State Prefix Cache 内部机制" (xLLM notes), §0: each GDN layer
 *     keeps a per-slot recurrent state made of a short-conv window and an ssm
 *     state, and every step overwrites it in place; §4 / §4.1-§4.3: the worker
 *     restores a checkpoint by copying it across layers, skipping attention-only
 *     layers, and writes has_initial_state; §6: one op per batch row.
 *   - "非连续 KV Cache" (vLLM Ascend design document), §1, §3, §3.2-§3.4: slots
 *     are pages of a page-aligned pool; each region is a view that advances by
 *     the physical page stride, so padding is skipped, never copied; §4-§5:
 *     indexed gather into dense rows and in-place scatter back; §6: the conv
 *     update and the recurrent gated delta rule.
 *   - "Kapitsa 源码拆解 05：前缀缓存与模型状态恢复", the section on what
 *     Attention and Gated DeltaNet keep: the gated delta rule (retention gate,
 *     prediction for k compared with v, correction by the difference, q reads
 *     the updated state); the section on partial reuse: restore at a saved
 *     position and recompute the rest.
 *
 * The recurrence, per token, v-head h reading k-head g = h / (Hv/Hk):
 *     y  = SiLU(conv over the window and the current input)   (depthwise)
 *     q^ = scale * q / sqrt(|q|^2 + eps),  k^ = k / sqrt(|k|^2 + eps)
 *     S <- alpha S;   u = S k^;   S <- S + beta (v - u) k^T;   o = S q^
 *
 * Conventions
 *   - Every device buffer and the stream belong to the caller.  The library
 *     never allocates or frees device memory and never synchronises: every
 *     call only validates on the host and enqueues kernels on `stream`.
 *   - Return value: 0 (GDN_OK) on success, GDN_WARN_COLD_FALLBACK (+1) for
 *     the restore soft failure, a negative GDN_E* code otherwise; nothing is
 *     launched when a negative code is returned.  gdn_last_error() gives a
 *     message for the last non-zero return on the calling thread.
 *   - Device faults (e.g. from a bad device pointer) surface at the caller's
 *     next synchronisation, as with any asynchronous GPU call.
 *   - Indices that live in device memory (state_indices, gather/scatter
 *     indices) cannot be checked on the host: an index outside
 *     [0, num_slots) marks a padding row -- no state is read or written and
 *     its outputs are zero.  Within one call the in-range indices must be
 *     distinct (two rows writing one slot race).
 *
 * Page layout (per layer; one layer = one cache group of the pool)
 *   slot s of layer l starts at layer_base[l] + s * page_stride_bytes.
 *   state region at ssm_offset_bytes:   fp32 [Hv][dk][dv]; entry (key j,
 *       value i) of head h at element (h*dk + j)*dv + i.
 *   window region at conv_offset_bytes: bf16 [W-1][C], oldest input first;
 *       it holds raw (pre-conv) inputs.
 *   the remaining bytes of the page are padding and are never accessed.
 *   Channel order of C: q (Hk*dk) | k (Hk*dk) | v (Hv*dv).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* gdn_stream_t; /* the same type as hipStream_t */

enum {
    GDN_OK = 0,
    GDN_WARN_COLD_FALLBACK = 1, /* restore: a requested hit copied no layer */
    GDN_EINVAL = -1,            /* bad argument (NULL, negative size, ...) */
    GDN_ERANGE = -2,            /* slot / layer / size out of range */
    GDN_EOVERLAP = -3,          /* restore: duplicate dst, or a src that is also a dst */
    GDN_EALIGN = -4,            /* a pointer, offset or stride breaks the alignment its call states */
    GDN_EUNSUPPORTED = -5,      /* geometry without a compiled kernel variant */
    GDN_EHIP = -6,              /* the HIP runtime refused a launch */
    GDN_ENOMEM = -11            /* host memory exhausted (no C++ exception crosses the ABI) */
};

/* ---------------------------------------------------------------------- */
/* Pool descriptor                                                          */
/* ---------------------------------------------------------------------- */
typedef struct gdn_pool gdn_pool; /* opaque, host-side, immutable; owns no device memory */

typedef struct {
    int32_t num_layers;           /* whole hybrid stack, attention-only layers included */
    void* const* layer_base;      /* [num_layers] device pointers (caller-owned, 16-byte
                                     aligned), each num_slots * page_stride_bytes long;
                                     NULL marks an attention-only layer (no GDN state) */
    int64_t num_slots;            /* pages per layer */
    int64_t page_stride_bytes;    /* physical page; >= payload, multiple of 16 */
    int64_t conv_offset_bytes;    /* window region offset in the page, multiple of 16 */
    int64_t ssm_offset_bytes;     /* state region offset in the page, multiple of 16 */
    int32_t conv_channels;        /* C; must be 2*Hk*dk + Hv*dv when Hv > 0 */
    int32_t conv_width;           /* W in [2, 8]; the window keeps W-1 inputs */
    int32_t num_k_heads;          /* Hk */
    int32_t num_v_heads;          /* Hv (multiple of Hk); 0 = conv-window-only pool,
                                     usable by restore / gather / scatter only */
    int32_t head_k_dim;           /* dk */
    int32_t head_v_dim;           /* dv */
} gdn_pool_desc;

/* Validate `desc` and build a pool handle (copies the layer table).
 * Checks: sizes positive, regions inside the page and not overlapping,
 * 16-byte alignment of strides, offsets and layer bases (GDN_EALIGN),
 * C == 2*Hk*dk + Hv*dv, Hv % Hk == 0.  A pool describes a memory layout, so
 * any such geometry is accepted: restore, gather and scatter work on all of
 * them.  The step kernels cover dk == dv in {16, 32, 64, 128} with conv
 * widths 2-4 (gdn_pool_step_support says which apply); on other pools
 * gdn_decode_step and gdn_prefill_varlen return GDN_EUNSUPPORTED.  *out is
 * set only on success. */
int gdn_pool_create(const gdn_pool_desc* desc, gdn_pool** out);
void gdn_pool_destroy(gdn_pool* pool);

/* Bytes of the state region and of the window region of one page. */
int gdn_pool_region_bytes(const gdn_pool* pool, int64_t* ssm_bytes, int64_t* conv_bytes);

/* Which step kernels exist for the pool's geometry: GDN_STEP_DECODE when
 * gdn_decode_step can run on it, GDN_STEP_PREFILL when gdn_prefill_varlen
 * and gdn_prefill_varlen_checkpoint can (0 for a conv-window-only pool or
 * head dims / conv width without a compiled kernel).  Returns the mask
 * (>= 0), or GDN_EINVAL for a NULL pool.  Host-only; touches no device. */
#define GDN_STEP_DECODE 1
#define GDN_STEP_PREFILL 2
int gdn_pool_step_support(const gdn_pool* pool);

/* Human-readable layout dump (shapes, strides, offsets, padding, which layers
 * are attention-only), NUL-terminated, truncated to `len`.  Returns the
 * length the full text needs (excluding the NUL), or a negative code.
 * Mirrors the layout debug log of the vLLM Ascend page, §7. */
int gdn_pool_describe(const gdn_pool* pool, char* buf, size_t len);

/* ---------------------------------------------------------------------- */
/* Worker-side restore ("Linear-State Prefix Cache 内部机制" §4, §4.2, §4.3) */
/* ---------------------------------------------------------------------- */
typedef struct {
    int32_t dst_slot;  /* the row's live slot */
    int32_t src_slot;  /* checkpoint slot found by the scheduler, or -1 (miss) */
    int32_t requested; /* non-zero: the row asked for a restore */
} gdn_restore_op;

/* Op i belongs to batch row i and acts on has_initial_state_dev[i] (device,
 * uint8, length n_ops, prefilled by the caller):
 *   requested == 0           -> nothing; hs[i] keeps its prefilled value;
 *   requested, src_slot < 0  -> miss: no copy; hs[i] = 0;
 *   requested, src_slot >= 0 -> for every layer whose base is not NULL copy
 *       the window and state payload bytes of page src_slot into page
 *       dst_slot (padding untouched); hs[i] = 1.  If the pool has no such
 *       layer nothing is copied, hs[i] = 0 and the call returns
 *       GDN_WARN_COLD_FALLBACK (soft failure: the row starts cold).
 * Host checks before any launch: slots of hits in range (GDN_ERANGE); dst
 * slots of hits distinct and no src equal to any hit's dst (GDN_EOVERLAP;
 * several hits may share one src).  ops_host is host memory and may be
 * reused as soon as the call returns.  Enqueued on `stream` without a host
 * sync: a forward on another stream must wait on an event recorded after it. */
int gdn_restore_slots(const gdn_pool* pool, const gdn_restore_op* ops_host, int32_t n_ops,
                      uint8_t* has_initial_state_dev, gdn_stream_t stream);

/* ---------------------------------------------------------------------- */
/* Gather / scatter of indexed rows ("非连续 KV Cache" §4, §5)              */
/* ---------------------------------------------------------------------- */
/* gather:  conv_dense[r] = window payload of page idx[r],
 *          ssm_dense[r]  = state payload of page idx[r]  (r < n);
 *          an out-of-range idx[r] gives zero rows.
 * scatter: the reverse; an out-of-range idx[r] is skipped; padding and
 *          slots not named are left untouched.
 * idx_dev: device int32 [n].  conv_dense: device bf16 [n][(W-1) * C]
 * (2-byte aligned); ssm_dense: device fp32 [n][Hv * dk * dv] (4-byte aligned;
 * may be NULL for a conv-window-only pool).  Rows are packed back to back in
 * the dense buffers.  Bit-exact copies.  Errors: GDN_EINVAL (NULL pointer,
 * n < 0), GDN_ERANGE (layer out of range or attention-only), GDN_EALIGN. */
int gdn_gather_states(const gdn_pool* pool, int32_t layer, const int32_t* idx_dev, int32_t n,
                      void* conv_dense, float* ssm_dense, gdn_stream_t stream);
int gdn_scatter_states(const gdn_pool* pool, int32_t layer, const int32_t* idx_dev, int32_t n,
                       const void* conv_dense, const float* ssm_dense, gdn_stream_t stream);

/* ---------------------------------------------------------------------- */
/* Decode step and varlen prefill ("非连续 KV Cache" §5-§6; the Kapitsa     */
/* page's delta-rule description)                                           */
/* ---------------------------------------------------------------------- */
typedef struct {
    const uint16_t* x;                  /* bf16 [tokens][C]: pre-conv q|k|v input */
    const uint16_t* conv_w;             /* bf16 [C][W]; tap W-1 multiplies the current input */
    const uint16_t* conv_b;             /* bf16 [C] or NULL */
    const float* alpha;                 /* fp32 [tokens][Hv]: the decay itself (not its log) */
    const float* beta;                  /* fp32 [tokens][Hv] */
    const int32_t* state_indices;       /* int32 [rows or sequences]: slot per row */
    const uint8_t* has_initial_state;   /* uint8 [rows or sequences]: 0 = start from zero */
    uint16_t* out;                      /* bf16 [tokens][Hv][dv] */
    float scale;                        /* multiplies q after its L2 norm */
    float l2_eps;                       /* added to |q|^2 and |k|^2 inside the sqrt */
} gdn_step_args;

/* One decode step of `rows` rows, one token each, on GDN layer `layer`.
 * Row r uses slot state_indices[r]; when has_initial_state[r] == 0 the
 * window and state are taken as zero and the page is not read.  The updated
 * window and state are written back into the same page.  All pointers in
 * `args` are device pointers (conv_b may be NULL).  rows == 0 is a no-op
 * that reads no buffer (they may then be NULL, as empty tensors are).
 * Alignment: x, conv_w and conv_b 4-byte aligned, out 8-byte aligned.
 * Errors: GDN_EINVAL (NULL pointer, rows < 0), GDN_ERANGE (layer out of
 * range or attention-only), GDN_EUNSUPPORTED (head dims), GDN_EALIGN. */
int gdn_decode_step(const gdn_pool* pool, int32_t layer, int32_t rows,
                    const gdn_step_args* args, gdn_stream_t stream);

/* Varlen prefill: sequence n covers tokens [cu[n], cu[n+1]) of x / alpha /
 * beta / out and owns slot state_indices[n].  The state is carried on chip
 * from token to token; the final window and state are written back in place.
 * cu_seqlens_dev: device int32 [num_seqs + 1], non-decreasing, cu[0] == 0,
 * cu[num_seqs] == total_tokens (not checkable on the host without a
 * synchronisation; the kernels skip a sequence whose range is empty or not
 * inside [0, total_tokens): no memory access, its slot and output rows are
 * left as they were).  max_seqlen is an upper bound of the lengths (host
 * hint).  A zero-length sequence leaves its slot untouched.  A call with
 * num_seqs, total_tokens or max_seqlen zero is a no-op whose buffers may be
 * NULL (cu_seqlens_dev and the checkpoint arrays included).  Alignment as
 * for gdn_decode_step: x, conv_w and conv_b 4-byte aligned, out 8-byte
 * aligned.  Errors as for gdn_decode_step. */
int gdn_prefill_varlen(const gdn_pool* pool, int32_t layer, int32_t num_seqs,
                       const int32_t* cu_seqlens_dev, int32_t max_seqlen, int64_t total_tokens,
                       const gdn_step_args* args, gdn_stream_t stream);

/* Varlen prefill that also writes a block-boundary checkpoint ("Linear-State
 * Prefix Cache 内部机制" §3.1: the checkpoint is the recurrent state at a
 * block-aligned boundary; here the boundary may fall inside the chunk the
 * call computes, so the state there is emitted into a separate page instead
 * of being lost).  Sequence n with 0 <= ckpt_slot_dev[n] < num_slots and
 * 1 <= ckpt_len_dev[n] <= its length gets, in page ckpt_slot_dev[n], the
 * window and state after its first ckpt_len_dev[n] tokens (payload only;
 * padding untouched); other values mean no checkpoint for that sequence.
 * ckpt_slot_dev, ckpt_len_dev: device int32 [num_seqs], both non-NULL
 * unless the call is a no-op (GDN_EINVAL).  A checkpoint slot must differ from every state_indices
 * entry and from the other checkpoint slots of the call (not checkable on
 * the host; two writers of one page race).  Everything else as
 * gdn_prefill_varlen, whose results it leaves unchanged. */
int gdn_prefill_varlen_checkpoint(const gdn_pool* pool, int32_t layer, int32_t num_seqs,
                                  const int32_t* cu_seqlens_dev, int32_t max_seqlen,
                                  int64_t total_tokens, const gdn_step_args* args,
                                  const int32_t* ckpt_slot_dev, const int32_t* ckpt_len_dev,
                                  gdn_stream_t stream);

/* Message for the last non-zero return on this thread ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
