/*
 * CPU oracle for the slot-indexed Gated DeltaNet state path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or table with the HIP library.
 *
 * Plain, slow and written to be checked by eye against the pages:
 *   - arithmetic in double precision, one token and one head at a time;
 *   - the recurrent state is held as fp32 between tokens, because the slot
 *     pool stores it as fp32;
 *   - the conv window holds raw bf16 inputs and is moved bit-exactly.
 *
 * Sources (cited by page title and section):
 *   [KAP]  "Kapitsa 源码拆解 05：前缀缓存与模型状态恢复", section on what
 *          Attention and Gated DeltaNet keep (the gated delta rule in prose:
 *          gate decides retention, prediction for k compared with v and the
 *          state corrected by the difference, q reads the updated state).
 *   [LSPC] "Linear-State Prefix Cache 内部机制", §0 (state = conv + ssm per
 *          slot, overwritten in place), §4.1 (has_initial_state), §4.2/§4.3
 *          (restore: per-op paths, cross-layer copy, attention-only layers
 *          skipped, soft failure when no layer is copied).
 *   [NCKV] "非连续 KV Cache" (vLLM Ascend design document), §3 and §3.4 (page
 *          stride, padding skipped by stride), §4/§5 (gather/scatter of
 *          indexed strided state rows, padding and unselected rows kept).
 *
 * Parity status: every function below is pinned by a CPU test (closed forms,
 * invariants, brute force, a library routine or the worked example of [NCKV]
 * §3.4); end-to-end numeric values are not printed by the pages.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32.  bf16 keeps the upper 16 bits of an IEEE-754 binary32.     */
/* ------------------------------------------------------------------------ */
static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 to bf16, nearest with ties to even.  NaN maps to a quiet
 * NaN (0x7FC0); infinities and signed zeros pass through. */
static uint16_t float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u; /* carries into the exponent correctly, up to infinity */
    return (uint16_t)upper;
}

void orc_f32_to_bf16(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = float_to_bf16(in[i]);
}

void orc_bf16_to_f32(const uint16_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_to_float(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Threads                                                                   */
/* ------------------------------------------------------------------------ */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Addressing ([NCKV] §3, §3.4): a slot is one physical page; the page of    */
/* slot s starts s * page_stride bytes into the layer's allocation, and each */
/* region sits at a fixed byte offset inside the page.  Whatever lies between */
/* the end of the payload and the next page is padding and is never touched. */
/* ------------------------------------------------------------------------ */
static uint8_t* page_of(uint8_t* pool, int64_t page_stride, int64_t slot)
{
    return pool + slot * page_stride;
}

/* ------------------------------------------------------------------------ */
/* One GDN layer over a batch of sequences.                                  */
/*                                                                           */
/* Sequence n covers tokens [cu_seqlens[n], cu_seqlens[n+1]) and owns slot   */
/* state_indices[n].  A decode step is the case where every sequence has one */
/* token.                                                                    */
/*                                                                           */
/* Steps per sequence, in the order the method states them:                  */
/*   1. select the initial conv window and state: the slot's contents when   */
/*      has_initial_state != 0, zeros otherwise (the page is not read at all, */
/*      [LSPC] §4.1);                                                        */
/*   2. depthwise causal conv over the window + current input, then SiLU;    */
/*      the window drops its oldest input and appends the current raw input; */
/*   3. split the conv output into q | k | v, L2-normalise q and k per k-head */
/*      (q also multiplied by `scale`);                                       */
/*   4. per v-head h (k-head g = h / (Hv/Hk)) and token:                      */
/*        S <- alpha S;  u = S k;  S <- S + beta (v - u) k^T;  o = S q        */
/*      ([KAP]); S is rounded to fp32 after every token;                      */
/*   5. write the window and the states back into the same slot ([LSPC] §0). */
/*                                                                           */
/* Layouts: x [T][C] bf16; conv_w [C][W] bf16 (tap W-1 multiplies the current */
/* input); conv_b [C] bf16 or NULL; alpha, beta [T][Hv] fp32;                */
/* window region [W-1][C] bf16, oldest input first; state region             */
/* [Hv][dk][dv] fp32, entry (key j, value i) of head h at (h*dk + j)*dv + i; */
/* out [T][Hv][dv] (double and bf16).                                        */
/* A state index outside [0, num_slots) marks a padding row: its outputs are  */
/* zero and its slot is not touched.  A zero-length sequence does nothing.    */
/* ------------------------------------------------------------------------ */

/* Step 2 for one sequence: conv outputs y[t][c] (double) for its L tokens.
 * `win` (in/out) is the window as raw bf16, [W-1][C]. */
static void conv_silu_sequence(int32_t L, int32_t C, int32_t W, uint16_t* win,
                               const uint16_t* x, const uint16_t* conv_w,
                               const uint16_t* conv_b, double* y)
{
    for (int32_t t = 0; t < L; ++t) {
        for (int32_t c = 0; c < C; ++c) {
            double pre = conv_b ? (double)bf16_to_float(conv_b[c]) : 0.0;
            for (int32_t w = 0; w < W - 1; ++w)
                pre += (double)bf16_to_float(conv_w[(int64_t)c * W + w]) *
                       (double)bf16_to_float(win[(int64_t)w * C + c]);
            pre += (double)bf16_to_float(conv_w[(int64_t)c * W + (W - 1)]) *
                   (double)bf16_to_float(x[(int64_t)t * C + c]);
            y[(int64_t)t * C + c] = pre / (1.0 + exp(-pre)); /* SiLU */
        }
        /* shift: drop the oldest input, append the current raw input */
        for (int32_t c = 0; c < C; ++c) {
            for (int32_t w = 0; w + 1 < W - 1; ++w)
                win[(int64_t)w * C + c] = win[(int64_t)(w + 1) * C + c];
            win[(int64_t)(W - 2) * C + c] = x[(int64_t)t * C + c];
        }
    }
}

/* Step 3: v / sqrt(sum v^2 + eps), times `mult`. */
static void l2_normalise(const double* v, int32_t n, double eps, double mult, double* out)
{
    double ss = 0.0;
    for (int32_t j = 0; j < n; ++j)
        ss += v[j] * v[j];
    double r = mult / sqrt(ss + eps);
    for (int32_t j = 0; j < n; ++j)
        out[j] = v[j] * r;
}

/* Step 4 for one v-head over one sequence.  S32 is [dk][dv] fp32 (in/out).
 * q_hat, k_hat: [L][dk] for this head's k-head; v: the conv output rows,
 * value channels of head h at v + t*C. */
static void delta_rule_head(int32_t L, int32_t dk, int32_t dv, float* S32,
                            const double* q_hat, const double* k_hat,
                            const double* y, int64_t y_stride, int64_t v_col,
                            const float* alpha, const float* beta, int64_t gate_stride,
                            double* out64, uint16_t* out16, int64_t out_stride)
{
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    for (int64_t e = 0; e < (int64_t)dk * dv; ++e)
        S[e] = (double)S32[e];

    for (int32_t t = 0; t < L; ++t) {
        const double a = (double)alpha[(int64_t)t * gate_stride];
        const double b = (double)beta[(int64_t)t * gate_stride];
        const double* k = k_hat + (int64_t)t * dk;
        const double* q = q_hat + (int64_t)t * dk;
        const double* v = y + (int64_t)t * y_stride + v_col;

        /* S <- a S */
        for (int64_t e = 0; e < (int64_t)dk * dv; ++e)
            S[e] *= a;
        /* u = S k   (u_i = sum_j S[j][i] k_j) */
        for (int32_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < dk; ++j)
                acc += S[(int64_t)j * dv + i] * k[j];
            u[i] = acc;
        }
        /* S <- S + b (v - u) k^T */
        for (int32_t j = 0; j < dk; ++j)
            for (int32_t i = 0; i < dv; ++i)
                S[(int64_t)j * dv + i] += b * (v[i] - u[i]) * k[j];
        /* o = S q   (with the updated S) */
        for (int32_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < dk; ++j)
                acc += S[(int64_t)j * dv + i] * q[j];
            out64[(int64_t)t * out_stride + i] = acc;
            out16[(int64_t)t * out_stride + i] = float_to_bf16((float)acc);
        }
        /* the state lives in an fp32 pool */
        for (int64_t e = 0; e < (int64_t)dk * dv; ++e)
            S[e] = (double)(float)S[e];
    }
    for (int64_t e = 0; e < (int64_t)dk * dv; ++e)
        S32[e] = (float)S[e];
    free(u);
    free(S);
}

int orc_gdn_layer(uint8_t* pool, int64_t num_slots, int64_t page_stride,
                  int64_t ssm_off, int64_t conv_off,
                  int32_t C, int32_t W, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                  int32_t num_seqs, const int32_t* cu_seqlens,
                  const int32_t* state_indices, const uint8_t* has_initial_state,
                  const uint16_t* x, const uint16_t* conv_w, const uint16_t* conv_b,
                  const float* alpha, const float* beta, double scale, double eps,
                  double* out64, uint16_t* out16)
{
    if (Hk <= 0 || Hv <= 0 || Hv % Hk != 0 || C != 2 * Hk * dk + Hv * dv || W < 2)
        return -1;
    const int32_t group = Hv / Hk;
    const int64_t out_stride = (int64_t)Hv * dv;
    const int64_t ssm_head = (int64_t)dk * dv;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t n = 0; n < num_seqs; ++n) {
        const int32_t t0 = cu_seqlens[n];
        const int32_t L = cu_seqlens[n + 1] - t0;
        const int32_t slot = state_indices[n];
        if (L < 0) {
            bad = 1;
            continue;
        }
        if (L == 0)
            continue;
        if (slot < 0 || slot >= num_slots) { /* padding row */
            for (int64_t e = 0; e < (int64_t)L * out_stride; ++e) {
                out64[(int64_t)t0 * out_stride + e] = 0.0;
                out16[(int64_t)t0 * out_stride + e] = 0;
            }
            continue;
        }
        uint8_t* page = page_of(pool, page_stride, slot);
        const int warm = has_initial_state[n] != 0;

        /* 1. initial window and state (cold: zeros, the page is not read) */
        uint16_t* win = (uint16_t*)calloc((size_t)(W - 1) * C, sizeof(uint16_t));
        float* S = (float*)calloc((size_t)Hv * ssm_head, sizeof(float));
        if (warm) {
            memcpy(win, page + conv_off, sizeof(uint16_t) * (size_t)(W - 1) * C);
            memcpy(S, page + ssm_off, sizeof(float) * (size_t)Hv * ssm_head);
        }

        /* 2. conv + SiLU for every token of the sequence */
        double* y = (double*)malloc(sizeof(double) * (size_t)L * C);
        conv_silu_sequence(L, C, W, win, x + (int64_t)t0 * C, conv_w, conv_b, y);

        /* 3. q | k | v split and L2 norms */
        double* q_hat = (double*)malloc(sizeof(double) * (size_t)L * Hk * dk);
        double* k_hat = (double*)malloc(sizeof(double) * (size_t)L * Hk * dk);
        for (int32_t t = 0; t < L; ++t)
            for (int32_t g = 0; g < Hk; ++g) {
                const double* yt = y + (int64_t)t * C;
                l2_normalise(yt + (int64_t)g * dk, dk, eps, scale,
                             q_hat + ((int64_t)g * L + t) * dk);
                l2_normalise(yt + (int64_t)Hk * dk + (int64_t)g * dk, dk, eps, 1.0,
                             k_hat + ((int64_t)g * L + t) * dk);
            }

        /* 4. gated delta rule, head by head */
        for (int32_t h = 0; h < Hv; ++h) {
            const int32_t g = h / group;
            delta_rule_head(L, dk, dv, S + (int64_t)h * ssm_head,
                            q_hat + (int64_t)g * L * dk, k_hat + (int64_t)g * L * dk,
                            y, C, (int64_t)2 * Hk * dk + (int64_t)h * dv,
                            alpha + (int64_t)t0 * Hv + h, beta + (int64_t)t0 * Hv + h, Hv,
                            out64 + (int64_t)t0 * out_stride + (int64_t)h * dv,
                            out16 + (int64_t)t0 * out_stride + (int64_t)h * dv, out_stride);
        }

        /* 5. write back in place */
        memcpy(page + conv_off, win, sizeof(uint16_t) * (size_t)(W - 1) * C);
        memcpy(page + ssm_off, S, sizeof(float) * (size_t)Hv * ssm_head);

        free(k_hat);
        free(q_hat);
        free(y);
        free(S);
        free(win);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Worker-side restore ([LSPC] §4, §4.2, §4.3).                               */
/*                                                                           */
/* Op i belongs to batch row i and names (dst, src, requested):              */
/*   not requested        -> nothing happens, hs[i] keeps its prefilled value;*/
/*   requested, src < 0   -> a miss: no copy, hs[i] = 0;                      */
/*   requested, src >= 0  -> for every layer that has a state pool (the      */
/*                           attention-only ones have none and are skipped)   */
/*                           copy the conv and state payload bytes of page   */
/*                           src into page dst; hs[i] = 1 if at least one    */
/*                           layer was copied, else 0 and the call reports   */
/*                           the soft failure (returns 1).                   */
/* Only payload bytes move; padding and every other page stay as they were.  */
/* Returns -1 if a copied op names a slot outside [0, num_slots).            */
/* ------------------------------------------------------------------------ */
int orc_restore(uint8_t* const* layer_pools, int32_t num_layers, int64_t num_slots,
                int64_t page_stride, int64_t ssm_off, int64_t ssm_bytes,
                int64_t conv_off, int64_t conv_bytes,
                const int32_t* dst, const int32_t* src, const uint8_t* requested,
                int32_t n_ops, uint8_t* hs)
{
    int soft_failure = 0;
    for (int32_t i = 0; i < n_ops; ++i) {
        if (!requested[i])
            continue;
        if (src[i] < 0) {
            hs[i] = 0;
            continue;
        }
        if (src[i] >= num_slots || dst[i] < 0 || dst[i] >= num_slots)
            return -1;
        int copied = 0;
        for (int32_t l = 0; l < num_layers; ++l) {
            if (layer_pools[l] == NULL)
                continue; /* attention-only layer */
            uint8_t* from = page_of(layer_pools[l], page_stride, src[i]);
            uint8_t* to = page_of(layer_pools[l], page_stride, dst[i]);
            memcpy(to + conv_off, from + conv_off, (size_t)conv_bytes);
            memcpy(to + ssm_off, from + ssm_off, (size_t)ssm_bytes);
            copied += 1;
        }
        hs[i] = copied > 0 ? 1 : 0;
        if (copied == 0)
            soft_failure = 1;
    }
    return soft_failure;
}

/* ------------------------------------------------------------------------ */
/* Gather / scatter of indexed strided state rows ([NCKV] §4, §5).           */
/* Dense row r of each region holds the payload of page idx[r].  Gather      */
/* writes zeros for an index outside [0, num_slots); scatter skips it.       */
/* ------------------------------------------------------------------------ */
void orc_gather(const uint8_t* pool, int64_t num_slots, int64_t page_stride,
                int64_t ssm_off, int64_t ssm_bytes, int64_t conv_off, int64_t conv_bytes,
                const int32_t* idx, int32_t n, uint8_t* ssm_dense, uint8_t* conv_dense)
{
    for (int32_t r = 0; r < n; ++r) {
        uint8_t* sd = ssm_dense + (int64_t)r * ssm_bytes;
        uint8_t* cd = conv_dense + (int64_t)r * conv_bytes;
        if (idx[r] < 0 || idx[r] >= num_slots) {
            memset(sd, 0, (size_t)ssm_bytes);
            memset(cd, 0, (size_t)conv_bytes);
            continue;
        }
        const uint8_t* page = pool + (int64_t)idx[r] * page_stride;
        memcpy(sd, page + ssm_off, (size_t)ssm_bytes);
        memcpy(cd, page + conv_off, (size_t)conv_bytes);
    }
}

void orc_scatter(uint8_t* pool, int64_t num_slots, int64_t page_stride,
                 int64_t ssm_off, int64_t ssm_bytes, int64_t conv_off, int64_t conv_bytes,
                 const int32_t* idx, int32_t n, const uint8_t* ssm_dense,
                 const uint8_t* conv_dense)
{
    for (int32_t r = 0; r < n; ++r) {
        if (idx[r] < 0 || idx[r] >= num_slots)
            continue;
        uint8_t* page = page_of(pool, page_stride, idx[r]);
        memcpy(page + ssm_off, ssm_dense + (int64_t)r * ssm_bytes, (size_t)ssm_bytes);
        memcpy(page + conv_off, conv_dense + (int64_t)r * conv_bytes, (size_t)conv_bytes);
    }
}

/* ------------------------------------------------------------------------ */
/* The two inner steps, exported so that tests can pin each on its own.      */
/* ------------------------------------------------------------------------ */
void orc_conv_silu(int32_t L, int32_t C, int32_t W, uint16_t* win, const uint16_t* x,
                   const uint16_t* conv_w, const uint16_t* conv_b, double* y)
{
    conv_silu_sequence(L, C, W, win, x, conv_w, conv_b, y);
}

/* q_hat, k_hat [L][dk]; v [L][dv]; alpha, beta [L]; S32 [dk][dv] in/out;
 * out64, out16 [L][dv]. */
void orc_delta_rule(int32_t L, int32_t dk, int32_t dv, float* S32, const double* q_hat,
                    const double* k_hat, const double* v, const float* alpha,
                    const float* beta, double* out64, uint16_t* out16)
{
    delta_rule_head(L, dk, dv, S32, q_hat, k_hat, v, dv, 0, alpha, beta, 1, out64, out16, dv);
}
