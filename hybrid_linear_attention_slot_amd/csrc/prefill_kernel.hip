// Varlen recurrent prefill of a Gated DeltaNet layer over a page-strided
// slot pool (gfx950).
//
// Sequence n covers tokens [cu[n], cu[n+1]) and owns slot state_indices[n].
// Its window and state are gathered once (or taken as zero when
// has_initial_state is 0, "Linear-State Prefix Cache 内部机制" §4.1), the
// causal conv + SiLU, the q/k L2 norms and the gated delta rule run token by
// token with the state kept on chip ("Kapitsa 源码拆解 05": the work per
// token does not grow with the history), and the final window and state are
// scattered back into the same page ("非连续 KV Cache" §5-§6).
//
// Parallel structure.  Every value column of a head's state evolves on its
// own once k, v, a, b of the token are known, so a workgroup takes one
// (sequence, v-head, slice of ISZ value columns) and keeps that slice of the
// state in registers for the whole sequence.  Its waves have two roles:
//   - consumer waves run the recurrence and nothing else.  A lane holds KPL
//     keys of one value column (keys 4 jl + 4 LPC m + e, so that the LPC
//     lanes of a column read one contiguous run of k from LDS); S k is a
//     lane-partial dot product finished with DPP sums over the LPC lanes,
//     d = b (v - a S_old k^) and S <- a S_old + d k^T.  A consumer writes d of
//     every token, and the state at the start of every chunk, to LDS;
//   - producer waves prepare the next chunk of CT tokens while the consumers
//     work on the current one (raw inputs loaded into registers a chunk
//     ahead, conv + SiLU, norm factors, decay products), and form the
//     outputs of a chunk from what the consumers left, on the matrix cores.
//     Within a chunk, with S_0 the state at its start, A_t the product of the
//     chunk's decays through token t and D the chunk's d values,
//         o_t = S_t q^_t = A_t S_0 q^_t + sum_{s<=t} (A_t / A_s) (k^_s . q^_t) d_s,
//     i.e. per 16-column block O = alpha (S_0 Q^T) + D M^T with M the masked,
//     decay-weighted 16x16 Q K^T of the chunk: three fp32 16x16x4 MFMA
//     products per chunk (S_0 Q^T and Q K^T while the consumers run the
//     chunk, D M^T after it).  The output is not on the recurrence's path, so
//     this takes a third of the per-token work off the serial chain.
// Consumers and producers meet at two barriers per chunk (one after the
// consumers have written the chunk's starting state, one at its end).  The L2
// norm factors are applied to reduced sums and coefficients, so k and q stay
// raw in LDS.  A run split at a multiple of the chunk length (16 tokens) and
// resumed from the written-back state gives the same bits as the straight
// run: the state is folded to its plain form at every chunk start, which is
// also the form written back, and a chunk's outputs depend only on that state
// and the chunk's own inputs.
//
// The conv window is rewritten by a second small kernel after this one, so
// that no workgroup of a sequence can overwrite the window another workgroup
// of the same sequence has yet to read.
#include <algorithm>
#include <type_traits>

#include "device_utils.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int DK, int DV>
struct PrefillShape {
    static constexpr int KPL = DK >= 128 ? 16 : (DK >= 32 ? 8 : 4); // keys per consumer lane
    static constexpr int LPC = DK / KPL;                            // lanes sharing one column
    static constexpr int CPW = 64 / LPC;                            // columns per consumer wave
    static constexpr int NCONS = (DV / CPW) < 4 ? (DV / CPW) : 4;   // consumer waves
    static constexpr int NPROD = 4;                                 // producer waves
    static constexpr int ISZ = NCONS * CPW;                         // value columns per workgroup
    static constexpr int NSL = DV / ISZ;                            // workgroups per head
    static constexpr int NT = 64 * (NCONS + NPROD);
    static constexpr int CT = 16;                                   // tokens per chunk
    static constexpr int YS = 2 * DK + ISZ + 4;   // conv outputs per token row (q|k|v slice|pad)
    static constexpr int SROW = DK + 4;           // starting-state row (one value column), padded
    static constexpr int NCB = ISZ / 16;          // 16-column output blocks
    static constexpr int KQ = DK / 4;             // keys per MFMA lane group
    static constexpr int QKP = DK / 2;            // q (and k) channel pairs
    static constexpr int NVP = ISZ / 2;           // v channel pairs
    static constexpr int TPW = CT / NPROD;        // tokens per producer wave
    static constexpr int NVJ = (TPW * NVP + 63) / 64; // v conv jobs per producer lane
    // Q K^T is split over the producer waves without an output block: GP
    // parts of the key range (a power of two dividing the KQ / 4 steps)
    static constexpr int GFREE = NPROD - NCB;
    static constexpr int GP = (GFREE >= 4 && (KQ / 4) % 4 == 0) ? 4
                            : (GFREE >= 2 && (KQ / 4) % 2 == 0) ? 2 : 1;
    static_assert(DK == DV, "square heads only");
    static_assert(KPL % 4 == 0 && DK % KPL == 0 && LPC >= 1 && LPC <= 64, "key split");
    static_assert(NCONS >= 1 && DV % ISZ == 0 && ISZ % 16 == 0, "column split");
    static_assert(CT == 16, "a chunk is one 16-wide MFMA tile and one 16-lane DPP row");
    static_assert(NCB <= NPROD, "each producer wave keeps at most one output block");
    static_assert(QKP <= 64, "one q/k channel pair per producer lane");
    static_assert(KQ % 4 == 0, "MFMA operands are read as float4 runs");
};

struct PrefillParams {
    uint8_t* layer;
    int64_t page_stride;
    int64_t ssm_off;
    int64_t conv_off;
    int32_t num_slots;
    int32_t num_seqs;
    int64_t total_tokens; // rows of x / alpha / beta / out
    int32_t C;
    int32_t Hk;
    int32_t Hv;
    const int32_t* cu;
    const uint16_t* x;
    const uint16_t* conv_w;
    const uint16_t* conv_b;
    const float* alpha;
    const float* beta;
    const int32_t* state_indices;
    const uint8_t* hs;
    uint16_t* out;
    const int32_t* ckpt_slot; // NULL, or per sequence: page that receives the
    const int32_t* ckpt_len;  // state after the first ckpt_len tokens
    float scale;
    float eps;
};

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lo_bf16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// The sequence at dispatch position r when sequences are placed by length:
// the first half of the positions takes the longest sequences (longest
// first), the second half the shortest (shortest first).  Each XCD fills its
// CUs in dispatch order, so the long sequences get a CU each and then share
// it with the short ones, which finish early.  Ranks break ties by index; up
// to 64 sequences (one per lane), identity beyond.
__device__ __forceinline__ int seq_at_position(const int32_t* cu, int N, int r)
{
    if (N > 64 || N < 2)
        return r;
    const int half = (N + 1) / 2;
    const int want = r < half ? r : N - 1 - (r - half);
    const int m = threadIdx.x & 63;
    int rank = -1;
    if (m < N) {
        const int lm = cu[m + 1] - cu[m];
        rank = 0;
        for (int j = 0; j < N; ++j) {
            const int lj = cu[j + 1] - cu[j];
            rank += (lj > lm || (lj == lm && j < m)) ? 1 : 0;
        }
    }
    const uint64_t hit = __ballot(rank == want);
    return __ffsll(static_cast<long long>(hit)) - 1;
}

// The scale of the state is folded into it once it falls below 2^-40 (bits
// of the float), so s stays within 2^40 of the state's magnitude.
constexpr uint32_t kFoldBelow = (127u - 40u) << 23;

// A token's coefficients in LDS (floats):
//   SC_SCALED  c rk, b, rk / c, c     (c: running product of the chunk's
//                                     decays through the token)
//   SC_PLAIN   a, b, rk, rq           (chunks that may need a fold)
constexpr int SC_SCALED = 0, SC_PLAIN = 4, SC_N = 8;

constexpr int kBufferWord3 = 0x00020000; // raw 32-bit buffer resource, gfx9-family layout

// A buffer resource's range from a wave-uniform byte count, capped at
// INT32_MAX; kept in a scalar register so loads through it need no loop
// over distinct resources.
__device__ __forceinline__ int range_bytes(int64_t n)
{
    const int r = n > int64_t(INT32_MAX) ? INT32_MAX : int(n);
    return __builtin_amdgcn_readfirstlane(r);
}

// v * (lane v of the row n lanes lower), or v * 1 for the first n lanes of
// each 16-lane row (DPP row_shr; an invalid source keeps the `old` operand)
template <int N>
__device__ __forceinline__ float row_shr_or_one(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(v),
                                                      0x110 + N, 0xF, 0xF, false));
}

__device__ __forceinline__ v4f mfma16(float a, float b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int DK, int DV, int W>
// four waves per SIMD: two 512-thread workgroups per CU (their LDS fits too)
__global__ __launch_bounds__((PrefillShape<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(4)))
void prefill_kernel(PrefillParams p)
{
    using Sh = PrefillShape<DK, DV>;
    constexpr int KPL = Sh::KPL, LPC = Sh::LPC, CPW = Sh::CPW, NCONS = Sh::NCONS;
    constexpr int ISZ = Sh::ISZ, CT = Sh::CT, YS = Sh::YS, SROW = Sh::SROW, NCB = Sh::NCB;
    constexpr int KQ = Sh::KQ, QKP = Sh::QKP, NVP = Sh::NVP, TPW = Sh::TPW, NVJ = Sh::NVJ;

    // Chunk k's inputs are written while chunk k-1 runs, read by the
    // consumers and the products while it runs, and its coefficients once more
    // by its epilogue while chunk k+1 runs, when chunk k+2 is being prepared:
    // hence two buffers for the conv outputs and three for the coefficients.
    __shared__ __align__(16) float ys[2][CT][YS];      // conv outputs (raw q | raw k | v)
    __shared__ __align__(16) float s0[ISZ][SROW];      // the state at the current chunk's start
    __shared__ __align__(16) float sc[3][CT][SC_N];    // per token coefficients (SC_*)
    __shared__ __align__(16) float alf[3][CT];         // output scale A_t rq_t per token
    __shared__ __align__(16) float dbuf[2][CT][ISZ];   // d per (token, value column)
    __shared__ __align__(16) float gq[2][Sh::GP][CT][CT]; // parts of a chunk's Q K^T
    __shared__ __align__(16) v4f pq[2][NCB][64];        // S_0 Q^T of a block, MFMA lane order
    __shared__ uint32_t nofold[3];                     // the chunk's decays need no fold

    // workgroup -> (k-head g, dispatch position of sequence n, v-head of the
    // group, slice): the workgroups of one (n, g) read the same q/k inputs and
    // share an XCD
    const int G = p.Hv / p.Hk;
    const int nblocks = p.num_seqs * p.Hv * Sh::NSL;
    const int id = xcd_contiguous_id(blockIdx.x, nblocks);
    const int per_g = p.num_seqs * G * Sh::NSL;
    const int g = id / per_g;
    const int r0 = id - g * per_g;
    const int pos = r0 / (G * Sh::NSL);
    const int n = __builtin_amdgcn_readfirstlane(seq_at_position(p.cu, p.num_seqs, pos));
    const int r1 = r0 - pos * (G * Sh::NSL);
    const int h = g * G + r1 / Sh::NSL;
    const int sl = r1 % Sh::NSL;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform: role and token
    const int lane = tid & 63;                                 // indices go to scalar registers
    // a sequence whose range is empty or not inside [0, total_tokens) is skipped
    const int64_t tb64 = p.cu[n], te64 = p.cu[n + 1];
    if (tb64 < 0 || te64 <= tb64 || te64 > p.total_tokens)
        return;
    const int tb = int(tb64);
    const int L = int(te64 - tb64);
    const int64_t out_tok = int64_t(p.Hv) * DV; // out elements per token
    uint16_t* out_base = p.out + int64_t(tb) * out_tok + int64_t(h) * DV + sl * ISZ;
    const int slot = p.state_indices[n];
    if (slot < 0 || slot >= p.num_slots) { // padding row: zero outputs, no state I/O
        for (int e = tid; e < L * (ISZ / 4); e += Sh::NT) {
            const int tt = e / (ISZ / 4), c4 = e - tt * (ISZ / 4);
            *reinterpret_cast<uint2*>(out_base + tt * out_tok + 4 * c4) = make_uint2(0u, 0u);
        }
        return;
    }
    const bool warm = p.hs[n] != 0;
    uint8_t* page = p.layer + int64_t(slot) * p.page_stride;
    const int nchunks = (L + CT - 1) / CT;

    // global channel of the workgroup's channel `ch` (q | k | v slice)
    auto chan = [&](int ch) -> int {
        if (ch < DK)
            return g * DK + ch;
        if (ch < 2 * DK)
            return p.Hk * DK + g * DK + (ch - DK);
        return 2 * p.Hk * DK + h * DV + sl * ISZ + (ch - 2 * DK);
    };
    auto chunk_len = [&](int k) { return min(CT, L - k * CT); };

    if (wave < NCONS) {
        // ======================= consumer waves =============================
        // (each consumer shares its SIMD with a producer wave; the two roles'
        // work per chunk is balanced, so neither takes issue priority)
        const int col = wave * CPW + lane / LPC; // value column inside the slice
        const int jl = lane % LPC;
        const int gcol = sl * ISZ + col;
        float* tile = reinterpret_cast<float*>(page + p.ssm_off) + int64_t(h) * DK * DV;
        float s[KPL];
#pragma unroll
        for (int m = 0; m < KPL / 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s[4 * m + e] = warm ? tile[(4 * jl + 4 * LPC * m + e) * DV + gcol] : 0.f;
        // d of tokens past a ragged chunk's end meets zeros in M; it must be
        // finite, so the buffers start at zero
        for (int e = tid; e < 2 * CT * ISZ; e += 64 * NCONS)
            (&dbuf[0][0][0])[e] = 0.f;
        // operands of one token; the next token's are fetched from LDS while
        // the current one is computed
        struct Ops {
            float4 k[KPL / 4];
            float4 g; // SC_SCALED or SC_PLAIN
            float v;
        };
        auto fetch = [&](Ops& r, int buf, int sb, int tt, auto checked) {
            const float* yt = ys[buf][tt];
#pragma unroll
            for (int m = 0; m < KPL / 4; ++m)
                r.k[m] = *reinterpret_cast<const float4*>(yt + DK + 4 * jl + 4 * LPC * m);
            r.g = *reinterpret_cast<const float4*>(
                &sc[sb][tt][decltype(checked)::value ? SC_PLAIN : SC_SCALED]);
            r.v = yt[2 * DK + col];
        };
        // The state is held as cs * s: the decays of a chunk's tokens gather in
        // the lane-uniform scale cs, so a token's update is one fma per
        // element.  The scale is folded back into s at the start of every
        // chunk, and at once should it fall below kFoldBelow.
        float cs = 1.f;
        auto fold = [&](float c) {
#pragma unroll
            for (int m = 0; m < KPL; ++m)
                s[m] *= c;
        };
        // `checked`: whether the scale may have to be folded within the chunk.
        // The producers rule that out for most chunks; the scale after each of
        // their tokens is then the running product of the chunk's decays,
        // which they also fold into the token's coefficients.
        auto step = [&](const Ops& r, int buf, int tt, auto checked) {
            constexpr bool kChecked = decltype(checked)::value;
            const float b = r.g.y;
            float ca, cu, rkc; // a S_old = ca s; ca rk; rk / ca
            if constexpr (kChecked) {
                ca = cs * r.g.x;
                if ((__builtin_amdgcn_readfirstlane(__float_as_uint(ca)) & 0x7FFFFFFFu) <
                    kFoldBelow) {
                    fold(ca);
                    ca = 1.f;
                }
                cu = ca * r.g.z;
                rkc = r.g.z * __builtin_amdgcn_rcpf(ca);
            } else {
                ca = r.g.w;
                cu = r.g.x;
                rkc = r.g.z;
            }
            float u0 = 0.f, u1 = 0.f;
#pragma unroll
            for (int m = 0; m < KPL / 4; ++m) {
                u0 = fmaf(s[4 * m + 0], r.k[m].x, u0);
                u1 = fmaf(s[4 * m + 1], r.k[m].y, u1);
                u0 = fmaf(s[4 * m + 2], r.k[m].z, u0);
                u1 = fmaf(s[4 * m + 3], r.k[m].w, u1);
            }
            const float u = group_sum<LPC>(u0 + u1); // s k (raw k)
            const float d = b * (r.v - cu * u);      // b (v - a S_old k^)
            // S <- a S_old + d k^ k^T = ca (s + (d rk / ca) k)
            const float dk = d * rkc;
#pragma unroll
            for (int m = 0; m < KPL / 4; ++m) {
                s[4 * m + 0] = fmaf(dk, r.k[m].x, s[4 * m + 0]);
                s[4 * m + 1] = fmaf(dk, r.k[m].y, s[4 * m + 1]);
                s[4 * m + 2] = fmaf(dk, r.k[m].z, s[4 * m + 2]);
                s[4 * m + 3] = fmaf(dk, r.k[m].w, s[4 * m + 3]);
            }
            cs = ca;
            // the LPC lanes of the column hold the same bits (each step of
            // group_sum adds the same two values in every lane), so all of
            // them store it: no exec-mask switch per token
            dbuf[buf][tt][col] = d;
        };
        // checkpoint emission: the state after token ck_tok (if any) is also
        // stored into the checkpoint page
        // (buffer stores: one VGPR offset per lane and per-store constants, so
        // the rarely used path holds no addresses across the token loop)
        int ck_tok = -1;
        float* ck_tile = tile;
        if (p.ckpt_slot) {
            const int cs = p.ckpt_slot[n], cl = p.ckpt_len[n];
            if (cs >= 0 && cs < p.num_slots && cl >= 1 && cl <= L) {
                ck_tok = cl - 1;
                ck_tile = reinterpret_cast<float*>(p.layer + int64_t(cs) * p.page_stride + p.ssm_off) +
                          int64_t(h) * DK * DV;
            }
        }
        // the chunk holding the checkpoint token (-1: none; -1 / CT would be 0)
        const int ck_chunk = ck_tok >= 0 ? ck_tok / CT : -1;
        const __amdgpu_buffer_rsrc_t ck_rs = __builtin_amdgcn_make_buffer_rsrc(
            ck_tile, short(0), ck_tok >= 0 ? DK * DV * 4 : 0, 0x00020000);
        const int voff = (4 * jl * DV + gcol) * 4;
        auto store_ck = [&]() {
#pragma unroll
            for (int m = 0; m < KPL / 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __float_as_uint(s[4 * m + e] * cs), ck_rs,
                        voff + (4 * LPC * m + e) * DV * 4, 0, 0);
        };
        __syncthreads(); // B: chunk 0 prepared, d buffers cleared
        for (int c = 0; c < nchunks; ++c) {
            const int buf = c & 1, sb = c % 3;
            const int nt = chunk_len(c);
            fold(cs);
            cs = 1.f;
            // the chunk's starting state, for the producers' output products
#pragma unroll
            for (int m = 0; m < KPL / 4; ++m)
                *reinterpret_cast<float4*>(&s0[col][4 * jl + 4 * LPC * m]) =
                    make_float4(s[4 * m], s[4 * m + 1], s[4 * m + 2], s[4 * m + 3]);
            __syncthreads(); // X: starting state written
            // the producers' verdict: no token of the chunk needs a fold
            const bool quiet = __builtin_amdgcn_readfirstlane(nofold[sb]) != 0u;
            Ops A, B;
            auto per_token = [&](auto checked) {
                for (int tt = 0; tt < nt; ++tt) {
                    fetch(A, buf, sb, tt, checked);
                    step(A, buf, tt, checked);
                    if (c * CT + tt == ck_tok)
                        store_ck();
                }
            };
            if (nt == CT && ck_chunk != c && quiet) {
                // full chunk: a fully unrolled loop without branches (every LDS
                // address is a base plus an immediate), in which the operands of
                // token t+1 are requested before token t is computed; the
                // scheduling barriers keep the compiler from sinking those reads
                // next to their use, so each token waits only for reads issued
                // a whole token earlier (the last fetch of the chunk re-reads
                // token CT-1 and is unused)
                constexpr std::false_type scaled{};
                fetch(A, buf, sb, 0, scaled);
#pragma unroll
                for (int tt = 0; tt < CT; tt += 2) {
                    fetch(B, buf, sb, tt + 1, scaled);
                    __builtin_amdgcn_sched_barrier(0);
                    step(A, buf, tt, scaled);
                    fetch(A, buf, sb, min(tt + 2, CT - 1), scaled);
                    __builtin_amdgcn_sched_barrier(0);
                    step(B, buf, tt + 1, scaled);
                }
            } else if (quiet) { // a ragged last chunk, or the chunk holding the checkpoint token
                per_token(std::false_type{});
            } else {
                per_token(std::true_type{});
            }
            __syncthreads(); // P: chunk done
        }
#pragma unroll
        for (int m = 0; m < KPL / 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                tile[(4 * jl + 4 * LPC * m + e) * DV + gcol] = s[4 * m + e] * cs;
        return;
    }

    // ========================= producer waves ===============================
    const int pw = wave - Sh::NCONS;
    const uint16_t* win = reinterpret_cast<const uint16_t*>(page + p.conv_off);

    // conv taps and bias of the lane's channel pairs: q and k pair `lane`
    // (lanes past DK/2 idle), v pair of each of the lane's v jobs
    float wq[2][W], wk[2][W], wv[NVJ][2][W];
    float bq[2], bk[2], bv[NVJ][2];
    auto load_taps = [&](int ch, float (&w2)[2][W], float (&b2)[2]) {
        const int c = chan(ch);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int w = 0; w < W; ++w)
                w2[i][w] = bf16_to_f32(p.conv_w[int64_t(c + i) * W + w]);
            b2[i] = p.conv_b ? bf16_to_f32(p.conv_b[c + i]) : 0.f;
        }
    };
    const int qkp = min(lane, QKP - 1); // q/k pair of the lane (clamped; idle lanes recompute)
    load_taps(2 * qkp, wq, bq);
    load_taps(DK + 2 * qkp, wk, bk);
    // v job jj of the lane: token t0 + vi[jj] of the wave's TPW, pair vpj[jj]
    int vi[NVJ], vpj[NVJ];
#pragma unroll
    for (int jj = 0; jj < NVJ; ++jj) {
        const int j = lane + 64 * jj;
        vi[jj] = j / NVP;
        vpj[jj] = j % NVP;
        load_taps(2 * DK + 2 * vpj[jj], wv[jj], bv[jj]);
    }

    // Raw inputs of chunk k for this wave's TPW tokens, loaded into registers
    // a chunk ahead: for q and k the lane's channel pair over the W-1 rows
    // before the wave's first token and its TPW rows; for v the W rows of each
    // job; the gates of token k CT + lane % CT.  All are buffer loads with the
    // row in the lane's offset: the range check returns zero for rows past
    // the sequence's end (their results are never stored) and for the rows
    // before its start when the sequence is cold, whose window resource is
    // empty, so no load waits on a branch and a cold page is never read.
    constexpr int HR = W - 1, NR = HR + TPW;
    constexpr uint32_t kOutOfRange = 0xFFFFFFF0u; // past any num_records below
    const int t0 = pw * TPW;
    uint32_t xq[NR], xk[NR], xv[NVJ][W];
    float2 pg;
    // byte offsets inside a row of x of the lane's q pair, k pair, and (from
    // the wave's first row) of each v job's first row
    const int rowb = p.C * 2;
    const int oq = chan(2 * qkp) * 2, ok = chan(DK + 2 * qkp) * 2;
    int ov[NVJ];
#pragma unroll
    for (int jj = 0; jj < NVJ; ++jj)
        ov[jj] = min(vi[jj], TPW - 1) * rowb + chan(2 * DK + 2 * vpj[jj]) * 2;
    auto ld = [](__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0);
    };
    auto issue = [&](int k) {
        if (k >= nchunks)
            return;
        const int rbase = k * CT + t0 - HR; // the wave's first row
        // the first of its rows inside the sequence; L (an empty range) when
        // the wave's tokens all lie past the end of a short last chunk
        const int xb = min(max(rbase, 0), L);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(p.x) + int64_t(tb + xb) * p.C, short(0),
            range_bytes(int64_t(L - xb) * rowb), kBufferWord3);
        if (rbase >= 0) {
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                xq[i] = ld(rs, oq + i * rowb);
                xk[i] = ld(rs, ok + i * rowb);
            }
#pragma unroll
            for (int jj = 0; jj < NVJ; ++jj)
#pragma unroll
                for (int w = 0; w < W; ++w)
                    xv[jj][w] = ld(rs, ov[jj] + w * rowb);
        } else {
            // the first chunk of wave 0: rows -HR .. -1 come from the window
            const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(win), short(0), warm ? HR * rowb : 0, kBufferWord3);
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const int r = i - HR; // rbase == -HR here
                xq[i] = r < 0 ? ld(rw, (HR + r) * rowb + oq) : ld(rs, r * rowb + oq);
                xk[i] = r < 0 ? ld(rw, (HR + r) * rowb + ok) : ld(rs, r * rowb + ok);
            }
#pragma unroll
            for (int jj = 0; jj < NVJ; ++jj) {
                const int cv = chan(2 * DK + 2 * vpj[jj]) * 2;
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    const int r = min(vi[jj], TPW - 1) + w - HR;
                    xv[jj][w] = ld(rw, r < 0 ? uint32_t((HR + r) * rowb + cv) : kOutOfRange) |
                                ld(rs, r >= 0 ? uint32_t(r * rowb + cv) : kOutOfRange);
                }
            }
        }
        // gates of token k CT + lane % CT (zero past the sequence's end)
        const int ht = p.Hv * 4;
        const int64_t g0 = int64_t(tb + k * CT) * p.Hv + h;
        const int grec = range_bytes(int64_t(L - k * CT) * ht);
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(p.alpha) + g0, short(0), grec, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(p.beta) + g0, short(0), grec, kBufferWord3);
        pg = make_float2(__uint_as_float(ld(ra, (lane % CT) * ht)),
                         __uint_as_float(ld(rb, (lane % CT) * ht)));
    };

    // conv + SiLU, norm factors and coefficients of chunk k into ys[k & 1],
    // sc[k % 3], alf[k % 3] and nofold[k % 3], for the wave's tokens
    // [t0, t0 + TPW).  The 2 TPW wave sums (|q|^2, |k|^2 of each token) are
    // reduced together, and lane i finishes the coefficients of the wave's
    // i-th token.
    auto prepare = [&](int k) {
        static_assert(TPW == 4, "the sums of 4 tokens are reduced together");
        if (k >= nchunks)
            return;
        const int buf = k & 1, sb = k % 3;
        const int nt = chunk_len(k);
        // v: one (token, pair) job per lane
#pragma unroll
        for (int jj = 0; jj < NVJ; ++jj) {
            const int tt = t0 + vi[jj];
            if (vi[jj] < TPW && tt < nt) {
                float a0 = bv[jj][0], a1 = bv[jj][1];
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    a0 = fmaf(wv[jj][0][w], lo_bf16(xv[jj][w]), a0);
                    a1 = fmaf(wv[jj][1][w], hi_bf16(xv[jj][w]), a1);
                }
                *reinterpret_cast<float2*>(&ys[buf][tt][2 * DK + 2 * vpj[jj]]) =
                    make_float2(silu(a0), silu(a1));
            }
        }
        // q, k: the lane walks the wave's tokens over its register rows
        auto conv1 = [&](const float (&wt)[W], float b, const uint32_t (&xr)[NR], int i, bool hi) {
            float acc = b;
#pragma unroll
            for (int w = 0; w < W; ++w)
                acc = fmaf(wt[w], hi ? hi_bf16(xr[i + w]) : lo_bf16(xr[i + w]), acc);
            return silu(acc);
        };
        float sq[TPW], sk[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            sq[i] = sk[i] = 0.f;
            const int tt = t0 + i;
            if (tt >= nt)
                break;
            const float q0 = conv1(wq[0], bq[0], xq, i, false);
            const float q1 = conv1(wq[1], bq[1], xq, i, true);
            const float k0 = conv1(wk[0], bk[0], xk, i, false);
            const float k1 = conv1(wk[1], bk[1], xk, i, true);
            if (lane < QKP) {
                *reinterpret_cast<float2*>(&ys[buf][tt][2 * lane]) = make_float2(q0, q1);
                *reinterpret_cast<float2*>(&ys[buf][tt][DK + 2 * lane]) = make_float2(k0, k1);
                sq[i] = fmaf(q0, q0, q1 * q1);
                sk[i] = fmaf(k0, k0, k1 * k1);
            }
        }
        // wave sums: halves (tokens 0|1 and 2|3 share a register), then rows
        // (row j then holds token (0, 2, 1, 3)[j]), then within the rows
        auto fold_halves = [](float a, float b) { // lanes 0-31: a, lanes 32-63: b
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b),
                                                           false, false);
            return __uint_as_float(r[0]) + __uint_as_float(r[1]);
        };
        auto fold_rows = [](float x, float y) { // rows: x0+x1, y0+y1, x2+x3, y2+y3
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y),
                                                           false, false);
            return __uint_as_float(r[0]) + __uint_as_float(r[1]);
        };
        auto token_sums = [&](const float (&v)[TPW]) {
            return group_sum<16>(fold_rows(fold_halves(v[0], v[1]), fold_halves(v[2], v[3])));
        };
        const float tsq = token_sums(sq), tsk = token_sums(sk);
        const int src = 16 * (((lane & 1) << 1) | ((lane >> 1) & 1)); // row of token lane & 3
        const float my_sq = __shfl(tsq, src, 64), my_sk = __shfl(tsk, src, 64);
        // running products of the chunk's decays: an inclusive scan over each
        // 16-lane row (lane i of a row: token i; lanes past the chunk's end
        // take 1).  Whether the state's scale can stay unfolded through the
        // chunk: every decay in [0, 1] and their product at least 2^-40, so
        // that no running product falls below it (NaN fails the test).
        const int ti = lane % CT;
        const float av = ti < nt ? pg.x : 1.f;
        float cp = av;
        cp *= row_shr_or_one<1>(cp);
        cp *= row_shr_or_one<2>(cp);
        cp *= row_shr_or_one<4>(cp);
        cp *= row_shr_or_one<8>(cp);
        if (pw == 0) {
            const bool ok = av >= 0.f && av <= 1.f;
            const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cp), 15));
            const bool quiet = __ballot(!ok) == 0 && total >= __uint_as_float(kFoldBelow);
            if (lane == 0)
                nofold[sb] = quiet ? 1u : 0u;
        }
        const int tt = t0 + (lane & 3);
        const float ct = __shfl(cp, tt, 64); // running product through token tt
        const float ga = __shfl(pg.x, tt, 64), gb = __shfl(pg.y, tt, 64);
        if (lane < TPW && tt < nt) {
            const float rq = p.scale * __builtin_amdgcn_rsqf(my_sq + p.eps);
            const float rk = __builtin_amdgcn_rsqf(my_sk + p.eps);
            float* o = sc[sb][tt];
            *reinterpret_cast<float4*>(o + SC_SCALED) =
                make_float4(ct * rk, gb, rk * __builtin_amdgcn_rcpf(ct), ct);
            *reinterpret_cast<float4*>(o + SC_PLAIN) = make_float4(ga, gb, rk, rq);
            alf[k % 3][tt] = ct * rq;
        }
    };

    // Output products of chunk k, while the consumers run it: producer wave
    // j < NCB forms S_0 Q^T for the slice's j-th 16-column block (to LDS for
    // the epilogue), the others form the GP parts of Q K^T over
    // slices of the key range (to LDS; a single part goes to wave 0 when no
    // wave is free).  MFMA lane l supplies A[l % 16][l / 16] and
    // B[l / 16][l % 16] and receives D[4 (l / 16) + r][l % 16] in r; the K
    // index of a step is permuted so that lane group l / 16 reads one run of
    // consecutive keys.
    constexpr int GP = Sh::GP;
    const int m16 = lane % 16, q4 = lane / 16;
    auto product = [&](const float* arow, const float* brow, int ngroups) {
        // four independent accumulation chains keep the matrix pipe busy
        v4f ac[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f},
                     {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int i = 0; i < ngroups; ++i) {
            const float4 a = *reinterpret_cast<const float4*>(arow + 4 * i);
            const float4 b = *reinterpret_cast<const float4*>(brow + 4 * i);
            ac[0] = mfma16(a.x, b.x, ac[0]);
            ac[1] = mfma16(a.y, b.y, ac[1]);
            ac[2] = mfma16(a.z, b.z, ac[2]);
            ac[3] = mfma16(a.w, b.w, ac[3]);
        }
        return (ac[0] + ac[1]) + (ac[2] + ac[3]);
    };
    auto products = [&](int k) {
        const int buf = k & 1;
        if (pw < NCB) // S_0[col][key] x Q[t][key], for the block's epilogue
            pq[buf][pw][lane] = product(&s0[16 * pw + m16][q4 * KQ], &ys[buf][m16][q4 * KQ], KQ / 4);
        const int gpart = Sh::GFREE > 0 ? pw - NCB : (pw == 0 ? 0 : -1);
        if (gpart >= 0 && gpart < GP) { // Q[t][key] x K[s][key] over a slice of the keys
            constexpr int NG = KQ / 4 / GP;
            const int k0 = q4 * KQ + 4 * NG * gpart;
            const v4f g4 = product(&ys[buf][m16][k0], &ys[buf][m16][DK + k0], NG);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                gq[buf][gpart][4 * q4 + r][m16] = g4[r];
        }
    };

    // Outputs of chunk k (after it): o = alf_t (S_0 Q^T) + D M^T for the
    // wave's column block, written as bf16 (a lane: 4 columns of token l % 16).
    // M[t][s] = (A_t / A_s) rq_t rk_s (q_t . k_s) for s <= t, else 0; chunks
    // without a fold take A_t rq_t (alf) and rk_s / A_s (SC_SCALED), the
    // others multiply the decays between s and t one by one.  A lane builds
    // the B operand it supplies, M[t = l % 16][s = 4 (l / 16) + j], j = 0..3.
    auto epilogue = [&](int k) {
        // block eb of the chunk; on the waves without a block when there are
        // enough of them (they carry the lighter products), else the block's own
        const int eb = Sh::GFREE >= NCB ? pw - (Sh::NPROD - NCB) : pw;
        if (eb < 0 || eb >= NCB)
            return;
        const int buf = k & 1, sb = k % 3;
        const int t_ = m16;
        float4 gsum = *reinterpret_cast<const float4*>(&gq[buf][0][t_][4 * q4]);
#pragma unroll
        for (int j = 1; j < GP; ++j) {
            const float4 e = *reinterpret_cast<const float4*>(&gq[buf][j][t_][4 * q4]);
            gsum.x += e.x;
            gsum.y += e.y;
            gsum.z += e.z;
            gsum.w += e.w;
        }
        const float gs[4] = {gsum.x, gsum.y, gsum.z, gsum.w};
        const float at = alf[k % 3][t_];
        const bool quiet = __builtin_amdgcn_readfirstlane(nofold[sb]) != 0u;
        float f[4];
        if (quiet) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                f[j] = at * sc[sb][4 * q4 + j][SC_SCALED + 2];
        } else {
            // the decays between s and t, one token at a time (rare)
            f[0] = f[1] = f[2] = f[3] = 1.f;
#pragma unroll 1
            for (int u = 1; u < CT; ++u) {
                const float au = sc[sb][u][SC_PLAIN];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    f[j] *= (u > 4 * q4 + j && u <= t_) ? au : 1.f;
            }
            const float rq = sc[sb][t_][SC_PLAIN + 3];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                f[j] *= rq * sc[sb][4 * q4 + j][SC_PLAIN + 2];
        }
        v4f acc = pq[buf][eb][lane] * at;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s_ = 4 * q4 + j;
            acc = mfma16(dbuf[buf][s_][16 * eb + m16], s_ <= t_ ? gs[j] * f[j] : 0.f, acc);
        }
        if (m16 < chunk_len(k)) {
            *reinterpret_cast<uint2*>(out_base + int64_t(k * CT + m16) * out_tok + 16 * eb + 4 * q4) =
                pack_bf16x4(acc[0], acc[1], acc[2], acc[3]);
        }
    };

    issue(0);
    prepare(0);
    issue(1);
    __syncthreads(); // B
    for (int c = 0; c < nchunks; ++c) {
        __syncthreads(); // X: the consumers have written the chunk's starting state
        if (c >= 1)
            epilogue(c - 1);
        products(c);
        prepare(c + 1);
        issue(c + 2);
        __syncthreads(); // P
    }
    epilogue(nchunks - 1);
}

// Final window of each sequence: the last W-1 entries of (old window, x).
struct WindowParams {
    uint8_t* layer;
    int64_t page_stride;
    int64_t conv_off;
    int32_t num_slots;
    int32_t C;
    int32_t W;
    int64_t total_tokens;
    const int32_t* cu;
    const uint16_t* x;
    const int32_t* state_indices;
    const uint8_t* hs;
    const int32_t* ckpt_slot; // as in PrefillParams
    const int32_t* ckpt_len;
};

constexpr int kWinThreads = 256;

__global__ __launch_bounds__(kWinThreads) void prefill_window_kernel(WindowParams p)
{
    const int cblocks = (p.C + kWinThreads - 1) / kWinThreads;
    const int n = blockIdx.x / cblocks;
    const int c = (blockIdx.x - n * cblocks) * kWinThreads + threadIdx.x;
    if (c >= p.C)
        return;
    const int64_t tb64 = p.cu[n], te64 = p.cu[n + 1];
    if (tb64 < 0 || te64 <= tb64 || te64 > p.total_tokens) // as in prefill_kernel
        return;
    const int tb = int(tb64);
    const int L = int(te64 - tb64);
    const int slot = p.state_indices[n];
    if (slot < 0 || slot >= p.num_slots)
        return;
    const bool warm = p.hs[n] != 0;
    uint16_t* win = reinterpret_cast<uint16_t*>(p.layer + int64_t(slot) * p.page_stride +
                                                p.conv_off);
    // the window after the first `len` tokens: the last W-1 of (old window, x)
    auto window_at = [&](int len, uint16_t (&nw)[7]) {
#pragma unroll
        for (int w = 0; w < 7; ++w) {
            if (w < p.W - 1) {
                const int pos = len - (p.W - 1) + w; // position relative to the first token
                nw[w] = pos >= 0 ? p.x[int64_t(tb + pos) * p.C + c]
                                 : (warm ? win[int64_t(p.W - 1 + pos) * p.C + c] : uint16_t(0));
            }
        }
    };
    uint16_t nw[7], cw[7];
    window_at(L, nw);
    uint16_t* ck_win = nullptr;
    if (p.ckpt_slot) {
        const int cs = p.ckpt_slot[n], cl = p.ckpt_len[n];
        if (cs >= 0 && cs < p.num_slots && cl >= 1 && cl <= L) {
            window_at(cl, cw); // reads the old window before it is rewritten below
            ck_win = reinterpret_cast<uint16_t*>(p.layer + int64_t(cs) * p.page_stride + p.conv_off);
        }
    }
#pragma unroll
    for (int w = 0; w < 7; ++w) {
        if (w < p.W - 1) {
            win[int64_t(w) * p.C + c] = nw[w];
            if (ck_win)
                ck_win[int64_t(w) * p.C + c] = cw[w];
        }
    }
}

template <int DK, int DV, int W>
int launch_prefill_t(const gdn_pool* pool, int32_t layer, int32_t num_seqs, int64_t total_tokens,
                     const int32_t* cu, const gdn_step_args* a, const int32_t* ckpt_slot,
                     const int32_t* ckpt_len, hipStream_t stream)
{
    using Sh = PrefillShape<DK, DV>;
    const gdn_pool_desc& d = pool->desc;
    PrefillParams p;
    p.layer = static_cast<uint8_t*>(pool->bases[layer]);
    p.page_stride = d.page_stride_bytes;
    p.ssm_off = d.ssm_offset_bytes;
    p.conv_off = d.conv_offset_bytes;
    p.num_slots = int32_t(d.num_slots);
    p.num_seqs = num_seqs;
    p.total_tokens = total_tokens;
    p.C = d.conv_channels;
    p.Hk = d.num_k_heads;
    p.Hv = d.num_v_heads;
    p.cu = cu;
    p.x = a->x;
    p.conv_w = a->conv_w;
    p.conv_b = a->conv_b;
    p.alpha = a->alpha;
    p.beta = a->beta;
    p.state_indices = a->state_indices;
    p.hs = a->has_initial_state;
    p.out = a->out;
    p.ckpt_slot = ckpt_slot;
    p.ckpt_len = ckpt_len;
    p.scale = a->scale;
    p.eps = a->l2_eps;
    const int64_t blocks = int64_t(num_seqs) * d.num_v_heads * Sh::NSL;
    if (blocks > INT32_MAX)
        return fail(GDN_ERANGE, "prefill grid too large");
    hipLaunchKernelGGL((prefill_kernel<DK, DV, W>), dim3(uint32_t(blocks)), dim3(Sh::NT), 0,
                       stream, p);
    int rc = check_launch("prefill");
    if (rc != GDN_OK)
        return rc;
    WindowParams w;
    w.layer = p.layer;
    w.page_stride = p.page_stride;
    w.conv_off = p.conv_off;
    w.num_slots = p.num_slots;
    w.C = p.C;
    w.W = W;
    w.total_tokens = total_tokens;
    w.cu = cu;
    w.x = a->x;
    w.state_indices = a->state_indices;
    w.hs = a->has_initial_state;
    w.ckpt_slot = ckpt_slot;
    w.ckpt_len = ckpt_len;
    const int64_t wblocks =
        int64_t(num_seqs) * ((d.conv_channels + kWinThreads - 1) / kWinThreads);
    if (wblocks > INT32_MAX)
        return fail(GDN_ERANGE, "prefill window grid too large");
    hipLaunchKernelGGL(prefill_window_kernel, dim3(uint32_t(wblocks)), dim3(kWinThreads), 0,
                       stream, w);
    return check_launch("prefill window");
}

template <int DK>
int dispatch_w(const gdn_pool* pool, int32_t layer, int32_t num_seqs, int64_t T, const int32_t* cu,
               const gdn_step_args* a, const int32_t* cs, const int32_t* cl, hipStream_t stream)
{
    switch (pool->desc.conv_width) {
    case 2: return launch_prefill_t<DK, DK, 2>(pool, layer, num_seqs, T, cu, a, cs, cl, stream);
    case 3: return launch_prefill_t<DK, DK, 3>(pool, layer, num_seqs, T, cu, a, cs, cl, stream);
    case 4: return launch_prefill_t<DK, DK, 4>(pool, layer, num_seqs, T, cu, a, cs, cl, stream);
    default: return fail(GDN_EUNSUPPORTED, "prefill: conv width %d", pool->desc.conv_width);
    }
}

} // namespace

bool prefill_supported(int dk, int dv, int W)
{
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128) && W >= 2 && W <= 4;
}

int launch_prefill(const gdn_pool* pool, int32_t layer, int32_t num_seqs, int64_t total_tokens,
                   const int32_t* cu, const gdn_step_args* a, const int32_t* ckpt_slot,
                   const int32_t* ckpt_len, hipStream_t stream)
{
    const int32_t *cs = ckpt_slot, *cl = ckpt_len;
    switch (pool->desc.head_k_dim) {
    case 16: return dispatch_w<16>(pool, layer, num_seqs, total_tokens, cu, a, cs, cl, stream);
    case 32: return dispatch_w<32>(pool, layer, num_seqs, total_tokens, cu, a, cs, cl, stream);
    case 64: return dispatch_w<64>(pool, layer, num_seqs, total_tokens, cu, a, cs, cl, stream);
    case 128: return dispatch_w<128>(pool, layer, num_seqs, total_tokens, cu, a, cs, cl, stream);
    default: return fail(GDN_EUNSUPPORTED, "prefill: head dim %d", pool->desc.head_k_dim);
    }
}

} // namespace gdn
