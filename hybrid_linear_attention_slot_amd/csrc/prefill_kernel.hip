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
// own once k, q, v, a, b of the token are known, so a workgroup takes one
// (sequence, v-head, slice of ISZ value columns) and keeps that slice of the
// state in registers for the whole sequence.  Its waves have two roles:
//   - consumer waves run the serial recurrence.  A lane holds KPL keys of one
//     value column (keys 4 jl + 4 LPC m + e, so that the LPC lanes of a
//     column read one contiguous run of k or q from LDS); S k and S q are
//     lane-partial dot products finished with DPP sums over the LPC lanes,
//     and  o = a (S_old q^) + d (k^.q^),  d = b (v - a S_old k^),  so one pass
//     over the state gives both the update and the output;
//   - producer waves prepare the next chunk of CT tokens while the consumers
//     work on the current one: they stage the raw inputs of the workgroup's
//     channels (q and k of its k-head, v of its slice) in an LDS ring with
//     coalesced 16-byte loads issued a chunk ahead, run the conv + SiLU, form
//     the per-token norm factors, and write the previous chunk's outputs to
//     HBM as bf16.
// Consumers and producers meet at one barrier per chunk; the per-token work
// on the critical path is the consumers' recurrence alone.  The L2 norm
// factors are applied to the reduced sums, so k and q stay raw in LDS.
// A run split at a multiple of the chunk length (16 tokens) and resumed from
// the written-back state gives the same bits as the straight run: the state
// is folded to its plain form at every chunk start, which is also the form
// written back.
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
    static constexpr int KPL = DK >= 64 ? 16 : (DK >= 32 ? 8 : 4); // keys per consumer lane
    static constexpr int LPC = DK / KPL;                            // lanes sharing one column
    static constexpr int CPW = 64 / LPC;                            // columns per consumer wave
    static constexpr int NCONS = (DV / CPW) < 4 ? (DV / CPW) : 4;   // consumer waves
    static constexpr int NPROD = 4;                                 // producer waves
    static constexpr int ISZ = NCONS * CPW;                         // value columns per workgroup
    static constexpr int NSL = DV / ISZ;                            // workgroups per head
    static constexpr int NT = 64 * (NCONS + NPROD);
    static constexpr int CT = 16;                                   // tokens per chunk
    static constexpr int RING = 3 * CT;                             // staged input rows
    static constexpr int NCH = 2 * DK + ISZ;                        // channels: q | k | v slice
    static constexpr int NPIECE = NCH / 8;                          // 16-byte pieces per row
    static constexpr int QKP = DK / 2;                              // q (and k) channel pairs
    static constexpr int NQK = (QKP + 63) / 64;                     // q/k pair slots per lane
    static constexpr int NVP = ISZ / 2;                             // v channel pairs
    static constexpr int PLANES = 64 * NPROD;
    static constexpr int LOADS = (CT * NPIECE + PLANES - 1) / PLANES; // pieces per producer lane
    static constexpr int OPR = ISZ / 8;                             // 8-column output pieces per row
    static constexpr int TPW = CT / NPROD;                          // tokens per producer wave
    static_assert(DK == DV, "square heads only");
    static_assert(KPL % 4 == 0 && DK % KPL == 0 && LPC >= 1 && LPC <= 64, "key split");
    static_assert(NCONS >= 1 && DV % ISZ == 0 && ISZ % 8 == 0, "column split");
    static_assert(CT == 16, "a chunk's decays are reduced over one 16-lane DPP row");
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
//   SC_SCALED  c rk, b, rk / c, c rq   (c: running product of the chunk's
//                                      decays through the token)
//   SC_KQ      k^.q^, c
//   SC_PLAIN   a, b, rk, rq            (chunks that may need a fold)
constexpr int SC_SCALED = 0, SC_KQ = 4, SC_PLAIN = 8;

// v * (lane v of the row n lanes lower), or v * 1 for the first n lanes of
// each 16-lane row (DPP row_shr; an invalid source keeps the `old` operand)
template <int N>
__device__ __forceinline__ float row_shr_or_one(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(v),
                                                      0x110 + N, 0xF, 0xF, false));
}

template <int RING>
__device__ __forceinline__ int ring_pos(int t) // t >= -RING
{
    return (t + RING) % RING;
}

template <int DK, int DV, int W>
// four waves per SIMD: two 512-thread workgroups per CU (their LDS fits too)
__global__ __launch_bounds__((PrefillShape<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(4)))
void prefill_kernel(PrefillParams p)
{
    using Sh = PrefillShape<DK, DV>;
    constexpr int KPL = Sh::KPL, LPC = Sh::LPC, CPW = Sh::CPW, NCONS = Sh::NCONS;
    constexpr int ISZ = Sh::ISZ, NCH = Sh::NCH, CT = Sh::CT, RING = Sh::RING;
    constexpr int NT = Sh::NT, PLANES = Sh::PLANES, NPIECE = Sh::NPIECE, QKP = Sh::QKP;

    __shared__ __align__(16) uint16_t raw[RING][NCH];  // staged raw inputs, row = token % RING
    __shared__ __align__(16) float ys[2][CT][NCH];     // conv outputs (raw q | raw k | v)
    __shared__ __align__(16) float sc[2][CT][12];      // per token coefficients (SC_*)
    __shared__ uint32_t nofold[2];                     // the chunk's decays need no fold
    __shared__ __align__(8) float gab[RING][2];        // staged alpha, beta
    __shared__ __align__(16) float ob[2][CT][ISZ];     // outputs of a chunk (fp32)

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
        for (int e = tid; e < L * (ISZ / 4); e += NT) {
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
        // The recurrence is the critical path and each consumer shares its
        // SIMD with a producer wave, which has a chunk of slack: when both can
        // issue, the consumer goes first.
        __builtin_amdgcn_s_setprio(3);
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
        // operands of one token; the next token's are fetched from LDS while
        // the current one is computed
        struct Ops {
            float4 k[KPL / 4], q[KPL / 4];
            float4 g; // SC_SCALED or SC_PLAIN
            float2 h; // k^.q^, running scale
            float v;
        };
        auto fetch = [&](Ops& r, int buf, int tt, auto checked) {
            const float* yt = ys[buf][tt];
#pragma unroll
            for (int m = 0; m < KPL / 4; ++m) {
                r.k[m] = *reinterpret_cast<const float4*>(yt + DK + 4 * jl + 4 * LPC * m);
                r.q[m] = *reinterpret_cast<const float4*>(yt + 4 * jl + 4 * LPC * m);
            }
            r.g = *reinterpret_cast<const float4*>(
                &sc[buf][tt][decltype(checked)::value ? SC_PLAIN : SC_SCALED]);
            r.h = *reinterpret_cast<const float2*>(&sc[buf][tt][SC_KQ]);
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
            const float b = r.g.y, kq = r.h.x;
            float ca, cu, rkc, cq; // a S_old = ca s; ca rk; rk / ca; ca rq
            if constexpr (kChecked) {
                ca = cs * r.g.x;
                if ((__builtin_amdgcn_readfirstlane(__float_as_uint(ca)) & 0x7FFFFFFFu) <
                    kFoldBelow) {
                    fold(ca);
                    ca = 1.f;
                }
                cu = ca * r.g.z;
                rkc = r.g.z * __builtin_amdgcn_rcpf(ca);
                cq = ca * r.g.w;
            } else {
                ca = r.h.y;
                cu = r.g.x;
                rkc = r.g.z;
                cq = r.g.w;
            }
            float u0 = 0.f, u1 = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
            for (int m = 0; m < KPL / 4; ++m) {
                u0 = fmaf(s[4 * m + 0], r.k[m].x, u0);
                u1 = fmaf(s[4 * m + 1], r.k[m].y, u1);
                o0 = fmaf(s[4 * m + 0], r.q[m].x, o0);
                o1 = fmaf(s[4 * m + 1], r.q[m].y, o1);
                u0 = fmaf(s[4 * m + 2], r.k[m].z, u0);
                u1 = fmaf(s[4 * m + 3], r.k[m].w, u1);
                o0 = fmaf(s[4 * m + 2], r.q[m].z, o0);
                o1 = fmaf(s[4 * m + 3], r.q[m].w, o1);
            }
            const float u = group_sum<LPC>(u0 + u1); // s k (raw k)
            const float o = group_sum<LPC>(o0 + o1); // s q (raw q)
            const float d = b * (r.v - cu * u); // b (v - a S_old k^)
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
            // a S_old q^ + d (k^.q^); the LPC lanes of the column hold the same
            // bits (each step of group_sum adds the same two values in every
            // lane), so all of them store it: no exec-mask switch per token
            const float ov = fmaf(cq, o, kq * d);
            ob[buf][tt][col] = ov;
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
        __syncthreads(); // A: history and chunk 0 staged
        __syncthreads(); // B: chunk 0 prepared
        for (int c = 0; c < nchunks; ++c) {
            const int buf = c & 1;
            const int nt = chunk_len(c);
            fold(cs);
            cs = 1.f;
            // the producers' verdict: no token of the chunk needs a fold
            const bool quiet = __builtin_amdgcn_readfirstlane(nofold[buf]) != 0u;
            Ops A, B;
            auto per_token = [&](auto checked) {
                for (int tt = 0; tt < nt; ++tt) {
                    fetch(A, buf, tt, checked);
                    step(A, buf, tt, checked);
                    if (c * CT + tt == ck_tok)
                        store_ck();
                }
            };
            if (nt == CT && ck_tok / CT != c && quiet) {
                // full chunk: a fully unrolled loop without branches (every LDS
                // address is a base plus an immediate), in which the operands of
                // token t+1 are requested before token t is computed; the
                // scheduling barriers keep the compiler from sinking those reads
                // next to their use, so each token waits only for reads issued
                // a whole token earlier (the last fetch of the chunk re-reads
                // token CT-1 and is unused)
                constexpr std::false_type scaled{};
                fetch(A, buf, 0, scaled);
#pragma unroll
                for (int tt = 0; tt < CT; tt += 2) {
                    fetch(B, buf, tt + 1, scaled);
                    __builtin_amdgcn_sched_barrier(0);
                    step(A, buf, tt, scaled);
                    fetch(A, buf, min(tt + 2, CT - 1), scaled);
                    __builtin_amdgcn_sched_barrier(0);
                    step(B, buf, tt + 1, scaled);
                }
            } else if (quiet) { // a ragged last chunk, or the chunk holding the checkpoint token
                per_token(std::false_type{});
            } else {
                per_token(std::true_type{});
            }
            __syncthreads();
        }
#pragma unroll
        for (int m = 0; m < KPL / 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                tile[(4 * jl + 4 * LPC * m + e) * DV + gcol] = s[4 * m + e] * cs;
        return;
    }

    // ========================= producer waves ===============================
    const int pw = wave - NCONS;
    const int plane = pw * 64 + lane;
    const uint16_t* win = reinterpret_cast<const uint16_t*>(page + p.conv_off);

    // conv taps and bias of the lane's channel pairs: q and k pair `lane`
    // (lanes past DK/2 idle), v pair `lane % NVP` of the slice
    static_assert(Sh::NQK == 1 && 64 % Sh::NVP == 0, "one q/k pair per lane; v pairs tile a wave");
    float wq[2][W], wk[2][W], wv[2][W];
    float bq[2], bk[2], bv[2];
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
    const int vp = lane % Sh::NVP;      // v pair of the lane
    load_taps(2 * qkp, wq, bq);
    load_taps(DK + 2 * qkp, wk, bk);
    load_taps(2 * DK + 2 * vp, wv, bv);

    // chunk k's raw rows and gates: issue (into registers), then stage (to LDS).
    // Every lane issues the same number of 16-byte loads whatever the chunk's
    // length (pieces past the last token re-read the last token's row and land
    // in ring rows no conv reads), so the waits for them are exact.
    // (a native vector type: an array of HIP's uint4 is kept in scratch memory
    // here, which turns the prefetch into a load, a wait and a spill)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 pf[Sh::LOADS];
    float2 pg;
    auto issue = [&](int k) {
        if (k >= nchunks)
            return;
        const int last = chunk_len(k) - 1;
#pragma unroll
        for (int i = 0; i < Sh::LOADS; ++i) {
            const int e = min(plane + PLANES * i, CT * NPIECE - 1);
            const int tt = e / NPIECE, pc = e - tt * NPIECE;
            pf[i] = *reinterpret_cast<const u32x4*>(p.x + int64_t(tb + k * CT + min(tt, last)) * p.C +
                                                   chan(8 * pc));
        }
        const int64_t gi = int64_t(tb + k * CT + min(plane % CT, last)) * p.Hv + h;
        pg = make_float2(p.alpha[gi], p.beta[gi]);
    };
    auto stage = [&](int k) {
        if (k >= nchunks)
            return;
#pragma unroll
        for (int i = 0; i < Sh::LOADS; ++i) {
            const int e = plane + PLANES * i;
            if (e < CT * NPIECE) {
                const int tt = e / NPIECE, pc = e - tt * NPIECE;
                *reinterpret_cast<u32x4*>(&raw[ring_pos<RING>(k * CT + tt)][8 * pc]) = pf[i];
            }
        }
        if (plane < CT)
            *reinterpret_cast<float2*>(gab[ring_pos<RING>(k * CT + plane)]) = pg;
    };

    // conv + SiLU and the norm factors of chunk k into ys[k & 1], sc[k & 1].
    // Producer wave pw takes the TPW consecutive tokens starting at pw * TPW.
    // For q and k each lane walks them in order for its channel pair, keeping
    // the W-1 previous inputs in registers (primed from the ring), so every
    // staged input is unpacked once; the v channels of the slice are fewer
    // than the lanes, so there a lane takes one (token, pair) job and reads
    // its window from the ring.  The 3 TPW wave sums (|q|^2, |k|^2, q.k of
    // each token) are reduced together, and lane i finishes the coefficients
    // of the wave's i-th token.
    auto prepare = [&](int k) {
        constexpr int TPW = Sh::TPW;
        static_assert(TPW == 4, "the sums of 4 tokens are reduced together");
        const int buf = k & 1;
        const int t0 = pw * TPW;
        const int t1 = min(t0 + TPW, chunk_len(k));
        if (t0 >= t1)
            return;
        const int base = (k % 3) * CT; // ring row of the chunk's first token
        auto row = [&](int tt) {       // tt in [-(W-1), CT)
            const int r = base + tt;
            return reinterpret_cast<const uint32_t*>(raw[r < 0 ? r + RING : r]);
        };
        // v: job j = lane + 64 jj is token t0 + j / NVP, pair vp
#pragma unroll
        for (int jj = 0; jj < (TPW * Sh::NVP + 63) / 64; ++jj) {
            const int i = (lane + 64 * jj) / Sh::NVP;
            const int tt = t0 + i;
            if (i < TPW && tt < t1) {
                float a0 = bv[0], a1 = bv[1];
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    const uint32_t xv = row(tt - (W - 1) + w)[2 * QKP + vp];
                    a0 = fmaf(wv[0][w], lo_bf16(xv), a0);
                    a1 = fmaf(wv[1][w], hi_bf16(xv), a1);
                }
                *reinterpret_cast<float2*>(ys[buf][tt] + 2 * DK + 2 * vp) =
                    make_float2(silu(a0), silu(a1));
            }
        }
        // q, k
        float hq[2][W - 1], hk[2][W - 1];
#pragma unroll
        for (int w = 0; w < W - 1; ++w) {
            const uint32_t* r = row(t0 - (W - 1) + w);
            const uint32_t xq = r[qkp], xk = r[QKP + qkp];
            hq[0][w] = lo_bf16(xq);
            hq[1][w] = hi_bf16(xq);
            hk[0][w] = lo_bf16(xk);
            hk[1][w] = hi_bf16(xk);
        }
        // conv of one channel: taps over the W-1 held inputs and the current one,
        // then the held inputs shift by one
        auto conv1 = [&](const float (&wt)[W], float b, float (&hist)[W - 1], float x) {
            float acc = b;
#pragma unroll
            for (int w = 0; w < W - 1; ++w)
                acc = fmaf(wt[w], hist[w], acc);
            acc = fmaf(wt[W - 1], x, acc);
#pragma unroll
            for (int w = 0; w + 1 < W - 1; ++w)
                hist[w] = hist[w + 1];
            hist[W - 2] = x;
            return silu(acc);
        };
        float sq[TPW], sk[TPW], qk[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            sq[i] = sk[i] = qk[i] = 0.f;
            const int tt = t0 + i;
            if (tt >= t1)
                break;
            const uint32_t* r = row(tt);
            float* yt = ys[buf][tt];
            const uint32_t xq = r[qkp], xk = r[QKP + qkp];
            const float q0 = conv1(wq[0], bq[0], hq[0], lo_bf16(xq));
            const float q1 = conv1(wq[1], bq[1], hq[1], hi_bf16(xq));
            const float k0 = conv1(wk[0], bk[0], hk[0], lo_bf16(xk));
            const float k1 = conv1(wk[1], bk[1], hk[1], hi_bf16(xk));
            if (lane < QKP) {
                *reinterpret_cast<float2*>(yt + 2 * lane) = make_float2(q0, q1);
                *reinterpret_cast<float2*>(yt + DK + 2 * lane) = make_float2(k0, k1);
                sq[i] = fmaf(q0, q0, q1 * q1);
                sk[i] = fmaf(k0, k0, k1 * k1);
                qk[i] = fmaf(q0, k0, q1 * k1);
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
        const float tsq = token_sums(sq), tsk = token_sums(sk), tqk = token_sums(qk);
        const int src = 16 * (((lane & 1) << 1) | ((lane >> 1) & 1)); // row of token lane & 3
        const float my_sq = __shfl(tsq, src, 64), my_sk = __shfl(tsk, src, 64),
                    my_qk = __shfl(tqk, src, 64);
        // running products of the chunk's decays: an inclusive scan over lanes
        // 0..15 (one DPP row; lanes past the chunk's end take 1).  Whether the
        // state's scale can stay unfolded through the chunk: every decay in
        // [0, 1] and their product at least 2^-40, so that no running product
        // falls below it (NaN fails the test).
        const int ntk = chunk_len(k);
        const float av = lane < ntk ? gab[base + lane][0] : 1.f;
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
                nofold[buf] = quiet ? 1u : 0u;
        }
        const float ct = __shfl(cp, min(t0 + lane, 15), 64); // running product through token t0+lane
        const int tt = t0 + lane;
        if (lane < TPW && tt < t1) {
            const float rq = p.scale / sqrtf(my_sq + p.eps);
            const float rk = 1.0f / sqrtf(my_sk + p.eps);
            const float2 ab = *reinterpret_cast<const float2*>(gab[base + tt]);
            float* o = sc[buf][tt];
            *reinterpret_cast<float4*>(o + SC_SCALED) =
                make_float4(ct * rk, ab.y, rk * __builtin_amdgcn_rcpf(ct), ct * rq);
            *reinterpret_cast<float2*>(o + SC_KQ) = make_float2(my_qk * rq * rk, ct);
            *reinterpret_cast<float4*>(o + SC_PLAIN) = make_float4(ab.x, ab.y, rk, rq);
        }
    };

    // chunk k's outputs from ob[k & 1] to HBM as bf16
    auto flush = [&](int k) {
        const int buf = k & 1;
        const int nt = chunk_len(k);
        for (int e = plane; e < nt * Sh::OPR; e += PLANES) {
            const int tt = e / Sh::OPR, c8 = e - tt * Sh::OPR;
            const float4 lo = *reinterpret_cast<const float4*>(&ob[buf][tt][8 * c8]);
            const float4 hi = *reinterpret_cast<const float4*>(&ob[buf][tt][8 * c8 + 4]);
            const uint2 a = pack_bf16x4(lo.x, lo.y, lo.z, lo.w);
            const uint2 b = pack_bf16x4(hi.x, hi.y, hi.z, hi.w);
            *reinterpret_cast<uint4*>(out_base + int64_t(k * CT + tt) * out_tok + 8 * c8) =
                make_uint4(a.x, a.y, b.x, b.y);
        }
    };

    // prologue: the W-1 inputs before the first token (window or zeros), chunk 0
    for (int e = plane; e < (W - 1) * NCH; e += PLANES) {
        const int w = e / NCH, ch = e - w * NCH;
        raw[ring_pos<RING>(w - (W - 1))][ch] = warm ? win[int64_t(w) * p.C + chan(ch)] : uint16_t(0);
    }
    issue(0);
    stage(0);
    __syncthreads(); // A
    issue(1);
    prepare(0);
    stage(1);
    __syncthreads(); // B
    for (int c = 0; c < nchunks; ++c) {
        // the loads are consumed by stage() after prepare(); the output stores
        // go last, so that no wait for loads also waits for fresh stores
        issue(c + 2);
        if (c + 1 < nchunks)
            prepare(c + 1);
        stage(c + 2);
        if (c >= 1)
            flush(c - 1);
        __syncthreads();
    }
    flush(nchunks - 1);
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
