// Varlen recurrent prefill of a Gated DeltaNet layer over a page-strided
// slot pool (gfx950).
//
// Sequence n covers tokens [cu[n], cu[n+1]) and owns slot state_indices[n].
// Its window and state are gathered once (or taken as zero when
// has_initial_state is 0, "Linear-State Prefix Cache 内部机制" §4.1), the
// causal conv + SiLU, the q/k L2 norms and the gated delta rule run over the
// sequence with the state kept on chip ("Kapitsa 源码拆解 05": the work per
// token does not grow with the history), and the final window and state are
// scattered back into the same page ("非连续 KV Cache" §5-§6).
//
// The recurrence, per token t of a v-head (state S: key x value),
//     d_t = b_t (v_t - a_t S_{t-1} k^_t),   S_t = a_t S_{t-1} + k^_t d_t^T,
//     o_t = S_t^T q^_t
// (decay first, prediction from the decayed state, output from the updated
// state), is evaluated sixteen tokens at a time.  With S_0 the state at a
// chunk's start, A_t the product of the chunk's decays through token t and
// r(t, s) = A_t / A_s the product of the decays after token s through t,
//     a_t S_{t-1} k^_t = A_t S_0 k^_t + sum_{s<t} r(t, s) (k^_s . k^_t) d_s,
// so the chunk's d solve a 16x16 unit lower-triangular system
//     (I + L) D = R,  L[t][s] = b_t r(t, s) (k^_s . k^_t) (s < t),
//                     R[t] = b_t (v_t - A_t S_0 k^_t),
// and then
//     S_16 = A_15 S_0 + sum_s r(15, s) k^_s d_s^T,
//     o_t  = A_t S_0^T q^_t + sum_{s<=t} r(t, s) (k^_s . q^_t) d_s.
// These are the same values the token-by-token recurrence produces (up to
// rounding); the chunk only changes the order of the arithmetic.  Every
// product over the key dimension, and the state update over the chunk's
// tokens, is a dense contraction, so it runs on the matrix cores in three
// bf16 products per fp32 product: with x = x_hi + x_lo (x_hi the bf16
// rounding of x, x_lo that of the remainder), a b ~ a_hi b_hi + a_hi b_lo +
// a_lo b_hi, exact bf16 x bf16 products accumulated in fp32 (operands carry
// 16 of fp32's 24 significand bits; measured state error ~1e-5 of the
// state's largest entry, against 1e-4 allowed).  A 16x16x32 bf16 MFMA costs
// 16 cycles, a 16x16x4 fp32 MFMA (the same fp32 product over 4 keys) 32, and
// an fp32 MFMA stops the other waves' vector issue on its SIMD while it runs,
// so the chunk's 16x16 products (T R, D M^T and the state update) are split
// the same way, each on two 16x16x32 MFMAs.
//
// Parallel structure.  A workgroup takes one (sequence, v-head, slice of ISZ
// value columns); its waves have two roles:
//   - a state wave owns a block of 16 value columns of the state for the
//     whole sequence, in MFMA accumulator layout (lane l, register (kb, r):
//     key 16 kb + 4 (l / 16) + r, column l % 16).  Per chunk it splits the
//     state into bf16 halves and forms P = K^ S_0 and S_0^T Q^^T (the state
//     is the B operand of the first and the A operand of the second, so it
//     never leaves the registers), R, D = T R with T = (I + L)^-1, the
//     outputs, and the new state.  It also forms the v its R needs (lane l:
//     column l % 16, tokens 4 (l / 16) + i) from its own loads of x, on the
//     vector units beside the key products on the matrix cores.  The q^ / k^
//     rows in LDS keep their keys in
//     the order in which a lane supplies them to a 16x16x32 MFMA (keys 32 c +
//     4 (l / 16) + i and 32 c + 16 + 4 (l / 16) + i, i < 4, side by side), so
//     a lane's operand is one 16-byte read and matches its state registers;
//   - eight conv waves prepare the chunks, two per 4 tokens: one takes the
//     q channel pairs, the other the k pairs (one pair per lane, so that each
//     norm is reduced within one wave).  Raw inputs are loaded into registers
//     a chunk ahead, then conv + SiLU and the L2-normalised q^ and k^ rows
//     (per chunk c); one chunk later the
//     chunk's Gram products k^ k^T and q^ k^T, L, its inverse T, the output
//     mask M (as two key halves) and the decay products are formed: in a
//     64-column workgroup a wave of its own forms L and T (so that no wave
//     carries both the conv and the inversion) and three conv waves the
//     halves of M and the decay products; in a whole-head one four conv
//     waves share the four parts.  One conv wave also writes each chunk's
//     gates and decay ratios.  A wave issues its own instructions at a
//     fraction of the SIMD's rate (two vector waves on one SIMD each keep
//     their solo speed, and a bf16 MFMA on one wave barely slows the vector
//     work of another), so the work of an interval is spread over many short
//     waves, and the wave that inverts I + L, whose chain waits on itself, is
//     wave 0 (the oldest wave of a SIMD issues first).
// A chunk is prepared in interval c (conv), finished in c + 1 (T, M, decays)
// and consumed by the state waves in c + 2; one barrier ends each interval,
// so q^/k^ rows are triple-buffered and T, M and the coefficients double-
// buffered (about 100 KB of LDS at head size 128: one workgroup per CU).
// The state is plain at every chunk boundary (no running scale), so a run
// split at a multiple of 16 tokens and resumed from the written-back state
// gives the same bits as the straight run.
//
// The conv window is rewritten by a second small kernel after this one, so
// that no workgroup of a sequence can overwrite the window another workgroup
// of the same sequence has yet to read.
#include <algorithm>
#include <atomic>

#include "device_utils.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

// SWR: state waves asked for per workgroup (4: slices of 64 value columns, so
// that a long sequence's heads spread over more CUs; 8: whole 128-column
// heads, so that a large batch repeats the q/k conv of a head once instead
// of twice).  Every value is computed the same way in both, bit for bit.
template <int DK, int DV, int SWR>
struct PrefillShape {
    static constexpr int CT = 16;              // tokens per chunk: one MFMA tile
    static constexpr int NKB = DK / 16;        // 16-key blocks of a column block of the state
    static constexpr int NB = DV / 16;         // 16-column blocks of a head
    static constexpr int SW = NB < SWR ? NB : SWR; // state waves per workgroup, one block each
    static constexpr int NSL = NB / SW;        // workgroups per (sequence, v-head)
    static constexpr int ISZ = 16 * SW;        // value columns per workgroup
    static constexpr int NPROD = 8;            // conv waves: q and k of 4 tokens each
    // a wave of its own for L and T when the workgroup has room for it (the
    // conv waves form the other finish parts, and all of them in a whole-head
    // workgroup)
    static constexpr int NFIN = SW <= 4 ? 1 : 0;
    static constexpr int NT = 64 * (SW + NPROD + NFIN);
    static constexpr int WPE = (SW + NPROD + NFIN + 3) / 4; // waves per SIMD (one workgroup per CU)
    static constexpr bool X32 = DK >= 32;      // key products in 32-key MFMA steps (else one 16-key step)
    static constexpr int KG = X32 ? 32 : 16;   // keys per MFMA step
    static constexpr int NKC = DK / KG;        // MFMA steps over the keys
    static constexpr int KS = DK + 8;          // row stride of the bf16 q^ / k^ rows (elements)
    // row stride of the transposed k^ rows (elements): per token group of 4,
    // the 4 hi and then the 4 lo halves (16 bytes); 80 bytes, so that the
    // 16-byte reads of 8 consecutive rows hit distinct banks
    static constexpr int KTS = 5 * 8;
    static constexpr int TS = CT + 4;          // row stride of 16-wide fp32 rows (floats)
    static constexpr int QKP = DK / 2;         // q (and k) channel pairs
    static constexpr int TPW = 2 * CT / NPROD; // tokens per conv wave
    // Roles of conv wave pw (wave SW + 1 + pw of the workgroup with a finish
    // wave; else wave 0 for pw = 0 and wave SW + pw; wave w runs on SIMD
    // w % 4): its type (0: q, 1: k; the k waves also write
    // the transposed rows, so they carry more), the finish part (see
    // `finish`) it forms, or -1, and the one wave that writes the gates and
    // decay ratios.  A SIMD shares its vector issue among its waves (older
    // waves first; one wave alone reaches about half of it), so the
    // assignment evens out the SIMDs' instruction counts: with a finish wave,
    // SIMD 0 also runs it and gets two q waves and no other part.
    static constexpr int conv_type(int pw) { return NFIN ? (pw + 1) & 1 : pw & 1; }
    static constexpr int conv_part(int pw)
    {
        if (NFIN)
            return pw == 1 ? 1 : pw == 0 ? 3 : pw == 2 ? 2 : -1;
        return pw == 0 ? 0 : pw == 2 ? 1 : pw == 6 ? 3 : pw == 3 ? 2 : -1;
    }
    static constexpr int RATIO_PW = NFIN ? 5 : 1;
    static_assert(DK == DV, "square heads only");
    static_assert(DK % 16 == 0 && NB % SW == 0, "16-wide blocks");
    static_assert(QKP <= 64, "one q/k channel pair per conv lane");
    static_assert(NPROD * TPW == 2 * CT, "two conv waves per token group");
};

// Per-chunk coefficients (rows of cf[2][CF_N][16]): for token t of the chunk
//   CF_B   b_t (0 past the sequence's end)
//   CF_A   A_t, the product of the chunk's decays through t
//   CF_E   r(15, t), the decay from after t to the chunk's end
//   CF_EM  r(m - 1, t) for t < m, else 0, when a checkpoint falls after the
//          chunk's first m < 16 tokens
//   CF_SC  [0] A_15, [1] A_{m-1} (the checkpoint's decay)
constexpr int CF_B = 0, CF_A = 1, CF_E = 2, CF_EM = 3, CF_SC = 4, CF_N = 5;

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

constexpr int kBufferWord3 = 0x00020000; // raw 32-bit buffer resource, gfx9-family layout

// A buffer resource's range from a wave-uniform byte count, capped at
// INT32_MAX; kept in a scalar register so loads through it need no loop
// over distinct resources.
__device__ __forceinline__ int range_bytes(int64_t n)
{
    // clamped at 0: a negative range would turn the range check off
    const int r = n > int64_t(INT32_MAX) ? INT32_MAX : (n < 0 ? 0 : int(n));
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short bf16x4 __attribute__((ext_vector_type(4))); // bit patterns

// 16x16x32 bf16: lane l supplies A[l % 16][8 (l / 16) + i] and
// B[8 (l / 16) + i][l % 16], i < 8, and holds D[4 (l / 16) + r][l % 16] in
// register r.  (Lane layout and cost measured on gfx950: 16 cycles, as for
// a 16x16x16 bf16 product; 32 for a 16x16x4 fp32 one.)
__device__ __forceinline__ v4f mfma_k32(bf16x8 a, bf16x8 b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
// x = hi + lo to 16 significand bits for x0 and x1 at once: hi the bf16
// rounding of x (nearest, ties to even), lo that of the exact remainder, as
// packed pairs (x0's half in the low 16 bits), one pair conversion per half
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo)
{
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2v));
    const f32x2 r = {x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2v));
}
// the low (kHi false) or high 16-bit halves of words w0 and w1 as one word (w0's first)
template <bool kHi>
__device__ __forceinline__ uint32_t halves(uint32_t w0, uint32_t w1)
{
    return __builtin_amdgcn_perm(w1, w0, kHi ? 0x07060302u : 0x05040100u);
}

// The three products of a x b in bf16 halves (the lo x lo term, 2^-16 of it,
// is dropped): a_hi b_hi + a_hi b_lo + a_lo b_hi.
__device__ __forceinline__ v4f mfma3_k32(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, v4f c)
{
    c = mfma_k32(ah, bh, c);
    c = mfma_k32(ah, bl, c);
    return mfma_k32(al, bh, c);
}
// [x | y] as a lane's 8 slots of a 16x16x32 operand
__device__ __forceinline__ bf16x8 pair(bf16x4 x, bf16x4 y)
{
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}
// The same three products of 16x16x16 operands in two 16x16x32 products:
// their summation slots are a dummy index, so lane l's eight slots can carry
// its four a_hi and then its four a_lo entries (a = [a_hi | a_lo]) against
// its four b_hi entries twice (bb = [b_hi | b_hi]): a_hi b_hi + a_lo b_hi;
// and against [b_lo | 0] (blz): a_hi b_lo.  One 16x16x32 product costs what
// a 16x16x16 one does.  Both are the same instruction on purpose: a
// 16x16x16 product accumulating onto a 16x16x32 one's result (or the
// reverse) with the compiler's wait states between them gave wrong sums on
// gfx950 (measured), while chains of one instruction are exact.
__device__ __forceinline__ v4f mfma3_k16(bf16x8 a, bf16x8 bb, bf16x8 blz, v4f c)
{
    c = mfma_k32(a, blz, c);
    return mfma_k32(a, bb, c);
}
__device__ __forceinline__ bf16x8 lo_zero(bf16x4 x) { return pair(x, bf16x4{0, 0, 0, 0}); }
__device__ __forceinline__ v4f mfma3_k16(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, v4f c)
{
    return mfma3_k16(pair(ah, al), pair(bh, bh), lo_zero(bl), c);
}

// LDS values one lane of a wave wrote, read by other lanes of the same wave:
// a wave's LDS operations complete in order, so waiting for its own LDS
// operations (lgkmcnt 0, not its outstanding global loads) and keeping the
// compiler from moving code across suffices.
__device__ __forceinline__ void lds_wave_sync()
{
    __builtin_amdgcn_s_waitcnt(0xC07F); // vmcnt and expcnt at their maximum: no wait
    __builtin_amdgcn_wave_barrier();
}

// Position of key `key` in a bf16 q^ / k^ row: 32-key groups where lane
// group q of a 16x16x32 MFMA finds its keys 4 q + i and 16 + 4 q + i (i < 4)
// at 8 q .. 8 q + 7; plain order for 16-key heads.
template <bool X32>
__device__ __forceinline__ int key_pos(int key)
{
    if constexpr (X32)
        return 32 * (key >> 5) + 8 * ((key >> 2) & 3) + 4 * ((key >> 4) & 1) + (key & 3);
    else
        return key;
}

template <int DK, int DV, int W, int SWR>
// one workgroup per CU (its LDS)
__global__ __launch_bounds__((PrefillShape<DK, DV, SWR>::NT))
__attribute__((amdgpu_waves_per_eu(PrefillShape<DK, DV, SWR>::WPE)))
void prefill_kernel(PrefillParams p)
{
    using Sh = PrefillShape<DK, DV, SWR>;
    constexpr int CT = Sh::CT, NKB = Sh::NKB, SW = Sh::SW, ISZ = Sh::ISZ, KS = Sh::KS;
    constexpr int TS = Sh::TS, QKP = Sh::QKP, TPW = Sh::TPW;
    static_assert(KS % 8 == 0 && Sh::KTS % 8 == 0, "16-byte operand reads");

    // chunk c's rows are written in interval c, read by the Gram stage in
    // c + 1 and by the state waves in c + 2: three buffers; T, M and the
    // coefficients are written in c + 1 and read in c + 2: two buffers
    // bf16 halves of the q^ / k^ rows ([hi, lo][token][key position]) and of
    // the k^ columns for the state update ([key][8 (t / 4) + i]: the hi
    // halves of tokens 4 (t / 4) .. + 3 for i < 4, then their lo halves)
    __shared__ __align__(16) uint16_t kr[3][2][CT][KS]; // k^ (L2-normalised)
    __shared__ __align__(16) uint16_t qr[3][2][CT][KS]; // q^ (normalised, times scale)
    __shared__ __align__(16) uint16_t kc[3][DK][Sh::KTS];
    __shared__ __align__(16) float gt[2][2][CT];    // decay (1 past the end), beta (0 past it)
    __shared__ __align__(16) float rt[2][CT][TS];   // r(t, s) for s < t, 1 for s >= t
    __shared__ __align__(16) float tm[2][CT][TS];   // T = (I + L)^-1
    // M[t][s] = r(t, s) q^_t . k^_s (s <= t), as two terms: the Gram products
    // over the first and the second half of the keys
    __shared__ __align__(16) float mm[2][2][CT][TS];
    __shared__ __align__(16) float cf[2][CF_N][CT]; // CF_* rows
    __shared__ __align__(16) float lw[CT][TS];      // L of the chunk being inverted
    __shared__ __align__(16) float yw[8][12];       // C A^-1 of the chunk being inverted
    // conv taps of the q and k channel pairs, [tap][q pairs | k pairs]
    __shared__ __align__(16) float2 taps[W][2 * QKP];

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
    const int m16 = lane % 16, q4 = lane / 16;
    // a sequence whose range is empty or not inside [0, total_tokens) is skipped
    const int64_t tb64 = p.cu[n], te64 = p.cu[n + 1];
    if (tb64 < 0 || te64 <= tb64 || te64 > p.total_tokens)
        return;
    const int tb = int(tb64);
    const int L = int(te64 - tb64);
    const int64_t out_tok = int64_t(p.Hv) * DV; // out elements per token
    // T's upper-right 8 x 8 block is zero in every chunk: written once here,
    // before the first barrier of every role
    for (int e = tid; e < 2 * 8 * 8; e += Sh::NT)
        tm[e >> 6][(e >> 3) & 7][8 + (e & 7)] = 0.f;
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
    const uint16_t* win = reinterpret_cast<const uint16_t*>(page + p.conv_off);
    const int rowb = p.C * 2;                     // bytes per row of x (and of the window)
    constexpr uint32_t kOutOfRange = 0xFFFFFFF0u; // past any num_records below
    constexpr int HR = W - 1;                     // window rows before a token
    const int nchunks = (L + CT - 1) / CT;
    auto chunk_len = [&](int k) { return min(CT, L - k * CT); };

    // checkpoint: the state after the first ck_len tokens, into another page
    int ck_c = -1, ck_m = CT; // its chunk, and how many of the chunk's tokens it includes
    float* ck_tile = nullptr;
    if (p.ckpt_slot) {
        const int cs = p.ckpt_slot[n], cl = p.ckpt_len[n];
        if (cs >= 0 && cs < p.num_slots && cl >= 1 && cl <= L) {
            ck_c = (cl - 1) / CT;
            ck_m = cl - ck_c * CT;
            ck_tile = reinterpret_cast<float*>(p.layer + int64_t(cs) * p.page_stride + p.ssm_off) +
                      int64_t(h) * DK * DV;
        }
    }
    // a checkpoint strictly inside its chunk needs the state after ck_m tokens
    const bool ck_mid = ck_c >= 0 && ck_m < chunk_len(ck_c);

    // global channel of the workgroup's channel `ch` (q | k | v slice)
    auto chan = [&](int ch) -> int {
        if (ch < DK)
            return g * DK + ch;
        if (ch < 2 * DK)
            return p.Hk * DK + g * DK + (ch - DK);
        return 2 * p.Hk * DK + h * DV + sl * ISZ + (ch - 2 * DK);
    };

    // Gates of token k CT + lane % CT of head h (zero past the sequence's end,
    // and everywhere when `use` is false): buffer loads whose range check
    // covers the sequence's tokens only.
    auto load_gates = [&](int k, bool use) {
        const int ht = p.Hv * 4;
        const int64_t g0 = int64_t(tb + k * CT) * p.Hv + h;
        const int grec = use ? range_bytes(int64_t(L - k * CT) * ht) : 0;
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(p.alpha) + g0, short(0), grec, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(p.beta) + g0, short(0), grec, kBufferWord3);
        return make_float2(
            __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra, (lane % CT) * ht, 0, 0)),
            __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (lane % CT) * ht, 0, 0)));
    };
    // Chunk k's gates and decay ratios into gt / rt[k & 1] from the gates of
    // its tokens (lane l: token l % 16 of row l / 16); tokens past the end
    // take decay 1 and beta 0.  r(t, s), the product of the decays after s
    // through t: for s = 4 j + (row), an inclusive scan over t of the decays
    // with the tokens up to s replaced by 1.
    auto write_ratios = [&](int k, float2 gate) {
        const int b2 = k & 1;
        const int nt = chunk_len(k);
        const int t_ = m16;
        const float at = t_ < nt ? gate.x : 1.f;
        if (lane < CT) {
            gt[b2][0][t_] = at;
            gt[b2][1][t_] = t_ < nt ? gate.y : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s_ = 4 * j + q4;
            float x = t_ > s_ ? at : 1.f;
            x *= row_shr_or_one<1>(x);
            x *= row_shr_or_one<2>(x);
            x *= row_shr_or_one<4>(x);
            x *= row_shr_or_one<8>(x);
            rt[b2][t_][s_] = x;
        }
    };

    // Chunk k's T, M and coefficients (interval k + 1), from its rows, gates
    // and decay ratios, in four parts: (0) L from the Gram matrix k^ k^T and
    // T = (I + L)^-1 by forward substitution, (1) and (3) the two key halves
    // of M from q^ k^T, (2) the decay products.  Part 0 writes and reads back
    // lw within one wave.
    // the lane's element (t, s) = (4 q4, m16) of a 16 x TS tile, in floats;
    // opaque, so that the loop reads it from a register instead of forming it
    // again with a multiply whose (unused) high half can alias a register
    // that a load is still writing, which would make the read wait
    int tile_lane = 4 * q4 * TS + m16;
    asm volatile("" : "+v"(tile_lane));
    auto finish = [&](int k, int part) {
        if (k >= nchunks || part >= 4)
            return;
        const int b3 = k % 3, b2 = k & 1;
        // r(4 q4 + r, m16) at rtl[r TS]: every lane reads, the mask is applied after
        const float* rtl = &rt[b2][0][0] + tile_lane;
        const int pw = part;
        if (pw != 2) {
            // Gram: G[t][s] = x_t . k^_s, x = k^ (part 0) or q^ (parts 1, 3:
            // MFMA steps [0, NKH) and [NKH, NKC)); register r: t = 4 q4 + r,
            // s = m16 (rows are A and B operands alike: lane l reads row l % 16)
            const uint16_t(*xh)[KS] = pw == 0 ? kr[b3][0] : qr[b3][0];
            const uint16_t(*xl)[KS] = pw == 0 ? kr[b3][1] : qr[b3][1];
            constexpr int NKH = Sh::NKC >= 2 ? Sh::NKC / 2 : Sh::NKC;
            const int c2b = pw == 3 ? NKH : 0, c2e = pw == 1 ? NKH : Sh::NKC;
            v4f gm = {0.f, 0.f, 0.f, 0.f};
            if constexpr (Sh::X32) {
#pragma unroll
                for (int c2 = 0; c2 < Sh::NKC; ++c2) {
                    if (c2 < c2b || c2 >= c2e)
                        continue;
                    const int kp = 32 * c2 + 8 * q4;
                    auto ld8 = [&](const uint16_t* row) {
                        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + kp));
                    };
                    gm = mfma3_k32(ld8(xh[m16]), ld8(xl[m16]), ld8(kr[b3][0][m16]),
                                   ld8(kr[b3][1][m16]), gm);
                }
            } else {
                auto ld4 = [&](const uint16_t* row) {
                    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(row + 4 * q4));
                };
                if (pw != 3) // one step: all of it in parts 0 and 1
                    gm = mfma3_k16(ld4(xh[m16]), ld4(xl[m16]), ld4(kr[b3][0][m16]), ld4(kr[b3][1][m16]), gm);
            }
            const int s_ = m16;
            if (pw == 0) {
                const float4 bt = *reinterpret_cast<const float4*>(&gt[b2][1][4 * q4]);
                const float bts[4] = {bt.x, bt.y, bt.z, bt.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t_ = 4 * q4 + r;
                    const float l = bts[r] * rtl[r * TS] * gm[r];
                    (&lw[0][0])[tile_lane + r * TS] = s_ < t_ ? l : 0.f;
                }
                // the wave's own LDS writes above are read back by other lanes
                lds_wave_sync();
                // T = (I + L)^-1 in 8 x 8 blocks: with A and B the diagonal
                // blocks of I + L and C its lower-left block,
                //     T = [[A^-1, 0], [-B^-1 C A^-1, B^-1]]
                // (T's upper-right block is zero from the kernel's start).
                // (1) lane m16 (lanes 16-63 repeat it): column m16 % 8 of A^-1
                // (m16 < 8) or B^-1 by forward substitution; the column index
                // is opaque so that the identity entries are formed per chunk,
                // not held across the chunk loop
                {
                    const int hb = 8 * (m16 >> 3);
                    int jc = m16 & 7;
                    asm volatile("" : "+v"(jc));
                    float x[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        float acc = r == jc ? 1.f : 0.f;
#pragma unroll
                        for (int c = 0; c < r; ++c)
                            acc = fmaf(-lw[hb + r][hb + c], x[c], acc);
                        x[r] = acc;
                    }
                    if (lane < CT) {
#pragma unroll
                        for (int r = 0; r < 8; ++r)
                            tm[b2][hb + r][hb + (m16 & 7)] = x[r];
                    }
                }
                lds_wave_sync();
                // (2) Y = C A^-1 and (3) T's lower-left block -B^-1 Y, one
                // entry (row lane / 8, column lane % 8) per lane
                const int r8 = lane >> 3, c8 = lane & 7;
                {
                    float y = 0.f;
#pragma unroll
                    for (int m = 0; m < 8; ++m)
                        y = fmaf(lw[8 + r8][m], tm[b2][m][c8], y);
                    yw[r8][c8] = y;
                }
                lds_wave_sync();
                {
                    float xv = 0.f;
#pragma unroll
                    for (int m = 0; m < 8; ++m)
                        xv = fmaf(tm[b2][8 + r8][8 + m], yw[m][c8], xv);
                    tm[b2][8 + r8][c8] = -xv;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t_ = 4 * q4 + r;
                    const float mv = rtl[r * TS] * gm[r];
                    (&mm[b2][pw == 3][0][0])[tile_lane + r * TS] = s_ <= t_ ? mv : 0.f;
                }
            }
        } else if (lane < CT) {
            // wave 2: A_t = a_0 r(t, 0), r(15, t), the checkpoint's r(m - 1, t)
            const int t_ = lane;
            const float a0 = gt[b2][0][0];
            cf[b2][CF_B][t_] = gt[b2][1][t_];
            cf[b2][CF_A][t_] = a0 * rt[b2][t_][0];
            cf[b2][CF_E][t_] = rt[b2][CT - 1][t_];
            cf[b2][CF_EM][t_] = t_ < ck_m ? rt[b2][ck_m - 1][t_] : 0.f;
            if (t_ == 0) {
                cf[b2][CF_SC][0] = a0 * rt[b2][CT - 1][0];
                cf[b2][CF_SC][1] = a0 * rt[b2][ck_m - 1][0];
            }
        }
    };

    // roles by wave: the wave that inverts I + L first (the oldest wave of a
    // SIMD gets the first issue slot, and its substitution chain is the least
    // able to wait): the finish wave, or in a whole-head workgroup conv wave
    // 0, which forms that part there; then the state waves (waves 1 .. SW),
    // then the other conv waves
    const int sw = wave - 1; // state wave index, for sw in [0, SW)
    if (sw >= 0 && sw < SW) {
        // ========================= state waves ==============================
        const int col0 = sl * ISZ + 16 * sw; // first column of the block in the head
        float* tile = reinterpret_cast<float*>(page + p.ssm_off) + int64_t(h) * DK * DV;
        // s[kb][r] = S[key 16 kb + 4 q4 + r][column col0 + m16], at byte
        // eoff + (16 kb + r) DV 4 of the head's tile.  State I/O goes through
        // buffer resources: the lane's offset eoff, the row r as the
        // instruction's immediate offset and the block 16 kb in the scalar
        // offset, so that the (rare) checkpoint stores inside the chunk loop
        // hold one resource and one address register across it.  Every access
        // lies inside the tile.
        const int eoff = ((4 * q4) * DV + col0 + m16) * 4;
        constexpr int kTileBytes = DK * DV * 4;
        v4f s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            s[kb] = v4f{0.f, 0.f, 0.f, 0.f};
        const __amdgpu_buffer_rsrc_t rt_tile =
            __builtin_amdgcn_make_buffer_rsrc(tile, short(0), kTileBytes, kBufferWord3);
        if (warm) { // a cold page is never read
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s[kb][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        rt_tile, eoff + r * DV * 4, 16 * kb * DV * 4, 0));
        }
        auto store_state = [&](__amdgpu_buffer_rsrc_t dst, const v4f (&x)[NKB]) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[kb][r]), dst,
                                                          eoff + r * DV * 4, 16 * kb * DV * 4, 0);
        };
        const __amdgpu_buffer_rsrc_t rt_ck = __builtin_amdgcn_make_buffer_rsrc(
            ck_tile ? ck_tile : tile, short(0), ck_tile ? kTileBytes : 0, kBufferWord3);

        // v of the block: lane l forms v[token 4 q4 + i][column col0 + m16],
        // i < 4, itself (the values its R needs), from its channel's HR + 4
        // rows, loaded one interval ahead with 16-bit buffer loads: the range
        // check returns zero past the sequence's end, and the window rows of
        // a cold sequence are an empty range.  The conv and SiLU run beside
        // the key products on the matrix cores.
        constexpr int NRV = HR + 4;
        const int vch = chan(2 * DK + 16 * sw + m16); // the lane's v channel
        const int vo = vch * 2;
        float vtap[W];
#pragma unroll
        for (int w = 0; w < W; ++w)
            vtap[w] = bf16_to_f32(p.conv_w[int64_t(vch) * W + w]);
        const float vbias = p.conv_b ? bf16_to_f32(p.conv_b[vch]) : 0.f;
        uint32_t vr[NRV]; // bf16 bits in the low half
        auto ld16 = [](__amdgpu_buffer_rsrc_t r, uint32_t off) {
            return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, int(off), 0, 0));
        };
        auto vrows = [&](int xb) { // rows of x from xb on (xb <= L)
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.x) + int64_t(tb + xb) * p.C,
                                                     short(0), range_bytes(int64_t(L - xb) * rowb),
                                                     kBufferWord3);
        };
        // chunk k >= 1: rows k CT - HR + 4 q4 + i, the first of them not before
        // the sequence's start (L, an empty range, once past its end)
        auto issue_v = [&](int k) {
            const __amdgpu_buffer_rsrc_t rs = vrows(min(k * CT - HR, L));
#pragma unroll
            for (int i = 0; i < NRV; ++i)
                vr[i] = ld16(rs, (4 * q4 + i) * rowb + vo);
        };
        { // chunk 0: the rows before the sequence's start come from the window
            const __amdgpu_buffer_rsrc_t rs = vrows(0);
            const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(win), short(0), warm ? HR * rowb : 0, kBufferWord3);
#pragma unroll
            for (int i = 0; i < NRV; ++i) {
                const int r = 4 * q4 + i - HR;
                vr[i] = ld16(rw, r < 0 ? uint32_t((HR + r) * rowb + vo) : kOutOfRange) |
                        ld16(rs, r >= 0 ? uint32_t(r * rowb + vo) : kOutOfRange);
            }
        }
        __syncthreads(); // the conv waves' taps are in LDS
        for (int c = 0; c < nchunks + 2; ++c) {
            const int k = c - 2;
            if (k >= 0) {
                const int b3 = k % 3, b2 = k & 1;
                const int nt = chunk_len(k);
                float vv[4]; // v[token 4 q4 + i][col0 + m16]
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float a = vbias;
#pragma unroll
                    for (int w = 0; w < W; ++w)
                        a = fmaf(vtap[w], __uint_as_float(vr[i + w] << 16), a);
                    vv[i] = silu(a);
                }
                // the next chunk's rows into the same registers, once read
                __builtin_amdgcn_sched_barrier(0);
                issue_v(k + 1);
                // P[t][col] = k^_t . S_0[:, col]  (register r: token 4 q4 + r)
                // O[col][t] = S_0[:, col] . q^_t  (register r: column 4 q4 + r, token m16)
                v4f P = {0.f, 0.f, 0.f, 0.f}, O = {0.f, 0.f, 0.f, 0.f};
                if constexpr (Sh::X32) {
#pragma unroll
                    for (int c2 = 0; c2 < Sh::NKC; ++c2) {
                        // the lane's 8 keys of the step: 32 c2 + 4 q4 + i, 32 c2 + 16 + 4 q4 + i
                        // (element i = s[2 c2 + i / 4][i % 4], two per word)
                        uint32_t h4[4], l4[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            split_bf16x2(s[2 * c2 + j / 2][2 * (j % 2)], s[2 * c2 + j / 2][2 * (j % 2) + 1],
                                         h4[j], l4[j]);
                        const bf16x8 sh = __builtin_bit_cast(bf16x8, make_uint4(h4[0], h4[1], h4[2], h4[3]));
                        const bf16x8 sl = __builtin_bit_cast(bf16x8, make_uint4(l4[0], l4[1], l4[2], l4[3]));
                        const int kp = 32 * c2 + 8 * q4;
                        auto ld8 = [&](const uint16_t* row) {
                            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + kp));
                        };
                        P = mfma3_k32(ld8(kr[b3][0][m16]), ld8(kr[b3][1][m16]), sh, sl, P);
                        O = mfma3_k32(sh, sl, ld8(qr[b3][0][m16]), ld8(qr[b3][1][m16]), O);
                    }
                } else {
                    uint32_t h2[2], l2[2];
                    split_bf16x2(s[0][0], s[0][1], h2[0], l2[0]);
                    split_bf16x2(s[0][2], s[0][3], h2[1], l2[1]);
                    const bf16x4 sh = __builtin_bit_cast(bf16x4, make_uint2(h2[0], h2[1]));
                    const bf16x4 sl = __builtin_bit_cast(bf16x4, make_uint2(l2[0], l2[1]));
                    auto ld4 = [&](const uint16_t* row) {
                        return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(row + 4 * q4));
                    };
                    P = mfma3_k16(ld4(kr[b3][0][m16]), ld4(kr[b3][1][m16]), sh, sl, P);
                    O = mfma3_k16(sh, sl, ld4(qr[b3][0][m16]), ld4(qr[b3][1][m16]), O);
                }
                // R[t] = b_t (v_t - A_t P_t), then D = T R
                const float4 bb = *reinterpret_cast<const float4*>(&cf[b2][CF_B][4 * q4]);
                const float4 aa = *reinterpret_cast<const float4*>(&cf[b2][CF_A][4 * q4]);
                const float4 tt = *reinterpret_cast<const float4*>(&tm[b2][m16][4 * q4]);
                const float R0 = bb.x * (vv[0] - aa.x * P[0]);
                const float R1 = bb.y * (vv[1] - aa.y * P[1]);
                const float R2 = bb.z * (vv[2] - aa.z * P[2]);
                const float R3 = bb.w * (vv[3] - aa.w * P[3]);
                // d[r] = d_{4 q4 + r}[col0 + m16]: one 16x16x16 product, the lane
                // holding T[m16][4 q4 + i] and R[4 q4 + i][m16] (bf16 splits: an
                // fp32 MFMA would stop the other waves' vector issue on this SIMD)
                auto split4 = [](float a, float b, float c, float e, bf16x4& h, bf16x4& l) {
                    uint32_t h0, l0, h1, l1;
                    split_bf16x2(a, b, h0, l0);
                    split_bf16x2(c, e, h1, l1);
                    h = __builtin_bit_cast(bf16x4, make_uint2(h0, h1));
                    l = __builtin_bit_cast(bf16x4, make_uint2(l0, l1));
                };
                bf16x4 th, tl, rh, rl;
                split4(tt.x, tt.y, tt.z, tt.w, th, tl);
                split4(R0, R1, R2, R3, rh, rl);
                const v4f d = mfma3_k16(th, tl, rh, rl, v4f{0.f, 0.f, 0.f, 0.f});
                // outputs: O^T = A_t O^T + D^T M^T (lane: 4 columns of token m16)
                const float4 m0 = *reinterpret_cast<const float4*>(&mm[b2][0][m16][4 * q4]);
                const float4 m1 = *reinterpret_cast<const float4*>(&mm[b2][1][m16][4 * q4]);
                const float4 mv = make_float4(m0.x + m1.x, m0.y + m1.y, m0.z + m1.z, m0.w + m1.w);
                O *= cf[b2][CF_A][m16];
                bf16x4 dh0, dl0, mh, ml;
                split4(d[0], d[1], d[2], d[3], dh0, dl0);
                split4(mv.x, mv.y, mv.z, mv.w, mh, ml);
                O = mfma3_k16(dh0, dl0, mh, ml, O);
                if (m16 < nt)
                    *reinterpret_cast<uint2*>(out_base + int64_t(k * CT + m16) * out_tok +
                                              16 * sw + 4 * q4) = pack_bf16x4(O[0], O[1], O[2], O[3]);
                // S <- A_15 S_0 + sum_s r(15, s) k^_s d_s^T (and, for a checkpoint
                // inside the chunk, the state after its first ck_m tokens): per
                // 16-key block, K^T (16 keys x 16 tokens) times the decayed D
                auto advance = [&](v4f (&x)[NKB], float a0, const float4& e) {
                    uint32_t h2[2], l2[2];
                    split_bf16x2(d[0] * e.x, d[1] * e.y, h2[0], l2[0]);
                    split_bf16x2(d[2] * e.z, d[3] * e.w, h2[1], l2[1]);
                    const bf16x4 dh = __builtin_bit_cast(bf16x4, make_uint2(h2[0], h2[1]));
                    const bf16x4 dl = __builtin_bit_cast(bf16x4, make_uint2(l2[0], l2[1]));
                    const bf16x8 dd = pair(dh, dh), dlz = lo_zero(dl);
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        // k^_hi and k^_lo of key 16 kb + m16, tokens 4 q4 .. + 3
                        const bf16x8 k8 = __builtin_bit_cast(
                            bf16x8, *reinterpret_cast<const uint4*>(&kc[b3][16 * kb + m16][8 * q4]));
                        x[kb] = mfma3_k16(k8, dd, dlz, s[kb] * a0);
                    }
                };
                if (k == ck_c && ck_mid) {
                    v4f sc[NKB];
                    advance(sc, cf[b2][CF_SC][1],
                            *reinterpret_cast<const float4*>(&cf[b2][CF_EM][4 * q4]));
                    store_state(rt_ck, sc);
                }
                advance(s, cf[b2][CF_SC][0], *reinterpret_cast<const float4*>(&cf[b2][CF_E][4 * q4]));
                if (k == ck_c && !ck_mid)
                    store_state(rt_ck, s);
            }
            __syncthreads(); // end of interval c
        }
        store_state(rt_tile, s);
        return;
    }

    if (Sh::NFIN && wave == 0) {
        // ========================= finish wave ==============================
        __syncthreads(); // the conv waves' taps are in LDS
        for (int c = 0; c < nchunks + 2; ++c) {
            if (c >= 1)
                finish(c - 1, 0);
            __syncthreads(); // end of interval c
        }
        return;
    }

    // ========================= conv waves ===================================
    // Conv wave pw takes tokens [t0, t0 + TPW) of each chunk: the q or the k
    // channel pairs (conv_type), one pair per lane, so that each of q^ and
    // k^ is normalised within one wave.
    const int pw = Sh::NFIN ? wave - SW - 1 : (wave == 0 ? 0 : wave - SW);
    const int ty = Sh::conv_type(pw); // 0: q, 1: k
    const bool rw_ = pw == Sh::RATIO_PW; // writes the gates and decay ratios
    const int t0 = (pw >> 1) * TPW;

    // conv taps of the slice's channel pairs into LDS (read back per chunk, so
    // that they hold no registers across the loop); biases stay in registers.
    // Both are scaled by -log2(e), so that a conv sum is y = -log2(e) x and
    // the SiLU's exponential is exp2(y) with no multiply; the factor cancels
    // in the L2 norm (see `prepare`).
    constexpr float kNegLog2e = -1.4426950408889634f;
    for (int e = 64 * pw + lane; e < W * 2 * QKP; e += 64 * Sh::NPROD) {
        const int w = e / (2 * QKP), pr = e - w * (2 * QKP);
        const int ch = pr < QKP ? 2 * pr : DK + 2 * (pr - QKP);
        const int c = chan(ch);
        taps[w][pr] = make_float2(kNegLog2e * bf16_to_f32(p.conv_w[int64_t(c) * W + w]),
                                  kNegLog2e * bf16_to_f32(p.conv_w[int64_t(c + 1) * W + w]));
    }
    auto bias2 = [&](int ch) {
        const int c = chan(ch);
        return p.conv_b ? make_float2(kNegLog2e * bf16_to_f32(p.conv_b[c]),
                                      kNegLog2e * bf16_to_f32(p.conv_b[c + 1]))
                        : make_float2(0.f, 0.f);
    };
    const int qkp = min(lane, QKP - 1);  // the lane's pair (clamped; idle lanes recompute)
    const int xch = ty * DK + 2 * qkp;   // its first channel in the slice's channel order
    const float2 bx = bias2(xch);

    // Raw inputs of chunk k for this wave's TPW tokens, loaded into registers
    // a chunk ahead: the lane's q or k channel pair over the W-1 rows before
    // the wave's first token and its TPW rows; the gates of token k CT + lane
    // % CT.  All are buffer loads with the
    // row in the lane's offset: the range check returns zero for rows past
    // the sequence's end and for the rows before its start when the sequence
    // is cold, whose window resource is empty, so no load waits on a branch
    // and a cold page is never read.  Rows past the end give finite values
    // whose tokens the coefficients then leave out (b = 0, decay 1).
    constexpr int NR = HR + TPW;
    uint32_t xr[NR];
    float2 pg;
    const int ox = chan(xch) * 2; // byte offset of the lane's pair inside a row of x
    auto ld = [](__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0);
    };
    // The in-loop form has no branch and no early return: a load skipped on
    // one path would make the compiler merge the two paths' registers with
    // copies, and a copy of a register still being loaded waits for the load.
    // Past the sequence's end the ranges are empty (the loads return zero).
    auto rows_resource = [&](int xb) { // rows from xb on (xb <= L)
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.x) + int64_t(tb + xb) * p.C,
                                                 short(0), range_bytes(int64_t(L - xb) * rowb),
                                                 kBufferWord3);
    };
    auto load_rows = [&](__amdgpu_buffer_rsrc_t rs) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
            xr[i] = ld(rs, ox + i * rowb);
    };
    // chunk k >= 1: the wave's first row k CT + t0 - HR is not before the
    // sequence's start (L, an empty range, once past its end)
    auto issue = [&](int k) { load_rows(rows_resource(min(k * CT + t0 - HR, L))); };
    // chunk 0: the first rows of the waves of tokens 0-3 come from the window
    auto issue_first = [&]() {
        const int rbase = t0 - HR;
        pg = load_gates(0, rw_);
        if (rbase >= 0) {
            issue(0);
        } else {
            const __amdgpu_buffer_rsrc_t rs = rows_resource(0);
            const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(win), short(0), warm ? HR * rowb : 0, kBufferWord3);
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const int r = i - HR; // rbase == -HR here
                xr[i] = r < 0 ? ld(rw, (HR + r) * rowb + ox) : ld(rs, r * rowb + ox);
            }
        }
    };

    // conv + SiLU of chunk k for the wave's tokens [t0, t0 + TPW): the bf16
    // halves of its q^ or k^ into qr / kr[k % 3] (and of k^ by key into
    // kc[k % 3]) once the wave has reduced the TPW sums |q|^2 or |k|^2 of its
    // tokens.  Every token is computed, also past
    // the sequence's end.  The ratio wave also writes the gates and the decay ratios
    // r(t, s) into gt / rt[k & 1].
    auto prepare = [&](int k) { // k < nchunks
        static_assert(TPW == 4, "the sums of 4 tokens are reduced together");
        const int b3 = k % 3;
        // the conv sums first: once they have read the raw rows, the next
        // chunk's loads go out (into the same registers) and have the rest of
        // the interval and the next one's start to arrive
        // q or k: the lane walks the wave's tokens over its register rows
        float2 tx[W];
#pragma unroll
        for (int w = 0; w < W; ++w)
            tx[w] = taps[w][ty * QKP + qkp];
        float2 xs[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            float a0 = bx.x, a1 = bx.y;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                a0 = fmaf(tx[w].x, lo_bf16(xr[i + w]), a0);
                a1 = fmaf(tx[w].y, hi_bf16(xr[i + w]), a1);
            }
            xs[i] = make_float2(a0, a1);
        }
        // keep the loads below the sums: loads moved above them would need
        // registers of their own, and the copies into the loop's registers
        // would wait for the loads at the interval's end
        __builtin_amdgcn_sched_barrier(0);
        issue(k + 1);
        float ss[TPW];
        const bool own = lane < QKP;
        // u = y sigmoid(-y ln 2) = -log2(e) silu(x) for y = -log2(e) x
        auto silu_scaled = [](float y) {
            return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
        };
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            xs[i] = make_float2(silu_scaled(xs[i].x), silu_scaled(xs[i].y));
            ss[i] = own ? fmaf(xs[i].x, xs[i].x, xs[i].y * xs[i].y) : 0.f;
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
        const float tsum = group_sum<16>(fold_rows(fold_halves(ss[0], ss[1]), fold_halves(ss[2], ss[3])));
        // row j of the sums holds token (0, 2, 1, 3)[j]; lane i < 4 takes token i's
        const int src = 16 * (((lane & 1) << 1) | ((lane >> 1) & 1));
        // with s = silu(x) = u / -log2(e): s / sqrt(|s|^2 + eps) = -u / sqrt(|u|^2 + log2(e)^2 eps)
        const float rx = (ty == 0 ? -p.scale : -1.f) *
                         __builtin_amdgcn_rsqf(__shfl(tsum, src, 64) + p.eps * (kNegLog2e * kNegLog2e));
        if (own) {
            // the lane's keys 2 lane and 2 lane + 1 sit side by side in a row
            const int kp = key_pos<Sh::X32>(2 * lane);
            uint16_t(*dst)[CT][KS] = ty == 0 ? qr[b3] : kr[b3];
            // per token, the two keys' halves as one word each (key 2 lane in
            // the low half)
            uint32_t xh[TPW], xl[TPW];
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rx), i));
                split_bf16x2(xs[i].x * f, xs[i].y * f, xh[i], xl[i]);
                *reinterpret_cast<uint32_t*>(&dst[0][t0 + i][kp]) = xh[i];
                *reinterpret_cast<uint32_t*>(&dst[1][t0 + i][kp]) = xl[i];
            }
            if (ty == 1) {
                // k^ columns of the two keys over the wave's 4 tokens: per key one 16-byte
                // store of the 4 hi halves, then the 4 lo halves
                *reinterpret_cast<uint4*>(&kc[b3][2 * lane][2 * t0]) =
                    make_uint4(halves<false>(xh[0], xh[1]), halves<false>(xh[2], xh[3]),
                               halves<false>(xl[0], xl[1]), halves<false>(xl[2], xl[3]));
                *reinterpret_cast<uint4*>(&kc[b3][2 * lane + 1][2 * t0]) =
                    make_uint4(halves<true>(xh[0], xh[1]), halves<true>(xh[2], xh[3]),
                               halves<true>(xl[0], xl[1]), halves<true>(xl[2], xl[3]));
            }
        }
        if (rw_)
            write_ratios(k, pg);
        pg = load_gates(k + 1, rw_); // after its last use, for the same reason
    };

    issue_first();
    __syncthreads(); // taps in LDS
    const int fp = Sh::conv_part(pw); // the finish part this wave forms, or -1
    // the previous chunk's finish part before the conv in a whole-head
    // workgroup (its conv waves then start the interval in different phases:
    // 2 % faster there), after it in a 64-column one (3 % faster there)
    for (int c = 0; c < nchunks; ++c) {
        if (!Sh::NFIN && c >= 1 && fp >= 0)
            finish(c - 1, fp);
        prepare(c); // also issues chunk c + 1's loads
        if (Sh::NFIN && c >= 1 && fp >= 0)
            finish(c - 1, fp);
        __syncthreads(); // end of interval c
    }
    // intervals nchunks and nchunks + 1: the last chunk's finish parts, then
    // the state waves' last chunk
    if (fp >= 0)
        finish(nchunks - 1, fp);
    __syncthreads();
    __syncthreads();
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

template <int DK, int DV, int W, int SWR>
int launch_prefill_t(const gdn_pool* pool, int32_t layer, int32_t num_seqs, int64_t total_tokens,
                     const int32_t* cu, const gdn_step_args* a, const int32_t* ckpt_slot,
                     const int32_t* ckpt_len, hipStream_t stream)
{
    using Sh = PrefillShape<DK, DV, SWR>;
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
    hipLaunchKernelGGL((prefill_kernel<DK, DV, W, SWR>), dim3(uint32_t(blocks)), dim3(Sh::NT), 0,
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

// Compute units of the calling thread's current device (looked up once per device).
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 0;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev < 64)
        cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

template <int DK, int SWR>
int dispatch_w(const gdn_pool* pool, int32_t layer, int32_t num_seqs, int64_t T, const int32_t* cu,
               const gdn_step_args* a, const int32_t* cs, const int32_t* cl, hipStream_t stream)
{
    switch (pool->desc.conv_width) {
    case 2: return launch_prefill_t<DK, DK, 2, SWR>(pool, layer, num_seqs, T, cu, a, cs, cl, stream);
    case 3: return launch_prefill_t<DK, DK, 3, SWR>(pool, layer, num_seqs, T, cu, a, cs, cl, stream);
    case 4: return launch_prefill_t<DK, DK, 4, SWR>(pool, layer, num_seqs, T, cu, a, cs, cl, stream);
    default: return fail(GDN_EUNSUPPORTED, "prefill: conv width %d", pool->desc.conv_width);
    }
}

// Head size 128: 64-column workgroups while they all fit on the GPU at once
// (the critical path is then the longest sequence, which gets twice the CUs),
// whole-head workgroups when the batch needs several rounds of them.
int dispatch_128(const gdn_pool* pool, int32_t layer, int32_t num_seqs, int64_t T,
                 const int32_t* cu, const gdn_step_args* a, const int32_t* cs, const int32_t* cl,
                 hipStream_t stream)
{
    const int cus = device_cus();
    if (cus <= 0)
        return fail(GDN_EHIP, "cannot query the device's compute units");
    if (int64_t(num_seqs) * pool->desc.num_v_heads * 2 <= cus)
        return dispatch_w<128, 4>(pool, layer, num_seqs, T, cu, a, cs, cl, stream);
    return dispatch_w<128, 8>(pool, layer, num_seqs, T, cu, a, cs, cl, stream);
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
    case 16: return dispatch_w<16, 4>(pool, layer, num_seqs, total_tokens, cu, a, cs, cl, stream);
    case 32: return dispatch_w<32, 4>(pool, layer, num_seqs, total_tokens, cu, a, cs, cl, stream);
    case 64: return dispatch_w<64, 4>(pool, layer, num_seqs, total_tokens, cu, a, cs, cl, stream);
    case 128: return dispatch_128(pool, layer, num_seqs, total_tokens, cu, a, cs, cl, stream);
    default: return fail(GDN_EUNSUPPORTED, "prefill: head dim %d", pool->desc.head_k_dim);
    }
}

} // namespace gdn
