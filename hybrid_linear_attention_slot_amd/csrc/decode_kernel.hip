// Fused decode step of a Gated DeltaNet layer over a page-strided slot pool
// (gfx950).
//
// Per batch row: gather the row's conv window and recurrent state from its
// slot ("非连续 KV Cache" §5: indexed access into the strided pool; zero
// state when has_initial_state is 0, "Linear-State Prefix Cache 内部机制"
// §4.1), run the depthwise causal conv update with SiLU ("非连续 KV Cache"
// §6, the decode-time conv update), L2-normalise q and k, apply the gated
// delta rule ("Kapitsa 源码拆解 05", section on what Gated DeltaNet keeps):
//     S <- a S;  u = S k;  S <- S + b (v - u) k^T;  o = S q
// and write window and state back into the same page ("Linear-State Prefix
// Cache 内部机制" §0: the slot is overwritten in place every step).
//
// Design (HBM-bound; MFMA is of no use for rank-1 updates and mat-vecs):
//   - one group of waves per (row, k-head g), one or more such groups per
//     workgroup (several for small heads, below).  A group owns the q and k
//     conv channels of g and the v channels of the Hv/Hk v-heads that read g,
//     so no two groups touch the same window channels, and q/k are computed
//     once.
//   - each v-head's dk x dv fp32 state tile is streamed once from HBM into
//     registers and once back.  The tile is stored key-major ([dk][dv], value
//     index contiguous).  Wave w owns the key rows [w KPW, (w+1) KPW) of every
//     tile and walks them RPI rows (1 KiB with dv = 128) per load or store
//     instruction, each lane holding one float4 of value columns; a wave's
//     consecutive memory instructions therefore touch consecutive kilobytes,
//     the order in which the HBM stream of this in-place read-modify-write
//     runs fastest.
//   - S k and S q are lane-partial dot products over the lane's key rows,
//     summed over the RPI lanes of a column with cross-lane moves and over
//     the waves through LDS (one barrier for both heads of a pair, fixed
//     summation order); o is formed without a second pass over S:
//     o = a (S_old q) + d (k.q)  with  d = b (v - a S_old k).
//   - the state loads of the first two heads are issued before the conv so
//     that the conv and the norms overlap them.
#include "device_utils.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int DK, int DV>
struct DecodeShape {
    static constexpr int LPR = DV / 4;                                 // lanes per key row (a float4 each)
    static constexpr int RPI = 64 / LPR;                               // key rows per memory instruction
    static constexpr int NWMAX = DK * DV / 1024;                       // waves with >= 4 rows per lane
    static constexpr int NW = NWMAX < 1 ? 1 : (NWMAX > 4 ? 4 : NWMAX); // waves per workgroup
    static constexpr int KPW = DK / NW;                                // key rows per wave
    static constexpr int JPL = KPW / RPI;                              // key rows per lane
    static constexpr int NT = 64 * NW;
    static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "value dim");
    static_assert(DK % NW == 0 && KPW % RPI == 0 && JPL >= 1, "key dim");
};

struct DecodeParams {
    uint8_t* layer;
    int64_t page_stride;
    int64_t ssm_off;
    int64_t conv_off;
    int32_t num_slots;
    int32_t C;
    int32_t Hk;
    int32_t Hv;
    const uint16_t* x;
    const uint16_t* conv_w;
    const uint16_t* conv_b;
    const float* alpha;
    const float* beta;
    const int32_t* state_indices;
    const uint8_t* hs;
    uint16_t* out;
    float scale;
    float eps;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over one page's state region.  Buffer instructions take the
// per-key offset in an SGPR, so a lane needs a single VGPR offset for all of
// its loads and stores, and the hardware drops accesses past num_records.
constexpr int kBufferWord3 = 0x00020000; // raw 32-bit buffer, gfx9-family layout
constexpr int kNonTemporal = 2;          // cache-policy bit: streamed once
// State stores are non-temporal at device scope (SC1 | NT).  On the 256-row,
// 32-head update this ran 5 % faster than NT alone (5.95 against 5.66 TB/s);
// SC1 or SC0 + SC1 without NT, SC0 + NT and cached stores were all slower,
// and so were SC1 + NT loads.
constexpr int kStoreDeviceNT = 16 | kNonTemporal;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t state_rsrc(float* ssm, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(ssm, short(0), bytes, kBufferWord3);
}

// Tile of head h: the lane's key rows RPI*m + (its first row), value columns
// of its float4 (voff = byte offset of that first element inside a head tile).
template <int DK, int DV, int JPL, int RPI>
__device__ __forceinline__ void load_tile(f32x4 (&s)[JPL], __amdgpu_buffer_rsrc_t r, int voff,
                                          int h)
{
#pragma unroll
    for (int m = 0; m < JPL; ++m)
        s[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             r, voff, (h * DK + RPI * m) * DV * 4, kNonTemporal));
}

// Stores take their whole offset in the VGPR and a literal zero soffset:
// the compiler only protects a 128-bit store's data registers from being
// overwritten too early (the store reads them after issue) when soffset is
// not an SGPR, and with an SGPR soffset that window was seen to corrupt the
// last lanes' data.
template <int DK, int DV, int RPI>
__device__ __forceinline__ void store_row(const f32x4& t, __amdgpu_buffer_rsrc_t r, int voff,
                                          int h, int m)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, t), r,
                                           voff + (h * DK + RPI * m) * DV * 4, 0, kStoreDeviceNT);
}

// Sum over the lanes l, l + S, l + 2S, ... of a wave (S a power of two).
template <int S>
__device__ __forceinline__ float strided_sum(float v)
{
#pragma unroll
    for (int st = S; st < 64; st *= 2)
        v += __shfl_xor(v, st, 64);
    return v;
}

template <int JPL>
__device__ __forceinline__ void zero_tile(f32x4 (&s)[JPL])
{
#pragma unroll
    for (int m = 0; m < JPL; ++m)
        s[m] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Conv inputs of one pair of adjacent channels (c, c+1), kept as the raw
// words that were loaded: nothing is unpacked until every load of the
// workgroup's first phase has been issued.
template <int W>
struct ConvPairIn {
    uint32_t x;          // current inputs, bf16 x2
    uint32_t win[W - 1]; // window rows, oldest first, bf16 x2
    uint32_t w[W];       // taps of c then taps of c+1: 2W bf16
    uint32_t b;          // bias of c and c+1, bf16 x2 (0 without bias)
};

__device__ __forceinline__ float lo_bf16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// bf16 number k of the packed sequence in `w`
template <int K, int W>
__device__ __forceinline__ float tap(const uint32_t (&w)[W])
{
    return (K & 1) ? hi_bf16(w[K >> 1]) : lo_bf16(w[K >> 1]);
}

template <int W>
__device__ __forceinline__ void load_conv_pair(ConvPairIn<W>& in, const DecodeParams& p, int row,
                                               int c, const uint32_t* wp, bool warm)
{
    in.x = *reinterpret_cast<const uint32_t*>(p.x + int64_t(row) * p.C + c);
#pragma unroll
    for (int w = 0; w < W - 1; ++w)
        in.win[w] = warm ? wp[w * (p.C / 2)] : 0u;
    const uint32_t* wsrc = reinterpret_cast<const uint32_t*>(p.conv_w + int64_t(c) * W);
#pragma unroll
    for (int k = 0; k < W; ++k)
        in.w[k] = wsrc[k];
    in.b = p.conv_b ? *reinterpret_cast<const uint32_t*>(p.conv_b + c) : 0u;
}

template <int W, int T = 0>
__device__ __forceinline__ void conv_taps(const ConvPairIn<W>& in, float& acc0, float& acc1)
{
    if constexpr (T < W - 1) {
        acc0 += tap<T, W>(in.w) * lo_bf16(in.win[T]);
        acc1 += tap<W + T, W>(in.w) * hi_bf16(in.win[T]);
        conv_taps<W, T + 1>(in, acc0, acc1);
    }
}

// SiLU(conv) of both channels into LDS; the window is rewritten shifted by
// one input with the current input appended.
template <int W>
__device__ __forceinline__ void finish_conv_pair(const ConvPairIn<W>& in, uint32_t* wp, int C,
                                                 float* y)
{
    float acc0 = lo_bf16(in.b), acc1 = hi_bf16(in.b);
    conv_taps<W>(in, acc0, acc1);
    acc0 += tap<W - 1, W>(in.w) * lo_bf16(in.x);
    acc1 += tap<2 * W - 1, W>(in.w) * hi_bf16(in.x);
#pragma unroll
    for (int w = 0; w + 1 < W - 1; ++w)
        wp[w * (C / 2)] = in.win[w + 1];
    wp[(W - 2) * (C / 2)] = in.x;
    y[0] = silu(acc0);
    y[1] = silu(acc1);
}

// One (row, k-head group).  WARM is a template parameter so that the cold
// path (no state loads) and the warm path each get exact memory waits.
// `red` holds the per-wave partial sums of S k and S q of two heads:
// [2 heads][u | o][NW waves][DV].
template <int DK, int DV, int W, bool WARM>
__device__ __forceinline__ void decode_group(const DecodeParams& p, float* ys, float* red, int row,
                                             int g, uint8_t* page, int tid)
{
    using Sh = DecodeShape<DK, DV>;
    constexpr int JPL = Sh::JPL, RPI = Sh::RPI, LPR = Sh::LPR, NW = Sh::NW;
    const int G = p.Hv / p.Hk;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c4 = lane % LPR;                     // float4 column of the lane
    const int key0 = wave * Sh::KPW + lane / LPR;  // first key row; then every RPI rows
    const int h0 = g * G;
    uint16_t* out_row = p.out + (int64_t(row) * p.Hv + h0) * DV;
    float* ssm = reinterpret_cast<float*>(page + p.ssm_off);
    const __amdgpu_buffer_rsrc_t rs = state_rsrc(ssm, p.Hv * DK * DV * 4);
    const int voff = (key0 * DV + 4 * c4) * 4;
    uint16_t* win = reinterpret_cast<uint16_t*>(page + p.conv_off);
    const int C = p.C;

    // workgroup channel pair -> global channel: q of g | k of g | v of the group
    const int nvc = 2 * DK + G * DV;
    auto chan = [&](int vc) -> int {
        if (vc < DK)
            return g * DK + vc;
        if (vc < 2 * DK)
            return p.Hk * DK + g * DK + (vc - DK);
        return 2 * p.Hk * DK + h0 * DV + (vc - 2 * DK);
    };

    // 1. conv inputs of the first channel pair, then the state tiles of the
    //    first two heads: the conv runs while the tiles are in flight
    ConvPairIn<W> cin;
    const int vc0 = 2 * tid;
    const int c0 = chan(vc0 < nvc ? vc0 : 0);
    if (vc0 < nvc)
        load_conv_pair<W>(cin, p, row, c0, reinterpret_cast<const uint32_t*>(win + c0), WARM);
    f32x4 s0[JPL], s1[JPL];
    if constexpr (WARM) {
        load_tile<DK, DV, JPL, RPI>(s0, rs, voff, h0);
        if (G > 1)
            load_tile<DK, DV, JPL, RPI>(s1, rs, voff, h0 + 1);
    } else {
        zero_tile<JPL>(s0);
        zero_tile<JPL>(s1);
    }

    // 2. conv + SiLU; groups with more channels than 2 per thread loop on
    if (vc0 < nvc)
        finish_conv_pair<W>(cin, reinterpret_cast<uint32_t*>(win + c0), C, ys + vc0);
    for (int vc = vc0 + 2 * Sh::NT; vc < nvc; vc += 2 * Sh::NT) {
        const int c = chan(vc);
        ConvPairIn<W> in;
        load_conv_pair<W>(in, p, row, c, reinterpret_cast<const uint32_t*>(win + c), WARM);
        finish_conv_pair<W>(in, reinterpret_cast<uint32_t*>(win + c), C, ys + vc);
    }
    __syncthreads();

    // 3. L2 norms and k.q; every wave reduces redundantly.  The dot products
    //    below run on the raw conv outputs; the norm factors are applied to
    //    their sums.  The lane's raw k and q values stay in registers.
    float sq = 0.f, sk = 0.f, qk = 0.f;
    for (int j = lane; j < DK; j += 64) {
        const float a = ys[j], b = ys[DK + j];
        sq += a * a;
        sk += b * b;
        qk += a * b;
    }
    sq = group_sum<64>(sq);
    sk = group_sum<64>(sk);
    qk = group_sum<64>(qk);
    const float rq = p.scale / sqrtf(sq + p.eps);
    const float rk = 1.0f / sqrtf(sk + p.eps);
    const float kq = qk * rq * rk;
    float kr[JPL];
#pragma unroll
    for (int m = 0; m < JPL; ++m)
        kr[m] = ys[DK + key0 + RPI * m];

    // 4. the gated delta rule for a pair of v-heads (hh, hh+1) whose tiles
    //    are held in s0, s1: partial sums, one exchange, then the update
    auto partials = [&](const f32x4 (&s)[JPL], float* rh) {
        f32x4 u = f32x4{0.f, 0.f, 0.f, 0.f}, o = u;
#pragma unroll
        for (int m = 0; m < JPL; ++m) {
            u += s[m] * kr[m];
            o += s[m] * ys[key0 + RPI * m];
        }
        u.x = strided_sum<LPR>(u.x);
        u.y = strided_sum<LPR>(u.y);
        u.z = strided_sum<LPR>(u.z);
        u.w = strided_sum<LPR>(u.w);
        o.x = strided_sum<LPR>(o.x);
        o.y = strided_sum<LPR>(o.y);
        o.z = strided_sum<LPR>(o.z);
        o.w = strided_sum<LPR>(o.w);
        if (lane < LPR) {
            *reinterpret_cast<f32x4*>(rh + wave * DV + 4 * c4) = u;
            *reinterpret_cast<f32x4*>(rh + (NW + wave) * DV + 4 * c4) = o;
        }
    };
    auto finish = [&](const f32x4 (&s)[JPL], const float* rh, int hh) {
        const int h = h0 + hh;
        f32x4 u = f32x4{0.f, 0.f, 0.f, 0.f}, o = u;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            u += *reinterpret_cast<const f32x4*>(rh + w * DV + 4 * c4);
            o += *reinterpret_cast<const f32x4*>(rh + (NW + w) * DV + 4 * c4);
        }
        const float a = p.alpha[int64_t(row) * p.Hv + h];
        const float b = p.beta[int64_t(row) * p.Hv + h];
        const f32x4 v = *reinterpret_cast<const f32x4*>(ys + 2 * DK + hh * DV + 4 * c4);
        // d = b (v - a S k^), with k^ = rk k
        const f32x4 d = b * (v - (a * rk) * u);
        const f32x4 dk = d * rk; // update S <- a S + d k^T with raw k
#pragma unroll
        for (int m = 0; m < JPL; ++m)
            store_row<DK, DV, RPI>(a * s[m] + dk * kr[m], rs, voff, h, m);
        if (wave == 0 && lane < LPR) {
            // o = a S q^ + d (k^.q^), with q^ = rq q
            const f32x4 ov = (a * rq) * o + d * kq;
            *reinterpret_cast<uint2*>(out_row + hh * DV + 4 * c4) =
                pack_bf16x4(ov.x, ov.y, ov.z, ov.w);
        }
    };
    constexpr int RH = 2 * NW * DV; // floats of one head's partial sums
    for (int hh = 0; hh < G; hh += 2) {
        const bool pair = hh + 1 < G;
        if (hh > 0) { // the next pair's tiles; red is free again after the barrier
            if constexpr (WARM) {
                load_tile<DK, DV, JPL, RPI>(s0, rs, voff, h0 + hh);
                if (pair)
                    load_tile<DK, DV, JPL, RPI>(s1, rs, voff, h0 + hh + 1);
            }
            __syncthreads();
        }
        partials(s0, red);
        if (pair)
            partials(s1, red + RH);
        __syncthreads();
        finish(s0, red, hh);
        if (pair)
            finish(s1, red + RH, hh + 1);
    }
}

template <int DK, int DV, int W, int KPG>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT * KPG)) __attribute__((amdgpu_waves_per_eu(2)))
void decode_kernel(DecodeParams p)
{
    using Sh = DecodeShape<DK, DV>;
    // per k-head: conv outputs q (DK) | k (DK) | v (G*DV), then partial sums
    extern __shared__ float lds[];
    const int G = p.Hv / p.Hk;
    const int per_row = p.Hk / KPG; // workgroups per row
    const int row = blockIdx.x / per_row;
    const int g0 = (blockIdx.x - row * per_row) * KPG;
    const int slot = p.state_indices[row];
    if (slot < 0 || slot >= p.num_slots) { // padding row: zero output, no state I/O
        uint16_t* out_row = p.out + (int64_t(row) * p.Hv + g0 * G) * DV;
        for (int e = threadIdx.x; e < KPG * G * DV; e += KPG * Sh::NT)
            out_row[e] = 0;
        return;
    }
    const int sub = KPG > 1 ? int(threadIdx.x) / Sh::NT : 0;
    float* ys = lds + sub * (2 * DK + G * DV + 4 * Sh::NW * DV);
    uint8_t* page = p.layer + int64_t(slot) * p.page_stride;
    float* red = ys + 2 * DK + G * DV;
    const int tid = KPG > 1 ? int(threadIdx.x) % Sh::NT : int(threadIdx.x);
    if (p.hs[row] != 0)
        decode_group<DK, DV, W, true>(p, ys, red, row, g0 + sub, page, tid);
    else
        decode_group<DK, DV, W, false>(p, ys, red, row, g0 + sub, page, tid);
}

template <int DK, int DV, int W, int KPG>
int launch_decode_t(const gdn_pool* pool, int32_t layer, int32_t rows, const gdn_step_args* a,
                    hipStream_t stream)
{
    using Sh = DecodeShape<DK, DV>;
    const gdn_pool_desc& d = pool->desc;
    DecodeParams p;
    p.layer = static_cast<uint8_t*>(pool->bases[layer]);
    p.page_stride = d.page_stride_bytes;
    p.ssm_off = d.ssm_offset_bytes;
    p.conv_off = d.conv_offset_bytes;
    p.num_slots = int32_t(d.num_slots);
    p.C = d.conv_channels;
    p.Hk = d.num_k_heads;
    p.Hv = d.num_v_heads;
    p.x = a->x;
    p.conv_w = a->conv_w;
    p.conv_b = a->conv_b;
    p.alpha = a->alpha;
    p.beta = a->beta;
    p.state_indices = a->state_indices;
    p.hs = a->has_initial_state;
    p.out = a->out;
    p.scale = a->scale;
    p.eps = a->l2_eps;
    const int G = d.num_v_heads / d.num_k_heads;
    const size_t lds = sizeof(float) * size_t(KPG) * size_t(2 * DK + G * DV + 2 * 2 * Sh::NW * DV);
    const int64_t blocks = int64_t(rows) * (d.num_k_heads / KPG);
    if (blocks > INT32_MAX)
        return fail(GDN_ERANGE, "decode grid too large");
    hipLaunchKernelGGL((decode_kernel<DK, DV, W, KPG>), dim3(uint32_t(blocks)), dim3(Sh::NT * KPG),
                       lds, stream, p);
    return check_launch("decode");
}

// k-heads per workgroup.  A small head moves few bytes per k-head, and
// workgroups of 256 threads or fewer with 32 KiB or less each kept the HBM
// short of work; 512-thread workgroups ran fastest (512 MiB of state per step:
// head size 64 5.70 against 5.38 TB/s with one k-head per workgroup, 32 5.86
// against 5.40, 16 4.20 against 4.0; twice as many k-heads per workgroup was
// slower at every size).  A pool whose k-head count the choice does not
// divide takes one k-head per workgroup.
constexpr int kpg_for(int dk) { return dk == 64 ? 2 : dk == 32 ? 8 : dk == 16 ? 8 : 1; }

template <int DK, int KPG>
int dispatch_kpg(const gdn_pool* pool, int32_t layer, int32_t rows, const gdn_step_args* a,
                 hipStream_t stream)
{
    switch (pool->desc.conv_width) {
    case 2: return launch_decode_t<DK, DK, 2, KPG>(pool, layer, rows, a, stream);
    case 3: return launch_decode_t<DK, DK, 3, KPG>(pool, layer, rows, a, stream);
    case 4: return launch_decode_t<DK, DK, 4, KPG>(pool, layer, rows, a, stream);
    default: return fail(GDN_EUNSUPPORTED, "decode: conv width %d", pool->desc.conv_width);
    }
}

template <int DK>
int dispatch_w(const gdn_pool* pool, int32_t layer, int32_t rows, const gdn_step_args* a,
               hipStream_t stream)
{
    constexpr int K = kpg_for(DK);
    if (K > 1 && pool->desc.num_k_heads % K == 0)
        return dispatch_kpg<DK, K>(pool, layer, rows, a, stream);
    return dispatch_kpg<DK, 1>(pool, layer, rows, a, stream);
}

} // namespace

bool decode_supported(int dk, int dv, int W)
{
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128) && W >= 2 && W <= 4;
}

int launch_decode(const gdn_pool* pool, int32_t layer, int32_t rows, const gdn_step_args* a,
                  hipStream_t stream)
{
    switch (pool->desc.head_k_dim) {
    case 16: return dispatch_w<16>(pool, layer, rows, a, stream);
    case 32: return dispatch_w<32>(pool, layer, rows, a, stream);
    case 64: return dispatch_w<64>(pool, layer, rows, a, stream);
    case 128: return dispatch_w<128>(pool, layer, rows, a, stream);
    default: return fail(GDN_EUNSUPPORTED, "decode: head dim %d", pool->desc.head_k_dim);
    }
}

} // namespace gdn
