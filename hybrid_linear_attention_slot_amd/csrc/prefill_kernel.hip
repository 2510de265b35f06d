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
// Parallel structure: every value row of a head's state evolves on its own
// once k, q, v, a, b of the token are known, so a workgroup takes one
// (sequence, v-head, slice of ISZ value rows).  Its waves never exchange
// partial sums: a wave owns 4*NCW value columns for all dk keys, the LPC
// lanes that share a float4 column split the keys, and S k / S q are finished
// with DPP sums inside the wave.  The sequence is processed in chunks of CT
// tokens:
//   A. stage the chunk's raw inputs of the workgroup's channels (q and k of
//      its k-head, v of its slice) into LDS with coalesced loads (as fp32);
//   B. conv + SiLU per channel, the W-1 previous inputs held in registers;
//   C. per token: L2 norms of q and k and k.q (one wave per token);
//   D. the serial recurrence over the chunk's tokens, reading k^, q^, v, a, b
//      from LDS; no barrier inside the chunk.
// The conv window is rewritten by a second small kernel after this one, so
// that no workgroup of a sequence can overwrite the window another workgroup
// of the same sequence has yet to read.
#include <algorithm>

#include "device_utils.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int DK, int DV>
struct PrefillShape {
    static constexpr int NCW = (DV / 4) < 4 ? (DV / 4) : 4;   // float4 columns per wave
    static constexpr int LPC = 64 / NCW;                      // lanes splitting one column's keys
    static constexpr int JPL = DK / LPC;                      // keys per lane
    static constexpr int NWP = (DV / (4 * NCW)) < 2 ? (DV / (4 * NCW)) : 2; // waves per workgroup
    static constexpr int ISZ = 4 * NCW * NWP;                 // value rows per workgroup
    static constexpr int NSL = DV / ISZ;                      // slices per head
    static constexpr int NT = 64 * NWP;
    static constexpr int NCH = 2 * DK + ISZ;                  // channels per workgroup
    static constexpr int CPT = (NCH + NT - 1) / NT;           // channel slots per thread
    static constexpr int CT = 32;                             // tokens per chunk
    static_assert(JPL >= 1 && DK % LPC == 0 && DV % ISZ == 0, "unsupported head dims");
};

struct PrefillParams {
    uint8_t* layer;
    int64_t page_stride;
    int64_t ssm_off;
    int64_t conv_off;
    int32_t num_slots;
    int32_t num_seqs;
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
    float scale;
    float eps;
};

template <int DK, int DV, int W>
__global__ __launch_bounds__((PrefillShape<DK, DV>::NT)) void prefill_kernel(PrefillParams p)
{
    using Sh = PrefillShape<DK, DV>;
    constexpr int JPL = Sh::JPL, LPC = Sh::LPC, NCH = Sh::NCH, CT = Sh::CT, NT = Sh::NT;
    // q | k | v-slice per token: raw inputs after phase A, conv outputs after
    // phase B (each thread reads and rewrites only its own channels), q and k
    // normalised in place by phase C
    __shared__ __align__(16) float ys[CT][NCH];
    __shared__ float s_kq[CT], s_a[CT], s_b[CT];

    const int nblocks = p.num_seqs * p.Hv * Sh::NSL;
    const int id = xcd_contiguous_id(blockIdx.x, nblocks);
    const int sl = id % Sh::NSL;
    const int h = (id / Sh::NSL) % p.Hv;
    const int n = id / (Sh::NSL * p.Hv);
    const int G = p.Hv / p.Hk;
    const int g = h / G;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int jl = lane % LPC;
    const int il = 4 * (wave * Sh::NCW + lane / LPC); // value column inside the slice
    const int i0 = sl * Sh::ISZ + il;                  // value column inside the head

    const int tb = p.cu[n];
    const int L = p.cu[n + 1] - tb;
    if (L <= 0)
        return;
    const int64_t out_stride = int64_t(p.Hv) * DV;
    uint16_t* out = p.out + int64_t(tb) * out_stride + int64_t(h) * DV + i0;
    const int slot = p.state_indices[n];
    if (slot < 0 || slot >= p.num_slots) { // padding row: zero outputs, no state I/O
        if (jl == 0)
            for (int t = 0; t < L; ++t)
                *reinterpret_cast<uint2*>(out + t * out_stride) = make_uint2(0u, 0u);
        return;
    }
    const bool warm = p.hs[n] != 0;
    uint8_t* page = p.layer + int64_t(slot) * p.page_stride;
    float* tile = reinterpret_cast<float*>(page + p.ssm_off) + int64_t(h) * DK * DV;
    const uint16_t* win = reinterpret_cast<const uint16_t*>(page + p.conv_off);

    // the workgroup's channel -> global conv channel
    auto chan = [&](int ch) -> int {
        if (ch < DK)
            return g * DK + ch;
        if (ch < 2 * DK)
            return p.Hk * DK + g * DK + (ch - DK);
        return 2 * p.Hk * DK + h * DV + sl * Sh::ISZ + (ch - 2 * DK);
    };

    // state slice into registers
    float4 s[JPL];
#pragma unroll
    for (int m = 0; m < JPL; ++m)
        s[m] = warm ? *reinterpret_cast<const float4*>(tile + (jl + LPC * m) * DV + i0)
                    : make_float4(0.f, 0.f, 0.f, 0.f);

    // per-thread conv channels: taps, bias and the last W-1 inputs
    float cw[Sh::CPT][W], cb[Sh::CPT], cwin[Sh::CPT][W > 1 ? W - 1 : 1];
#pragma unroll
    for (int k = 0; k < Sh::CPT; ++k) {
        const int ch = tid + k * NT;
        const int c = chan(ch < NCH ? ch : 0);
#pragma unroll
        for (int w = 0; w < W; ++w)
            cw[k][w] = bf16_to_f32(p.conv_w[int64_t(c) * W + w]);
        cb[k] = p.conv_b ? bf16_to_f32(p.conv_b[c]) : 0.f;
#pragma unroll
        for (int w = 0; w < W - 1; ++w)
            cwin[k][w] = warm ? bf16_to_f32(win[int64_t(w) * p.C + c]) : 0.f;
    }

    for (int t0 = 0; t0 < L; t0 += CT) {
        const int nt = min(CT, L - t0);
        // A. stage raw inputs
        for (int e = tid; e < nt * NCH; e += NT) {
            const int tt = e / NCH, ch = e - tt * NCH;
            ys[tt][ch] = bf16_to_f32(p.x[int64_t(tb + t0 + tt) * p.C + chan(ch)]);
        }
        if (tid < nt) {
            s_a[tid] = p.alpha[int64_t(tb + t0 + tid) * p.Hv + h];
            s_b[tid] = p.beta[int64_t(tb + t0 + tid) * p.Hv + h];
        }
        __syncthreads();
        // B. conv + SiLU
#pragma unroll
        for (int k = 0; k < Sh::CPT; ++k) {
            const int ch = tid + k * NT;
            if (ch < NCH) {
                for (int tt = 0; tt < nt; ++tt) {
                    const float xv = ys[tt][ch];
                    float acc = cb[k];
#pragma unroll
                    for (int w = 0; w < W - 1; ++w)
                        acc += cw[k][w] * cwin[k][w];
                    acc += cw[k][W - 1] * xv;
#pragma unroll
                    for (int w = 0; w + 1 < W - 1; ++w)
                        cwin[k][w] = cwin[k][w + 1];
                    cwin[k][W - 2] = xv;
                    ys[tt][ch] = silu(acc);
                }
            }
        }
        __syncthreads();
        // C. norms, one wave per token
        for (int tt = wave; tt < nt; tt += Sh::NWP) {
            float sq = 0.f, sk = 0.f, qk = 0.f;
            for (int j = lane; j < DK; j += 64) {
                const float a = ys[tt][j], b = ys[tt][DK + j];
                sq += a * a;
                sk += b * b;
                qk += a * b;
            }
            sq = group_sum<64>(sq);
            sk = group_sum<64>(sk);
            qk = group_sum<64>(qk);
            const float rq = p.scale / sqrtf(sq + p.eps);
            const float rk = 1.0f / sqrtf(sk + p.eps);
            for (int j = lane; j < DK; j += 64) {
                ys[tt][j] *= rq;
                ys[tt][DK + j] *= rk;
            }
            if (lane == 0)
                s_kq[tt] = qk * rq * rk;
        }
        __syncthreads();
        // D. recurrence
        for (int tt = 0; tt < nt; ++tt) {
            float kh[JPL], qh[JPL];
#pragma unroll
            for (int m = 0; m < JPL; ++m) {
                qh[m] = ys[tt][jl + LPC * m];
                kh[m] = ys[tt][DK + jl + LPC * m];
            }
            const float4 v = *reinterpret_cast<const float4*>(&ys[tt][2 * DK + il]);
            const float a = s_a[tt], b = s_b[tt], kq = s_kq[tt];
            float4 u = make_float4(0.f, 0.f, 0.f, 0.f), o = u;
#pragma unroll
            for (int m = 0; m < JPL; ++m) {
                u.x += s[m].x * kh[m];
                u.y += s[m].y * kh[m];
                u.z += s[m].z * kh[m];
                u.w += s[m].w * kh[m];
                o.x += s[m].x * qh[m];
                o.y += s[m].y * qh[m];
                o.z += s[m].z * qh[m];
                o.w += s[m].w * qh[m];
            }
            u.x = group_sum<LPC>(u.x);
            u.y = group_sum<LPC>(u.y);
            u.z = group_sum<LPC>(u.z);
            u.w = group_sum<LPC>(u.w);
            o.x = group_sum<LPC>(o.x);
            o.y = group_sum<LPC>(o.y);
            o.z = group_sum<LPC>(o.z);
            o.w = group_sum<LPC>(o.w);
            float4 d;
            d.x = b * (v.x - a * u.x);
            d.y = b * (v.y - a * u.y);
            d.z = b * (v.z - a * u.z);
            d.w = b * (v.w - a * u.w);
#pragma unroll
            for (int m = 0; m < JPL; ++m) {
                s[m].x = fmaf(d.x, kh[m], a * s[m].x);
                s[m].y = fmaf(d.y, kh[m], a * s[m].y);
                s[m].z = fmaf(d.z, kh[m], a * s[m].z);
                s[m].w = fmaf(d.w, kh[m], a * s[m].w);
            }
            if (jl == 0) {
                *reinterpret_cast<uint2*>(out + int64_t(t0 + tt) * out_stride) =
                    pack_bf16x4(fmaf(d.x, kq, a * o.x), fmaf(d.y, kq, a * o.y),
                                fmaf(d.z, kq, a * o.z), fmaf(d.w, kq, a * o.w));
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int m = 0; m < JPL; ++m)
        *reinterpret_cast<float4*>(tile + (jl + LPC * m) * DV + i0) = s[m];
}

// Final window of each sequence: the last W-1 entries of (old window, x).
struct WindowParams {
    uint8_t* layer;
    int64_t page_stride;
    int64_t conv_off;
    int32_t num_slots;
    int32_t C;
    int32_t W;
    const int32_t* cu;
    const uint16_t* x;
    const int32_t* state_indices;
    const uint8_t* hs;
};

constexpr int kWinThreads = 256;

__global__ __launch_bounds__(kWinThreads) void prefill_window_kernel(WindowParams p)
{
    const int cblocks = (p.C + kWinThreads - 1) / kWinThreads;
    const int n = blockIdx.x / cblocks;
    const int c = (blockIdx.x - n * cblocks) * kWinThreads + threadIdx.x;
    if (c >= p.C)
        return;
    const int tb = p.cu[n];
    const int L = p.cu[n + 1] - tb;
    const int slot = p.state_indices[n];
    if (L <= 0 || slot < 0 || slot >= p.num_slots)
        return;
    const bool warm = p.hs[n] != 0;
    uint16_t* win = reinterpret_cast<uint16_t*>(p.layer + int64_t(slot) * p.page_stride +
                                                p.conv_off);
    uint16_t nw[7];
#pragma unroll
    for (int w = 0; w < 7; ++w) {
        if (w < p.W - 1) {
            const int pos = L - (p.W - 1) + w; // position relative to the first token
            nw[w] = pos >= 0 ? p.x[int64_t(tb + pos) * p.C + c]
                             : (warm ? win[int64_t(p.W - 1 + pos) * p.C + c] : uint16_t(0));
        }
    }
#pragma unroll
    for (int w = 0; w < 7; ++w)
        if (w < p.W - 1)
            win[int64_t(w) * p.C + c] = nw[w];
}

template <int DK, int DV, int W>
int launch_prefill_t(const gdn_pool* pool, int32_t layer, int32_t num_seqs, const int32_t* cu,
                     const gdn_step_args* a, hipStream_t stream)
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
    w.cu = cu;
    w.x = a->x;
    w.state_indices = a->state_indices;
    w.hs = a->has_initial_state;
    const int64_t wblocks =
        int64_t(num_seqs) * ((d.conv_channels + kWinThreads - 1) / kWinThreads);
    if (wblocks > INT32_MAX)
        return fail(GDN_ERANGE, "prefill window grid too large");
    hipLaunchKernelGGL(prefill_window_kernel, dim3(uint32_t(wblocks)), dim3(kWinThreads), 0,
                       stream, w);
    return check_launch("prefill window");
}

template <int DK>
int dispatch_w(const gdn_pool* pool, int32_t layer, int32_t num_seqs, const int32_t* cu,
               const gdn_step_args* a, hipStream_t stream)
{
    switch (pool->desc.conv_width) {
    case 2: return launch_prefill_t<DK, DK, 2>(pool, layer, num_seqs, cu, a, stream);
    case 3: return launch_prefill_t<DK, DK, 3>(pool, layer, num_seqs, cu, a, stream);
    case 4: return launch_prefill_t<DK, DK, 4>(pool, layer, num_seqs, cu, a, stream);
    default: return fail(GDN_EUNSUPPORTED, "prefill: conv width %d", pool->desc.conv_width);
    }
}

} // namespace

bool prefill_supported(int dk, int dv, int W)
{
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128) && W >= 2 && W <= 4;
}

int launch_prefill(const gdn_pool* pool, int32_t layer, int32_t num_seqs, const int32_t* cu,
                   const gdn_step_args* a, hipStream_t stream)
{
    switch (pool->desc.head_k_dim) {
    case 16: return dispatch_w<16>(pool, layer, num_seqs, cu, a, stream);
    case 32: return dispatch_w<32>(pool, layer, num_seqs, cu, a, stream);
    case 64: return dispatch_w<64>(pool, layer, num_seqs, cu, a, stream);
    case 128: return dispatch_w<128>(pool, layer, num_seqs, cu, a, stream);
    default: return fail(GDN_EUNSUPPORTED, "prefill: head dim %d", pool->desc.head_k_dim);
    }
}

} // namespace gdn
