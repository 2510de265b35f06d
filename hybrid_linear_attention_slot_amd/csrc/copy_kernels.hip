// Restore, gather and scatter of slot payloads (gfx950).
//
// Restore: the worker-side cross-layer copy of a checkpoint page into a live
// page ("Linear-State Prefix Cache 内部机制" §4, §4.3): for every layer that
// owns a state pool, the window and state payloads of page src are copied
// into page dst; attention-only layers have no pool and are skipped.
// Gather / scatter: indexed strided rows to dense rows and back
// ("非连续 KV Cache" §4, §5).  Only payload bytes move; the padding between
// the end of a payload and the next page is skipped by stride, never read or
// written ("非连续 KV Cache" §3.2-§3.4).
//
// The copies are HBM-bound.  Each workgroup of 1024 threads moves 128 KiB at
// a time: every lane issues eight 16-byte loads before its eight stores, so a
// wave keeps 8 KiB in flight and every load instruction of the workgroup reads
// 16 KiB of consecutive bytes (on the 48-layer restore this ran 10 % faster
// than 256-thread workgroups moving 32 KiB).  The restore launches one
// workgroup per 128 KiB chunk of each (pair, layer, region): tens of thousands
// of them, so the last partial round of the GPU's resident workgroups is a
// small share.  A gather or scatter call moves only one layer's rows (about a
// thousand chunks), so there every resident workgroup takes an equal
// contiguous share of the call's 16-byte units instead and all of them finish
// together.  Regions whose bytes are not a multiple of 16 (or dense rows not
// 16-byte aligned) use 2-byte element copies.
#include <algorithm>
#include <atomic>

#include "device_utils.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 1024;
constexpr int kCopyUnroll = 8;
constexpr int64_t kChunkBytes = int64_t(kCopyThreads) * kCopyUnroll * 16; // 128 KiB

constexpr int kMaxLayersPerLaunch = 64;
constexpr int kMaxPairsPerLaunch = 96;
constexpr int kMaxHsPerLaunch = 96;

// Copy chunk `chunk` of a `bytes`-long region (dst/src 16-byte aligned when
// `vec` is true; bytes always even).
__device__ __forceinline__ void copy_region_chunk(uint8_t* __restrict__ dst,
                                                  const uint8_t* __restrict__ src, int64_t bytes,
                                                  int64_t chunk, bool vec)
{
    const int64_t begin = chunk * kChunkBytes;
    const int64_t end = min(begin + kChunkBytes, bytes);
    if (vec) {
        const uint4* s = reinterpret_cast<const uint4*>(src);
        uint4* d = reinterpret_cast<uint4*>(dst);
        const int64_t u_end = end >> 4; // whole 16-byte units of this chunk
        if (end - begin == kChunkBytes) {
            // full chunk: all eight loads in flight before the first store
            // streamed once: non-temporal, all eight loads ahead of the stores
            const u32x4* sv = reinterpret_cast<const u32x4*>(src);
            u32x4* dv = reinterpret_cast<u32x4*>(dst);
            // each load instruction of the workgroup covers 16 KiB of consecutive
            // bytes (for long contiguous copies this order streams faster than
            // giving each wave its own part)
            const int64_t u0 = (begin >> 4) + threadIdx.x;
            u32x4 v[kCopyUnroll];
#pragma unroll
            for (int k = 0; k < kCopyUnroll; ++k)
                v[k] = __builtin_nontemporal_load(&sv[u0 + int64_t(k) * kCopyThreads]);
#pragma unroll
            for (int k = 0; k < kCopyUnroll; ++k)
                __builtin_nontemporal_store(v[k], &dv[u0 + int64_t(k) * kCopyThreads]);
            return;
        }
        for (int64_t u = (begin >> 4) + threadIdx.x; u < u_end; u += kCopyThreads)
            d[u] = s[u];
        // bytes past the last whole unit
        for (int64_t b = (u_end << 4) + 2 * threadIdx.x; b < end; b += 2 * kCopyThreads)
            *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
    } else {
        for (int64_t b = begin + 2 * threadIdx.x; b < end; b += 2 * kCopyThreads)
            *reinterpret_cast<uint16_t*>(dst + b) = *reinterpret_cast<const uint16_t*>(src + b);
    }
}

__device__ __forceinline__ void zero_region_chunk(uint8_t* __restrict__ dst, int64_t bytes,
                                                  int64_t chunk, bool vec)
{
    const int64_t begin = chunk * kChunkBytes;
    const int64_t end = min(begin + kChunkBytes, bytes);
    if (vec) {
        const int64_t u_end = end >> 4;
        uint4* d = reinterpret_cast<uint4*>(dst);
        for (int64_t u = (begin >> 4) + threadIdx.x; u < u_end; u += kCopyThreads)
            d[u] = make_uint4(0, 0, 0, 0);
        for (int64_t b = (u_end << 4) + 2 * threadIdx.x; b < end; b += 2 * kCopyThreads)
            *reinterpret_cast<uint16_t*>(dst + b) = 0;
    } else {
        for (int64_t b = begin + 2 * threadIdx.x; b < end; b += 2 * kCopyThreads)
            *reinterpret_cast<uint16_t*>(dst + b) = 0;
    }
}

// Two payload regions per page: 0 = state, 1 = window.
struct Regions {
    int64_t off[2];
    int64_t bytes[2];
    int32_t chunks[2]; // ceil(bytes / kChunkBytes)
};

// Everything a launch needs travels in the kernel arguments (no device
// allocation): at most 64 layers, 96 pairs and 96 hs entries per launch.
struct RestoreArgs {
    uint8_t* base[kMaxLayersPerLaunch];
    int32_t dst[kMaxPairsPerLaunch];
    int32_t src[kMaxPairsPerLaunch];
    int32_t hs_row[kMaxHsPerLaunch];
    uint8_t hs_val[kMaxHsPerLaunch];
    uint8_t* hs;
    int64_t page_stride;
    Regions r;
    int32_t n_layers;
    int32_t n_pairs;
    int32_t n_hs;
};
static_assert(sizeof(RestoreArgs) <= 4096, "kernel-argument budget");

// Grid: one workgroup per (pair, layer, region chunk); at least one.
__global__ __launch_bounds__(kCopyThreads) void restore_kernel(RestoreArgs a)
{
    if (blockIdx.x == 0 && threadIdx.x < a.n_hs)
        a.hs[a.hs_row[threadIdx.x]] = a.hs_val[threadIdx.x];
    const int per_pl = a.r.chunks[0] + a.r.chunks[1];
    if (per_pl == 0)
        return;
    const int pl = blockIdx.x / per_pl;
    if (pl >= a.n_pairs * a.n_layers)
        return;
    int chunk = blockIdx.x - pl * per_pl;
    const int pair = pl / a.n_layers;
    const int layer = pl - pair * a.n_layers;
    const int reg = chunk < a.r.chunks[0] ? 0 : 1;
    if (reg == 1)
        chunk -= a.r.chunks[0];
    uint8_t* base = a.base[layer];
    const uint8_t* from = base + int64_t(a.src[pair]) * a.page_stride + a.r.off[reg];
    uint8_t* to = base + int64_t(a.dst[pair]) * a.page_stride + a.r.off[reg];
    copy_region_chunk(to, from, a.r.bytes[reg], chunk, true);
}

struct RowCopyArgs {
    uint8_t* base;
    const int32_t* idx;
    uint8_t* dense[2]; // per region, [n][bytes]
    int64_t page_stride;
    int64_t num_slots;
    Regions r;
    int32_t n;
    int32_t vec[2]; // dense rows of the region are 16-byte aligned
};

template <bool kGather>
__global__ __launch_bounds__(kCopyThreads) void rows_kernel(RowCopyArgs a)
{
    const int per_row = a.r.chunks[0] + a.r.chunks[1];
    const int row = blockIdx.x / per_row;
    if (row >= a.n)
        return;
    int chunk = blockIdx.x - row * per_row;
    const int reg = chunk < a.r.chunks[0] ? 0 : 1;
    if (reg == 1)
        chunk -= a.r.chunks[0];
    const int64_t bytes = a.r.bytes[reg];
    uint8_t* dense = a.dense[reg] + int64_t(row) * bytes;
    const int32_t slot = a.idx[row];
    const bool valid = slot >= 0 && slot < a.num_slots;
    if (!valid) {
        if (kGather)
            zero_region_chunk(dense, bytes, chunk, a.vec[reg] != 0);
        return;
    }
    uint8_t* page = a.base + int64_t(slot) * a.page_stride + a.r.off[reg];
    if (kGather)
        copy_region_chunk(dense, page, bytes, chunk, a.vec[reg] != 0);
    else
        copy_region_chunk(page, dense, bytes, chunk, a.vec[reg] != 0);
}

// Copy n consecutive 16-byte units (n < 2^27) through buffer resources of
// exactly n units: whole 128 KiB blocks with eight loads in flight per lane
// ahead of the stores, then the remainder as one more block whose lanes past
// the end fall outside the resources (loads return zero, stores are dropped).
// The raw buffer intrinsics leave the SGPR offset out of the range check (it
// covers the VGPR offset), so every access of the remainder carries its whole
// offset in the VGPR; the whole blocks' loads, always in range, take the
// block offset in an SGPR.
// Stores always take their whole offset in the VGPR (a 128-bit store with an
// SGPR offset can read its data registers after a later write to them).
// The remainder is not guarded round by round: behind a branch per round the
// compiler waited for every earlier memory operation, stores included, before
// each store, which serialised the remainder's stores and made each call's
// last workgroups finish late (gather / scatter 1.5-2 % slower).
constexpr int kBufferWord3 = 0x00020000; // raw 32-bit buffer resource, gfx9-family layout
constexpr int kNonTemporal = 2;          // cache-policy bit: streamed once
constexpr int kDeviceNonTemporal = 16 | kNonTemporal; // SC1 | NT
constexpr int64_t kMaxPieceUnits = int64_t(1) << 27; // 2 GiB per buffer resource

// A wave-uniform value the compiler computed in vector registers (64-bit
// division is vector code) moved to scalar registers, so that buffer resources
// built from it need no loop over distinct values.
__device__ __forceinline__ int64_t uniform64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v)));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
    return int64_t((uint64_t(hi) << 32) | lo);
}

template <int kStorePolicy>
__device__ __forceinline__ void copy_units(uint8_t* dst, const uint8_t* src, int64_t n)
{
    constexpr int kBlockUnits = kCopyThreads * kCopyUnroll;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(src), short(0), int(n * 16), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rd =
        __builtin_amdgcn_make_buffer_rsrc(dst, short(0), int(n * 16), kBufferWord3);
    const int lane = int(threadIdx.x) * 16;
    const int ni = int(n);
    int i = 0;
    for (; i + kBlockUnits <= ni; i += kBlockUnits) {
        u32x4 v[kCopyUnroll];
#pragma unroll
        for (int k = 0; k < kCopyUnroll; ++k)
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane, (i + k * kCopyThreads) * 16,
                                                         kNonTemporal);
#pragma unroll
        for (int k = 0; k < kCopyUnroll; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(v[k], rd, lane + (i + k * kCopyThreads) * 16,
                                                   0, kStorePolicy);
    }
    if (i == ni)
        return;
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int k = 0; k < kCopyUnroll; ++k)
        v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane + (i + k * kCopyThreads) * 16, 0,
                                                     kNonTemporal);
#pragma unroll
    for (int k = 0; k < kCopyUnroll; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(v[k], rd, lane + (i + k * kCopyThreads) * 16, 0,
                                               kStorePolicy);
}

template <int kStorePolicy>
__device__ __forceinline__ void zero_units(uint8_t* dst, int64_t n)
{
    const __amdgpu_buffer_rsrc_t rd =
        __builtin_amdgcn_make_buffer_rsrc(dst, short(0), int(n * 16), kBufferWord3);
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int j = int(threadIdx.x); j < int(n); j += kCopyThreads)
        __builtin_amdgcn_raw_buffer_store_b128(z, rd, j * 16, 0, kStorePolicy);
}

// Gather / scatter with 16-byte aligned regions and dense rows.  The call's
// units are numbered row by row (row r: its state units, then its window
// units); workgroup w of the grid takes units [U w / G, U (w + 1) / G) and
// walks the (row, region) pieces they cover.  All indices are wave-uniform.
// Stores are non-temporal at device scope (SC1 | NT): over alternating runs of
// the 64-page calls on 48 layers, each layer with dense rows of its own, a
// gather ran 1-2 % and a scatter about 1.5 % faster than with NT alone.
template <bool kGather>
__global__ __launch_bounds__(kCopyThreads) void rows_balanced_kernel(RowCopyArgs a)
{
    const int64_t us = a.r.bytes[0] >> 4, uw = a.r.bytes[1] >> 4;
    const int64_t upr = us + uw; // units per row
    const int64_t total = upr * a.n;
    constexpr int kStorePolicy = kDeviceNonTemporal;
    const int64_t end = total * (blockIdx.x + 1) / gridDim.x;
    int64_t u = total * blockIdx.x / gridDim.x;
    while (u < end) {
        const int64_t row = u / upr;
        const int64_t ur = u - row * upr;
        const int reg = ur < us ? 0 : 1;
        const int64_t off = reg == 0 ? ur : ur - us;         // units into the region
        const int64_t len =
            uniform64(min(min(end - u, (reg == 0 ? us : uw) - off), kMaxPieceUnits));
        uint8_t* dense = reinterpret_cast<uint8_t*>(uniform64(
            reinterpret_cast<int64_t>(a.dense[reg] + row * a.r.bytes[reg] + off * 16)));
        const int32_t slot = __builtin_amdgcn_readfirstlane(a.idx[uniform64(row)]);
        if (slot >= 0 && slot < a.num_slots) {
            uint8_t* page = reinterpret_cast<uint8_t*>(uniform64(reinterpret_cast<int64_t>(
                a.base + int64_t(slot) * a.page_stride + a.r.off[reg] + off * 16)));
            if (kGather)
                copy_units<kStorePolicy>(dense, page, len);
            else
                copy_units<kStorePolicy>(page, dense, len);
        } else if (kGather) {
            zero_units<kStorePolicy>(dense, len);
        }
        u += len;
    }
}

// Workgroups of `kernel` the device can hold at once (CUs x occupancy),
// looked up once per device.
int resident_copy_workgroups(const void* kernel)
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
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kCopyThreads, 0) !=
            hipSuccess)
        return 0;
    const int r = std::max(1, cus) * std::max(1, per_cu);
    if (dev < 64)
        cache[dev].store(r, std::memory_order_relaxed);
    return r;
}

Regions regions_of(const gdn_pool* pool)
{
    Regions r;
    r.off[0] = pool->desc.ssm_offset_bytes;
    r.bytes[0] = pool->ssm_bytes;
    r.off[1] = pool->desc.conv_offset_bytes;
    r.bytes[1] = pool->conv_bytes;
    for (int k = 0; k < 2; ++k)
        r.chunks[k] = int32_t((r.bytes[k] + kChunkBytes - 1) / kChunkBytes);
    return r;
}

int launch_rows(bool gather, const gdn_pool* pool, int32_t layer, const int32_t* idx, int32_t n,
                const void* ssm_dense, const void* conv_dense, hipStream_t stream)
{
    RowCopyArgs a;
    a.base = static_cast<uint8_t*>(pool->bases[layer]);
    a.idx = idx;
    a.dense[0] = static_cast<uint8_t*>(const_cast<void*>(ssm_dense));
    a.dense[1] = static_cast<uint8_t*>(const_cast<void*>(conv_dense));
    a.page_stride = pool->desc.page_stride_bytes;
    a.num_slots = pool->desc.num_slots;
    a.r = regions_of(pool);
    a.n = n;
    for (int k = 0; k < 2; ++k)
        a.vec[k] = ((reinterpret_cast<uintptr_t>(a.dense[k]) & 15u) == 0 && (a.r.bytes[k] & 15) == 0)
                       ? 1
                       : 0;
    const int64_t per_row = a.r.chunks[0] + a.r.chunks[1];
    const int64_t blocks = per_row * n;
    if (blocks == 0)
        return GDN_OK;
    if (a.vec[0] && a.vec[1]) {
        // balanced: two resident rounds of workgroups (the second round fills
        // the slots the first frees, which evens out the finish; one round, or
        // three or four, ran 3-6 % slower), none with less than one 128 KiB
        // block of work
        const void* k = gather ? reinterpret_cast<const void*>(&rows_balanced_kernel<true>)
                               : reinterpret_cast<const void*>(&rows_balanced_kernel<false>);
        const int resident = resident_copy_workgroups(k);
        if (resident <= 0)
            return fail(GDN_EHIP, "cannot query the device's workgroup capacity");
        const int64_t units = (a.r.bytes[0] + a.r.bytes[1]) / 16 * n;
        const int64_t per_block = int64_t(kCopyThreads) * kCopyUnroll;
        const int64_t grid = std::max<int64_t>(
            1, std::min<int64_t>(2 * int64_t(resident), (units + per_block - 1) / per_block));
        if (gather)
            hipLaunchKernelGGL(rows_balanced_kernel<true>, dim3(uint32_t(grid)),
                               dim3(kCopyThreads), 0, stream, a);
        else
            hipLaunchKernelGGL(rows_balanced_kernel<false>, dim3(uint32_t(grid)),
                               dim3(kCopyThreads), 0, stream, a);
        return check_launch(gather ? "gather" : "scatter");
    }
    if (blocks > INT32_MAX)
        return fail(GDN_ERANGE, "too many rows for one launch");
    if (gather)
        hipLaunchKernelGGL(rows_kernel<true>, dim3(uint32_t(blocks)), dim3(kCopyThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(rows_kernel<false>, dim3(uint32_t(blocks)), dim3(kCopyThreads), 0,
                           stream, a);
    return check_launch(gather ? "gather" : "scatter");
}

} // namespace

int launch_restore(const gdn_pool* pool, const std::vector<HitPair>& pairs,
                   const std::vector<HsWrite>& hs, uint8_t* hs_dev, hipStream_t stream)
{
    const Regions r = regions_of(pool);
    const std::vector<int32_t>& layers = pool->linear;
    const size_t n_layer_chunks =
        std::max<size_t>(1, (layers.size() + kMaxLayersPerLaunch - 1) / kMaxLayersPerLaunch);
    const size_t n_pair_chunks =
        std::max<size_t>(1, (pairs.size() + kMaxPairsPerLaunch - 1) / kMaxPairsPerLaunch);
    const size_t n_hs_chunks = (hs.size() + kMaxHsPerLaunch - 1) / kMaxHsPerLaunch;
    // Launch (pair chunk p, layer chunk q); the hs writes ride on the first
    // launches, and extra launches carry any hs writes left over.
    size_t hs_next = 0;
    const size_t n_launches = std::max(n_pair_chunks * n_layer_chunks, n_hs_chunks);
    for (size_t k = 0; k < n_launches; ++k) {
        RestoreArgs a = {};
        a.page_stride = pool->desc.page_stride_bytes;
        a.r = r;
        a.hs = hs_dev;
        const size_t p = k / n_layer_chunks, q = k % n_layer_chunks;
        if (p < n_pair_chunks && !pairs.empty() && !layers.empty()) {
            const size_t p0 = p * kMaxPairsPerLaunch;
            a.n_pairs = int32_t(std::min<size_t>(kMaxPairsPerLaunch, pairs.size() - p0));
            for (int i = 0; i < a.n_pairs; ++i) {
                a.dst[i] = pairs[p0 + i].dst;
                a.src[i] = pairs[p0 + i].src;
            }
            const size_t l0 = q * kMaxLayersPerLaunch;
            a.n_layers = int32_t(std::min<size_t>(kMaxLayersPerLaunch, layers.size() - l0));
            for (int i = 0; i < a.n_layers; ++i)
                a.base[i] = static_cast<uint8_t*>(pool->bases[layers[l0 + i]]);
        }
        a.n_hs = int32_t(std::min<size_t>(kMaxHsPerLaunch, hs.size() - hs_next));
        for (int i = 0; i < a.n_hs; ++i) {
            a.hs_row[i] = hs[hs_next + i].row;
            a.hs_val[i] = uint8_t(hs[hs_next + i].value);
        }
        hs_next += a.n_hs;
        const int64_t blocks =
            std::max<int64_t>(1, int64_t(a.n_pairs) * a.n_layers * (r.chunks[0] + r.chunks[1]));
        if (a.n_pairs == 0 && a.n_hs == 0)
            continue;
        if (blocks > INT32_MAX)
            return fail(GDN_ERANGE, "restore grid too large");
        hipLaunchKernelGGL(restore_kernel, dim3(uint32_t(blocks)), dim3(kCopyThreads), 0, stream,
                           a);
        int rc = check_launch("restore");
        if (rc != GDN_OK)
            return rc;
    }
    return GDN_OK;
}

int launch_gather(const gdn_pool* pool, int32_t layer, const int32_t* idx, int32_t n,
                  void* ssm_dense, void* conv_dense, hipStream_t stream)
{
    return launch_rows(true, pool, layer, idx, n, ssm_dense, conv_dense, stream);
}

int launch_scatter(const gdn_pool* pool, int32_t layer, const int32_t* idx, int32_t n,
                   const void* ssm_dense, const void* conv_dense, hipStream_t stream)
{
    return launch_rows(false, pool, layer, idx, n, ssm_dense, conv_dense, stream);
}

} // namespace gdn
