// Device helpers shared by the gfx950 kernels of the GDN state library:
// bf16 conversion, cross-lane sums over groups of consecutive lanes, and the
// SiLU.  Wavefronts are 64 lanes wide; a DPP "row" is 16 lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even; NaN becomes the quiet NaN 0x7FC0.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Four floats -> four bf16 packed in a uint2 (element 0 in the low half).
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d)
{
    uint2 r;
    r.x = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
    r.y = static_cast<uint32_t>(f32_to_bf16(c)) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
    return r;
}

// x * sigmoid(x) with the hardware reciprocal (about 1 ulp); for x -> -inf the
// exponential overflows to +inf and the result is -0.
__device__ __forceinline__ float silu(float x)
{
    return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// DPP lane permutations (all source lanes valid, so `old` is never used).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over each aligned group of N consecutive lanes (N in 2,4,...,64); every
// lane of the group gets the group's sum.  After the in-group steps below
// each lane already holds the sum of its aligned sub-group, so a mirror
// pairing is as good as an xor pairing for the next level.
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
    v += dpp_mov<kDppQuadXor1>(v);
    if constexpr (N >= 4)
        v += dpp_mov<kDppQuadXor2>(v);
    if constexpr (N >= 8)
        v += dpp_mov<kDppRowHalfMirror>(v);
    if constexpr (N >= 16)
        v += dpp_mov<kDppRowMirror>(v);
    if constexpr (N >= 32)
        v += __shfl_xor(v, 16, 64);
    if constexpr (N >= 64)
        v += __shfl_xor(v, 32, 64);
    return v;
}

constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// Sum over the whole wavefront as a wave-uniform value: sums within each row
// of 16 lanes, then rows 1 and 3 add the last lane of rows 0 and 2, then rows
// 2 and 3 add lane 31; lane 63 then holds the total and is read out.  Only
// DPP moves, no LDS permutes.
__device__ __forceinline__ float wave_total(float v)
{
    v = group_sum<16>(v);
    v += __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast15, 0xA, 0xF, false));
    v += __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast31, 0xC, 0xF, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Hardware dispatches workgroup b to XCD b % 8.  Renumber so that each XCD
// receives a contiguous run of logical ids (neighbours share its L2).
__device__ __forceinline__ int xcd_contiguous_id(int b, int nblocks)
{
    if (nblocks % 8 != 0)
        return b;
    return (b % 8) * (nblocks / 8) + b / 8;
}

} // namespace gdn
