// q4_lanes.h -- cross-lane sums inside a 64-lane CDNA wavefront, shared by
// the GEMV and GEMM kernels of libq4 (device code only).
//
// The pages' "subgroup reduction" variant of the int4 matmul ("Zero-TVM：手写
// WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权", section 完整的推理流水线)
// adds per-lane partial sums across a subgroup; on gfx950 the cheapest
// exchanges are DPP inside a quad row, ds_swizzle inside a 32-lane half and
// one bpermute across the halves.
#ifndef Q4_LANES_H
#define Q4_LANES_H

#include <hip/hip_runtime.h>

namespace q4 {
namespace lanes {

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, false));
}

template <int XOR>
__device__ __forceinline__ float swizzle_xor(float v)
{
    // ds_swizzle bit-mask mode inside 32-lane halves: and 0x1F, or 0, xor XOR
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                 (XOR << 10) | 0x1F));
}

// Sum over aligned groups of L lanes (L a power of two <= 64); every lane of
// a group gets the sum.
template <int L>
__device__ __forceinline__ float reduce(float v)
{
    if (L >= 2)
        v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: xor 1
    if (L >= 4)
        v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: xor 2
    if (L >= 8)
        v += swizzle_xor<4>(v);
    if (L >= 16)
        v += swizzle_xor<8>(v);
    if (L >= 32)
        v += swizzle_xor<16>(v);
    if (L >= 64)
        v += __shfl_xor(v, 32);
    return v;
}

}  // namespace lanes
}  // namespace q4

#endif
