// q4_merge.h -- merging the per-chunk attention records of one head (device
// code only), shared by the chunk-combine kernel of the paged attention and
// by the matmul that takes the merged attention output as its x, so both
// produce the same bits.
//
// Source: "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权"
// (zingnex.cn), section 内核融合 (attention over the paged cache; the split
// over the context and the merge of its parts is this library's design).
//
// A chunk record is (M, L, A[d]) in f32: M the chunk's largest score in base-2
// units, L = sum_t 2^(s_t - M), A[i] = sum_t 2^(s_t - M) V_t[i].  Records are
// stored [head][chunk][d + 2].
#ifndef Q4_MERGE_H
#define Q4_MERGE_H

#include <hip/hip_runtime.h>
#include <math.h>

namespace q4 {

// 2^x in f32 (v_exp_f32; 2^-inf = 0).
__device__ __forceinline__ float exp2_f32(float x) { return __builtin_amdgcn_exp2f(x); }

// Fold chunk record (mc, lc, ac) into the running (m, l, a) of one output
// element: the state of the union of their positions.  Explicit fmaf, so the
// rounding does not depend on how a compiler contracts each call site.
__device__ __forceinline__ void merge_record(float &m, float &l, float &a, float mc, float lc,
                                             float ac)
{
    const float mn = fmaxf(m, mc);
    const float e1 = m == -INFINITY ? 0.f : exp2_f32(m - mn);
    const float e2 = mc == -INFINITY ? 0.f : exp2_f32(mc - mn);
    l = fmaf(l, e1, lc * e2);
    a = fmaf(a, e1, ac * e2);
    m = mn;
}

// The merged output, rounded once to f16 (a head with no position: 0/0 = NaN).
__device__ __forceinline__ uint16_t merged_f16(float l, float a)
{
    return __builtin_bit_cast(uint16_t, (_Float16)(a / l));
}

}  // namespace q4

#endif
