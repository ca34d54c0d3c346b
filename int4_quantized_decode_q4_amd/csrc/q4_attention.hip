// q4_attention.hip -- paged-attention decode for one token on gfx950: the
// attention step between the fused QKV projection and the output projection
// of a decoder layer, reading the paged K/V cache that step writes.
//
// Source: "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权"
// (zingnex.cn), section 内核融合 (attention merges paged attention with the
// page-table reads) and section 完整的推理流水线 (vLLM-style page table).
//
// Design (split over the context, as flash-decoding does for one query):
//  * a block owns one query head and a chunk of 256 positions (16 pages); its
//    4 wavefronts take 64 positions each, 16 at a time: 4 lanes per
//    position, each lane d/4 dims, so one step reads 16 whole K rows and 16
//    whole V rows of one page (the page index is uniform over the step);
//  * the next step's rows are requested before the current one is used;
//  * scores: f16 pairs through v_dot2_f32_f16, summed over the 4 lanes of a
//    position with DPP, times the caller's scale; an online softmax per
//    wavefront (running max and sum, the accumulator rescaled when the max
//    grows), exp in f32;
//  * the 4 wavefronts are combined in LDS; with one chunk the block writes
//    the f16 output, otherwise it writes (max, sum, weighted V) to the
//    workspace and a second launch combines the chunks.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "q4_internal.h"
#include "q4_lanes.h"

namespace q4 {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

constexpr int kChunk = 256;   // positions per block
constexpr int kStep = 16;     // positions per wavefront step

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float dot8(uint4 a, uint4 b, float acc)
{
    acc = __builtin_amdgcn_fdot2(as_h2(a.x), as_h2(b.x), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(a.y), as_h2(b.y), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(a.z), as_h2(b.z), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(a.w), as_h2(b.w), acc, false);
    return acc;
}

__device__ __forceinline__ void axpy8(float p, uint4 v, float *acc)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const h2 h = as_h2(w[i]);
        acc[2 * i] = fmaf(p, (float)h.x, acc[2 * i]);
        acc[2 * i + 1] = fmaf(p, (float)h.y, acc[2 * i + 1]);
    }
}

// DL = d / 32: 16-byte loads per lane per row (each lane d/4 dims).
template <int DL>
__global__ __launch_bounds__(256) void attention_decode_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ cache,
    const int32_t *__restrict__ page_table, int32_t n_pages, int32_t ctx, int32_t nq,
    int32_t nkv, float scale, uint16_t *__restrict__ out, float *__restrict__ partial)
{
    constexpr int D = 32 * DL;
    constexpr int LD = 8 * DL;   // dims per lane
    __shared__ float wm[4], wl[4];
    __shared__ float wacc[4][D];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int h = blockIdx.x % nq, chunk = blockIdx.x / nq;
    const int g = h / (nq / nkv);
    const int sub = lane & 3, slot = lane >> 2;
    const int64_t row_stride = (int64_t)nkv * D;   // halves between slots of a page

    uint4 qv[DL];
#pragma unroll
    for (int j = 0; j < DL; ++j)
        qv[j] = reinterpret_cast<const uint4 *>(q + (int64_t)h * D + sub * LD)[j];

    const int t_begin = chunk * kChunk + w * (kChunk / 4);
    const int t_end = min(t_begin + kChunk / 4, ctx);
    struct Rows {
        uint4 k[DL], v[DL];
        bool ok;
    };
    auto load = [&](Rows &r, int t0) {
        // t0 % 16 == 0: the step is one page; entries outside the cache read nothing
        r.ok = false;
        if (t0 < t_end) {
            const int32_t page = page_table[t0 >> 4];
            if (page >= 0 && page < n_pages) {
                r.ok = true;
                const uint16_t *base = cache + ((int64_t)page * 2 * 16 + slot) * row_stride +
                                       (int64_t)g * D + sub * LD;
                const uint4 *kp = reinterpret_cast<const uint4 *>(base);
                const uint4 *vp = reinterpret_cast<const uint4 *>(base + 16 * row_stride);
#pragma unroll
                for (int j = 0; j < DL; ++j) {
                    r.k[j] = kp[j];
                    r.v[j] = vp[j];
                }
            }
        }
    };

    float acc[LD];
#pragma unroll
    for (int i = 0; i < LD; ++i)
        acc[i] = 0.f;
    float m = -INFINITY, l = 0.f;
    Rows ra, rb;
    load(ra, t_begin);
    for (int t0 = t_begin; t0 < t_end; t0 += 2 * kStep) {
        load(rb, t0 + kStep);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            Rows &r = half == 0 ? ra : rb;
            const int ts = t0 + half * kStep;
            if (ts >= t_end)
                break;
            const int t = ts + slot;
            // slots past the context (or of an absent page) hold whatever the
            // cache holds there: their score is -inf and their V row zero
            const bool valid = r.ok && t < t_end;
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < DL; ++j)
                s = dot8(qv[j], r.k[j], s);
            s = lanes::reduce<4>(s) * scale;
            if (!valid)
                s = -INFINITY;
            const float smax = wave_max(s);
            if (smax != -INFINITY) {   // a step with nothing valid changes nothing
                const float mn = fmaxf(m, smax);
                const float alpha = expf(m - mn);   // 0 while m is still -inf
                const float p = valid ? expf(s - mn) : 0.f;
                // each position's p sits in its 4 lanes: count it once
                l = l * alpha + lanes::reduce<64>(sub == 0 ? p : 0.f);
#pragma unroll
                for (int i = 0; i < LD; ++i)
                    acc[i] *= alpha;
                const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int j = 0; j < DL; ++j)
                    axpy8(p, valid ? r.v[j] : zero, acc + 8 * j);
                m = mn;
            }
            if (half == 0)
                load(ra, t0 + 2 * kStep);
        }
    }
    // sum the 16 positions' accumulators (lanes with the same dim slice)
#pragma unroll
    for (int i = 0; i < LD; ++i) {
        float v = acc[i];
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[i] = v;
    }
    if (lane < 4) {
#pragma unroll
        for (int i = 0; i < LD; ++i)
            wacc[w][lane * LD + i] = acc[i];
    }
    if (lane == 0) {
        wm[w] = m;
        wl[w] = l;
    }
    __syncthreads();
    const float M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
    float e[4], L = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        e[i] = wm[i] == -INFINITY ? 0.f : expf(wm[i] - M);
        L += wl[i] * e[i];
    }
    for (int i = threadIdx.x; i < D; i += blockDim.x) {
        const float A = ((wacc[0][i] * e[0] + wacc[1][i] * e[1]) + wacc[2][i] * e[2]) + wacc[3][i] * e[3];
        if (partial == nullptr) {
            out[(int64_t)h * D + i] = __builtin_bit_cast(uint16_t, (_Float16)(A / L));
        } else {
            float *rec = partial + ((int64_t)h * gridDim.x / nq + chunk) * (D + 2);
            rec[2 + i] = A;
            if (i == 0) {
                rec[0] = M;
                rec[1] = L;
            }
        }
    }
}

// Combine the chunks of each head: out = sum A_s e^(M_s - M) / sum L_s e^(M_s - M).
__global__ __launch_bounds__(256) void attention_combine_kernel(const float *__restrict__ partial,
                                                                int32_t chunks, int32_t d,
                                                                uint16_t *__restrict__ out)
{
    const int h = blockIdx.x;
    const float *rec = partial + (int64_t)h * chunks * (d + 2);
    float M = -INFINITY;
    for (int c = 0; c < chunks; ++c)
        M = fmaxf(M, rec[(int64_t)c * (d + 2)]);
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        float num = 0.f, den = 0.f;
        for (int c = 0; c < chunks; ++c) {
            const float *r = rec + (int64_t)c * (d + 2);
            const float e = r[0] == -INFINITY ? 0.f : expf(r[0] - M);
            num += r[2 + i] * e;
            den += r[1] * e;
        }
        out[(int64_t)h * d + i] = __builtin_bit_cast(uint16_t, (_Float16)(num / den));
    }
}

template <int DL>
hipError_t launch_dl(const uint16_t *q, const uint16_t *cache, const int32_t *pt, int32_t n_pages,
                     int32_t ctx, int32_t nq, int32_t nkv, float scale, uint16_t *out, float *ws,
                     hipStream_t stream)
{
    const int chunks = (ctx + kChunk - 1) / kChunk;
    float *partial = chunks > 1 ? ws : nullptr;
    hipLaunchKernelGGL((attention_decode_kernel<DL>), dim3((unsigned)(nq * chunks)), dim3(256), 0,
                       stream, q, cache, pt, n_pages, ctx, nq, nkv, scale, out, partial);
    if (chunks > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(attention_combine_kernel, dim3((unsigned)nq), dim3(128), 0, stream,
                           ws, chunks, 32 * DL, out);
    }
    return hipGetLastError();
}

}  // namespace

int64_t attention_workspace_bytes(int64_t ctx, int64_t nq, int64_t d)
{
    const int64_t chunks = (ctx + kChunk - 1) / kChunk;
    return chunks > 1 ? nq * chunks * (d + 2) * 4 : 0;
}

hipError_t launch_attention(const uint16_t *q, const uint16_t *cache, const int32_t *page_table,
                            int32_t n_pages, int32_t ctx, int32_t nq, int32_t nkv, int32_t d,
                            float scale, uint16_t *out, void *ws, hipStream_t stream)
{
    float *w = static_cast<float *>(ws);
    switch (d / 32) {
    case 1: return launch_dl<1>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, w, stream);
    case 2: return launch_dl<2>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, w, stream);
    case 3: return launch_dl<3>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, w, stream);
    case 4: return launch_dl<4>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, w, stream);
    case 5: return launch_dl<5>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, w, stream);
    case 6: return launch_dl<6>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, w, stream);
    case 7: return launch_dl<7>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, w, stream);
    case 8: return launch_dl<8>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, w, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace q4
