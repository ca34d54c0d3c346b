// q4_kernels.hip -- gfx950 kernels of libq4: repacking, and the int4
// dequantizing GEMV family (plain f16 output, f32 LM-head output with argmax,
// fused gate/up SiLU).
//
// Sources: "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权"
// (zingnex.cn), section 完整的推理流水线 (the int4 dequantizing matmul and its
// variants: rows-per-invocation tiling, subgroup reduction, f32 LM head; the
// greedy argmax) and section 内核融合 (gate + up + SiLU in one pass).  The
// WGSL kernels there were written for browser GPUs; what is kept is the
// structure (several rows per invocation so x is reused, a cross-lane
// reduction, fused epilogues), re-designed for 64-lane CDNA4 wavefronts.
//
// GEMV design (one 64-lane wavefront per tile of TR = 128/L rows):
//   * lane (s, c) = (lane / L, lane % L) owns rows 2s, 2s+1 of the tile and CG
//     fixed groups of 32 k; its slice of x is loaded once per wavefront into
//     VGPRs (x-stationary), pre-paired to match the dequant below;
//   * per pass, the wavefront issues 2*CG fully coalesced 1 KiB loads of codes
//     (one 16-byte unit per lane each) plus one load of the lane's 2*CG scales;
//   * dequant in registers: (w & 0x000F000F) | 0x64006400 reinterpreted as two
//     f16 is (1024 + q_a, 1024 + q_b) exactly; subtracting 1032 gives q - 8
//     exactly.  The 0x00F000F0 mask gives 16*q without a shift and is offset
//     by 1152, so one word needs 1 shift + 4 and-or + 4 packed subtracts + 4
//     v_dot2_f32_f16; the x16 products go to their own f32 sum, scaled by
//     1/16 (exact) once per group; the group sum is scaled by the f16 scale in
//     f32.  Products of f16 x and small integers are exact in f32;
//   * the L lanes of a row are reduced with DPP (xor 1, 2), ds_swizzle (xor 4,
//     8, 16) and one bpermute (xor 32); every lane ends with the same sum.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "q4_geometry.h"
#include "q4_internal.h"

namespace q4 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

__device__ __forceinline__ uint16_t f16_bits(float v)
{
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

__device__ __forceinline__ float f16_value(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}

// ---------------------------------------------------------------- packing --

// One thread per destination 16-byte code unit (and the scale beside it):
// a pure permutation of the canonical words, padding where the logical
// (row, group) lies outside the matrix.
__global__ void pack_kernel(const uint32_t *__restrict__ w0, const uint16_t *__restrict__ s0,
                            const uint32_t *__restrict__ w1, const uint16_t *__restrict__ s1,
                            int64_t rows, int64_t k, int gate_up, int L, int CG, int P,
                            int64_t units, uint8_t *__restrict__ dst)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= units)
        return;
    const int lane = (int)(idx & 63);
    int64_t rest = idx >> 6;
    const int uj = (int)(rest % (2 * CG));
    rest /= 2 * CG;
    const int p = (int)(rest % P);
    const int64_t t = rest / P;
    const int u = uj / CG, j = uj % CG;
    const int s = lane / L, c = lane % L;
    const int64_t TR = 128 / L;
    const int64_t r = t * TR + 2 * s + u;
    const int64_t G = k / 32;
    const int64_t g = (int64_t)p * L * CG + (int64_t)c * CG + j;

    uint4 words = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
    uint16_t scale = 0;
    if (r < rows && g < G) {
        const uint32_t *sw = w0;
        const uint16_t *ss = s0;
        int64_t row = r;
        if (gate_up) {
            row = r >> 1;
            sw = (r & 1) ? w1 : w0;
            ss = (r & 1) ? s1 : s0;
        }
        words = *reinterpret_cast<const uint4 *>(sw + row * (k / 8) + 4 * g);
        scale = ss[row * G + g];
    }
    uint8_t *base = dst + (t * P + p) * (int64_t)CG * 2304;
    *reinterpret_cast<uint4 *>(base + (int64_t)uj * 1024 + lane * 16) = words;
    *reinterpret_cast<uint16_t *>(base + (int64_t)2 * CG * 1024 + lane * 4 * CG + uj * 2) = scale;
}

// One thread per logical (row, group) of the real matrix.
__global__ void unpack_kernel(const uint8_t *__restrict__ src, int64_t rows, int64_t k,
                              int L, int CG, int P, uint32_t *__restrict__ words,
                              uint16_t *__restrict__ scales)
{
    const int64_t G = k / 32;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * G)
        return;
    const int64_t r = idx / G, g = idx % G;
    const int64_t TR = 128 / L;
    const int64_t t = r / TR;
    const int s = (int)((r % TR) >> 1), u = (int)(r & 1);
    const int64_t p = g / ((int64_t)L * CG);
    const int c = (int)((g % ((int64_t)L * CG)) / CG), j = (int)(g % CG);
    const int lane = s * L + c;
    const uint8_t *base = src + (t * P + p) * (int64_t)CG * 2304;
    const uint4 v = *reinterpret_cast<const uint4 *>(base + (int64_t)(u * CG + j) * 1024 + lane * 16);
    *reinterpret_cast<uint4 *>(words + r * (k / 8) + 4 * g) = v;
    scales[r * G + g] =
        *reinterpret_cast<const uint16_t *>(base + (int64_t)2 * CG * 1024 + lane * 4 * CG + (u * CG + j) * 2);
}

// ----------------------------------------------------------- GEMV family --

// x pairs for one group of 32 k, ordered per word of codes as
// (x0,x4) (x1,x5) (x2,x6) (x3,x7) to match dot_word's nibble pairs.
__device__ __forceinline__ void load_x_group(uint32_t *xp, const uint16_t *__restrict__ x,
                                             int64_t g, int64_t G)
{
    if (g >= G) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            xp[i] = 0u;
        return;
    }
    const uint4 *src = reinterpret_cast<const uint4 *>(x + g * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // q = word of codes, 8 k each
        const uint4 n = src[q];    // natural pairs (x0,x1) (x2,x3) (x4,x5) (x6,x7)
        xp[4 * q + 0] = (n.x & 0xFFFFu) | (n.z << 16);
        xp[4 * q + 1] = (n.x >> 16) | (n.z & 0xFFFF0000u);
        xp[4 * q + 2] = (n.y & 0xFFFFu) | (n.w << 16);
        xp[4 * q + 3] = (n.y >> 16) | (n.w & 0xFFFF0000u);
    }
}

// 8 codes (canonical nibble order) against their 4 prepared x pairs.
__device__ __forceinline__ void dot_word(uint32_t w, const uint32_t *xp, float &p1, float &p16)
{
    const h2 k1 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 k16 = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t a0 = (w & 0x000F000Fu) | 0x64006400u;   // 1024 + q0, 1024 + q4
    const uint32_t a1 = (w & 0x00F000F0u) | 0x64006400u;   // 1024 + 16 q1, 1024 + 16 q5
    const uint32_t b = w >> 8;
    const uint32_t a2 = (b & 0x000F000Fu) | 0x64006400u;   // q2, q6
    const uint32_t a3 = (b & 0x00F000F0u) | 0x64006400u;   // 16 q3, 16 q7
    p1 = __builtin_amdgcn_fdot2(as_h2(a0) - k1, as_h2(xp[0]), p1, false);
    p16 = __builtin_amdgcn_fdot2(as_h2(a1) - k16, as_h2(xp[1]), p16, false);
    p1 = __builtin_amdgcn_fdot2(as_h2(a2) - k1, as_h2(xp[2]), p1, false);
    p16 = __builtin_amdgcn_fdot2(as_h2(a3) - k16, as_h2(xp[3]), p16, false);
}

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

// Sum over aligned groups of L lanes; every lane of a group gets the sum.
template <int L>
__device__ __forceinline__ float reduce_lanes(float v)
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

__device__ __forceinline__ void better(float &bv, int &bi, float ov, int oi)
{
    if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
    }
}

__device__ __forceinline__ void wave_argmax(float &bv, int &bi)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        better(bv, bi, ov, oi);
    }
}

// Block-wide (max, lowest index) of per-thread candidates; result in thread 0.
__device__ void block_argmax(float &bv, int &bi, float *sv, int *si)
{
    wave_argmax(bv, bi);
    const int wid = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sv[wid] = bv;
        si[wid] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0)
        for (int w = 1; w < nwaves; ++w)
            better(bv, bi, sv[w], si[w]);
    __syncthreads();
}

__device__ __forceinline__ unsigned long long pack_vi(float v, int i)
{
    return (unsigned long long)__builtin_bit_cast(unsigned int, v) |
           ((unsigned long long)(unsigned int)i << 32);
}

// Argmax across blocks: each block publishes its candidate, the last block
// to arrive combines all of them in index order and resets the counter.
__device__ void grid_argmax(float bv, int bi, ArgmaxScratch am)
{
    __shared__ float sv[16];
    __shared__ int si[16];
    __shared__ int is_last;
    block_argmax(bv, bi, sv, si);
    if (threadIdx.x == 0) {
        __hip_atomic_store(am.partials + blockIdx.x, pack_vi(bv, bi), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __threadfence();
        const unsigned prev = atomicAdd(am.counter, 1u);
        is_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!is_last)
        return;
    __threadfence();
    float v = -INFINITY;
    int i = 0x7fffffff;
    for (unsigned b = threadIdx.x; b < gridDim.x; b += blockDim.x) {
        const unsigned long long pv =
            __hip_atomic_load(am.partials + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        better(v, i, __builtin_bit_cast(float, (unsigned int)(pv & 0xFFFFFFFFull)),
               (int)(unsigned int)(pv >> 32));
    }
    block_argmax(v, i, sv, si);
    if (threadIdx.x == 0) {
        *am.result = i;
        __hip_atomic_store(am.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// rows: logical rows of the layout (gate/up: 2 * n_out); n_out: output length.
template <int L, int CG, int EPI>
__global__ __launch_bounds__(256) void gemv_family_kernel(
    const uint8_t *__restrict__ wd, const uint16_t *__restrict__ x, void *__restrict__ out,
    int64_t rows, int64_t k, int passes, int64_t tiles, int64_t n_out, ArgmaxScratch am)
{
    constexpr int TR = 128 / L;
    constexpr int64_t PB = (int64_t)CG * 2304;
    const int lane = threadIdx.x & 63;
    const int s = lane / L, c = lane % L;
    const int64_t G = k >> 5;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t wave0 = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);

    uint32_t xp[CG][16];
    int have_pass = -1;
    float bv = -INFINITY;
    int bi = 0x7fffffff;

    for (int64_t t = wave0; t < tiles; t += nwaves) {
        float acc[2] = {0.f, 0.f};
        for (int p = 0; p < passes; ++p) {
            if (p != have_pass) {
#pragma unroll
                for (int j = 0; j < CG; ++j)
                    load_x_group(xp[j], x, (int64_t)p * L * CG + (int64_t)c * CG + j, G);
                have_pass = p;
            }
            const uint8_t *base = wd + (t * passes + p) * PB;
            uint4 cu[2][CG];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < CG; ++j)
                    cu[u][j] = *reinterpret_cast<const uint4 *>(base + (u * CG + j) * 1024 + lane * 16);
            uint32_t sc[CG];
            const uint32_t *sp = reinterpret_cast<const uint32_t *>(base + 2 * CG * 1024 + lane * 4 * CG);
#pragma unroll
            for (int j = 0; j < CG; ++j)
                sc[j] = sp[j];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < CG; ++j) {
                    float p1 = 0.f, p16 = 0.f;
                    dot_word(cu[u][j].x, &xp[j][0], p1, p16);
                    dot_word(cu[u][j].y, &xp[j][4], p1, p16);
                    dot_word(cu[u][j].z, &xp[j][8], p1, p16);
                    dot_word(cu[u][j].w, &xp[j][12], p1, p16);
                    const int e = u * CG + j;
                    const float sv = f16_value((uint16_t)(sc[e >> 1] >> ((e & 1) * 16)));
                    acc[u] = fmaf(sv, fmaf(p16, 0.0625f, p1), acc[u]);
                }
        }
        const float y0 = reduce_lanes<L>(acc[0]);
        const float y1 = reduce_lanes<L>(acc[1]);
        const int64_t r0 = t * TR + 2 * s;   // even
        if (c == 0) {
            if (EPI == EPI_F16) {
                uint16_t *y = static_cast<uint16_t *>(out);
                if (r0 + 1 < rows)
                    *reinterpret_cast<uint32_t *>(y + r0) =
                        (uint32_t)f16_bits(y0) | ((uint32_t)f16_bits(y1) << 16);
                else if (r0 < rows)
                    y[r0] = f16_bits(y0);
            } else if (EPI == EPI_F32) {
                float *y = static_cast<float *>(out);
                if (r0 + 1 < rows) {
                    *reinterpret_cast<float2 *>(y + r0) = make_float2(y0, y1);
                    better(bv, bi, y0, (int)r0);
                    better(bv, bi, y1, (int)r0 + 1);
                } else if (r0 < rows) {
                    y[r0] = y0;
                    better(bv, bi, y0, (int)r0);
                }
            } else {  // EPI_SILU: logical rows (2i, 2i+1) = (gate i, up i)
                const int64_t i = r0 >> 1;
                if (i < n_out) {
                    const float h = y0 / (1.0f + expf(-y0)) * y1;
                    static_cast<uint16_t *>(out)[i] = f16_bits(h);
                }
            }
        }
    }
    if (EPI == EPI_F32 && am.counter != nullptr)
        grid_argmax(bv, bi, am);
}

// ----------------------------------------------------------------- launch --

// One wavefront per tile up to this many wavefronts; beyond it wavefronts
// loop over tiles with a grid stride.
constexpr int64_t kMaxWaves = 256 * 32;

int64_t gemv_blocks(int64_t tiles)
{
    const int64_t waves = tiles < kMaxWaves ? tiles : kMaxWaves;
    return (waves + 3) / 4;
}

int64_t argmax_workspace_bytes(int64_t tiles)
{
    return kArgmaxHeader + 8 * gemv_blocks(tiles);
}

hipError_t launch_pack(const uint32_t *w0, const uint16_t *s0, const uint32_t *w1,
                       const uint16_t *s1, int64_t rows, int64_t k, bool gate_up,
                       const Geometry &geo, void *dst, hipStream_t stream)
{
    const int64_t units = geo.tiles * geo.P * 2 * geo.CG * 64;
    const int64_t blocks = (units + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w0, s0, w1, s1,
                       rows, k, gate_up ? 1 : 0, geo.L, geo.CG, geo.P, units,
                       static_cast<uint8_t *>(dst));
    return hipGetLastError();
}

hipError_t launch_unpack(const void *src, int64_t rows, int64_t k, const Geometry &geo,
                         uint32_t *words, uint16_t *scales, hipStream_t stream)
{
    const int64_t items = rows * (k / 32);
    const int64_t blocks = (items + 255) / 256;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t *>(src), rows, k, geo.L, geo.CG, geo.P, words,
                       scales);
    return hipGetLastError();
}

template <int L, int CG>
static void launch_lcg(Epilogue epi, dim3 grid, hipStream_t stream, const uint8_t *wd,
                       const uint16_t *x, void *out, int64_t rows, int64_t k, int passes,
                       int64_t tiles, int64_t n_out, ArgmaxScratch am)
{
    switch (epi) {
    case EPI_F16:
        hipLaunchKernelGGL((gemv_family_kernel<L, CG, EPI_F16>), grid, dim3(256), 0, stream, wd, x,
                           out, rows, k, passes, tiles, n_out, am);
        break;
    case EPI_F32:
        hipLaunchKernelGGL((gemv_family_kernel<L, CG, EPI_F32>), grid, dim3(256), 0, stream, wd, x,
                           out, rows, k, passes, tiles, n_out, am);
        break;
    case EPI_SILU:
        hipLaunchKernelGGL((gemv_family_kernel<L, CG, EPI_SILU>), grid, dim3(256), 0, stream, wd,
                           x, out, rows, k, passes, tiles, n_out, am);
        break;
    }
}

template <int L>
static bool launch_l(int CG, Epilogue epi, dim3 grid, hipStream_t stream, const uint8_t *wd,
                     const uint16_t *x, void *out, int64_t rows, int64_t k, int passes,
                     int64_t tiles, int64_t n_out, ArgmaxScratch am)
{
    switch (CG) {
    case 1: launch_lcg<L, 1>(epi, grid, stream, wd, x, out, rows, k, passes, tiles, n_out, am); return true;
    case 2: launch_lcg<L, 2>(epi, grid, stream, wd, x, out, rows, k, passes, tiles, n_out, am); return true;
    case 3: launch_lcg<L, 3>(epi, grid, stream, wd, x, out, rows, k, passes, tiles, n_out, am); return true;
    case 4: launch_lcg<L, 4>(epi, grid, stream, wd, x, out, rows, k, passes, tiles, n_out, am); return true;
    }
    return false;
}

hipError_t launch_gemv_family(const Geometry &geo, Epilogue epi, const void *wdata,
                              const uint16_t *x, void *out, int64_t rows, int64_t k,
                              int64_t n_out, ArgmaxScratch am, hipStream_t stream)
{
    const dim3 grid((unsigned)gemv_blocks(geo.tiles));
    const uint8_t *wd = static_cast<const uint8_t *>(wdata);
    bool ok = false;
    switch (geo.L) {
    case 64: ok = launch_l<64>(geo.CG, epi, grid, stream, wd, x, out, rows, k, geo.P, geo.tiles, n_out, am); break;
    case 32: ok = launch_l<32>(geo.CG, epi, grid, stream, wd, x, out, rows, k, geo.P, geo.tiles, n_out, am); break;
    case 16: ok = launch_l<16>(geo.CG, epi, grid, stream, wd, x, out, rows, k, geo.P, geo.tiles, n_out, am); break;
    case 8: ok = launch_l<8>(geo.CG, epi, grid, stream, wd, x, out, rows, k, geo.P, geo.tiles, n_out, am); break;
    case 4: ok = launch_l<4>(geo.CG, epi, grid, stream, wd, x, out, rows, k, geo.P, geo.tiles, n_out, am); break;
    case 2: ok = launch_l<2>(geo.CG, epi, grid, stream, wd, x, out, rows, k, geo.P, geo.tiles, n_out, am); break;
    case 1: ok = launch_l<1>(geo.CG, epi, grid, stream, wd, x, out, rows, k, geo.P, geo.tiles, n_out, am); break;
    }
    if (!ok)
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace q4
