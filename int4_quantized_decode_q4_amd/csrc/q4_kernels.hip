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
//
// The int3 variant of the same matmul (the Zero-TVM README, where it says
// where the shaders live, names one generator for an int4/int3 family) runs
// the block kernel with a 12-byte lane unit instead of 16; see the int3
// dequant below for its word layout.
#include <hip/hip_runtime.h>
#include <type_traits>
#include <math.h>
#include <stdint.h>

#include "q4_device.h"
#include "q4_geometry.h"
#include "q4_internal.h"
#include "q4_lanes.h"

namespace q4 {


// ---------------------------------------------------------------- packing --

// One thread per destination 16-byte code unit (and the scale beside it):
// a pure permutation of the canonical words, padding where the logical
// (row, group) lies outside the matrix.
// Canonical row behind logical row r of a rotary-paired layout with heads of
// d rows: logical rows 2p, 2p + 1 hold dims i, i + d/2 of head p / (d/2).
__host__ __device__ __forceinline__ int64_t rope_source_row(int64_t r, int64_t d)
{
    const int64_t p = r >> 1, half = d >> 1;
    return (p / half) * d + p % half + (r & 1) * half;
}

__global__ void pack_kernel(const uint32_t *__restrict__ w0, const uint16_t *__restrict__ s0,
                            const uint32_t *__restrict__ w1, const uint16_t *__restrict__ s1,
                            int64_t rows, int64_t k, int mode, int64_t d, int L, int CG, int P,
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
        if (mode == PACK_GATE_UP) {
            row = r >> 1;
            sw = (r & 1) ? w1 : w0;
            ss = (r & 1) ? s1 : s0;
        } else if (mode == PACK_ROPE) {
            row = rope_source_row(r, d);
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
                              int mode, int64_t d, int L, int CG, int P,
                              uint32_t *__restrict__ words, uint16_t *__restrict__ scales)
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
    // rotary pairs come back in the original row order
    const int64_t row = mode == PACK_ROPE ? rope_source_row(r, d) : r;
    *reinterpret_cast<uint4 *>(words + row * (k / 8) + 4 * g) = v;
    scales[row * G + g] =
        *reinterpret_cast<const uint16_t *>(base + (int64_t)2 * CG * 1024 + lane * 4 * CG + (u * CG + j) * 2);
}

// ------------------------------------------------------------ int3 packing --
//
// Canonical int3 rows are bit streams (code k in stream bits 3k .. 3k+2, LSB
// first over little-endian words), 3 words per group of 32 codes; the device
// unit of a group is 3 words with code 10i + m at bits 3m and 10i + 5 + m at
// bits 16 + 3m of word i (m = 0..4), and bit i of codes 30 / 31 at bits 15 /
// 31 of word i.  Padding is code 4 (a zero weight) with scale 0.

// code i of a group from its 3 canonical words
__device__ __forceinline__ uint32_t canonical3_code(const uint32_t (&w)[3], int i)
{
    const int b = 3 * i, wi = b >> 5, sh = b & 31;
    uint64_t v = w[wi];
    if (wi < 2)
        v |= (uint64_t)w[wi + 1] << 32;
    return (uint32_t)(v >> sh) & 7u;
}

__device__ __forceinline__ void device3_words(const uint32_t (&codes)[32], uint32_t (&d)[3])
{
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        uint32_t v = ((codes[30] >> i) & 1u) << 15 | ((codes[31] >> i) & 1u) << 31;
#pragma unroll
        for (int m = 0; m < 5; ++m)
            v |= codes[10 * i + m] << (3 * m) | codes[10 * i + 5 + m] << (16 + 3 * m);
        d[i] = v;
    }
}

// One thread per destination 12-byte unit (and the scale beside it).  With a
// second source (w3b, scb: the up half of a gate/up pair) logical row r reads
// row r / 2 of the gate (even r) or of the up matrix (odd r).
__global__ void pack3_kernel(const uint32_t *__restrict__ w3a, const uint16_t *__restrict__ sca,
                             const uint32_t *__restrict__ w3b, const uint16_t *__restrict__ scb,
                             int64_t rows, int64_t k, int L, int CG, int P, int64_t units,
                             uint8_t *__restrict__ dst)
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
    const int64_t r = t * (128 / L) + 2 * s + u;
    const int64_t G = k / 32;
    const int64_t g = (int64_t)p * L * CG + (int64_t)c * CG + j;
    uint32_t codes[32];
    uint16_t scale = 0;
    if (r < rows && g < G) {
        const bool up = w3b != nullptr && (r & 1);
        const int64_t row = w3b != nullptr ? r >> 1 : r;
        const uint32_t *src = (up ? w3b : w3a) + row * (3 * G) + 3 * g;
        const uint32_t w[3] = {src[0], src[1], src[2]};
#pragma unroll
        for (int i = 0; i < 32; ++i)
            codes[i] = canonical3_code(w, i);
        scale = (up ? scb : sca)[row * G + g];
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            codes[i] = 4u;
    }
    uint32_t d[3];
    device3_words(codes, d);
    uint8_t *base = dst + (t * P + p) * (int64_t)CG * 1792;
    uint32_t *out = reinterpret_cast<uint32_t *>(base + (int64_t)uj * 768 + lane * 12);
    out[0] = d[0];
    out[1] = d[1];
    out[2] = d[2];
    *reinterpret_cast<uint16_t *>(base + (int64_t)2 * CG * 768 + lane * 4 * CG + uj * 2) = scale;
}

// One thread per logical (row, group) of the real matrix: device unit back
// to the canonical stream.
__global__ void unpack3_kernel(const uint8_t *__restrict__ src, int64_t rows, int64_t k, int L,
                               int CG, int P, uint32_t *__restrict__ w3, uint16_t *__restrict__ sc)
{
    const int64_t G = k / 32;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * G)
        return;
    const int64_t r = idx / G, g = idx % G;
    const int64_t t = r / (128 / L);
    const int s = (int)((r % (128 / L)) >> 1), u = (int)(r & 1);
    const int64_t p = g / ((int64_t)L * CG);
    const int c = (int)((g % ((int64_t)L * CG)) / CG), j = (int)(g % CG);
    const int lane = s * L + c;
    const uint8_t *base = src + (t * P + p) * (int64_t)CG * 1792;
    const uint32_t *d = reinterpret_cast<const uint32_t *>(base + (int64_t)(u * CG + j) * 768 + lane * 12);
    uint64_t lo = 0;   // stream bits 0..63 of the group
    uint32_t hi = 0;   // bits 64..95
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const uint32_t v = d[i];
#pragma unroll
        for (int m = 0; m < 10; ++m) {
            const int code_i = 10 * i + m;
            const uint32_t q = (v >> (m < 5 ? 3 * m : 16 + 3 * (m - 5))) & 7u;
            const int b = 3 * code_i;
            if (b + 3 <= 64)
                lo |= (uint64_t)q << b;
            else if (b >= 64)
                hi |= q << (b - 64);
            else {   // code 21: bits 63..65
                lo |= (uint64_t)q << b;
                hi |= q >> (64 - b);
            }
        }
    }
    uint32_t q30 = 0, q31 = 0;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        q30 |= ((d[i] >> 15) & 1u) << i;
        q31 |= ((d[i] >> 31) & 1u) << i;
    }
    hi |= q30 << (90 - 64) | q31 << (93 - 64);
    uint32_t *dst = w3 + r * (3 * G) + 3 * g;
    dst[0] = (uint32_t)lo;
    dst[1] = (uint32_t)(lo >> 32);
    dst[2] = hi;
    sc[r * G + g] = *reinterpret_cast<const uint16_t *>(base + (int64_t)2 * CG * 768 + lane * 4 * CG +
                                                        (u * CG + j) * 2);
}

// ----------------------------------------------------------- GEMV family --

// x pairs for one group of 32 k, ordered per word of codes as
// (x0,x4) (x1,x5) (x2,x6) (x3,x7) to match dot_word's nibble pairs.

__device__ __forceinline__ void pair3_into(uint32_t *xp, const uint32_t (&n)[16]);

// x pairs of one group (int4: per word of codes; int3: see pair3_into)
template <int FMT = 4>
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
    if constexpr (FMT == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q)   // q = word of codes, 8 k each
            pair_into(xp + 4 * q, src[q]);
    } else {
        uint32_t n[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = src[q];
            n[4 * q] = v.x;
            n[4 * q + 1] = v.y;
            n[4 * q + 2] = v.z;
            n[4 * q + 3] = v.w;
        }
        pair3_into(xp, n);
    }
}

// ------------------------------------------------ residual add + RMSNorm --
// The add_norm step ([P1] 内核融合) run inside the matmul that consumes it:
// h = f16(x + r), the matmul sees f16(h * gamma / sqrt(mean(h^2) + eps)),
// all in f32.  Every block computes the mean square over all of k itself
// (k <= a few thousand halves, from L2), so no launch or grid barrier is
// needed; block 0 stores h when the caller asks for it.


// Sum of one value per thread over the block, in a fixed order (every thread
// gets the same bits).  scratch: 16 floats of LDS.
__device__ float block_sum(float v, float *scratch)
{
    v = lanes::reduce<64>(v);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();   // a previous use of scratch has been read
    if ((threadIdx.x & 63) == 0)
        scratch[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; ++i)
        t += scratch[i];
    return t;
}

// 1 / sqrt(mean(h^2) + eps) over all of k, by the whole block from global
// memory; block 0 also stores h when asked.
__device__ float norm_prepass(const uint16_t *__restrict__ x, const NormArgs &nm, int64_t k,
                              float *scratch)
{
    const uint4 *x4 = reinterpret_cast<const uint4 *>(x);
    const uint4 *r4 = reinterpret_cast<const uint4 *>(nm.r);
    uint4 *h4 = reinterpret_cast<uint4 *>(nm.h_out);
    float ss = 0.f;
    for (int64_t i = threadIdx.x; i < k / 8; i += blockDim.x) {
        uint4 h = x4[i];
        if (r4 != nullptr)
            h = residual_add8(h, r4[i]);
        ss += sumsq8(h);
        if (h4 != nullptr && blockIdx.x == 0)
            h4[i] = h;
    }
    return inv_rms(block_sum(ss, scratch), k, nm.eps);
}

// The normalised x pairs of group g (zeros past the end).
__device__ __forceinline__ void norm_x_group(uint32_t *xp, const uint16_t *__restrict__ x,
                                             const NormArgs &nm, float inv, int64_t g, int64_t G)
{
    if (g >= G) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            xp[i] = 0u;
        return;
    }
    const uint4 *x4 = reinterpret_cast<const uint4 *>(x + g * 32);
    const uint4 *r4 = reinterpret_cast<const uint4 *>(nm.r + g * 32);
    const uint4 *g4 = reinterpret_cast<const uint4 *>(nm.gamma + g * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint4 h = x4[q];
        if (nm.r != nullptr)
            h = residual_add8(h, r4[q]);
        pair_into(xp + 4 * q, norm8(h, g4[q], inv));
    }
}


// int3 (codes 0..7, w = (q - 4) * s).  A group's 32 codes c0..c31 sit in 3
// device words; word i holds codes 10i + m at bits 3m and 10i + 5 + m at bits
// 16 + 3m (m = 0..4), and bit i of c30 / c31 at bit 15 / 31.  So each word
// gives 5 f16 pairs (code 10i + m, code 10i + 5 + m) with the magic trick:
// the codes at bits 0, 3, 6 of each half are masked in place, read as
// 1024 + q, 1024 + 8q and 1024 + 64q, and offset by 1028, 1056 and 1280 to
// q - 4 times 1, 8 and 64; the codes at bits 9 and 12 take one shift by 9
// first.  The last pair (c30, c31) is assembled from the three top bits of
// each half.  Per group: 3 x (1 shift + 5 and-or + 5 subtract + 5 dot) plus
// 3 shifts, 3 and-or, 1 subtract and 1 dot -- about 56 VALU for 32 weights,
// against 52 for int4, on 12 bytes of codes instead of 16.
struct DequantConsts3 {
    uint32_t m0, m3, m6, b1, b2, b4, magic;
};

__device__ __forceinline__ DequantConsts3 dequant_consts3()
{
    DequantConsts3 k;
    asm("v_mov_b32 %0, 0x00070007" : "=v"(k.m0));
    asm("v_mov_b32 %0, 0x00380038" : "=v"(k.m3));
    asm("v_mov_b32 %0, 0x01C001C0" : "=v"(k.m6));
    asm("v_mov_b32 %0, 0x00010001" : "=v"(k.b1));
    asm("v_mov_b32 %0, 0x00020002" : "=v"(k.b2));
    asm("v_mov_b32 %0, 0x00040004" : "=v"(k.b4));
    asm("v_mov_b32 %0, 0x64006400" : "=v"(k.magic));
    return k;
}

// x pairs of one group for dot_unit3: xp[5i + m] = (x[10i + m], x[10i + 5 + m]),
// xp[15] = (x30, x31), from the natural pairs n[q] = (x[2q], x[2q + 1]).
__device__ __forceinline__ void pair3_into(uint32_t *xp, const uint32_t (&n)[16])
{
    auto half = [&](int i) -> uint32_t { return (n[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu; };
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int m = 0; m < 5; ++m)
            xp[5 * i + m] = half(10 * i + m) | (half(10 * i + 5 + m) << 16);
    xp[15] = n[15];
}

__device__ __forceinline__ float dot_unit3(uint4 c, const uint32_t *xp, const DequantConsts3 &m)
{
    const h2 k1 = {(_Float16)1028.0f, (_Float16)1028.0f};
    const h2 k8 = {(_Float16)1056.0f, (_Float16)1056.0f};
    const h2 k64 = {(_Float16)1280.0f, (_Float16)1280.0f};
    const uint32_t w[3] = {c.x, c.y, c.z};
    float p1 = 0.f, p8 = 0.f, p64 = 0.f;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const uint32_t v = w[i], t = v >> 9;
        const uint32_t a0 = (v & m.m0) | m.magic;   // 1024 + q(10i), 1024 + q(10i+5)
        const uint32_t a1 = (v & m.m3) | m.magic;   // 1024 + 8 q(10i+1), ..
        const uint32_t a2 = (v & m.m6) | m.magic;   // 1024 + 64 q(10i+2), ..
        const uint32_t a3 = (t & m.m0) | m.magic;   // 1024 + q(10i+3), ..
        const uint32_t a4 = (t & m.m3) | m.magic;   // 1024 + 8 q(10i+4), ..
        p1 = __builtin_amdgcn_fdot2(as_h2(a0) - k1, as_h2(xp[5 * i + 0]), p1, false);
        p8 = __builtin_amdgcn_fdot2(as_h2(a1) - k8, as_h2(xp[5 * i + 1]), p8, false);
        p64 = __builtin_amdgcn_fdot2(as_h2(a2) - k64, as_h2(xp[5 * i + 2]), p64, false);
        p1 = __builtin_amdgcn_fdot2(as_h2(a3) - k1, as_h2(xp[5 * i + 3]), p1, false);
        p8 = __builtin_amdgcn_fdot2(as_h2(a4) - k8, as_h2(xp[5 * i + 4]), p8, false);
    }
    uint32_t e = ((w[0] >> 15) & m.b1) | m.magic;   // bit 0 of c30 and c31
    e = ((w[1] >> 14) & m.b2) | e;                   // bit 1
    e = ((w[2] >> 13) & m.b4) | e;                   // bit 2: 1024 + c30, 1024 + c31
    p1 = __builtin_amdgcn_fdot2(as_h2(e) - k1, as_h2(xp[15]), p1, false);
    return fmaf(p64, 0.015625f, fmaf(p8, 0.125f, p1));
}

// Per-format pieces of the block kernel: FMT 4 (int4, 16-byte lane units) or
// 3 (int3, 12-byte lane units); a pass is CG * (2 * UB + 256) bytes.
template <int FMT>
struct Fmt;
template <>
struct Fmt<4> {
    static constexpr int UB = 1024;
    using Consts = DequantConsts;
    static __device__ __forceinline__ Consts consts() { return dequant_consts(); }
    static __device__ __forceinline__ float dot(uint4 c, const uint32_t *xp, const Consts &m)
    {
        return dot_unit4(c, xp, m);
    }
};
template <>
struct Fmt<3> {
    static constexpr int UB = 768;
    using Consts = DequantConsts3;
    static __device__ __forceinline__ Consts consts() { return dequant_consts3(); }
    static __device__ __forceinline__ float dot(uint4 c, const uint32_t *xp, const Consts &m)
    {
        return dot_unit3(c, xp, m);
    }
};

template <int L>
__device__ __forceinline__ float reduce_lanes(float v)
{
    return lanes::reduce<L>(v);
}

__device__ __forceinline__ void better(float &bv, int &bi, float ov, int oi)
{
    if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
    }
}

// (max, lowest index) over the lanes of a wavefront whose lane index is a
// multiple of STRIDE (the other lanes hold no candidate): the xor steps of
// STRIDE and above only, so a GEMV kernel whose rows are finished by lane
// c == 0 of each L-lane row group takes log2(64 / L) steps instead of 6
template <int STRIDE>
__device__ __forceinline__ void wave_argmax(float &bv, int &bi)
{
#pragma unroll
    for (int off = 32; off >= STRIDE; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        better(bv, bi, ov, oi);
    }
}

// Block-wide (max, lowest index) of per-thread candidates over a block of
// NWAVES wavefronts; result in thread 0.  The caller orders any later use of
// sv / si (a block barrier).  The wave count is a template constant: reading
// blockDim.x costs a load from the dispatch packet, and waiting for it waited
// for every store the wavefront still had in flight.
template <int STRIDE, int NWAVES>
__device__ void block_argmax(float &bv, int &bi, float *sv, int *si)
{
    wave_argmax<STRIDE>(bv, bi);
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sv[wid] = bv;
        si[wid] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0)
#pragma unroll
        for (int w = 1; w < NWAVES; ++w)
            better(bv, bi, sv[w], si[w]);
}

__device__ __forceinline__ unsigned long long pack_vi(float v, int i)
{
    return (unsigned long long)__builtin_bit_cast(unsigned int, v) |
           ((unsigned long long)(unsigned int)i << 32);
}

// Argmax across blocks, in the matmul's own launch: each block publishes its
// candidate and counts itself in; the block that completes the count
// combines every candidate (max value, then lowest index: the result does
// not depend on the order they arrive in) and writes the index.  The count
// is two-level -- 16 counters on separate 256-byte lines, each finished by
// the last block of its line, which then adds to one top counter -- so no
// more than (blocks / 16) atomics queue on one address.  A block's candidate
// store is complete before its atomic (vmcnt wait), and the candidates are
// read back with device-coherent loads, so no fence is needed; every counter
// is reset to zero by the block that completes it, ready for the next call.
constexpr int kArgmaxLines = 16;

template <int STRIDE, int NWAVES>
__device__ void grid_argmax(float bv, int bi, ArgmaxScratch am)
{
    static_assert(NWAVES <= 16, "one LDS slot per wavefront");
    __shared__ float sv[16];
    __shared__ int si[16];
    __shared__ int last;
    block_argmax<STRIDE, NWAVES>(bv, bi, sv, si);
    const int nb = gridDim.x, b = blockIdx.x;
    if (threadIdx.x == 0) {
        __hip_atomic_store(am.partials + b, pack_vi(bv, bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const int line = b % kArgmaxLines;
        const int lines = nb < kArgmaxLines ? nb : kArgmaxLines;
        const unsigned in_line = (unsigned)((nb - 1 - line) / kArgmaxLines + 1);
        uint32_t *ctr = am.counters + 64 * line;
        int l = 0;
        if (__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == in_line - 1) {
            __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t *top = am.counters + 64 * kArgmaxLines;
            if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (unsigned)lines - 1) {
                __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                l = 1;
            }
        }
        last = l;
    }
    __syncthreads();
    if (last) {
        float v = -INFINITY;
        int i = 0x7fffffff;
        for (int p = threadIdx.x; p < nb; p += 64 * NWAVES) {
            const unsigned long long k =
                __hip_atomic_load(am.partials + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            better(v, i, __builtin_bit_cast(float, (unsigned int)(k & 0xFFFFFFFFull)), (int)(unsigned int)(k >> 32));
        }
        block_argmax<1, NWAVES>(v, i, sv, si);
        if (threadIdx.x == 0)
            *am.result = i;
    }
}

// Registers of one pass of one tile: 2*CG code units and 2*CG scales.
template <int CG>
struct TileRegs {
    uint4 c[2][CG];
    uint32_t s[CG];
};

template <int CG>
__device__ __forceinline__ void load_tile(TileRegs<CG> &r, const uint8_t *__restrict__ base, int lane)
{
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < CG; ++j)
            r.c[u][j] = *reinterpret_cast<const uint4 *>(base + (u * CG + j) * 1024 + lane * 16);
    const uint32_t *sp = reinterpret_cast<const uint32_t *>(base + 2 * CG * 1024 + lane * 4 * CG);
#pragma unroll
    for (int j = 0; j < CG; ++j)
        r.s[j] = sp[j];
}

// acc[u] += sum over the lane's CG groups of scale * sum_k x_k (q_k - 8)
template <int CG>
__device__ __forceinline__ void compute_tile(const TileRegs<CG> &r, const uint32_t (&xp)[CG][16],
                                             float (&acc)[2], const DequantConsts &m)
{
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < CG; ++j) {
            float p1 = 0.f, p16 = 0.f;
            dot_word(r.c[u][j].x, &xp[j][0], p1, p16, m);
            dot_word(r.c[u][j].y, &xp[j][4], p1, p16, m);
            dot_word(r.c[u][j].z, &xp[j][8], p1, p16, m);
            dot_word(r.c[u][j].w, &xp[j][12], p1, p16, m);
            const int e = u * CG + j;
            const float sv = f16_value((uint16_t)(r.s[e >> 1] >> ((e & 1) * 16)));
            acc[u] = fmaf(sv, fmaf(p16, 0.0625f, p1), acc[u]);
        }
}

// Epilogue of the finished sums y0, y1 of logical rows r0 (even) and r0 + 1.
template <int EPI>
__device__ __forceinline__ void store_rows(float y0, float y1, int64_t r0, void *__restrict__ out,
                                           int64_t rows, int64_t n_out, float &bv, int &bi,
                                           const typename RopeParam<EPI>::type &rp)
{
    if constexpr (EPI == EPI_F16) {
        uint16_t *y = static_cast<uint16_t *>(out);
        if (r0 + 1 < rows)
            *reinterpret_cast<uint32_t *>(y + r0) =
                (uint32_t)f16_bits(y0) | ((uint32_t)f16_bits(y1) << 16);
        else if (r0 < rows)
            y[r0] = f16_bits(y0);
    } else if constexpr (EPI == EPI_F32) {
        float *y = static_cast<float *>(out);
        if (r0 + 1 < rows) {
            *reinterpret_cast<float2 *>(y + r0) = make_float2(y0, y1);
            better(bv, bi, y0, (int)r0);
            better(bv, bi, y1, (int)r0 + 1);
        } else if (r0 < rows) {
            y[r0] = y0;
            better(bv, bi, y0, (int)r0);
        }
    } else if constexpr (EPI == EPI_SILU) {  // logical rows (2i, 2i+1) = (gate i, up i)
        const int64_t i = r0 >> 1;
        if (i < n_out) {
            const float h = y0 / (1.0f + expf(-y0)) * y1;
            static_cast<uint16_t *>(out)[i] = f16_bits(h);
        }
    } else if constexpr (EPI == EPI_ROPE) {
        // logical rows (2p, 2p+1) = dims (i, i + d/2) of head p / (d/2)
        if (r0 >= rows)
            return;
        const int64_t p = r0 >> 1, half = rp.d >> 1;
        const int64_t blk = p / half, i = p % half;
        float a = y0, b = y1;
        if (blk < rp.nq + rp.nkv) {   // q and k heads turn
            const float cs = rp.cs[i][0], sn = rp.cs[i][1];
            a = y0 * cs - y1 * sn;
            b = y1 * cs + y0 * sn;
        }
        const uint16_t ha = f16_bits(a), hb = f16_bits(b);
        uint16_t *y = static_cast<uint16_t *>(out);
        y[blk * rp.d + i] = ha;
        y[blk * rp.d + i + half] = hb;
        if (rp.cache != nullptr && blk >= rp.nq) {   // k and v heads: the page slot of pos
            const int64_t kv = blk >= rp.nq + rp.nkv ? 1 : 0;
            const int64_t head = blk - rp.nq - kv * rp.nkv;
            const int32_t page = rp.page_table[rp.pos >> 4];
            if (page >= 0 && page < rp.n_pages) {
                uint16_t *dst = rp.cache + ((((int64_t)page * 2 + kv) * rp.nkv + head) * 16 + (rp.pos & 15)) * rp.d + i;
                dst[0] = ha;
                dst[half] = hb;
            }
        }
    }
}

// Cross-lane reduction of a finished tile and its epilogue.
template <int L, int EPI>
__device__ __forceinline__ void finish_tile(const float (&acc)[2], int64_t t, int s, int c,
                                            void *__restrict__ out, int64_t rows, int64_t n_out,
                                            float &bv, int &bi,
                                            const typename RopeParam<EPI>::type &rp)
{
    constexpr int TR = 128 / L;
    const float y0 = reduce_lanes<L>(acc[0]);
    const float y1 = reduce_lanes<L>(acc[1]);
    if (c == 0)
        store_rows<EPI>(y0, y1, t * TR + 2 * s, out, rows, n_out, bv, bi, rp);
}

// ------------------------------------------------------------ GEMV kernels --
//
// rows: logical rows of the layout (gate/up: 2 * n_out); n_out: output length.
// The three kernels (block, split, multi-pass) share the unit arithmetic
// above and differ in how tiles are assigned and how many are kept in flight.

#ifndef Q4_STREAM_DEPTH
#define Q4_STREAM_DEPTH 6
#endif
#ifndef Q4_BLOCK_WAVES
#define Q4_BLOCK_WAVES 4
#endif
constexpr int kBlockWaves = Q4_BLOCK_WAVES;


// Load unit i (u = i / CG, j = i % CG) of a tile into its register slot
// (int3: 12 bytes, the fourth word unused).
typedef unsigned v3u __attribute__((ext_vector_type(3)));

template <int CG, int FMT = 4>
__device__ __forceinline__ void load_unit(TileRegs<CG> &r, __amdgpu_buffer_rsrc_t rs, int lane, int i)
{
    if constexpr (FMT == 4) {
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, i * 1024, 0);
        r.c[i / CG][i % CG] = make_uint4(v.x, v.y, v.z, v.w);
    } else {
        const v3u v = __builtin_amdgcn_raw_buffer_load_b96(rs, lane * 12, i * 768, 0);
        r.c[i / CG][i % CG] = make_uint4(v.x, v.y, v.z, 0u);
    }
}

template <int CG, int FMT = 4>
__device__ __forceinline__ void load_scales(TileRegs<CG> &r, __amdgpu_buffer_rsrc_t rs, int lane)
{
#pragma unroll
    for (int j = 0; j < CG; ++j)
        r.s[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4 * CG + 4 * j, 2 * CG * Fmt<FMT>::UB, 0);
}

// One tile, unit by unit: compute unit i of `cur`, then issue the load that
// keeps PD units in flight: unit i + PD of `cur`, or past its end a unit of
// `nxt`, the wavefront's next tile (a zero-size resource when there is none).
template <int FMT, int CG, int PD>
__device__ __forceinline__ void stream_tile(TileRegs<CG> &cur, TileRegs<CG> &nxt,
                                            __amdgpu_buffer_rsrc_t cur_rs,
                                            __amdgpu_buffer_rsrc_t nxt_rs, int lane,
                                            const uint32_t (&xp)[CG][16], float (&acc)[2],
                                            const typename Fmt<FMT>::Consts &m)
{
    constexpr int NU = 2 * CG;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const int u = i / CG, j = i % CG;
        const float p = Fmt<FMT>::dot(cur.c[u][j], &xp[j][0], m);
        const int e = u * CG + j;
        const float sv = f16_value((uint16_t)(cur.s[e >> 1] >> ((e & 1) * 16)));
        acc[u] = fmaf(sv, p, acc[u]);
        // the unit's arithmetic must be issued before the next load: the
        // compiler would otherwise hoist every load of the tile to its top
        // (and sink the arithmetic below them), defeating the pipeline
        asm volatile("" ::"v"(acc[u]) : "memory");
        const int pi = i + PD;
        if (pi < NU) {
            load_unit<CG, FMT>(cur, cur_rs, lane, pi);
        } else {
            if (pi == NU)
                load_scales<CG, FMT>(nxt, nxt_rs, lane);
            load_unit<CG, FMT>(nxt, nxt_rs, lane, pi - NU);
        }
    }
}

// Block kernel (single-pass weights): a block of kBlockWaves wavefronts
// takes that many consecutive tiles at a time, one per wavefront, and
// strides over the matrix by the grid (about two blocks per CU, so each
// wavefront streams a few tiles).  The block stages x in LDS once; each
// wavefront then builds its x pairs from LDS, so x costs one L2 read per
// block instead of one per wavefront, and few blocks keep that cost small.
// Each wavefront streams its tiles unit by unit (one 1 KiB load per 16-byte
// lane unit) with Q4_STREAM_DEPTH units in flight -- by default a whole
// tile, so while a tile is reduced the next one is already on its way.
constexpr int kBlockXHalves = 8192;   // largest single-pass k

template <int FMT = 4>
__device__ __forceinline__ void lds_x_group(uint32_t *xp, const uint4 *xs, int64_t g, int64_t G)
{
    if (g >= G) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            xp[i] = 0u;
        return;
    }
    if constexpr (FMT == 4) {
        // staged already paired (pair_chunk)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = xs[g * 4 + q];
            xp[4 * q] = v.x;
            xp[4 * q + 1] = v.y;
            xp[4 * q + 2] = v.z;
            xp[4 * q + 3] = v.w;
        }
    } else {
        uint32_t n[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = xs[g * 4 + q];
            n[4 * q] = v.x;
            n[4 * q + 1] = v.y;
            n[4 * q + 2] = v.z;
            n[4 * q + 3] = v.w;
        }
        pair3_into(xp, n);
    }
}

template <int L, int CG, int EPI, bool NORM, int FMT = 4>
__global__ __launch_bounds__(64 * kBlockWaves) void gemv_block_kernel(
    const uint8_t *__restrict__ wd, const uint16_t *__restrict__ x, void *__restrict__ out,
    int64_t rows, int64_t k, int64_t tiles, int64_t n_out, ArgmaxScratch am, NormArgs nm,
    typename RopeParam<EPI>::type rp)
{
    constexpr int PD = Q4_STREAM_DEPTH < 2 * CG ? Q4_STREAM_DEPTH : 2 * CG;
    constexpr int64_t PB = (int64_t)CG * (2 * Fmt<FMT>::UB + 256);
    __shared__ uint4 xs[kBlockXHalves / 8];
    const int lane = threadIdx.x & 63;
    // wave-uniform by construction; said explicitly so that the tile index and
    // its buffer resource live in SGPRs (no waterfall loop around each load)
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int s = lane / L, c = lane % L;
    const int64_t G = k >> 5;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    const typename Fmt<FMT>::Consts m = Fmt<FMT>::consts();

    // x and the head of the weight stream are requested together: x through
    // a resource of k halves (loads past it return zeros), up to 4 x 16 bytes
    // per thread (the largest single-pass k; only the rounds k needs are
    // issued), written to LDS once both are in flight
    const __amdgpu_buffer_rsrc_t xrs = tile_rsrc(reinterpret_cast<const uint8_t *>(x), (int)(k * 2));
    constexpr int kThreads = 64 * kBlockWaves;
    constexpr int kXRounds = kBlockXHalves / 8 / kThreads;
    const int xrounds = (int)((k / 8 + kThreads - 1) / kThreads);
    v4u xv[kXRounds];
#pragma unroll
    for (int q = 0; q < kXRounds; ++q)
        if (q < xrounds)
            xv[q] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (threadIdx.x + kThreads * q) * 16, 0, 0);
    // with the norm: the residual (a zero-size resource when there is none)
    // and gamma, requested with x
    v4u rv[NORM ? kXRounds : 1], gv[NORM ? kXRounds : 1];
    if constexpr (NORM) {
        const __amdgpu_buffer_rsrc_t rrs =
            tile_rsrc(reinterpret_cast<const uint8_t *>(nm.r), nm.r != nullptr ? (int)(k * 2) : 0);
        const __amdgpu_buffer_rsrc_t grs = tile_rsrc(reinterpret_cast<const uint8_t *>(nm.gamma), (int)(k * 2));
#pragma unroll
        for (int q = 0; q < kXRounds; ++q)
            if (q < xrounds) {
                rv[q] = __builtin_amdgcn_raw_buffer_load_b128(rrs, (threadIdx.x + kThreads * q) * 16, 0, 0);
                gv[q] = __builtin_amdgcn_raw_buffer_load_b128(grs, (threadIdx.x + kThreads * q) * 16, 0, 0);
            }
    }
    int64_t t = (int64_t)blockIdx.x * kBlockWaves + w;
    const int64_t step = (int64_t)gridDim.x * kBlockWaves;
    auto rs_of = [&](int64_t tt) {
        return tt < tiles ? tile_rsrc(wd + tt * PB, (int)PB) : tile_rsrc(wd, 0);
    };
    TileRegs<CG> ra, rb;
    {
        const __amdgpu_buffer_rsrc_t r0 = rs_of(t);
        load_scales<CG, FMT>(ra, r0, lane);
#pragma unroll
        for (int i = 0; i < PD; ++i)
            load_unit<CG, FMT>(ra, r0, lane, i);
    }
    // with the norm: each thread keeps its chunks of h in registers and
    // parks its wavefront's part of the sum of squares in LDS; after one
    // barrier every thread has the block's sum, normalises its own chunks
    // into LDS, and the staging barrier below publishes them
    if constexpr (NORM) {
        __shared__ float nss[kBlockWaves];
        uint4 hv[kXRounds];
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < kXRounds; ++q)
            if (q < xrounds) {   // chunks past k read as zero and add nothing
                hv[q] = as_uint4(xv[q]);
                if (nm.r != nullptr)
                    hv[q] = residual_add8(hv[q], as_uint4(rv[q]));
                ss += sumsq8(hv[q]);
                const int64_t ci = threadIdx.x + kThreads * q;
                if (nm.h_out != nullptr && blockIdx.x == 0 && ci < k / 8)
                    reinterpret_cast<uint4 *>(nm.h_out)[ci] = hv[q];
            }
        ss = lanes::reduce<64>(ss);
        if (lane == 0)
            nss[w] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < kBlockWaves; ++i)
            tot += nss[i];
        const float inv = inv_rms(tot, k, nm.eps);
#pragma unroll
        for (int q = 0; q < kXRounds; ++q)
            if (q < xrounds)
                xs[threadIdx.x + kThreads * q] = (FMT == 4)
                                                      ? pair_chunk(norm8(hv[q], as_uint4(gv[q]), inv))
                                                      : norm8(hv[q], as_uint4(gv[q]), inv);
    } else {
#pragma unroll
        for (int q = 0; q < kXRounds; ++q)
            if (q < xrounds)
                xs[threadIdx.x + kThreads * q] = (FMT == 4) ? pair_chunk(as_uint4(xv[q]))
                                                                             : as_uint4(xv[q]);
    }
    __syncthreads();
    uint32_t xp[CG][16];
#pragma unroll
    for (int j = 0; j < CG; ++j)
        lds_x_group<FMT>(xp[j], xs, (int64_t)c * CG + j, G);
    while (t < tiles) {
        {
            const int64_t nt = t + step;
            float acc[2] = {0.f, 0.f};
            stream_tile<FMT, CG, PD>(ra, rb, rs_of(t), rs_of(nt), lane, xp, acc, m);
            finish_tile<L, EPI>(acc, t, s, c, out, rows, n_out, bv, bi, rp);
            t = nt;
        }
        if (t >= tiles)
            break;
        {
            const int64_t nt = t + step;
            float acc[2] = {0.f, 0.f};
            stream_tile<FMT, CG, PD>(rb, ra, rs_of(t), rs_of(nt), lane, xp, acc, m);
            finish_tile<L, EPI>(acc, t, s, c, out, rows, n_out, bv, bi, rp);
            t = nt;
        }
    }
    if (EPI == EPI_F32 && am.partials != nullptr)
        grid_argmax<L, kBlockWaves>(bv, bi, am);   // candidates in lanes c == 0
}

// Split kernel (single-pass weights, long k, few tiles): a block of CG
// wavefronts owns the tiles blockIdx.x, + gridDim.x, ... (at most
// kSplitMaxTiles of them); wavefront j takes group slot j of every lane in
// all of them, so a lane keeps the x slice of one group in VGPRs for the
// whole launch and streams 2 code units per tile, with the next
// Q4_SPLIT_DEPTH - 1 tiles already in flight.  Each tile's row sums are
// reduced across lanes inside the wavefront and parked in LDS; after one
// barrier at the end the CG slot sums of a row are added in slot order
// (deterministic) and the epilogue runs.
constexpr int kSplitMaxTiles = 8;
#ifndef Q4_SPLIT_DEPTH
#define Q4_SPLIT_DEPTH 2
#endif

template <int L, int CG, int EPI, bool NORM, int FMT = 4>
__global__ __launch_bounds__(64 * CG) void gemv_split_kernel(
    const uint8_t *__restrict__ wd, const uint16_t *__restrict__ x, void *__restrict__ out,
    int64_t rows, int64_t k, int64_t tiles, int64_t n_out, ArgmaxScratch am, NormArgs nm,
    typename RopeParam<EPI>::type rp)
{
    constexpr int HP = 64 / L;   // row pairs per tile
    constexpr int TR = 128 / L;
    constexpr int UB = Fmt<FMT>::UB;
    constexpr int PB = CG * (2 * UB + 256);
    constexpr int D = Q4_SPLIT_DEPTH;
    __shared__ float part[kSplitMaxTiles][CG][HP][2];
    const int lane = threadIdx.x & 63;
    const int j = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int s = lane / L, c = lane % L;
    uint32_t xp[16];
    if constexpr (!NORM)
        load_x_group<FMT>(xp, x, (int64_t)c * CG + j, k >> 5);
    const typename Fmt<FMT>::Consts m = Fmt<FMT>::consts();
    const int64_t count =
        (int64_t)blockIdx.x < tiles ? (tiles - 1 - (int64_t)blockIdx.x) / gridDim.x + 1 : 0;

    // this wavefront's two units and two scales inside a tile
    const int wo0 = j * UB + lane * (UB / 64), wo1 = (CG + j) * UB + lane * (UB / 64);
    const int so0 = 2 * CG * UB + lane * 4 * CG + j * 2, so1 = so0 + CG * 2;
    struct Regs {
        v4u w0, w1;
        uint16_t s0, s1;
    };
    auto load = [&](Regs &r, int64_t i) {   // the block's i-th tile; none past count
        const bool live = i < count;
        const __amdgpu_buffer_rsrc_t rs =
            tile_rsrc(wd + (live ? (int64_t)blockIdx.x + i * gridDim.x : 0) * PB, live ? PB : 0);
        if constexpr (FMT == 4) {
            r.w0 = __builtin_amdgcn_raw_buffer_load_b128(rs, wo0, 0, 0);
            r.w1 = __builtin_amdgcn_raw_buffer_load_b128(rs, wo1, 0, 0);
        } else {
            const v3u a = __builtin_amdgcn_raw_buffer_load_b96(rs, wo0, 0, 0);
            const v3u b = __builtin_amdgcn_raw_buffer_load_b96(rs, wo1, 0, 0);
            r.w0 = v4u{a.x, a.y, a.z, 0u};
            r.w1 = v4u{b.x, b.y, b.z, 0u};
        }
        r.s0 = __builtin_amdgcn_raw_buffer_load_b16(rs, so0, 0, 0);
        r.s1 = __builtin_amdgcn_raw_buffer_load_b16(rs, so1, 0, 0);
    };
    Regs ring[D];
#pragma unroll
    for (int q = 0; q < D; ++q)
        load(ring[q], q);
    if constexpr (NORM) {
        // after the first tiles are requested: the block's pass over x for
        // the mean square, then this lane's group, normalised
        __shared__ float nscr[16];
        const float inv = norm_prepass(x, nm, k, nscr);
        norm_x_group(xp, x, nm, inv, (int64_t)c * CG + j, k >> 5);
    }
    for (int64_t i0 = 0; i0 < count; i0 += D) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
            const int64_t i = i0 + q;
            if (i >= count)
                break;
            float acc0, acc1;
            if constexpr (FMT == 4) {
                float a1 = 0.f, a16 = 0.f, b1 = 0.f, b16 = 0.f;
                dot_word(ring[q].w0.x, &xp[0], a1, a16, m);
                dot_word(ring[q].w0.y, &xp[4], a1, a16, m);
                dot_word(ring[q].w0.z, &xp[8], a1, a16, m);
                dot_word(ring[q].w0.w, &xp[12], a1, a16, m);
                dot_word(ring[q].w1.x, &xp[0], b1, b16, m);
                dot_word(ring[q].w1.y, &xp[4], b1, b16, m);
                dot_word(ring[q].w1.z, &xp[8], b1, b16, m);
                dot_word(ring[q].w1.w, &xp[12], b1, b16, m);
                acc0 = f16_value(ring[q].s0) * fmaf(a16, 0.0625f, a1);
                acc1 = f16_value(ring[q].s1) * fmaf(b16, 0.0625f, b1);
            } else {
                const v4u a = ring[q].w0, b = ring[q].w1;
                acc0 = f16_value(ring[q].s0) * dot_unit3(make_uint4(a.x, a.y, a.z, 0u), xp, m);
                acc1 = f16_value(ring[q].s1) * dot_unit3(make_uint4(b.x, b.y, b.z, 0u), xp, m);
            }
            // the tile's arithmetic is issued before its registers are refilled
            asm volatile("" ::"v"(acc0), "v"(acc1) : "memory");
            load(ring[q], i + D);
            const float y0 = reduce_lanes<L>(acc0);
            const float y1 = reduce_lanes<L>(acc1);
            if (c == 0) {
                part[i][j][s][0] = y0;
                part[i][j][s][1] = y1;
            }
        }
    }
    __syncthreads();
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int o = threadIdx.x; o < count * HP; o += 64 * CG) {
        const int i = o / HP, ss = o % HP;
        float y0 = part[i][0][ss][0], y1 = part[i][0][ss][1];
#pragma unroll
        for (int jj = 1; jj < CG; ++jj) {
            y0 += part[i][jj][ss][0];
            y1 += part[i][jj][ss][1];
        }
        const int64_t t = (int64_t)blockIdx.x + (int64_t)i * gridDim.x;
        store_rows<EPI>(y0, y1, t * TR + 2 * ss, out, rows, n_out, bv, bi, rp);
    }
    if (EPI == EPI_F32 && am.partials != nullptr)
        grid_argmax<1, CG>(bv, bi, am);   // candidates in any thread; CG wavefronts
}

// Multi-pass kernel (k > 8192): a grid-stride loop over tiles that reloads
// the x slice for every pass.  int3 (FMT 3, no norm prologue) reads its
// 12-byte units through a buffer resource per pass and takes the block
// kernel's unit arithmetic.
template <int L, int CG, int EPI, bool NORM, int FMT = 4>
__global__ __launch_bounds__(256) void gemv_multipass_kernel(
    const uint8_t *__restrict__ wd, const uint16_t *__restrict__ x, void *__restrict__ out,
    int64_t rows, int64_t k, int passes, int64_t tiles, int64_t n_out, ArgmaxScratch am,
    NormArgs nm, typename RopeParam<EPI>::type rp)
{
    static_assert(FMT == 4 || !NORM, "the int3 kernels have no norm prologue");
    constexpr int64_t PB = (int64_t)CG * (2 * Fmt<FMT>::UB + 256);
    const int lane = threadIdx.x & 63;
    const int s = lane / L, c = lane % L;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    const typename Fmt<FMT>::Consts m = Fmt<FMT>::consts();
    float inv = 0.f;
    if constexpr (NORM) {
        __shared__ float nscr[16];
        inv = norm_prepass(x, nm, k, nscr);
    }
    for (int64_t t = wave; t < tiles; t += nwaves) {
        float acc[2] = {0.f, 0.f};
        for (int p = 0; p < passes; ++p) {
            TileRegs<CG> r;
            if constexpr (FMT == 4) {
                load_tile(r, wd + (t * passes + p) * PB, lane);
            } else {
                const __amdgpu_buffer_rsrc_t rs = tile_rsrc(wd + (t * passes + p) * PB, (int)PB);
#pragma unroll
                for (int i = 0; i < 2 * CG; ++i)
                    load_unit<CG, 3>(r, rs, lane, i);
                load_scales<CG, 3>(r, rs, lane);
            }
            uint32_t xp[CG][16];
#pragma unroll
            for (int j = 0; j < CG; ++j) {
                const int64_t g = (int64_t)p * L * CG + (int64_t)c * CG + j;
                if constexpr (NORM)
                    norm_x_group(xp[j], x, nm, inv, g, k >> 5);
                else
                    load_x_group<FMT>(xp[j], x, g, k >> 5);
            }
            if constexpr (FMT == 4) {
                compute_tile(r, xp, acc, m);
            } else {
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int j = 0; j < CG; ++j) {
                        const float d = Fmt<3>::dot(r.c[u][j], &xp[j][0], m);
                        const int e = u * CG + j;
                        const float sv = f16_value((uint16_t)(r.s[e >> 1] >> ((e & 1) * 16)));
                        acc[u] = fmaf(sv, d, acc[u]);
                    }
            }
        }
        finish_tile<L, EPI>(acc, t, s, c, out, rows, n_out, bv, bi, rp);
    }
    if (EPI == EPI_F32 && am.partials != nullptr)
        grid_argmax<L, 4>(bv, bi, am);   // candidates in lanes c == 0; 256 threads
}

// ----------------------------------------------------------------- launch --

#ifndef Q4_SPLIT_BELOW_TILES
#define Q4_SPLIT_BELOW_TILES 2000
#endif
#ifndef Q4_BLOCKS_PER_CU
#define Q4_BLOCKS_PER_CU 2
#endif
#ifndef Q4_SPLIT_MIN_CG
#define Q4_SPLIT_MIN_CG 4
#endif
#ifndef Q4_SPLIT_BLOCKS_PER_CU
#define Q4_SPLIT_BLOCKS_PER_CU 2
#endif

enum Mode { MODE_SPLIT = 1, MODE_MULTIPASS = 2, MODE_BLOCK = 3 };

struct GemvPlan {
    Mode mode;
    int64_t blocks;
    int threads;
};

// The launch plan depends only on the weight's geometry and the device's
// compute units.  Every kernel's result is independent of its grid size (a
// tile's row sums are formed inside one wavefront or added in slot order), so
// a given shape gives the same bits on any device.
static GemvPlan plan_gemv(const Geometry &geo, int64_t kCUs)
{
    if (geo.P > 1) {
        const int64_t waves = geo.tiles < kCUs * 8 ? geo.tiles : kCUs * 8;
        return {MODE_MULTIPASS, (waves + 3) / 4, 256};
    }
    // long k (4 groups per lane) and few tiles: one wavefront per tile would
    // leave the GPU short of wavefronts and each with a long serial chain, so
    // the group slots of a tile go to separate wavefronts
    if (geo.CG >= Q4_SPLIT_MIN_CG && geo.tiles < Q4_SPLIT_BELOW_TILES) {
        int64_t blocks = kCUs * Q4_SPLIT_BLOCKS_PER_CU;
        if (blocks > geo.tiles)
            blocks = geo.tiles;
        if (blocks * kSplitMaxTiles < geo.tiles)
            blocks = (geo.tiles + kSplitMaxTiles - 1) / kSplitMaxTiles;
        return {MODE_SPLIT, blocks, 64 * geo.CG};
    }
    const int64_t groups = (geo.tiles + kBlockWaves - 1) / kBlockWaves;
    const int64_t cap = kCUs * Q4_BLOCKS_PER_CU;
    return {MODE_BLOCK, groups < cap ? groups : cap, 64 * kBlockWaves};
}

int64_t argmax_workspace_bytes(const Geometry &geo)
{
    static_assert(kArgmaxCounterBytes == 256 * (kArgmaxLines + 1), "counter region");
    return kArgmaxCounterBytes + 8 * plan_gemv(geo, device_cus()).blocks;
}

hipError_t launch_pack(const uint32_t *w0, const uint16_t *s0, const uint32_t *w1,
                       const uint16_t *s1, int64_t rows, int64_t k, PackMode mode, int64_t d,
                       const Geometry &geo, void *dst, hipStream_t stream)
{
    const int64_t units = geo.tiles * geo.P * 2 * geo.CG * 64;
    const int64_t blocks = (units + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w0, s0, w1, s1,
                       rows, k, (int)mode, d, geo.L, geo.CG, geo.P, units,
                       static_cast<uint8_t *>(dst));
    return hipGetLastError();
}

hipError_t launch_unpack(const void *src, int64_t rows, int64_t k, PackMode mode, int64_t d,
                         const Geometry &geo, uint32_t *words, uint16_t *scales,
                         hipStream_t stream)
{
    const int64_t items = rows * (k / 32);
    const int64_t blocks = (items + 255) / 256;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t *>(src), rows, k, (int)mode, d, geo.L, geo.CG,
                       geo.P, words, scales);
    return hipGetLastError();
}

hipError_t launch_pack3(const uint32_t *w3, const uint16_t *s, const uint32_t *w3_up,
                        const uint16_t *s_up, int64_t rows, int64_t k, const Geometry &geo,
                        void *dst, hipStream_t stream)
{
    const int64_t units = geo.tiles * geo.P * 2 * geo.CG * 64;
    hipLaunchKernelGGL(pack3_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream,
                       w3, s, w3_up, s_up, rows, k, geo.L, geo.CG, geo.P, units,
                       static_cast<uint8_t *>(dst));
    return hipGetLastError();
}

hipError_t launch_unpack3(const void *src, int64_t rows, int64_t k, const Geometry &geo,
                          uint32_t *w3, uint16_t *s, hipStream_t stream)
{
    const int64_t items = rows * (k / 32);
    hipLaunchKernelGGL(unpack3_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const uint8_t *>(src), rows, k, geo.L, geo.CG, geo.P, w3, s);
    return hipGetLastError();
}

// int3 matmuls: the int4 plan (block, split or multi-pass kernel) with
// 12-byte units; epilogues f16 (GEMV), f32 + argmax (LM head) and SiLU
// (gate/up interleaved rows; n_out = rows / 2).
template <int L, int CG, int EPI>
static void launch_gemv3_lce(const GemvPlan &plan, const Geometry &geo, const uint8_t *wd,
                             const uint16_t *x, void *out, int64_t rows, int64_t k, int64_t n_out,
                             ArgmaxScratch am, hipStream_t stream)
{
    const dim3 grid((unsigned)plan.blocks), block((unsigned)plan.threads);
    const NormArgs nm{nullptr, nullptr, nullptr, 0.f};
    if (plan.mode == MODE_SPLIT)
        hipLaunchKernelGGL((gemv_split_kernel<L, CG, EPI, false, 3>), grid, block, 0, stream, wd, x,
                           out, rows, k, geo.tiles, n_out, am, nm, NoRope{});
    else if (plan.mode == MODE_MULTIPASS)
        hipLaunchKernelGGL((gemv_multipass_kernel<L, CG, EPI, false, 3>), grid, block, 0, stream, wd, x,
                           out, rows, k, geo.P, geo.tiles, n_out, am, nm, NoRope{});
    else
        hipLaunchKernelGGL((gemv_block_kernel<L, CG, EPI, false, 3>), grid, block, 0, stream, wd, x,
                           out, rows, k, geo.tiles, n_out, am, nm, NoRope{});
}

template <int L, int CG>
static bool launch_gemv3_lc(Epilogue epi, const GemvPlan &plan, const Geometry &geo,
                            const uint8_t *wd, const uint16_t *x, void *out, int64_t rows,
                            int64_t k, int64_t n_out, ArgmaxScratch am, hipStream_t stream)
{
    switch (epi) {
    case EPI_F16: launch_gemv3_lce<L, CG, EPI_F16>(plan, geo, wd, x, out, rows, k, n_out, am, stream); return true;
    case EPI_F32: launch_gemv3_lce<L, CG, EPI_F32>(plan, geo, wd, x, out, rows, k, n_out, am, stream); return true;
    case EPI_SILU: launch_gemv3_lce<L, CG, EPI_SILU>(plan, geo, wd, x, out, rows, k, n_out, am, stream); return true;
    default: return false;
    }
}

template <int L>
static bool launch_gemv3_l(Epilogue epi, const GemvPlan &plan, const Geometry &geo,
                           const uint8_t *wd, const uint16_t *x, void *out, int64_t rows, int64_t k,
                           int64_t n_out, ArgmaxScratch am, hipStream_t stream)
{
    switch (geo.CG) {
    case 1: return launch_gemv3_lc<L, 1>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream);
    case 2: return launch_gemv3_lc<L, 2>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream);
    case 3: return launch_gemv3_lc<L, 3>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream);
    case 4: return launch_gemv3_lc<L, 4>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream);
    }
    return false;
}

hipError_t launch_gemv3(const Geometry &geo, Epilogue epi, const void *wdata, const uint16_t *x,
                        void *out, int64_t rows, int64_t k, int64_t n_out, ArgmaxScratch am,
                        hipStream_t stream)
{
    if (geo.P == 1 && k > kBlockXHalves)
        return hipErrorInvalidValue;
    const GemvPlan plan = plan_gemv(geo, device_cus());
    const uint8_t *wd = static_cast<const uint8_t *>(wdata);
    bool ok = false;
    switch (geo.L) {
    case 64: ok = launch_gemv3_l<64>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream); break;
    case 32: ok = launch_gemv3_l<32>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream); break;
    case 16: ok = launch_gemv3_l<16>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream); break;
    case 8: ok = launch_gemv3_l<8>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream); break;
    case 4: ok = launch_gemv3_l<4>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream); break;
    case 2: ok = launch_gemv3_l<2>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream); break;
    case 1: ok = launch_gemv3_l<1>(epi, plan, geo, wd, x, out, rows, k, n_out, am, stream); break;
    }
    if (!ok)
        return hipErrorInvalidValue;
    return hipGetLastError();
}

struct GemvArgs {
    const uint8_t *wd;
    const uint16_t *x;
    void *out;
    int64_t rows, k, n_out;
    const Geometry *geo;
    ArgmaxScratch am;
    NormArgs nm;
    const RopeTab *rp;   // EPI_ROPE only
};

template <int EPI>
static typename RopeParam<EPI>::type rope_param(const GemvArgs &a)
{
    if constexpr (EPI == EPI_ROPE)
        return *a.rp;
    else
        return NoRope{};
}

template <int L, int CG, int EPI, bool NORM>
static void launch_lcen(const GemvPlan &plan, const GemvArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)plan.blocks), block((unsigned)plan.threads);
    switch (plan.mode) {
    case MODE_SPLIT:
        hipLaunchKernelGGL((gemv_split_kernel<L, CG, EPI, NORM>), grid, block, 0, stream, a.wd, a.x,
                           a.out, a.rows, a.k, a.geo->tiles, a.n_out, a.am, a.nm, rope_param<EPI>(a));
        break;
    case MODE_MULTIPASS:
        hipLaunchKernelGGL((gemv_multipass_kernel<L, CG, EPI, NORM>), grid, block, 0, stream, a.wd,
                           a.x, a.out, a.rows, a.k, a.geo->P, a.geo->tiles, a.n_out, a.am, a.nm, rope_param<EPI>(a));
        break;
    case MODE_BLOCK:
        hipLaunchKernelGGL((gemv_block_kernel<L, CG, EPI, NORM>), grid, block, 0, stream, a.wd, a.x,
                           a.out, a.rows, a.k, a.geo->tiles, a.n_out, a.am, a.nm, rope_param<EPI>(a));
        break;
    }
}

template <int L, int CG>
static void launch_lc(Epilogue epi, bool norm, const GemvPlan &plan, const GemvArgs &a,
                      hipStream_t stream)
{
    switch (epi) {
    case EPI_F16:
        if (norm)
            launch_lcen<L, CG, EPI_F16, true>(plan, a, stream);
        else
            launch_lcen<L, CG, EPI_F16, false>(plan, a, stream);
        break;
    case EPI_F32: launch_lcen<L, CG, EPI_F32, false>(plan, a, stream); break;
    case EPI_SILU:
        if (norm)
            launch_lcen<L, CG, EPI_SILU, true>(plan, a, stream);
        else
            launch_lcen<L, CG, EPI_SILU, false>(plan, a, stream);
        break;
    case EPI_ROPE:
        if (norm)
            launch_lcen<L, CG, EPI_ROPE, true>(plan, a, stream);
        else
            launch_lcen<L, CG, EPI_ROPE, false>(plan, a, stream);
        break;
    }
}

template <int L>
static bool launch_l(Epilogue epi, bool norm, const GemvPlan &plan, const GemvArgs &a,
                     hipStream_t stream)
{
    switch (a.geo->CG) {
    case 1: launch_lc<L, 1>(epi, norm, plan, a, stream); return true;
    case 2: launch_lc<L, 2>(epi, norm, plan, a, stream); return true;
    case 3: launch_lc<L, 3>(epi, norm, plan, a, stream); return true;
    case 4: launch_lc<L, 4>(epi, norm, plan, a, stream); return true;
    }
    return false;
}

hipError_t launch_gemv_family(const Geometry &geo, Epilogue epi, const void *wdata,
                              const uint16_t *x, void *out, int64_t rows, int64_t k,
                              int64_t n_out, ArgmaxScratch am, const NormArgs *norm,
                              const RopeArgs *rope, hipStream_t stream)
{
    if (norm != nullptr && epi == EPI_F32)
        return hipErrorInvalidValue;   // the LM head takes no norm prologue
    if ((epi == EPI_ROPE) != (rope != nullptr))
        return hipErrorInvalidValue;
    if (rope != nullptr && (rope->d < 2 || rope->d / 2 > kRopeMaxHalf))
        return hipErrorInvalidValue;
    const GemvPlan plan = plan_gemv(geo, device_cus());
    RopeTab tab{};
    if (rope != nullptr) {
        // the twiddles in f64 on the host, passed to the kernel as f32
        tab.d = rope->d;
        tab.nq = rope->nq;
        tab.nkv = rope->nkv;
        tab.pos = rope->pos;
        tab.cache = rope->cache;
        tab.page_table = rope->page_table;
        tab.n_pages = rope->n_pages;
        for (int i = 0; i < rope->d / 2; ++i) {
            const double ang = (double)rope->pos * pow(rope->base, -2.0 * (double)i / (double)rope->d);
            tab.cs[i][0] = (float)cos(ang);
            tab.cs[i][1] = (float)sin(ang);
        }
    }
    const GemvArgs a{static_cast<const uint8_t *>(wdata), x, out, rows, k, n_out, &geo, am,
                     norm != nullptr ? *norm : NormArgs{nullptr, nullptr, nullptr, 0.f}, &tab};
    const bool nrm = norm != nullptr;
    bool ok = false;
    switch (geo.L) {
    case 64: ok = launch_l<64>(epi, nrm, plan, a, stream); break;
    case 32: ok = launch_l<32>(epi, nrm, plan, a, stream); break;
    case 16: ok = launch_l<16>(epi, nrm, plan, a, stream); break;
    case 8: ok = launch_l<8>(epi, nrm, plan, a, stream); break;
    case 4: ok = launch_l<4>(epi, nrm, plan, a, stream); break;
    case 2: ok = launch_l<2>(epi, nrm, plan, a, stream); break;
    case 1: ok = launch_l<1>(epi, nrm, plan, a, stream); break;
    }
    if (!ok)
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace q4
