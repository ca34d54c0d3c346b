// q4_gemm.hip -- batched form of the int4 dequantizing matmul,
// Y[m][n] = sum_k X[m][k] * (q[n][k] - 8) * s[n][k/32], on gfx950.
//
// Source: "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权"
// (zingnex.cn), section 技术限制与诚实声明: batched-prefill shaders exist for
// prompt processing; the pages give no design for them.
//
// Kernels:
//  * VALU, m = 1 (or a layout the MFMA kernels do not take): the streaming
//    kernel -- CG wavefronts per block walk tiles, wavefront j takes group
//    slot j of every lane, so each lane keeps that group's x slices for up to
//    8 activation rows in VGPRs for the whole launch and one pass over W
//    serves 8 rows; codes are dequantized once per word (exact q - 8) and
//    reused for every row.  Multi-pass layouts (k > 8192) use a per-tile
//    variant that re-reads the x slices of each pass.
//  * MFMA, m >= 2: the K-split kernel.  A block owns 64 or 128 weight rows
//    and 32 to 128 activation rows; its wavefronts split K, each staging its
//    own X slices in its own LDS region (no block barrier until the end,
//    where the partial tiles are added in wavefront order).  Each lane loads
//    the 16-byte unit of codes that is its own A operand of
//    v_mfma_f32_32x32x16_f16 (row lane % 32, one of two groups by lane / 32)
//    and dequantizes it to f16 (q - 8) * s (one rounding, relative error
//    <= 2^-11) in registers; the step's four MFMAs take word w of every unit.
//    Inside each 8-k word the k order of both operands is (0,4,1,5,2,6,3,7)
//    -- the order the nibble masks produce -- which leaves the contraction
//    unchanged.
//  * MFMA, m > 128 with k > 4096: the weight-direct kernel, the same operand
//    scheme on v_mfma_f32_16x16x32_f16 with 128 x 128 block tiles whose X
//    slab of a step is shared by the block's 4 wavefronts.
// int3 weights (12-byte units of 32 codes, one pass) run through the same
// kernels with their own dequant: exact (q - 4) pairs on the VALU path, f16
// (q - 4) * s put back in k order for the MFMA kernel (X is not re-paired).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "q4_geometry.h"
#include "q4_internal.h"
#include "q4_lanes.h"

namespace q4 {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ float f16_value(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ uint16_t f16_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

struct Masks {
    uint32_t lo, hi, magic, magic_hi;
};

// masks in VGPRs so that (w & mask) | magic is a single v_and_or_b32
__device__ __forceinline__ Masks masks()
{
    Masks k;
    asm("v_mov_b32 %0, 0x000F000F" : "=v"(k.lo));
    asm("v_mov_b32 %0, 0x00F000F0" : "=v"(k.hi));
    asm("v_mov_b32 %0, 0x64006400" : "=v"(k.magic));
    asm("v_mov_b32 %0, 0x54005400" : "=v"(k.magic_hi));
    return k;
}

// Word of 8 codes -> (q-8) as f16 pairs (k0,k4) (k1,k5) (k2,k6) (k3,k7), all
// exact: 0x6400 | q is 1024 + q, and 0x5400 | (q << 4) is 64 + q (the f16
// ulp at 64 is 1/16), so subtracting 1032 or 72 leaves q - 8.
__device__ __forceinline__ void dequant_word_unit(uint32_t w, const Masks &m, h2 &a0, h2 &a1,
                                                  h2 &a2, h2 &a3)
{
    const h2 k1 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 k2 = {(_Float16)72.0f, (_Float16)72.0f};
    const uint32_t b = w >> 8;
    a0 = as_h2((w & m.lo) | m.magic) - k1;
    a1 = as_h2((w & m.hi) | m.magic_hi) - k2;
    a2 = as_h2((b & m.lo) | m.magic) - k1;
    a3 = as_h2((b & m.hi) | m.magic_hi) - k2;
}

// Word of 8 codes -> (q-8) as f16 pairs (k0,k4) (k1,k5) (k2,k6) (k3,k7), exact
// (the x16 pairs carry 16 (q - 8)).
__device__ __forceinline__ void dequant_word(uint32_t w, const Masks &m, h2 &a0, h2 &a1, h2 &a2,
                                             h2 &a3)
{
    const h2 k1 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 k16 = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t b = w >> 8;
    a0 = as_h2((w & m.lo) | m.magic) - k1;
    a1 = as_h2((w & m.hi) | m.magic) - k16;
    a2 = as_h2((b & m.lo) | m.magic) - k1;
    a3 = as_h2((b & m.hi) | m.magic) - k16;
}

// ------------------------------------------------------------ int3 units --
//
// An int3 lane unit is 12 bytes (3 words) for one group of 32 codes: word i
// holds codes 10i + m at bits 3m and 10i + 5 + m at bits 16 + 3m (m = 0..4),
// bit i of codes 30 / 31 at bits 15 / 31.  Dequantised here to exact
// (q - 4) f16 pairs P[5i + m] = (c(10i+m), c(10i+5+m)), P[15] = (c30, c31):
// a code masked in place at bits 0, 3 or 6 of a half reads as 1024 + q,
// 128 + q or 16 + q under the exponents 0x6400, 0x5800, 0x4C00 (f16 ulp 1,
// 1/8, 1/64), and 1028, 132 or 20 is subtracted.
struct Masks3 {
    uint32_t m0, m3, m6, b1, b2, b4, e1024, e128, e16;
};

__device__ __forceinline__ Masks3 masks3()
{
    Masks3 k;
    asm("v_mov_b32 %0, 0x00070007" : "=v"(k.m0));
    asm("v_mov_b32 %0, 0x00380038" : "=v"(k.m3));
    asm("v_mov_b32 %0, 0x01C001C0" : "=v"(k.m6));
    asm("v_mov_b32 %0, 0x00010001" : "=v"(k.b1));
    asm("v_mov_b32 %0, 0x00020002" : "=v"(k.b2));
    asm("v_mov_b32 %0, 0x00040004" : "=v"(k.b4));
    asm("v_mov_b32 %0, 0x64006400" : "=v"(k.e1024));
    asm("v_mov_b32 %0, 0x58005800" : "=v"(k.e128));
    asm("v_mov_b32 %0, 0x4C004C00" : "=v"(k.e16));
    return k;
}

__device__ __forceinline__ void dequant_unit3(uint32_t w0, uint32_t w1, uint32_t w2, const Masks3 &k,
                                              h2 (&P)[16])
{
    const h2 o1 = {(_Float16)1028.0f, (_Float16)1028.0f};
    const h2 o8 = {(_Float16)132.0f, (_Float16)132.0f};
    const h2 o64 = {(_Float16)20.0f, (_Float16)20.0f};
    const uint32_t w[3] = {w0, w1, w2};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const uint32_t v = w[i], t = v >> 9;
        P[5 * i + 0] = as_h2((v & k.m0) | k.e1024) - o1;
        P[5 * i + 1] = as_h2((v & k.m3) | k.e128) - o8;
        P[5 * i + 2] = as_h2((v & k.m6) | k.e16) - o64;
        P[5 * i + 3] = as_h2((t & k.m0) | k.e1024) - o1;
        P[5 * i + 4] = as_h2((t & k.m3) | k.e128) - o8;
    }
    uint32_t e = ((w0 >> 15) & k.b1) | k.e1024;
    e = ((w1 >> 14) & k.b2) | e;
    e = ((w2 >> 13) & k.b4) | e;
    P[15] = as_h2(e) - o1;
}

// the 32 values of a unit's pairs back in k order, 8 halves per uint4
__device__ __forceinline__ void pairs3_to_k(const h2 (&P)[16], uint4 (&out)[4])
{
    auto half = [&](int kk) -> uint32_t {
        const int pi = kk == 30 ? 15 : kk == 31 ? 15 : 5 * (kk / 10) + (kk % 10) % 5;
        const int hi = kk == 30 ? 0 : kk == 31 ? 1 : (kk % 10) >= 5;
        return (as_u32(P[pi]) >> (16 * hi)) & 0xFFFFu;
    };
    uint32_t d[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
        d[q] = half(2 * q) | (half(2 * q + 1) << 16);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        out[q] = make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
}

// x of one group (32 halves in k order, 4 uint4) -> the pairs matching P
__device__ __forceinline__ void pair3_x(const uint4 (&n)[4], uint4 (&xp)[4])
{
    const uint32_t nn[16] = {n[0].x, n[0].y, n[0].z, n[0].w, n[1].x, n[1].y, n[1].z, n[1].w,
                             n[2].x, n[2].y, n[2].z, n[2].w, n[3].x, n[3].y, n[3].z, n[3].w};
    auto half = [&](int kk) -> uint32_t { return (nn[kk >> 1] >> ((kk & 1) * 16)) & 0xFFFFu; };
    uint32_t d[16];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int mm = 0; mm < 5; ++mm)
            d[5 * i + mm] = half(10 * i + mm) | (half(10 * i + 5 + mm) << 16);
    d[15] = nn[15];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        xp[q] = make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
}

// Per-format sizes: lane unit bytes US and unit slot bytes UB (64 lanes).
template <int FMT>
struct GFmt {
    static constexpr int US = FMT == 4 ? 16 : 12;
    static constexpr int UB = 64 * US;
    static constexpr int PASS = 2 * UB + 256;   // bytes per group slot per pass (x CG)
};

typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v3u __attribute__((ext_vector_type(3)));

template <int FMT>
__device__ __forceinline__ v4u load_unit_g(__amdgpu_buffer_rsrc_t rs, int off)
{
    if constexpr (FMT == 4) {
        return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    } else {
        const v3u v = __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, 0);
        return v4u{v.x, v.y, v.z, 0u};
    }
}

template <int FMT>
__device__ __forceinline__ v4u load_unit_gs(__amdgpu_buffer_rsrc_t rs, int voff, int soff)
{
    if constexpr (FMT == 4) {
        return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
    } else {
        const v3u v = __builtin_amdgcn_raw_buffer_load_b96(rs, voff, soff, 0);
        return v4u{v.x, v.y, v.z, 0u};
    }
}

// natural x pairs of one word (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> (x0,x4)(x1,x5)(x2,x6)(x3,x7)
__device__ __forceinline__ uint4 pair_word(uint4 n)
{
    uint4 r;
    r.x = (n.x & 0xFFFFu) | (n.z << 16);
    r.y = (n.x >> 16) | (n.z & 0xFFFF0000u);
    r.z = (n.y & 0xFFFFu) | (n.w << 16);
    r.w = (n.y >> 16) | (n.w & 0xFFFF0000u);
    return r;
}

// ------------------------------------------------------------ VALU path --

constexpr int kValuRows = 8;   // activation rows per pass over W

// Single-pass layouts: the streaming VALU kernel.  A block of CG wavefronts
// walks tiles blockIdx.x, + gridDim.x, ...; wavefront j takes group slot j
// of every lane, so a lane meets the same group of 32 k in every tile and
// keeps that group's x slices for all MC activation rows in VGPRs for the
// whole launch.  PT tiles of codes and scales are in flight per wavefront.
// Each code word is dequantized once (exact q - 8) and reused for every
// row; per tile the lane sums of a row are reduced across its L lanes, and
// the CG slot sums are added in slot order through LDS (one barrier per
// tile, double-buffered).
#ifndef Q4_VALU_TILES_IN_FLIGHT
#define Q4_VALU_TILES_IN_FLIGHT 2
#endif
#ifndef Q4_VALU_BLOCKS_PER_CU
#define Q4_VALU_BLOCKS_PER_CU 2
#endif

template <int L, int CG, int MC, int PT, int FMT = 4>
__global__ __launch_bounds__(64 * CG) void gemm_valu_stream_kernel(
    const uint8_t *__restrict__ wd, const uint16_t *__restrict__ X, uint16_t *__restrict__ Y,
    int64_t m0, int64_t n, int64_t k, int64_t tiles)
{
    constexpr int TR = 128 / L;
    constexpr int HP = 64 / L;   // row pairs per tile
    constexpr int PB = CG * GFmt<FMT>::PASS;
    constexpr int UB = GFmt<FMT>::UB, US = GFmt<FMT>::US;
    __shared__ float part[2][CG][HP][MC][2];
    const int lane = threadIdx.x & 63;
    const int j = threadIdx.x >> 6;
    const int s = lane / L, c = lane % L;
    const int64_t G = k >> 5;
    const int64_t g = (int64_t)c * CG + j;
    const Masks mk = FMT == 4 ? masks() : Masks{};
    const Masks3 mk3 = FMT == 3 ? masks3() : Masks3{};

    // x pairs of this lane's group for every row: int4 per word (pair_word),
    // int3 for the whole unit (pair3_x)
    uint4 xq[MC][4];
#pragma unroll
    for (int r = 0; r < MC; ++r) {
        const uint4 *src = reinterpret_cast<const uint4 *>(X + (m0 + r) * k + g * 32);
        if constexpr (FMT == 4) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xq[r][q] = g < G ? pair_word(src[q]) : make_uint4(0, 0, 0, 0);
        } else {
            uint4 nat[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                nat[q] = g < G ? src[q] : make_uint4(0, 0, 0, 0);
            pair3_x(nat, xq[r]);
        }
    }

    // this lane's two units and two scales inside a tile
    const int wo0 = j * UB + lane * US, wo1 = (CG + j) * UB + lane * US;
    const int so0 = 2 * CG * UB + lane * 4 * CG + j * 2, so1 = so0 + CG * 2;
    struct Regs {
        v4u w0, w1;
        uint32_t s0, s1;
    };
    auto load = [&](Regs &r, int64_t t) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(wd + (t < tiles ? t : 0) * PB), (short)0, t < tiles ? PB : 0,
            0x00020000);
        r.w0 = load_unit_g<FMT>(rs, wo0);
        r.w1 = load_unit_g<FMT>(rs, wo1);
        r.s0 = __builtin_amdgcn_raw_buffer_load_b32(rs, so0 & ~3, 0, 0);
        r.s1 = __builtin_amdgcn_raw_buffer_load_b32(rs, so1 & ~3, 0, 0);
    };

    const int64_t stride = gridDim.x;
    Regs ring[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q)
        load(ring[q], (int64_t)blockIdx.x + q * stride);
    int buf = 0;
    for (int64_t t = blockIdx.x; t < tiles; t += PT * stride) {
#pragma unroll
        for (int q = 0; q < PT; ++q) {
            const int64_t tt = t + q * stride;
            if (tt >= tiles)
                break;
            float p[MC][2];
#pragma unroll
            for (int r = 0; r < MC; ++r)
                p[r][0] = p[r][1] = 0.f;
            if constexpr (FMT == 4) {
                const uint32_t w0[4] = {ring[q].w0.x, ring[q].w0.y, ring[q].w0.z, ring[q].w0.w};
                const uint32_t w1[4] = {ring[q].w1.x, ring[q].w1.y, ring[q].w1.z, ring[q].w1.w};
#pragma unroll
                for (int wq = 0; wq < 4; ++wq) {
                    h2 a0, a1, a2, a3, b0, b1, b2, b3;
                    dequant_word_unit(w0[wq], mk, a0, a1, a2, a3);
                    dequant_word_unit(w1[wq], mk, b0, b1, b2, b3);
#pragma unroll
                    for (int r = 0; r < MC; ++r) {
                        p[r][0] = __builtin_amdgcn_fdot2(a0, as_h2(xq[r][wq].x), p[r][0], false);
                        p[r][1] = __builtin_amdgcn_fdot2(b0, as_h2(xq[r][wq].x), p[r][1], false);
                        p[r][0] = __builtin_amdgcn_fdot2(a1, as_h2(xq[r][wq].y), p[r][0], false);
                        p[r][1] = __builtin_amdgcn_fdot2(b1, as_h2(xq[r][wq].y), p[r][1], false);
                        p[r][0] = __builtin_amdgcn_fdot2(a2, as_h2(xq[r][wq].z), p[r][0], false);
                        p[r][1] = __builtin_amdgcn_fdot2(b2, as_h2(xq[r][wq].z), p[r][1], false);
                        p[r][0] = __builtin_amdgcn_fdot2(a3, as_h2(xq[r][wq].w), p[r][0], false);
                        p[r][1] = __builtin_amdgcn_fdot2(b3, as_h2(xq[r][wq].w), p[r][1], false);
                    }
                }
            } else {
                h2 A[16], B[16];
                dequant_unit3(ring[q].w0.x, ring[q].w0.y, ring[q].w0.z, mk3, A);
                dequant_unit3(ring[q].w1.x, ring[q].w1.y, ring[q].w1.z, mk3, B);
#pragma unroll
                for (int r = 0; r < MC; ++r) {
                    const uint32_t xr[16] = {xq[r][0].x, xq[r][0].y, xq[r][0].z, xq[r][0].w,
                                             xq[r][1].x, xq[r][1].y, xq[r][1].z, xq[r][1].w,
                                             xq[r][2].x, xq[r][2].y, xq[r][2].z, xq[r][2].w,
                                             xq[r][3].x, xq[r][3].y, xq[r][3].z, xq[r][3].w};
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        p[r][0] = __builtin_amdgcn_fdot2(A[i], as_h2(xr[i]), p[r][0], false);
                        p[r][1] = __builtin_amdgcn_fdot2(B[i], as_h2(xr[i]), p[r][1], false);
                    }
                }
            }
            const float sc0 = f16_value((uint16_t)(ring[q].s0 >> ((so0 & 2) * 8)));
            const float sc1 = f16_value((uint16_t)(ring[q].s1 >> ((so1 & 2) * 8)));
            // the tile's arithmetic is issued before its registers are refilled
            asm volatile("" ::"v"(p[0][0]), "v"(p[0][1]) : "memory");
            load(ring[q], tt + PT * stride);   // past the end: a zero-size resource
#pragma unroll
            for (int r = 0; r < MC; ++r) {
                const float v0 = lanes::reduce<L>(sc0 * p[r][0]);
                const float v1 = lanes::reduce<L>(sc1 * p[r][1]);
                if (c == 0) {
                    part[buf][j][s][r][0] = v0;
                    part[buf][j][s][r][1] = v1;
                }
            }
            __syncthreads();
            for (int o = threadIdx.x; o < MC * TR; o += 64 * CG) {
                const int r = o / TR, row = o % TR;
                float y = part[buf][0][row >> 1][r][row & 1];
#pragma unroll
                for (int jj = 1; jj < CG; ++jj)
                    y += part[buf][jj][row >> 1][r][row & 1];
                const int64_t nn = tt * TR + row;
                if (nn < n)
                    Y[(m0 + r) * n + nn] = f16_bits(y);
            }
            buf ^= 1;
        }
    }
}

// Multi-pass layouts (k > 8192): block = CG wavefronts on one tile at a
// time; wavefront j takes group slot j of every lane, and the x slices of
// each pass are read again for every tile.  Rows m0 .. m0 + MC - 1 of X
// (MC <= kValuRows) per launch.
template <int L, int CG, int MC, int FMT = 4>
__global__ __launch_bounds__(256) void gemm_valu_multipass_kernel(const uint8_t *__restrict__ wd,
                                                        const uint16_t *__restrict__ X,
                                                        uint16_t *__restrict__ Y, int64_t m0,
                                                        int64_t n, int64_t k, int passes,
                                                        int64_t tiles)
{
    constexpr int TR = 128 / L;
    const int64_t PB = (int64_t)CG * GFmt<FMT>::PASS;
    __shared__ float part[CG][64][2 * MC];
    const int lane = threadIdx.x & 63;
    const int j = threadIdx.x >> 6;
    const int s = lane / L, c = lane % L;
    const int64_t G = k >> 5;
    const Masks mk = FMT == 4 ? masks() : Masks{};
    const Masks3 mk3 = FMT == 3 ? masks3() : Masks3{};
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        float acc[MC][2];
#pragma unroll
        for (int r = 0; r < MC; ++r)
            acc[r][0] = acc[r][1] = 0.f;
        for (int p = 0; p < passes; ++p) {
            const int64_t g = (int64_t)p * L * CG + (int64_t)c * CG + j;
            const uint8_t *base = wd + (t * passes + p) * PB;
            if constexpr (FMT == 3) {
                // exact (q - 4) pairs of the lane's two units; x re-paired to match
                constexpr int UB = GFmt<3>::UB;
                const uint32_t *u0 = reinterpret_cast<const uint32_t *>(base + j * UB + lane * 12);
                const uint32_t *u1 = reinterpret_cast<const uint32_t *>(base + (CG + j) * UB + lane * 12);
                const uint16_t *sp = reinterpret_cast<const uint16_t *>(base + 2 * CG * UB + lane * 4 * CG);
                const float s0 = f16_value(sp[j]), s1 = f16_value(sp[CG + j]);
                h2 A[16], B[16];
                dequant_unit3(u0[0], u0[1], u0[2], mk3, A);
                dequant_unit3(u1[0], u1[1], u1[2], mk3, B);
#pragma unroll
                for (int r = 0; r < MC; ++r) {
                    uint4 nat[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                                    make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
                    if (g < G) {
                        const uint4 *src = reinterpret_cast<const uint4 *>(X + (m0 + r) * k + g * 32);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            nat[q] = src[q];
                    }
                    uint4 xp[4];
                    pair3_x(nat, xp);
                    const uint32_t xr[16] = {xp[0].x, xp[0].y, xp[0].z, xp[0].w, xp[1].x, xp[1].y,
                                             xp[1].z, xp[1].w, xp[2].x, xp[2].y, xp[2].z, xp[2].w,
                                             xp[3].x, xp[3].y, xp[3].z, xp[3].w};
                    float a = 0.f, b = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        a = __builtin_amdgcn_fdot2(A[i], as_h2(xr[i]), a, false);
                        b = __builtin_amdgcn_fdot2(B[i], as_h2(xr[i]), b, false);
                    }
                    acc[r][0] = fmaf(s0, a, acc[r][0]);
                    acc[r][1] = fmaf(s1, b, acc[r][1]);
                }
                continue;
            }
            const uint4 c0 = *reinterpret_cast<const uint4 *>(base + j * 1024 + lane * 16);
            const uint4 c1 = *reinterpret_cast<const uint4 *>(base + (CG + j) * 1024 + lane * 16);
            const uint16_t *sp =
                reinterpret_cast<const uint16_t *>(base + 2 * CG * 1024 + lane * 4 * CG);
            const float s0 = f16_value(sp[j]), s1 = f16_value(sp[CG + j]);
            h2 d0[4][4], d1[4][4];   // [word][pair]
            const uint32_t w0[4] = {c0.x, c0.y, c0.z, c0.w}, w1[4] = {c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                dequant_word(w0[q], mk, d0[q][0], d0[q][1], d0[q][2], d0[q][3]);
                dequant_word(w1[q], mk, d1[q][0], d1[q][1], d1[q][2], d1[q][3]);
            }
#pragma unroll
            for (int r = 0; r < MC; ++r) {
                uint4 xq[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                               make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
                if (g < G) {
                    const uint4 *src = reinterpret_cast<const uint4 *>(X + (m0 + r) * k + g * 32);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        xq[q] = pair_word(src[q]);
                }
                float a1 = 0.f, a16 = 0.f, b1 = 0.f, b16 = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    a1 = __builtin_amdgcn_fdot2(d0[q][0], as_h2(xq[q].x), a1, false);
                    a16 = __builtin_amdgcn_fdot2(d0[q][1], as_h2(xq[q].y), a16, false);
                    a1 = __builtin_amdgcn_fdot2(d0[q][2], as_h2(xq[q].z), a1, false);
                    a16 = __builtin_amdgcn_fdot2(d0[q][3], as_h2(xq[q].w), a16, false);
                    b1 = __builtin_amdgcn_fdot2(d1[q][0], as_h2(xq[q].x), b1, false);
                    b16 = __builtin_amdgcn_fdot2(d1[q][1], as_h2(xq[q].y), b16, false);
                    b1 = __builtin_amdgcn_fdot2(d1[q][2], as_h2(xq[q].z), b1, false);
                    b16 = __builtin_amdgcn_fdot2(d1[q][3], as_h2(xq[q].w), b16, false);
                }
                acc[r][0] = fmaf(s0, fmaf(a16, 0.0625f, a1), acc[r][0]);
                acc[r][1] = fmaf(s1, fmaf(b16, 0.0625f, b1), acc[r][1]);
            }
        }
#pragma unroll
        for (int r = 0; r < MC; ++r) {
            part[j][lane][2 * r] = acc[r][0];
            part[j][lane][2 * r + 1] = acc[r][1];
        }
        __syncthreads();
        if (j == 0) {
            const int64_t r0 = t * TR + 2 * s;
#pragma unroll
            for (int r = 0; r < MC; ++r) {
                float y0 = part[0][lane][2 * r], y1 = part[0][lane][2 * r + 1];
#pragma unroll
                for (int q = 1; q < CG; ++q) {
                    y0 += part[q][lane][2 * r];
                    y1 += part[q][lane][2 * r + 1];
                }
                y0 = lanes::reduce<L>(y0);
                y1 = lanes::reduce<L>(y1);
                if (c == 0) {
                    uint16_t *yr = Y + (m0 + r) * n;
                    if (r0 < n)
                        yr[r0] = f16_bits(y0);
                    if (r0 + 1 < n)
                        yr[r0 + 1] = f16_bits(y1);
                }
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ MFMA path --

constexpr int kGroupsPerStep = 4;                 // K step: 4 groups = 128 k
constexpr int kStepK = 32 * kGroupsPerStep;
constexpr int kLdsRow = kStepK + 8;               // halves per LDS row (+16 B against bank conflicts)

// Weight-direct MFMA kernel: the weight operand never passes through LDS.
// The k order inside one v_mfma_f32_16x16x32_f16 is free as long as both
// operands use the same one, so lane l (row i = l % 16, k block b = l / 16)
// takes the whole 16-byte unit of weight row i and group slot b of the K
// step (4 groups = 128 k), and the step's four MFMAs use word w = 0..3 of
// every lane's unit: MFMA w contracts word w of the step's four groups.
// Each lane dequantizes its own unit with its own scale straight into the A
// operand.  The four wavefronts of a block own different weight rows (16 NT
// each, BN = 64 NT) and share BM = 16 MT activation rows, whose X slab of
// the step is paired into LDS once per block (double-buffered, one barrier
// per step) and read back as B operands.  Per step a wavefront does 4 NT MT
// MFMAs against 4 NT unit dequantizations and 4 MT LDS fragment reads; the
// per-step part of every load address is uniform and rides in the buffer
// instruction's scalar offset, so a load costs no address arithmetic.
template <int L, int CG, int NT, int MT, int FMT = 4>
__global__ __launch_bounds__(256) void gemm_mfma_wx_kernel(const uint8_t *__restrict__ wd,
                                                           int64_t wbytes,
                                                           const uint16_t *__restrict__ X,
                                                           uint16_t *__restrict__ Y, int64_t m,
                                                           int64_t n, int64_t k, int64_t nblocks_n,
                                                           int64_t padded_nblocks_n)
{
    constexpr int BN = 64 * NT, BM = 16 * MT;
    constexpr int TR = 128 / L;
    constexpr int PB = CG * GFmt<FMT>::PASS;
    constexpr int UB = GFmt<FMT>::UB, US = GFmt<FMT>::US;
    constexpr int CBLOCKS = L / kGroupsPerStep > 0 ? L / kGroupsPerStep : 1;   // L >= 4 on this path
    constexpr int STEPS = CG * CBLOCKS;
    constexpr int XC = BM * 16 / 256;                 // 16-byte X chunks per thread per step (MT)
    // steps in flight: about 112 VGPRs of operands (5 per weight unit and
    // scale, 4 per X chunk), at least 2, at most the whole K
    constexpr int PER = 5 * NT + 4 * XC;
    constexpr int DW = 112 / PER > 2 ? 112 / PER : 2;
    constexpr int D = DW < STEPS ? DW : (STEPS > 0 ? STEPS : 1);
    __shared__ _Float16 Xs[2][BM][kLdsRow];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int ri = lane & 15, kb = lane >> 4;
    const int64_t G = k >> 5;

    // XCD-aware order: the M blocks of one weight slab run on one XCD
    const int64_t mblocks = gridDim.x / padded_nblocks_n;
    const int64_t b = blockIdx.x;
    const int64_t grp = b / (8 * mblocks), within = b % (8 * mblocks);
    const int64_t nb = grp * 8 + within % 8;
    const int64_t mb = within / 8;
    if (nb >= nblocks_n)
        return;
    const int64_t nw0 = nb * BN + wv * 16 * NT, mrow0 = mb * BM;

    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(wd), (short)0, (int)wbytes, 0x00020000);
    const int xbytes = (int)(m * k * 2);
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(X), (short)0, xbytes, 0x00020000);
    const Masks mk = FMT == 4 ? masks() : Masks{};
    const Masks3 mk3 = FMT == 3 ? masks3() : Masks3{};

    // Per-lane parts of the unit, scale and X offsets (32-bit: this path takes
    // weights and X below 2 GiB); a step adds a uniform part, passed as the
    // buffer instruction's scalar offset.  A lane past the end of the weight or
    // of X gets num_records as its own offset, so it reads zeros whether or not
    // the scalar offset takes part in the range check.
    int wvo[NT], svo[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int64_t row = nw0 + 16 * t + ri;
        const int64_t tile = row / TR;
        const int sl = (int)((row % TR) >> 1);
        const int uu = (int)(row & 1);
        const int64_t uo = tile * PB + (int64_t)uu * CG * UB + (int64_t)(sl * L + kb) * US;
        const int64_t so = tile * PB + 2 * CG * UB + (int64_t)(sl * L + kb) * 4 * CG + uu * CG * 2;
        wvo[t] = uo < wbytes ? (int)uo : (int)wbytes;
        svo[t] = so < wbytes ? (int)so : (int)wbytes;
    }
    // X slab of a step: thread q = tid + 256 h takes row q / 16, group slot
    // cl = (q / 4) % 4, word q % 4 (four threads read one group's 64
    // contiguous bytes); group slot cl of step (j, cb) is group
    // (4 cb + cl) CG + j, which exists while 4 cb CG + j < G - cl CG
    int xvo[XC], xthr[XC];
#pragma unroll
    for (int h = 0; h < XC; ++h) {
        const int q = tid + 256 * h;
        const int mr = q >> 4, cl = (q >> 2) & 3, wq = q & 3;
        const int64_t mm = mrow0 + mr;
        xvo[h] = mm < m ? (int)((mm * k + cl * CG * 32 + wq * 8) * 2) : xbytes;
        xthr[h] = (int)(G - cl * CG);
    }

    struct WRegs {
        v4u w[NT];
        uint32_t s[NT];
    };
    struct XRegs {
        v4u x[XC];
    };
    auto load_w = [&](WRegs &r, int st) {
        if (st >= STEPS)
            return;                                   // past the end: never used
        const int j = st / CBLOCKS, cb = st % CBLOCKS;
        const int su = j * UB + cb * kGroupsPerStep * US;
        const int ss = cb * kGroupsPerStep * 4 * CG + j * 2;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            r.w[t] = load_unit_gs<FMT>(rs, wvo[t], su);
            r.s[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, svo[t], ss, 0);
        }
    };
    auto load_x = [&](XRegs &r, int st) {
        if (st >= STEPS)
            return;
        const int j = st / CBLOCKS, cb = st % CBLOCKS;
        const int ug = cb * kGroupsPerStep * CG + j;
#pragma unroll
        for (int h = 0; h < XC; ++h)
            r.x[h] = __builtin_amdgcn_raw_buffer_load_b128(xrs, ug < xthr[h] ? xvo[h] : xbytes, ug * 64, 0);
    };
    auto store_x = [&](const XRegs &r, int buf) {
#pragma unroll
        for (int h = 0; h < XC; ++h) {
            const int q = tid + 256 * h;
            {
                const int mr = q >> 4, cl = (q >> 2) & 3, wq = q & 3;
                const uint4 xv = make_uint4(r.x[h].x, r.x[h].y, r.x[h].z, r.x[h].w);
                *reinterpret_cast<uint4 *>(&Xs[buf][mr][cl * 32 + wq * 8]) = FMT == 4 ? pair_word(xv) : xv;
            }
        }
    };
    auto compute = [&](const WRegs &r, int buf, f4 (&acc)[NT][MT]) {
        if constexpr (FMT == 4) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                h8 af[NT], bf[MT];
#pragma unroll
                for (int jj = 0; jj < MT; ++jj)
                    bf[jj] = *reinterpret_cast<const h8 *>(&Xs[buf][jj * 16 + ri][kb * 32 + w * 8]);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(r.s[t] & 0xFFFFu));
                    const h2 sc = {sv, sv};
                    const uint32_t word = w == 0 ? r.w[t].x : w == 1 ? r.w[t].y : w == 2 ? r.w[t].z : r.w[t].w;
                    h2 a0, a1, a2, a3;
                    dequant_word_unit(word, mk, a0, a1, a2, a3);
                    // one f16 rounding of (q - 8) * s
                    af[t] = __builtin_bit_cast(h8, make_uint4(as_u32(a0 * sc), as_u32(a1 * sc),
                                                              as_u32(a2 * sc), as_u32(a3 * sc)));
                }
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int jj = 0; jj < MT; ++jj)
                        acc[t][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t], bf[jj], acc[t][jj], 0, 0, 0);
            }
        } else {
            // one f16 rounding of (q - 4) * s, back in k order; X stays natural
            uint4 ak[NT][4];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(r.s[t] & 0xFFFFu));
                const h2 sc = {sv, sv};
                h2 P[16];
                dequant_unit3(r.w[t].x, r.w[t].y, r.w[t].z, mk3, P);
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    P[q] = P[q] * sc;
                pairs3_to_k(P, ak[t]);
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                h8 bf[MT];
#pragma unroll
                for (int jj = 0; jj < MT; ++jj)
                    bf[jj] = *reinterpret_cast<const h8 *>(&Xs[buf][jj * 16 + ri][kb * 32 + w * 8]);
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int jj = 0; jj < MT; ++jj)
                        acc[t][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, ak[t][w]),
                                                                           bf[jj], acc[t][jj], 0, 0, 0);
            }
        }
    };

    f4 acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int jj = 0; jj < MT; ++jj)
            acc[t][jj] = f4{0.f, 0.f, 0.f, 0.f};
    // W of steps s .. s + D - 1 and X of steps s + 1 .. s + D in registers;
    // X of step s in LDS buffer s & 1
    WRegs wr[D];
    XRegs xr[D];
    XRegs x0;
    load_x(x0, 0);
#pragma unroll
    for (int i = 0; i < D; ++i) {
        load_w(wr[i], i);
        load_x(xr[(i + 1) % D], i + 1);
    }
    store_x(x0, 0);
    __syncthreads();
    for (int st = 0; st < STEPS; st += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int cur = st + i;
            if (cur < STEPS) {
                if (cur + 1 < STEPS)
                    store_x(xr[(i + 1) % D], (cur + 1) & 1);   // the buffer step cur - 1 read
                compute(wr[i], cur & 1, acc);
                load_w(wr[i], cur + D);                        // past the end reads nothing
                load_x(xr[(i + 1) % D], cur + 1 + D);
                __syncthreads();
            }
        }
    }
    // D[i][j]: lane holds weight rows 4 (lane / 16) + r of tile t, activation
    // row lane % 16 of tile jj
    const bool vec = (n & 3) == 0 && (reinterpret_cast<uintptr_t>(Y) & 7) == 0;
#pragma unroll
    for (int jj = 0; jj < MT; ++jj) {
        const int64_t mm = mrow0 + jj * 16 + ri;
        if (mm >= m)
            continue;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int64_t nn = nw0 + 16 * t + 4 * kb;
            if (vec && nn + 3 < n) {
                const uint32_t lo = f16_bits(acc[t][jj][0]) | ((uint32_t)f16_bits(acc[t][jj][1]) << 16);
                const uint32_t hi = f16_bits(acc[t][jj][2]) | ((uint32_t)f16_bits(acc[t][jj][3]) << 16);
                *reinterpret_cast<uint2 *>(Y + mm * n + nn) = make_uint2(lo, hi);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (nn + r < n)
                        Y[mm * n + nn + r] = f16_bits(acc[t][jj][r]);
            }
        }
    }
}

// K-split MFMA kernel (v_mfma_f32_32x32x16_f16).  A block owns BN = 32 NA
// weight rows (NA A tiles of 32) and BM = 32 MT activation rows, and its NW
// wavefronts split K instead of the rows: wavefront w takes a contiguous
// run of the row's steps, a step being one group pair (c, c + 1) of lane
// positions at one group slot j -- groups (2p) CG + j and (2p + 1) CG + j.
// Lane l (row l % 32 of a tile, half h = l / 32) loads the 16-byte unit of
// its row and of group 2p + h (so each row's two units of a step are 32
// contiguous bytes), dequantizes it to f16 (q - 8) * s in registers, and
// the step's MFMAs take word w = 0..3 of every unit; the B operand of word
// w, half h, is the same 8 k of activation row l % 32 (paired as the codes
// are).  Each wavefront stages its own X slab of a step (BM rows x the two
// groups) in its own LDS region and reads it back as B operands, so no
// block barrier is needed until the end, where the NW partial tiles are
// added in wavefront order through the same LDS (32 activation rows at a
// time) and rounded once to f16.  Per step a wavefront does 4 NA MT MFMAs
// against 4 NA dequantized words and 4 MT LDS fragment reads; every weight
// byte is dequantized once per M block, every X byte passes through LDS
// once per weight slab.  XR < BM: only the first XR activation rows exist
// (m <= XR), so only those are loaded and staged; the slab rows past them
// are zeroed once.
template <int L, int CG, int NA, int MT, int NW, int D, int FMT = 4, int XR = 32 * MT>
__global__ __launch_bounds__(64 * NW) void gemm_mfma_ks_kernel(const uint8_t *__restrict__ wd,
                                                               int64_t wbytes,
                                                               const uint16_t *__restrict__ X,
                                                               uint16_t *__restrict__ Y, int64_t m,
                                                               int64_t n, int64_t k, int64_t nblocks_n,
                                                               int64_t padded_nblocks_n)
{
    constexpr int BM = 32 * MT, BN = 32 * NA;
    constexpr int TR = 128 / L;
    constexpr int PB = CG * GFmt<FMT>::PASS;
    constexpr int UB = GFmt<FMT>::UB, US = GFmt<FMT>::US;
    constexpr int NP = L / 2;                        // lane-position pairs of a row (L >= 4 here)
    constexpr int PW = NP > NW ? (NP + NW - 1) / NW : 1;   // pairs per wavefront
    constexpr int SW = PW * CG;                      // steps per wavefront: (pair, slot), slot fastest
    constexpr int XROW = 64 + 8;                     // halves per slab row (+16 B: rows 4 banks apart)
    constexpr int XBUF = BM * XROW;                  // halves per slab buffer
    constexpr int PROW = BN + 4;                     // floats per row of a partial tile
    constexpr int REGION = 4 * XBUF > 4 * 32 * PROW ? 4 * XBUF : 4 * 32 * PROW;   // bytes per wavefront
    constexpr int XC = XR / 8;                       // 16-byte X pieces per lane per step
    constexpr int OPT = BN / (2 * NW);               // outputs per thread per 32 rows of the final sum
    static_assert((OPT == 2 || OPT % 4 == 0) && BN % OPT == 0 && D >= 2, "unsupported BN / NW / D");
    static_assert(XR % 8 == 0 && XR <= BM, "X rows per slab");
    __shared__ __attribute__((aligned(16))) uint8_t lds[NW * REGION];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ri = lane & 31, kh = lane >> 5;
    const int64_t G = k >> 5;

    // XCD-aware order: the M blocks of one weight slab run on one XCD
    const int64_t mblocks = gridDim.x / padded_nblocks_n;
    const int64_t b = blockIdx.x;
    const int64_t grp = b / (8 * mblocks), within = b % (8 * mblocks);
    const int64_t nb = grp * 8 + within % 8;
    const int64_t mb = within / 8;
    if (nb >= nblocks_n)
        return;
    const int64_t n0 = nb * BN, m0 = mb * BM;

    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(wd), (short)0, (int)wbytes, 0x00020000);
    const int xbytes = (int)(m * k * 2);
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(X), (short)0, xbytes, 0x00020000);
    const Masks mk = FMT == 4 ? masks() : Masks{};
    const Masks3 mk3 = FMT == 3 ? masks3() : Masks3{};

    // per-lane unit and scale offsets (lane position c = h of pair 0, slot
    // j = 0); a step (p, j) adds the uniform 2p US + j UB (units) and a pair
    // 2p 4 CG (its scale block: the 4 CG bytes of both rows of a lane pair
    // and every slot) through the scalar offset; rows past n read zero
    int wvo[NA], svo[NA], shalf[NA];
#pragma unroll
    for (int t = 0; t < NA; ++t) {
        const int64_t row = n0 + 32 * t + ri;
        const int64_t tile = row / TR;
        const int sl = (int)((row % TR) >> 1);
        const int uu = (int)(row & 1);
        const int64_t uo = tile * PB + (int64_t)uu * CG * UB + (int64_t)(sl * L + kh) * US;
        const int64_t so = tile * PB + 2 * CG * UB + (int64_t)(sl * L + kh) * 4 * CG;
        wvo[t] = (row < n && uo < wbytes) ? (int)uo : (int)wbytes;
        svo[t] = (row < n && so < wbytes) ? (int)so : (int)wbytes;
        shalf[t] = uu * CG;                          // this row's first half in the block
    }
    // X pieces of a step: piece q = lane + 64 i is row q / 8, half (q / 4) % 2,
    // 16-byte chunk q % 4 of that half's group; the step adds ga * 64 bytes
    // (ga = its first group); a half whose group is past k reads zeros
    int xvo[XC], xthr[XC];
#pragma unroll
    for (int i = 0; i < XC; ++i) {
        const int q = lane + 64 * i;
        const int rr = q >> 3, hh = (q >> 2) & 1, ch = q & 3;
        const int64_t mm = m0 + rr;
        xvo[i] = mm < m ? (int)((mm * k + hh * CG * 32 + ch * 8) * 2) : xbytes;
        xthr[i] = (int)(G - hh * CG);
    }

    struct Regs {
        v4u w[NA];
        v4u x[XC];
    };
    // Every load is issued unconditionally (a branch around loads makes the
    // compiler wait for all of them at the join): a pair past the row's end
    // (the last wavefronts' tail) reads zeros through out-of-range offsets.
    const int p0 = wv * PW;
    auto load = [&](Regs &r, int i) {
        if (i >= SW)
            return;                                   // compile-time: never used
        const int pr = p0 + i / CG, j = i % CG;
        const bool live = pr < NP;
        const int p = live ? pr : 0;
        const int ga = 2 * p * CG + j;
#pragma unroll
        for (int q = 0; q < XC; ++q)
            r.x[q] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (live && ga < xthr[q]) ? xvo[q] : xbytes,
                                                           ga * 64, 0);
#pragma unroll
        for (int t = 0; t < NA; ++t)
            r.w[t] = load_unit_gs<FMT>(rs, live ? wvo[t] : (int)wbytes, 2 * p * US + j * UB);
    };
    // scale blocks of the wavefront's pairs in SR slots, the block of pair
    // pi + SR - 1 requested when pair pi starts (at least two steps ahead)
    constexpr int SA = CG == 1 ? 4 : 2;
    constexpr int SR = PW < SA ? PW : SA;
    v4u sblk[SR][NA];
    auto load_s = [&](int pi) {
        if (pi >= PW)
            return;                                   // compile-time: never used
        const bool live = p0 + pi < NP;
        const int so = 2 * (live ? p0 + pi : 0) * 4 * CG;
#pragma unroll
        for (int t = 0; t < NA; ++t) {
            const int vo = live ? svo[t] : (int)wbytes;
            v4u &d = sblk[pi % SR][t];
            if constexpr (CG == 1) {
                d = v4u{__builtin_amdgcn_raw_buffer_load_b32(rs, vo, so, 0), 0u, 0u, 0u};
            } else if constexpr (CG == 2) {
                const v2u v = __builtin_amdgcn_raw_buffer_load_b64(rs, vo, so, 0);
                d = v4u{v.x, v.y, 0u, 0u};
            } else if constexpr (CG == 3) {
                const v3u v = __builtin_amdgcn_raw_buffer_load_b96(rs, vo, so, 0);
                d = v4u{v.x, v.y, v.z, 0u};
            } else {
                d = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, so, 0);
            }
        }
    };
#pragma unroll
    for (int pi = 0; pi < SR; ++pi)
        load_s(pi);
    // f16 scale of tile t at step i: half u CG + j of the pair's block
    auto scale_of = [&](int i, int t) -> _Float16 {
        const int pi = i / CG, j = i % CG;
        const int hi = shalf[t] + j;
        const v4u b = sblk[pi % SR][t];
        const uint32_t d = (hi >> 1) == 0 ? b.x : (hi >> 1) == 1 ? b.y : (hi >> 1) == 2 ? b.z : b.w;
        return __builtin_bit_cast(_Float16, (uint16_t)((hi & 1) ? (d >> 16) : (d & 0xFFFFu)));
    };
    uint8_t *const base = lds + wv * REGION;
    auto xslab = [&](int buf) { return reinterpret_cast<_Float16 *>(base) + buf * XBUF; };
    auto store_x = [&](const Regs &r, int buf) {
        _Float16 *xs = xslab(buf);
#pragma unroll
        for (int q = 0; q < XC; ++q) {
            const int qq = lane + 64 * q;
            const int rr = qq >> 3, hh = (qq >> 2) & 1, ch = qq & 3;
            const uint4 v = make_uint4(r.x[q].x, r.x[q].y, r.x[q].z, r.x[q].w);
            *reinterpret_cast<uint4 *>(xs + rr * XROW + hh * 32 + ch * 8) = FMT == 4 ? pair_word(v) : v;
        }
    };
    f16v acc[NA][MT];
#pragma unroll
    for (int t = 0; t < NA; ++t)
#pragma unroll
        for (int f = 0; f < MT; ++f)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[t][f][e] = 0.f;
    auto compute = [&](const Regs &r, int i) {
        const _Float16 *xs = xslab(i & 1);
        uint4 ak[NA][4];
#pragma unroll
        for (int t = 0; t < NA; ++t) {
            const _Float16 sv = scale_of(i, t);
            const h2 sc = {sv, sv};
            if constexpr (FMT == 4) {
                const uint32_t wds[4] = {r.w[t].x, r.w[t].y, r.w[t].z, r.w[t].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    h2 a0, a1, a2, a3;
                    dequant_word_unit(wds[w], mk, a0, a1, a2, a3);
                    // one f16 rounding of (q - 8) * s
                    ak[t][w] = make_uint4(as_u32(a0 * sc), as_u32(a1 * sc), as_u32(a2 * sc), as_u32(a3 * sc));
                }
            } else {
                // one f16 rounding of (q - 4) * s, back in k order; X natural
                h2 P[16];
                dequant_unit3(r.w[t].x, r.w[t].y, r.w[t].z, mk3, P);
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    P[q] = P[q] * sc;
                pairs3_to_k(P, ak[t]);
            }
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            h8 bf[MT];
#pragma unroll
            for (int f = 0; f < MT; ++f)
                bf[f] = *reinterpret_cast<const h8 *>(xs + (32 * f + ri) * XROW + kh * 32 + w * 8);
#pragma unroll
            for (int t = 0; t < NA; ++t)
#pragma unroll
                for (int f = 0; f < MT; ++f)
                    acc[t][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, ak[t][w]), bf[f],
                                                                      acc[t][f], 0, 0, 0);
        }
    };

    // W and X of steps i .. i + D - 1 in registers; X of step i in LDS
    // buffer i & 1 (written during step i - 1).  The slab is private to the
    // wavefront: LDS accesses of one wavefront complete in order, and the
    // empty asm statements keep the compiler from moving them across.
    Regs ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i)
        load(ring[i], i);
    if constexpr (XR < BM) {
        // rows XR .. BM - 1 of both slab buffers: 16-byte zeros, 8 per row
#pragma unroll
        for (int q = lane; q < 2 * (BM - XR) * 8; q += 64) {
            const int buf = q / ((BM - XR) * 8), rr = XR + (q / 8) % (BM - XR), ch = q % 8;
            *reinterpret_cast<uint4 *>(xslab(buf) + rr * XROW + ch * 8) = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    store_x(ring[0], 0);
#pragma unroll
    for (int i = 0; i < SW; ++i) {
        if (i + 1 < SW)
            store_x(ring[(i + 1) % D], (i + 1) & 1);
        asm volatile("" ::: "memory");
        compute(ring[i % D], i);
        asm volatile("" ::: "memory");
        load(ring[i % D], i + D);
        if (i % CG == 0 && i > 0)
            load_s(i / CG + SR - 1);
    }

    // partial tiles, 32 activation rows at a time: each wavefront writes its
    // rows 32 f .. 32 f + 31 ([m][n] f32; lane holds activation row 32 f +
    // l % 32, weight rows 32 t + 8 a + 4 h + e) into its own region, then
    // every thread adds OPT outputs over the wavefronts in order
    float *P = reinterpret_cast<float *>(base);
    constexpr int CPR = BN / OPT;
    const int mm = tid / CPR, c = tid % CPR;
    const int64_t gn = n0 + c * OPT;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int f = 0; f < MT; ++f) {
        if (f > 0)
            __syncthreads();                      // the previous rows have been read
#pragma unroll
        for (int t = 0; t < NA; ++t)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *reinterpret_cast<f4 *>(P + ri * PROW + 32 * t + 8 * a + 4 * kh) =
                    f4{acc[t][f][4 * a], acc[t][f][4 * a + 1], acc[t][f][4 * a + 2], acc[t][f][4 * a + 3]};
        __syncthreads();
        float sum[OPT];
#pragma unroll
        for (int e = 0; e < OPT; ++e)
            sum[e] = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float *Pw = reinterpret_cast<const float *>(lds + w * REGION) + mm * PROW + c * OPT;
            if constexpr (OPT == 2) {
                const float2 v = *reinterpret_cast<const float2 *>(Pw);
                sum[0] += v.x;
                sum[1] += v.y;
            } else {
#pragma unroll
                for (int e = 0; e < OPT; e += 4) {
                    const f4 v = *reinterpret_cast<const f4 *>(Pw + e);
                    sum[e] += v[0];
                    sum[e + 1] += v[1];
                    sum[e + 2] += v[2];
                    sum[e + 3] += v[3];
                }
            }
        }
        const int64_t gm = m0 + 32 * f + mm;
        if (gm < m) {
            uint16_t *yr = Y + gm * n + gn;
            if (OPT == 2 && (n % 2) == 0 && (reinterpret_cast<uintptr_t>(Y) & 3) == 0 && gn + 2 <= n) {
                *reinterpret_cast<uint32_t *>(yr) = f16_bits(sum[0]) | ((uint32_t)f16_bits(sum[OPT - 1]) << 16);
            } else if (OPT >= 4 && (n % OPT) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0 && gn + OPT <= n) {
#pragma unroll
                for (int e = 0; e + 3 < OPT; e += 4) {
                    const uint32_t lo = f16_bits(sum[e]) | ((uint32_t)f16_bits(sum[e + 1]) << 16);
                    const uint32_t hi = f16_bits(sum[e + 2]) | ((uint32_t)f16_bits(sum[e + 3]) << 16);
                    *reinterpret_cast<uint2 *>(yr + e) = make_uint2(lo, hi);
                }
            } else {
#pragma unroll
                for (int e = 0; e < OPT; ++e)
                    if (gn + e < n)
                        yr[e] = f16_bits(sum[e]);
            }
        }
    }
}

template <int L, int CG, int FMT>
hipError_t launch_valu_lc(const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                          int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    constexpr int PT = Q4_VALU_TILES_IN_FLIGHT;
    const bool single = geo.P == 1;
    const int64_t cus = device_cus();
    const int64_t cap = single ? cus * Q4_VALU_BLOCKS_PER_CU : cus * 8;
    const dim3 grid((unsigned)(geo.tiles < cap ? geo.tiles : cap)), block(64 * CG);
    for (int64_t m0 = 0; m0 < m; m0 += kValuRows) {
        const int64_t mc = m - m0 < kValuRows ? m - m0 : kValuRows;
        switch (mc) {
#define Q4_VALU_CASE(R)                                                                            \
    case R:                                                                                        \
        if (single)                                                                                \
            hipLaunchKernelGGL((gemm_valu_stream_kernel<L, CG, R, PT, FMT>), grid, block, 0, stream, \
                               wd, X, Y, m0, n, k, geo.tiles);                                     \
        else                                                                                       \
            hipLaunchKernelGGL((gemm_valu_multipass_kernel<L, CG, R, FMT>), grid, block, 0, stream, wd, \
                               X, Y, m0, n, k, geo.P, geo.tiles);                                  \
        break;
            Q4_VALU_CASE(1)
            Q4_VALU_CASE(2)
            Q4_VALU_CASE(3)
            Q4_VALU_CASE(4)
            Q4_VALU_CASE(5)
            Q4_VALU_CASE(6)
            Q4_VALU_CASE(7)
            Q4_VALU_CASE(8)
#undef Q4_VALU_CASE
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <int L, int CG, int NT, int MT, int FMT>
hipError_t launch_mfma_wx(const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                          int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    constexpr int BN = 64 * NT, BM = 16 * MT;
    const int64_t nbn = (n + BN - 1) / BN;
    const int64_t mbl = (m + BM - 1) / BM;
    const int64_t padded = mbl > 1 ? (nbn + 7) / 8 * 8 : nbn;
    const int64_t wbytes = geo.tiles * geo.tile_bytes;
    const dim3 grid((unsigned)(padded * mbl));
    hipLaunchKernelGGL((gemm_mfma_wx_kernel<L, CG, NT, MT, FMT>), grid, dim3(256), 0, stream, wd, wbytes,
                       X, Y, m, n, k, nbn, padded);
    return hipGetLastError();
}

template <int L, int CG, int NA, int MT, int NW, int D, int FMT, int XR = 32 * MT>
hipError_t launch_mfma_ks(const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                          int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    constexpr int BM = 32 * MT, BN = 32 * NA;
    const int64_t nbn = (n + BN - 1) / BN;
    const int64_t mbl = (m + BM - 1) / BM;
    const int64_t padded = mbl > 1 ? (nbn + 7) / 8 * 8 : nbn;
    const int64_t wbytes = geo.tiles * geo.tile_bytes;
    hipLaunchKernelGGL((gemm_mfma_ks_kernel<L, CG, NA, MT, NW, D, FMT, XR>), dim3((unsigned)(padded * mbl)),
                       dim3(64 * NW), 0, stream, wd, wbytes, X, Y, m, n, k, nbn, padded);
    return hipGetLastError();
}

template <int L, int CG, int FMT>
hipError_t launch_mfma_lc(const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                          int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    // K-split kernel tiles (A tiles NA x 32 weight rows, MT x 32 activation
    // rows, NW wavefronts, D steps in flight) with the measured fastest per
    // m on 16384 x 3072, us at m = 4 / 16 / 32 / 64 / 128 / 192 / 256: 10.8 /
    // 11.9 / 13.8 / 19.3 / 26.6 / 38.1 / 41.2, against 13.0 / 12.9 / 18.4 /
    // 25.9 / 34.5 / 45.6 / 47.8 for the X-resident and weight-direct kernels
    // they replaced; up to 8 and 16 rows only those X rows are staged (m =
    // 16: 11.9 against 12.4 us staging all 32).  Beyond k = 4096 the 4-wavefront tiles unroll too many
    // steps per wavefront and spill: two 64-row M blocks of 8 wavefronts up
    // to m = 128, the weight-direct kernel above.
    if (m <= 8)
        return launch_mfma_ks<L, CG, 2, 1, 16, 2, FMT, 8>(geo, wd, X, m, n, k, Y, stream);
    if (m <= 16)
        return launch_mfma_ks<L, CG, 2, 1, 16, 2, FMT, 16>(geo, wd, X, m, n, k, Y, stream);
    if (m <= 32)
        return launch_mfma_ks<L, CG, 2, 1, 16, 2, FMT>(geo, wd, X, m, n, k, Y, stream);
    if (m <= 64)
        return launch_mfma_ks<L, CG, 2, 2, 8, 3, FMT>(geo, wd, X, m, n, k, Y, stream);
    if constexpr (L * CG <= 128) {
        if (m <= 128)
            return launch_mfma_ks<L, CG, 4, 2, 8, 2, FMT>(geo, wd, X, m, n, k, Y, stream);
        return launch_mfma_ks<L, CG, 4, 4, 4, 2, FMT>(geo, wd, X, m, n, k, Y, stream);
    } else {
        if (m <= 128)
            return launch_mfma_ks<L, CG, 2, 2, 8, 3, FMT>(geo, wd, X, m, n, k, Y, stream);
        return launch_mfma_wx<L, CG, 2, 8, FMT>(geo, wd, X, m, n, k, Y, stream);
    }
}

template <int L, int FMT>
hipError_t launch_l(bool mfma, const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                    int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    switch (geo.CG) {
#define Q4_CG_CASE(C)                                                                 \
    case C:                                                                           \
        if (mfma)                                                                     \
            return launch_mfma_lc<L, C, FMT>(geo, wd, X, m, n, k, Y, stream);         \
        return launch_valu_lc<L, C, FMT>(geo, wd, X, m, n, k, Y, stream);
        Q4_CG_CASE(1)
        Q4_CG_CASE(2)
        Q4_CG_CASE(3)
        Q4_CG_CASE(4)
#undef Q4_CG_CASE
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool gemm_mfma_eligible(const Geometry &geo) { return geo.P == 1 && geo.L >= 4; }

template <int FMT>
static hipError_t launch_gemm_fmt(const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                                  int64_t n, int64_t k, uint16_t *Y, bool mfma, hipStream_t stream)
{
    switch (geo.L) {
    case 64: return launch_l<64, FMT>(mfma, geo, wd, X, m, n, k, Y, stream);
    case 32: return launch_l<32, FMT>(mfma, geo, wd, X, m, n, k, Y, stream);
    case 16: return launch_l<16, FMT>(mfma, geo, wd, X, m, n, k, Y, stream);
    case 8: return launch_l<8, FMT>(mfma, geo, wd, X, m, n, k, Y, stream);
    case 4: return launch_l<4, FMT>(mfma, geo, wd, X, m, n, k, Y, stream);
    case 2: return launch_l<2, FMT>(false, geo, wd, X, m, n, k, Y, stream);
    case 1: return launch_l<1, FMT>(false, geo, wd, X, m, n, k, Y, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(const Geometry &geo, const void *wdata, const uint16_t *X, int64_t m,
                       int64_t n, int64_t k, uint16_t *Y, int path, hipStream_t stream, bool int3)
{
    const uint8_t *wd = static_cast<const uint8_t *>(wdata);
    // from 2 rows on the MFMA kernels are faster (16384 x 3072: 10.9 against
    // 12.3 us at m = 2, 11.2 against 17.1 us at m = 4); one row with Y not
    // 4-byte aligned (else the GEMV kernels) takes the VALU kernel's single
    // exact pass over W
    bool mfma = (path == GEMM_PATH_MFMA) || (path == GEMM_PATH_AUTO && m >= 2);
    if (mfma && !gemm_mfma_eligible(geo))
        mfma = false;
    // the MFMA kernel addresses the weight and X through 32-bit buffer offsets
    if (mfma && (geo.tiles * geo.tile_bytes >= ((int64_t)1 << 31) || m * k * 2 >= ((int64_t)1 << 31)))
        mfma = false;
    if (int3)
        return launch_gemm_fmt<3>(geo, wd, X, m, n, k, Y, mfma, stream);
    return launch_gemm_fmt<4>(geo, wd, X, m, n, k, Y, mfma, stream);
}

}  // namespace q4
