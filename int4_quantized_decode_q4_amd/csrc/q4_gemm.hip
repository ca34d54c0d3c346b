// q4_gemm.hip -- batched form of the int4 dequantizing matmul,
// Y[m][n] = sum_k X[m][k] * (q[n][k] - 8) * s[n][k/32], on gfx950.
//
// Source: "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权"
// (zingnex.cn), section 技术限制与诚实声明: batched-prefill shaders exist for
// prompt processing; the pages give no design for them.
//
// Kernels:
//  * VALU, m < 4 (or a layout the MFMA kernels do not take): the streaming
//    kernel -- CG wavefronts per block walk tiles, wavefront j takes group
//    slot j of every lane, so each lane keeps that group's x slices for up to
//    8 activation rows in VGPRs for the whole launch and one pass over W
//    serves 8 rows; codes are dequantized once per word (exact q - 8) and
//    reused for every row.  Multi-pass layouts (k > 8192) use a per-tile
//    variant that re-reads the x slices of each pass.
//  * MFMA, small m (m <= 16, or m <= 32 with n < 8192): a block owns 16
//    weight rows and its 4 wavefronts split the K steps, each an independent
//    pipeline with its own LDS slice (no block barrier until the final
//    in-order sum of the 4 partial tiles).
//  * MFMA, larger m: a block owns 64 or 128 weight rows and BM activation
//    rows; K is walked in steps of 4 groups (128 k) with a register ring of
//    steps in flight.
// In both MFMA kernels each 16-byte unit of codes is dequantized to f16
// (q - 8) * s (one rounding, relative error <= 2^-11) into LDS, the X slab of
// the same k range is staged in LDS, and v_mfma_f32_16x16x32_f16 contracts
// them with f32 accumulation.  Inside each 8-k word the k order in LDS is
// (0,4,1,5,2,6,3,7) for both operands -- the order the nibble masks produce
// -- which leaves the contraction unchanged.
// int3 weights (12-byte units of 32 codes, one pass) run through the same
// kernels with their own dequant: exact (q - 4) pairs on the VALU path, f16
// (q - 4) * s put back in k order for the MFMA kernels (X is not re-paired).
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

#ifndef Q4_GEMM_DEPTH_LARGE
#define Q4_GEMM_DEPTH_LARGE 2
#endif
constexpr int kGroupsPerStep = 4;                 // K step: 4 groups = 128 k
constexpr int kStepK = 32 * kGroupsPerStep;
constexpr int kLdsRow = kStepK + 8;               // halves per LDS row (+16 B against bank conflicts)

// Block tile BN x BM = (16 NT WN) x (16 MT WM): 4 wavefronts in a WN x WM
// grid, each owning NT x MT MFMA tiles of 16 x 16.  K steps of 4 groups in
// layout order (for a row: 4 consecutive 16-byte units, 64 contiguous
// bytes).  The next step's units, scales and X chunks are loaded into
// registers while the current step's MFMAs run; dequant and the LDS stores
// happen between two barriers.
template <int L, int CG, int NT, int MT, int WN, int WM, int FMT = 4>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(const uint8_t *__restrict__ wd,
                                                        int64_t wbytes,
                                                        const uint16_t *__restrict__ X,
                                                        uint16_t *__restrict__ Y, int64_t m,
                                                        int64_t n, int64_t k, int64_t nblocks_n,
                                                        int64_t padded_nblocks_n)
{
    static_assert(WN * WM == 4, "four wavefronts");
    constexpr int BN = 16 * NT * WN, BM = 16 * MT * WM;
    constexpr int TR = 128 / L;
    constexpr int PB = CG * GFmt<FMT>::PASS;
    constexpr int UB = GFmt<FMT>::UB, US = GFmt<FMT>::US;
    constexpr int WU = BN * kGroupsPerStep / 256;     // weight units per thread per step
    constexpr int XC = BM * kGroupsPerStep * 4 / 256; // 16-byte X chunks per thread per step
    static_assert(WU >= 1 && XC >= 1, "tile too small for 256 threads");
    constexpr int CBLOCKS = L / kGroupsPerStep;
    constexpr int STEPS = CG * CBLOCKS;
    constexpr int D = BM <= 32 ? 4 : (BM <= 64 ? 2 : Q4_GEMM_DEPTH_LARGE);   // steps in flight
    __shared__ _Float16 Ws[BN][kLdsRow];
    __shared__ _Float16 Xs[BM][kLdsRow];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wn = wv % WN, wm = wv / WN;
    const int64_t G = k >> 5;

    // XCD-aware order: block ids b, b + 8, b + 16, ... go to the same XCD,
    // so the M-blocks of one weight slab are spread by a stride of 8 and
    // share that XCD's L2 for the slab.
    const int64_t mblocks = gridDim.x / padded_nblocks_n;
    const int64_t b = blockIdx.x;
    const int64_t grp = b / (8 * mblocks), within = b % (8 * mblocks);
    const int64_t nb = grp * 8 + within % 8;
    const int64_t mb = within / 8;
    if (nb >= nblocks_n)
        return;
    const int64_t n0 = nb * BN, mrow0 = mb * BM;
    const int64_t t0 = n0 / TR;

    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(wd), (short)0, (int)wbytes, 0x00020000);
    const Masks mk = FMT == 4 ? masks() : Masks{};
    const Masks3 mk3 = FMT == 3 ? masks3() : Masks3{};

    // per-thread fixed parts of the weight unit addresses
    int64_t ubase[WU];   // tile byte offset + lane' * US without the (u, j) unit term
    int64_t sbase[WU];   // tile byte offset of the lane's scale block
    int urow[WU], ucl[WU], uu[WU];
#pragma unroll
    for (int h = 0; h < WU; ++h) {
        const int q = tid + 256 * h;
        const int rr = q / kGroupsPerStep, cl = q % kGroupsPerStep;
        const int64_t tile = t0 + rr / TR;
        const int sl = (rr % TR) >> 1;
        urow[h] = rr;
        ucl[h] = cl;
        uu[h] = rr & 1;
        ubase[h] = tile * PB + (int64_t)(sl * L + cl) * US;
        sbase[h] = tile * PB + 2 * CG * UB + (int64_t)(sl * L + cl) * 4 * CG;
    }

    // X through a buffer resource too: chunks outside X (rows past m, groups
    // past k, steps past the end) read as zero without touching memory
    const int xbytes = (int)(m * k * 2);
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(X), (short)0, xbytes, 0x00020000);

    // D steps of operands kept in flight in registers
    struct StepRegs {
        v4u w[WU];
        uint32_t s[WU];
        v4u x[XC];
    };
    StepRegs ring[D];
    auto load_step = [&](StepRegs &r, int st) {
        const bool live = st < STEPS;
        const int j = st / CBLOCKS, cb = st % CBLOCKS;
#pragma unroll
        for (int h = 0; h < WU; ++h) {
            const int64_t off = ubase[h] + (int64_t)(uu[h] * CG + j) * UB + cb * kGroupsPerStep * US;
            const int64_t soff = sbase[h] + (int64_t)cb * kGroupsPerStep * 4 * CG + (uu[h] * CG + j) * 2;
            // rows past the end of the weight read as zero through the buffer bounds
            const int wo = (int)(live && off < wbytes ? off : wbytes);
            const int so = (int)(live && (soff & ~3ll) < wbytes ? (soff & ~3ll) : wbytes);
            r.w[h] = load_unit_g<FMT>(rs, wo);
            r.s[h] = __builtin_amdgcn_raw_buffer_load_b32(rs, so, 0, 0) >> ((soff & 2) * 8);
        }
#pragma unroll
        for (int h = 0; h < XC; ++h) {
            const int q = tid + 256 * h;
            const int mr = q / (kGroupsPerStep * 4), rest = q % (kGroupsPerStep * 4);
            const int cl = rest >> 2, wq = rest & 3;
            const int64_t g = (int64_t)(cb * kGroupsPerStep + cl) * CG + j;
            const int64_t mm = mrow0 + mr;
            const int xo = (live && mm < m && g < G) ? (int)((mm * k + g * 32 + wq * 8) * 2) : xbytes;
            r.x[h] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xo, 0, 0);
        }
    };
    auto store_step = [&](const StepRegs &r) {
#pragma unroll
        for (int h = 0; h < WU; ++h) {
            const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(r.s[h] & 0xFFFFu));
            const h2 sc = {sv, sv};
            uint4 *dst = reinterpret_cast<uint4 *>(&Ws[urow[h]][ucl[h] * 32]);
            if constexpr (FMT == 4) {
                const uint32_t ws4[4] = {r.w[h].x, r.w[h].y, r.w[h].z, r.w[h].w};
#pragma unroll
                for (int wq = 0; wq < 4; ++wq) {
                    h2 a0, a1, a2, a3;
                    dequant_word_unit(ws4[wq], mk, a0, a1, a2, a3);
                    // one f16 rounding of (q - 8) * s
                    dst[wq] = make_uint4(as_u32(a0 * sc), as_u32(a1 * sc), as_u32(a2 * sc), as_u32(a3 * sc));
                }
            } else {
                // one f16 rounding of (q - 4) * s, then back to k order (X stays natural)
                h2 P[16];
                dequant_unit3(r.w[h].x, r.w[h].y, r.w[h].z, mk3, P);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    P[i] = P[i] * sc;
                uint4 o[4];
                pairs3_to_k(P, o);
#pragma unroll
                for (int wq = 0; wq < 4; ++wq)
                    dst[wq] = o[wq];
            }
        }
#pragma unroll
        for (int h = 0; h < XC; ++h) {
            const int q = tid + 256 * h;
            const int mr = q / (kGroupsPerStep * 4), rest = q % (kGroupsPerStep * 4);
            const int cl = rest >> 2, wq = rest & 3;
            const uint4 xv = make_uint4(r.x[h].x, r.x[h].y, r.x[h].z, r.x[h].w);
            *reinterpret_cast<uint4 *>(&Xs[mr][cl * 32 + wq * 8]) = FMT == 4 ? pair_word(xv) : xv;
        }
    };
    auto mfma_step = [&](f4 (&acc)[NT][MT]) {
#pragma unroll
        for (int ss = 0; ss < kGroupsPerStep; ++ss) {
            const int kk = ss * 32 + 8 * (lane >> 4);
            h8 af[NT], bf[MT];
#pragma unroll
            for (int i = 0; i < NT; ++i)
                af[i] = *reinterpret_cast<const h8 *>(&Ws[(wn * NT + i) * 16 + (lane & 15)][kk]);
#pragma unroll
            for (int jj = 0; jj < MT; ++jj)
                bf[jj] = *reinterpret_cast<const h8 *>(&Xs[(wm * MT + jj) * 16 + (lane & 15)][kk]);
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int jj = 0; jj < MT; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[jj], acc[i][jj], 0, 0, 0);
        }
    };

    f4 acc[NT][MT];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int jj = 0; jj < MT; ++jj)
            acc[i][jj] = f4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i = 0; i < D; ++i)
        load_step(ring[i], i);
    for (int st = 0; st < STEPS; st += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            if (st + i < STEPS) {
                __syncthreads();          // the previous step's fragments have been read
                store_step(ring[i]);
                __syncthreads();
                load_step(ring[i], st + i + D);   // D steps ahead; past the end reads nothing
                mfma_step(acc);
            }
        }
    }
    // D[i][j]: lane holds rows i = 4 (lane / 16) + r (weight rows), column
    // j = lane % 16 (activation row)
#pragma unroll
    for (int jj = 0; jj < MT; ++jj) {
        const int64_t mm = mrow0 + (wm * MT + jj) * 16 + (lane & 15);
        if (mm >= m)
            continue;
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t nn = n0 + (wn * NT + i) * 16 + 4 * (lane >> 4) + r;
                if (nn < n)
                    Y[mm * n + nn] = f16_bits(acc[i][jj][r]);
            }
    }
}

// Small-m MFMA kernel (m <= 32): a block owns 16 weight rows x BM = 16 MT
// activation rows, and its 4 wavefronts split the K steps (wavefront w takes
// steps w, w + 4, ...).  Each wavefront is an independent pipeline -- up to
// six steps of operands in flight in registers, a private LDS slice, no
// block barrier -- and the four partial sums are added in wavefront order at the
// end (deterministic).  Many small blocks keep enough weight bytes in flight
// for the HBM-bound regime.
template <int L, int CG, int MT, int FMT = 4>
__global__ __launch_bounds__(256) void gemm_mfma_small_kernel(const uint8_t *__restrict__ wd,
                                                              int64_t wbytes,
                                                              const uint16_t *__restrict__ X,
                                                              uint16_t *__restrict__ Y, int64_t m,
                                                              int64_t n, int64_t k)
{
    constexpr int BM = 16 * MT;
    constexpr int TR = 128 / L;
    constexpr int PB = CG * GFmt<FMT>::PASS;
    constexpr int UB = GFmt<FMT>::UB, US = GFmt<FMT>::US;
    constexpr int XC = BM * kGroupsPerStep * 4 / 64;   // X chunks per lane per step
    constexpr int CBLOCKS = L / kGroupsPerStep;
    constexpr int STEPS = CG * CBLOCKS;
    // a wavefront with at most 6 steps keeps all of them in flight; longer
    // K streams 3 steps deep (measured best for k = 3072 and 8192)
    constexpr int WSTEPS = (STEPS + 3) / 4;
    constexpr int D = WSTEPS <= 6 ? (WSTEPS > 0 ? WSTEPS : 1) : 3;
    static_assert(TR <= 16, "16-row blocks need at least 8 lanes per row");
    __shared__ _Float16 Ws[4][16][kLdsRow];
    __shared__ _Float16 Xs[4][BM][kLdsRow];
    __shared__ float red[4][MT][4][64];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t G = k >> 5;
    const int64_t mblocks = (m + BM - 1) / BM;
    const int64_t nb = blockIdx.x / mblocks, mb = blockIdx.x % mblocks;
    const int64_t n0 = nb * 16, mrow0 = mb * BM;

    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(wd), (short)0, (int)wbytes, 0x00020000);
    const int xbytes = (int)(m * k * 2);
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(X), (short)0, xbytes, 0x00020000);
    const Masks mk = FMT == 4 ? masks() : Masks{};
    const Masks3 mk3 = FMT == 3 ? masks3() : Masks3{};

    // this lane's weight unit in every step: row lane / 4, group slot lane % 4
    const int rr = lane >> 2, cl = lane & 3;
    const int64_t row = n0 + rr;
    const int64_t tile = row / TR;
    const int sl = (int)((row % TR) >> 1), uu = (int)(row & 1);
    const int64_t ubase = tile * PB + (int64_t)(sl * L + cl) * US;
    const int64_t sbase = tile * PB + 2 * CG * UB + (int64_t)(sl * L + cl) * 4 * CG;

    struct StepRegs {
        v4u w;
        uint32_t s;
        v4u x[XC];
    };
    auto load_step = [&](StepRegs &r, int st) {
        const bool live = st < STEPS;
        const int j = st / CBLOCKS, cb = st % CBLOCKS;
        const int64_t off = ubase + (int64_t)(uu * CG + j) * UB + cb * kGroupsPerStep * US;
        const int64_t soff = sbase + (int64_t)cb * kGroupsPerStep * 4 * CG + (uu * CG + j) * 2;
        const int wo = (int)(live && off < wbytes ? off : wbytes);
        const int so = (int)(live && (soff & ~3ll) < wbytes ? (soff & ~3ll) : wbytes);
        r.w = load_unit_g<FMT>(rs, wo);
        r.s = __builtin_amdgcn_raw_buffer_load_b32(rs, so, 0, 0) >> ((soff & 2) * 8);
#pragma unroll
        for (int h = 0; h < XC; ++h) {
            const int q = lane + 64 * h;
            const int mr = q / (kGroupsPerStep * 4), rest = q % (kGroupsPerStep * 4);
            const int xcl = rest >> 2, wq = rest & 3;
            const int64_t g = (int64_t)(cb * kGroupsPerStep + xcl) * CG + j;
            const int64_t mm = mrow0 + mr;
            const int xo = (live && mm < m && g < G) ? (int)((mm * k + g * 32 + wq * 8) * 2) : xbytes;
            r.x[h] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xo, 0, 0);
        }
    };
    auto run_step = [&](const StepRegs &r, f4 (&acc)[MT]) {
        {
            const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(r.s & 0xFFFFu));
            const h2 sc = {sv, sv};
            uint4 *dst = reinterpret_cast<uint4 *>(&Ws[wv][rr][cl * 32]);
            if constexpr (FMT == 4) {
                const uint32_t ws4[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
#pragma unroll
                for (int wq = 0; wq < 4; ++wq) {
                    h2 a0, a1, a2, a3;
                    dequant_word_unit(ws4[wq], mk, a0, a1, a2, a3);
                    dst[wq] = make_uint4(as_u32(a0 * sc), as_u32(a1 * sc), as_u32(a2 * sc), as_u32(a3 * sc));
                }
            } else {
                h2 P[16];
                dequant_unit3(r.w.x, r.w.y, r.w.z, mk3, P);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    P[i] = P[i] * sc;
                uint4 o[4];
                pairs3_to_k(P, o);
#pragma unroll
                for (int wq = 0; wq < 4; ++wq)
                    dst[wq] = o[wq];
            }
        }
#pragma unroll
        for (int h = 0; h < XC; ++h) {
            const int q = lane + 64 * h;
            const int mr = q / (kGroupsPerStep * 4), rest = q % (kGroupsPerStep * 4);
            const int xcl = rest >> 2, wq = rest & 3;
            const uint4 xv = make_uint4(r.x[h].x, r.x[h].y, r.x[h].z, r.x[h].w);
            *reinterpret_cast<uint4 *>(&Xs[wv][mr][xcl * 32 + wq * 8]) = FMT == 4 ? pair_word(xv) : xv;
        }
        // the wavefront's own LDS slice: its writes must land before its reads
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int ss = 0; ss < kGroupsPerStep; ++ss) {
            const int kk = ss * 32 + 8 * (lane >> 4);
            const h8 a = *reinterpret_cast<const h8 *>(&Ws[wv][lane & 15][kk]);
#pragma unroll
            for (int jj = 0; jj < MT; ++jj) {
                const h8 bx = *reinterpret_cast<const h8 *>(&Xs[wv][jj * 16 + (lane & 15)][kk]);
                acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bx, acc[jj], 0, 0, 0);
            }
        }
        // fragments read before the next step overwrites the slice
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };

    f4 acc[MT];
#pragma unroll
    for (int jj = 0; jj < MT; ++jj)
        acc[jj] = f4{0.f, 0.f, 0.f, 0.f};
    StepRegs ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i)
        load_step(ring[i], wv + 4 * i);
    for (int st = wv; st < STEPS; st += 4 * D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int cur = st + 4 * i;
            if (cur < STEPS) {
                run_step(ring[i], acc);
                load_step(ring[i], cur + 4 * D);   // past the end reads nothing
            }
        }
    }
#pragma unroll
    for (int jj = 0; jj < MT; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            red[wv][jj][r][lane] = acc[jj][r];
    __syncthreads();
    if (wv == 0) {
#pragma unroll
        for (int jj = 0; jj < MT; ++jj) {
            const int64_t mm = mrow0 + jj * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = ((red[0][jj][r][lane] + red[1][jj][r][lane]) + red[2][jj][r][lane]) +
                                red[3][jj][r][lane];
                const int64_t nn = n0 + 4 * (lane >> 4) + r;
                if (mm < m && nn < n)
                    Y[mm * n + nn] = f16_bits(v);
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
    const int64_t cap = single ? 256 * Q4_VALU_BLOCKS_PER_CU : 256 * 8;
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

template <int L, int CG, int NT, int MT, int WN, int WM, int FMT>
hipError_t launch_mfma_cfg(const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                           int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    constexpr int BN = 16 * NT * WN, BM = 16 * MT * WM;
    const int64_t nbn = (n + BN - 1) / BN;
    const int64_t padded = (nbn + 7) / 8 * 8;   // whole groups of 8 for the XCD order
    const int64_t wbytes = geo.tiles * geo.tile_bytes;
    const dim3 grid((unsigned)(padded * ((m + BM - 1) / BM)));
    hipLaunchKernelGGL((gemm_mfma_kernel<L, CG, NT, MT, WN, WM, FMT>), grid, dim3(256), 0, stream, wd,
                       wbytes, X, Y, m, n, k, nbn, padded);
    return hipGetLastError();
}

template <int L, int CG, int MT, int FMT>
hipError_t launch_mfma_small(const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                             int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    const int64_t wbytes = geo.tiles * geo.tile_bytes;
    const dim3 grid((unsigned)(((n + 15) / 16) * ((m + 16 * MT - 1) / (16 * MT))));
    hipLaunchKernelGGL((gemm_mfma_small_kernel<L, CG, MT, FMT>), grid, dim3(256), 0, stream, wd, wbytes,
                       X, Y, m, n, k);
    return hipGetLastError();
}

template <int L, int CG, int FMT>
hipError_t launch_mfma_lc(const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                          int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    // m <= 16: the small kernel always; m <= 32: only while the 64-row tile
    // kernel would have too few blocks (n < 8192) to stream the weights
    if (L >= 8 && m <= 16)
        return launch_mfma_small<L >= 8 ? L : 8, CG, 1, FMT>(geo, wd, X, m, n, k, Y, stream);
    if (L >= 8 && m <= 32 && n < 8192)
        return launch_mfma_small<L >= 8 ? L : 8, CG, 2, FMT>(geo, wd, X, m, n, k, Y, stream);
    if (m <= 16)
        return launch_mfma_cfg<L, CG, 1, 1, 4, 1, FMT>(geo, wd, X, m, n, k, Y, stream);  // 64 x 16
    if (m <= 32)
        return launch_mfma_cfg<L, CG, 2, 1, 2, 2, FMT>(geo, wd, X, m, n, k, Y, stream);  // 64 x 32
    if (m <= 64)
        return launch_mfma_cfg<L, CG, 2, 2, 2, 2, FMT>(geo, wd, X, m, n, k, Y, stream);  // 64 x 64
    // up to 128 rows a 128 x 128 tile would leave half the compute units of a
    // 16384-row weight idle (128 blocks): 128 x 64 takes m = 128 from 57.5 to
    // 40.3 us; above, 128 x 128 is the faster of the two (60.0 against 63.5 us
    // at m = 256)
    if (m <= 128)
        return launch_mfma_cfg<L, CG, 4, 2, 2, 2, FMT>(geo, wd, X, m, n, k, Y, stream);  // 128 x 64
    return launch_mfma_cfg<L, CG, 4, 4, 2, 2, FMT>(geo, wd, X, m, n, k, Y, stream);      // 128 x 128
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
    // from 4 rows on the MFMA kernels are faster (16384 x 3072: 13.7 against
    // 17.4 us at m = 4, 17.4 against 44 us at m = 12); at 1-2 rows the VALU
    // kernel's single exact pass over W wins
    bool mfma = (path == GEMM_PATH_MFMA) || (path == GEMM_PATH_AUTO && m >= 4);
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
