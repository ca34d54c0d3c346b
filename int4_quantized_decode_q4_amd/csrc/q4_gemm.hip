// q4_gemm.hip -- batched form of the int4 dequantizing matmul,
// Y[m][n] = sum_k X[m][k] * (q[n][k] - 8) * s[n][k/32], on gfx950.
//
// Source: "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权"
// (zingnex.cn), section 技术限制与诚实声明: batched-prefill shaders exist for
// prompt processing; the pages give no design for them.
//
// Two paths:
//  * m < 16 (or a layout the MFMA kernel does not take): a VALU kernel in
//    the shape of the split GEMV -- CG wavefronts share a tile, each lane
//    holds the x slices of one group for up to 8 activation rows in VGPRs, so
//    one pass over W serves 8 rows; codes are dequantized once per word and
//    reused for every row.  Exact dequant as in the GEMV.
//  * m >= 16: an MFMA kernel.  A block owns 64 weight rows and BM activation
//    rows; K is walked in steps of 8 groups (256 k) in the order the layout
//    stores them, so each step reads, per weight row, 8 consecutive 16-byte
//    units (128 contiguous bytes).  Each unit is dequantized to f16
//    (q - 8) * s (one rounding, relative error <= 2^-11) into LDS; the X slab
//    of the same 256 k is staged in LDS; v_mfma_f32_16x16x32_f16 contracts
//    them with f32 accumulation.  Inside each 8-k word the k order in LDS is
//    (0,4,1,5,2,6,3,7) for both operands -- the order the nibble masks
//    produce -- which leaves the contraction unchanged.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "q4_geometry.h"
#include "q4_internal.h"

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

template <int L>
__device__ __forceinline__ float reduce_lanes(float v)
{
    if (L >= 2)
        v += __shfl_xor(v, 1);
    if (L >= 4)
        v += __shfl_xor(v, 2);
    if (L >= 8)
        v += __shfl_xor(v, 4);
    if (L >= 16)
        v += __shfl_xor(v, 8);
    if (L >= 32)
        v += __shfl_xor(v, 16);
    if (L >= 64)
        v += __shfl_xor(v, 32);
    return v;
}

// Block = CG wavefronts; wavefront j takes group slot j of every lane of a
// tile.  Rows m0 .. m0 + MC - 1 of X (MC <= kValuRows) per launch.
template <int L, int CG, int MC>
__global__ __launch_bounds__(256) void gemm_valu_kernel(const uint8_t *__restrict__ wd,
                                                        const uint16_t *__restrict__ X,
                                                        uint16_t *__restrict__ Y, int64_t m0,
                                                        int64_t n, int64_t k, int passes,
                                                        int64_t tiles)
{
    constexpr int TR = 128 / L;
    const int64_t PB = (int64_t)CG * 2304;
    __shared__ float part[CG][64][2 * MC];
    const int lane = threadIdx.x & 63;
    const int j = threadIdx.x >> 6;
    const int s = lane / L, c = lane % L;
    const int64_t G = k >> 5;
    const Masks mk = masks();
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        float acc[MC][2];
#pragma unroll
        for (int r = 0; r < MC; ++r)
            acc[r][0] = acc[r][1] = 0.f;
        for (int p = 0; p < passes; ++p) {
            const int64_t g = (int64_t)p * L * CG + (int64_t)c * CG + j;
            const uint8_t *base = wd + (t * passes + p) * PB;
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
                y0 = reduce_lanes<L>(y0);
                y1 = reduce_lanes<L>(y1);
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

constexpr int kBN = 64;          // weight rows per block
constexpr int kStepK = 256;      // k per step (8 groups)
constexpr int kLdsRow = kStepK + 8;   // halves per LDS row (padding against bank conflicts)

// One block: weight rows n0 .. n0+63 x activation rows mb*BM .. +BM-1.
// 4 wavefronts; wavefront w computes the 16 x BM output slab of rows
// n0 + 16w .. n0 + 16w + 15.
template <int L, int CG, int BM>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(const uint8_t *__restrict__ wd,
                                                        int64_t wbytes,
                                                        const uint16_t *__restrict__ X,
                                                        uint16_t *__restrict__ Y, int64_t m,
                                                        int64_t n, int64_t k, int64_t nblocks_n,
                                                        int64_t padded_nblocks_n)
{
    constexpr int TR = 128 / L;
    constexpr int PB = CG * 2304;
    constexpr int MT = BM / 16;
    __shared__ _Float16 Ws[kBN][kLdsRow];
    __shared__ _Float16 Xs[BM][kLdsRow];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int64_t G = k >> 5;

    // XCD-aware order: consecutive block ids go to different XCDs, so the
    // M-blocks of one weight slab are spread by a stride of 8 block ids and
    // land on the same XCD (sharing that XCD's L2 for the slab).
    const int64_t mblocks = gridDim.x / padded_nblocks_n;
    const int64_t b = blockIdx.x;
    const int64_t group = b / (8 * mblocks), within = b % (8 * mblocks);
    const int64_t nb = group * 8 + within % 8;
    const int64_t mb = within / 8;
    if (nb >= nblocks_n)
        return;
    const int64_t n0 = nb * kBN, mrow0 = mb * BM;
    const int64_t t0 = n0 / TR;

    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(wd), (short)0, (int)wbytes, 0x00020000);
    const Masks mk = masks();

    f4 acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
        acc[i] = f4{0.f, 0.f, 0.f, 0.f};

    for (int j = 0; j < CG; ++j) {
        for (int cb = 0; cb < L / 8; ++cb) {
            // W: 64 rows x 8 units; thread takes units q = tid and tid + 256
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q = tid + 256 * h;
                const int rr = q >> 3, cc = q & 7;
                const int64_t tile = t0 + rr / TR;
                const int sl = (rr % TR) >> 1, u = rr & 1;
                const int lanep = sl * L + cb * 8 + cc;
                const int64_t tb = tile * PB;
                // a tile past the end of the weight reads as zero (buffer bounds)
                const int64_t off = tb + (u * CG + j) * 1024 + lanep * 16;
                const int64_t soff = tb + 2 * CG * 1024 + lanep * 4 * CG + (u * CG + j) * 2;
                const bool inb = tb < wbytes;
                v4u cw = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
                uint32_t sw = 0;
                if (inb) {
                    cw = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
                    sw = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(soff & ~3ll), 0, 0);
                }
                const uint16_t sb = (uint16_t)(sw >> ((soff & 2) * 8));
                const h2 sc = {__builtin_bit_cast(_Float16, sb), __builtin_bit_cast(_Float16, sb)};
                uint32_t outw[16];
                const uint32_t ws4[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
                for (int wq = 0; wq < 4; ++wq) {
                    h2 a0, a1, a2, a3;
                    dequant_word_unit(ws4[wq], mk, a0, a1, a2, a3);
                    // one f16 rounding of (q - 8) * s
                    outw[4 * wq + 0] = as_u32(a0 * sc);
                    outw[4 * wq + 1] = as_u32(a1 * sc);
                    outw[4 * wq + 2] = as_u32(a2 * sc);
                    outw[4 * wq + 3] = as_u32(a3 * sc);
                }
                uint4 *dst = reinterpret_cast<uint4 *>(&Ws[rr][cc * 32]);
#pragma unroll
                for (int z = 0; z < 4; ++z)
                    dst[z] = make_uint4(outw[4 * z], outw[4 * z + 1], outw[4 * z + 2], outw[4 * z + 3]);
            }
            // X: BM rows x 8 groups x 4 words of 8 halves
            for (int q = tid; q < BM * 32; q += 256) {
                const int mr = q >> 5, rest = q & 31, cc = rest >> 2, wq = rest & 3;
                const int64_t g = (int64_t)(cb * 8 + cc) * CG + j;
                const int64_t mm = mrow0 + mr;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (mm < m && g < G)
                    v = pair_word(*reinterpret_cast<const uint4 *>(X + mm * k + g * 32 + wq * 8));
                *reinterpret_cast<uint4 *>(&Xs[mr][cc * 32 + wq * 8]) = v;
            }
            __syncthreads();
#pragma unroll
            for (int ss = 0; ss < kStepK / 32; ++ss) {
                const int kk = ss * 32 + 8 * (lane >> 4);
                const h8 a = *reinterpret_cast<const h8 *>(&Ws[16 * wv + (lane & 15)][kk]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const h8 bx = *reinterpret_cast<const h8 *>(&Xs[16 * mt + (lane & 15)][kk]);
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bx, acc[mt], 0, 0, 0);
                }
            }
            __syncthreads();
        }
    }
    // D[i][j]: lane holds rows i = 4 (lane / 16) + r (weight rows), column
    // j = lane % 16 (activation row)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t mm = mrow0 + 16 * mt + (lane & 15);
        if (mm >= m)
            continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t nn = n0 + 16 * wv + 4 * (lane >> 4) + r;
            if (nn < n)
                Y[mm * n + nn] = f16_bits(acc[mt][r]);
        }
    }
}

template <int L, int CG>
hipError_t launch_valu_lc(const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                          int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    const int64_t cap = 256 * 8;
    const dim3 grid((unsigned)(geo.tiles < cap ? geo.tiles : cap)), block(64 * CG);
    for (int64_t m0 = 0; m0 < m; m0 += kValuRows) {
        const int64_t mc = m - m0 < kValuRows ? m - m0 : kValuRows;
        switch (mc) {
#define Q4_VALU_CASE(R)                                                                           \
    case R:                                                                                       \
        hipLaunchKernelGGL((gemm_valu_kernel<L, CG, R>), grid, block, 0, stream, wd, X, Y, m0, n, \
                           k, geo.P, geo.tiles);                                                  \
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

template <int L, int CG>
hipError_t launch_mfma_lc(const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                          int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    const int64_t nbn = (n + kBN - 1) / kBN;
    const int64_t padded_nbn = (nbn + 7) / 8 * 8;   // whole groups of 8 for the XCD order
    const int64_t wbytes = geo.tiles * geo.tile_bytes;
    if (m <= 16) {
        const dim3 grid((unsigned)(padded_nbn * ((m + 15) / 16)));
        hipLaunchKernelGGL((gemm_mfma_kernel<L, CG, 16>), grid, dim3(256), 0, stream, wd, wbytes, X,
                           Y, m, n, k, nbn, padded_nbn);
    } else if (m <= 32) {
        const dim3 grid((unsigned)(padded_nbn * ((m + 31) / 32)));
        hipLaunchKernelGGL((gemm_mfma_kernel<L, CG, 32>), grid, dim3(256), 0, stream, wd, wbytes, X,
                           Y, m, n, k, nbn, padded_nbn);
    } else {
        const dim3 grid((unsigned)(padded_nbn * ((m + 63) / 64)));
        hipLaunchKernelGGL((gemm_mfma_kernel<L, CG, 64>), grid, dim3(256), 0, stream, wd, wbytes, X,
                           Y, m, n, k, nbn, padded_nbn);
    }
    return hipGetLastError();
}

template <int L>
hipError_t launch_l(bool mfma, const Geometry &geo, const uint8_t *wd, const uint16_t *X, int64_t m,
                    int64_t n, int64_t k, uint16_t *Y, hipStream_t stream)
{
    switch (geo.CG) {
#define Q4_CG_CASE(C)                                                                 \
    case C:                                                                           \
        if (mfma)                                                                     \
            return launch_mfma_lc<L, C>(geo, wd, X, m, n, k, Y, stream);              \
        return launch_valu_lc<L, C>(geo, wd, X, m, n, k, Y, stream);
        Q4_CG_CASE(1)
        Q4_CG_CASE(2)
        Q4_CG_CASE(3)
        Q4_CG_CASE(4)
#undef Q4_CG_CASE
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool gemm_mfma_eligible(const Geometry &geo) { return geo.P == 1 && geo.L >= 8; }

hipError_t launch_gemm(const Geometry &geo, const void *wdata, const uint16_t *X, int64_t m,
                       int64_t n, int64_t k, uint16_t *Y, int path, hipStream_t stream)
{
    const uint8_t *wd = static_cast<const uint8_t *>(wdata);
    bool mfma = (path == GEMM_PATH_MFMA) || (path == GEMM_PATH_AUTO && m >= 16);
    if (mfma && !gemm_mfma_eligible(geo))
        mfma = false;
    // the MFMA kernel addresses the weight through 32-bit buffer offsets
    if (mfma && geo.tiles * geo.tile_bytes >= ((int64_t)1 << 31))
        mfma = false;
    switch (geo.L) {
    case 64: return launch_l<64>(mfma, geo, wd, X, m, n, k, Y, stream);
    case 32: return launch_l<32>(mfma, geo, wd, X, m, n, k, Y, stream);
    case 16: return launch_l<16>(mfma, geo, wd, X, m, n, k, Y, stream);
    case 8: return launch_l<8>(mfma, geo, wd, X, m, n, k, Y, stream);
    case 4: return launch_l<4>(false, geo, wd, X, m, n, k, Y, stream);
    case 2: return launch_l<2>(false, geo, wd, X, m, n, k, Y, stream);
    case 1: return launch_l<1>(false, geo, wd, X, m, n, k, Y, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace q4
