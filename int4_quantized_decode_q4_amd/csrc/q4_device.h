// q4_device.h -- device helpers shared by the GEMV kernels of libq4
// (q4_kernels.hip) and the persistent chain kernel (q4_chain.hip): f16 bit
// conversions, the x pairing and int4 dequant arithmetic of one 8-code word,
// the residual add + RMSNorm pieces, and buffer resources.  Device code only.
//
// The dequant is the magic-number integer-to-float conversion: a small
// integer OR-ed into the mantissa of a power-of-two float reads as that power
// plus the integer.  Here a 4-bit code q in the mantissa of the f16 pattern
// 0x6400 (1024.0, mantissa ulp exactly 1) is the f16 value 1024 + q, so one
// packed subtract leaves q - 8; a code 4 bits higher in the same half reads
// as 1024 + 16 q.  The method is published for int4 -> f16 weights by Kim et
// al., "Who Says Elephants Can't Run: Bringing Large Scale MoE Models into
// Cloud Scale Production" (2022), and is the conversion behind AMD Composable
// Kernel's pk_int4 type.  The arrangement below -- pairs (q_i, q_i+4) against
// x pairs (x_i, x_i+4), the 16 q products in their own f32 sum, one scale
// multiply per group -- is this library's.
#ifndef Q4_DEVICE_H
#define Q4_DEVICE_H

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace q4 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

__device__ __forceinline__ uint16_t f16_bits(float v)
{
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

__device__ __forceinline__ float f16_value(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}

// natural x pairs (x0,x1) (x2,x3) (x4,x5) (x6,x7) of one 8-k word ->
// (x0,x4) (x1,x5) (x2,x6) (x3,x7), the order the dequant produces
__device__ __forceinline__ void pair_into(uint32_t *xp, uint4 n)
{
    xp[0] = (n.x & 0xFFFFu) | (n.z << 16);
    xp[1] = (n.x >> 16) | (n.z & 0xFFFF0000u);
    xp[2] = (n.y & 0xFFFFu) | (n.w << 16);
    xp[3] = (n.y >> 16) | (n.w & 0xFFFF0000u);
}

// the same permutation as one 16-byte chunk: (x0,x4) (x1,x5) (x2,x6) (x3,x7)
__device__ __forceinline__ uint4 pair_chunk(uint4 n)
{
    uint32_t p[4];
    pair_into(p, n);
    return make_uint4(p[0], p[1], p[2], p[3]);
}

__device__ __forceinline__ uint4 residual_add8(uint4 xv, uint4 rv)
{
    const uint32_t a[4] = {xv.x, xv.y, xv.z, xv.w}, b[4] = {rv.x, rv.y, rv.z, rv.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const h2 p = as_h2(a[i]), q = as_h2(b[i]);
        // the f32 sum of two f16 is exact: one rounding, to f16
        const _Float16 lo = (_Float16)((float)p.x + (float)q.x);
        const _Float16 hi = (_Float16)((float)p.y + (float)q.y);
        o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float sumsq8(uint4 v)
{
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const h2 p = as_h2(a[i]);
        s += (float)p.x * (float)p.x;
        s += (float)p.y * (float)p.y;
    }
    return s;
}

// f16(h * gamma * inv) of 8 halves; h * gamma is exact in f32
__device__ __forceinline__ uint4 norm8(uint4 hv, uint4 gv, float inv)
{
    const uint32_t a[4] = {hv.x, hv.y, hv.z, hv.w}, b[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const h2 p = as_h2(a[i]), q = as_h2(b[i]);
        const _Float16 lo = (_Float16)((float)p.x * (float)q.x * inv);
        const _Float16 hi = (_Float16)((float)p.y * (float)q.y * inv);
        o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint4 as_uint4(v4u v) { return make_uint4(v.x, v.y, v.z, v.w); }

__device__ __forceinline__ float inv_rms(float sumsq, int64_t k, float eps)
{
    return 1.0f / sqrtf(sumsq / (float)k + eps);
}

// The dequant masks and the f16 exponent pattern, held in VGPRs.  gfx9 VOP3
// instructions take no literal operands and read at most one SGPR, so with
// plain constants the compiler splits (w & mask) | magic into a VOP2 and and
// a VOP2 or (two instructions); from registers it is one v_and_or_b32.
struct DequantConsts {
    uint32_t lo, hi, magic;
};

__device__ __forceinline__ DequantConsts dequant_consts()
{
    DequantConsts k;
    asm("v_mov_b32 %0, 0x000F000F" : "=v"(k.lo));
    asm("v_mov_b32 %0, 0x00F000F0" : "=v"(k.hi));
    asm("v_mov_b32 %0, 0x64006400" : "=v"(k.magic));
    return k;
}

// 8 codes (canonical nibble order) against their 4 prepared x pairs.
__device__ __forceinline__ void dot_word(uint32_t w, const uint32_t *xp, float &p1, float &p16,
                                         const DequantConsts &m)
{
    const h2 k1 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 k16 = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t a0 = (w & m.lo) | m.magic;   // 1024 + q0, 1024 + q4
    const uint32_t a1 = (w & m.hi) | m.magic;   // 1024 + 16 q1, 1024 + 16 q5
    const uint32_t b = w >> 8;
    const uint32_t a2 = (b & m.lo) | m.magic;   // q2, q6
    const uint32_t a3 = (b & m.hi) | m.magic;   // 16 q3, 16 q7
    p1 = __builtin_amdgcn_fdot2(as_h2(a0) - k1, as_h2(xp[0]), p1, false);
    p16 = __builtin_amdgcn_fdot2(as_h2(a1) - k16, as_h2(xp[1]), p16, false);
    p1 = __builtin_amdgcn_fdot2(as_h2(a2) - k1, as_h2(xp[2]), p1, false);
    p16 = __builtin_amdgcn_fdot2(as_h2(a3) - k16, as_h2(xp[3]), p16, false);
}

// The 16-byte unit of one (row, group): 4 words of 8 codes.
__device__ __forceinline__ float dot_unit4(uint4 c, const uint32_t *xp, const DequantConsts &m)
{
    float p1 = 0.f, p16 = 0.f;
    dot_word(c.x, xp + 0, p1, p16, m);
    dot_word(c.y, xp + 4, p1, p16, m);
    dot_word(c.z, xp + 8, p1, p16, m);
    dot_word(c.w, xp + 12, p1, p16, m);
    return fmaf(p16, 0.0625f, p1);
}

// Buffer resources: a tile (one pass) is addressed through a V# whose
// num_records is the tile's byte size, or 0 when the wavefront has no such
// tile; buffer loads past num_records return zeros without touching memory,
// so prefetches need no branch and the compiler's vmcnt waits stay exact.
constexpr int kBufferWord3 = 0x00020000;   // gfx9-family raw buffer format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, bytes,
                                             kBufferWord3);
}

}  // namespace q4

#endif
