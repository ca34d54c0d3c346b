// q4_attention.hip -- paged-attention decode for one token on gfx950: the
// attention step between the fused QKV projection and the output projection
// of a decoder layer, reading the paged K/V cache that step writes.
//
// Source: "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权"
// (zingnex.cn), section 内核融合 (attention merges paged attention with the
// page-table reads) and section 完整的推理流水线 (vLLM-style page table).
//
// Design (split over the context, as flash-decoding does for one query):
//  * the cache is head-major inside a page ([page][K|V][head][slot][dim]),
//    so the 16 K rows (and the 16 V rows) one head takes from a page are one
//    contiguous run of 32 d bytes;
//  * a block owns one query head and a chunk of positions, sized from the
//    context so the grid holds about one block per compute unit (measured
//    best: more, shorter blocks and more wavefronts per block were slower);
//    its 4 wavefronts take a quarter each, 16 positions (one page) at a
//    time: 4 lanes per position, each lane d/4 dims interleaved in 16-byte
//    pieces, so every load instruction reads 16 whole 64-byte spans; the
//    wavefront's page indices are read once, one per lane;
//  * the next step's rows are requested before the current one is used, by
//    buffer loads through a resource that spans the head's K and V runs of
//    the step's page; a step past the wavefront's end or on an absent page
//    gets a resource of size 0, whose loads return zeros without touching
//    memory, so every load is issued unconditionally and the compiler's
//    vmcnt waits stay exact (a branch around the loads makes it wait for
//    all of them);
//  * scores: f16 pairs through v_dot2_f32_f16, summed over the 4 lanes of a
//    position with DPP, times scale * log2(e), so the softmax runs in base 2
//    (e^(s - m) = 2^((s - m) log2 e); one v_exp_f32 per exponential); every
//    lane runs its own online softmax (running max and sum, the accumulator
//    rescaled when the max grows) and the lanes of a dim slice merge their
//    states once at the end, so a step has no wavefront-wide exchange;
//  * the 4 wavefronts are combined in LDS; with one chunk the block writes
//    the f16 output, otherwise it writes (max, sum, weighted V) to the
//    workspace and a second launch merges the chunks of each head (merging
//    in the last block of a head instead needs an agent-scope release per
//    block and an acquire in the last one, which write back and invalidate
//    the L2; measured slower than the second launch).
//
// The optional int8 cache (same section 完整的推理流水线: an int8 KV path that
// halves the cache) stores each (token, kv head) row as int8 codes with one
// f32 scale (max |x| / 127): pages [page][K|V][kv head] of 16 d codes + 16
// scales.  kv_append_int8_kernel quantises the k and v heads a fused QKV step
// produced (a head's row spans many GEMV tiles, so its max cannot be taken in
// that kernel's epilogue); the attention kernel's int8 instantiation reads
// 8-byte pieces (the same dims per lane as the f16 one), turns 4 codes into
// two exact f16 pairs with one xor, one shift and two and-or (excess-128 bytes
// under the 0x6400 exponent) and applies the K scale once per score and the
// V scale folded into the softmax weight.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "q4_internal.h"
#include "q4_lanes.h"

namespace q4 {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
constexpr int kBufferWord3 = 0x00020000;   // gfx9-family raw buffer format

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// bytes of one int8 block ([page][K|V][head]): 16 rows of d codes + 16 f32 scales
__host__ __device__ constexpr int64_t kv8_block_bytes(int64_t d) { return 16 * d + 64; }

// 4 int8 codes (one word) -> f16 pairs (c0, c2) and (c1, c3), exact: the
// codes as excess-128 bytes under the 0x6400 exponent are 1024 + 128 + c
struct CodePairs {
    h2 a, b;
};
__device__ __forceinline__ CodePairs int8_pairs(uint32_t w)
{
    const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t u = w ^ 0x80808080u;
    const uint32_t lo = (u & 0x00FF00FFu) | 0x64006400u;
    const uint32_t hi = ((u >> 8) & 0x00FF00FFu) | 0x64006400u;
    return {as_h2(lo) - off, as_h2(hi) - off};
}

// q pairs (d0, d1) (d2, d3) .. of one 8-dim piece -> (d0, d2) (d1, d3) (d4, d6) (d5, d7)
__device__ __forceinline__ uint4 pair_for_int8(uint4 n)
{
    return make_uint4((n.x & 0xFFFFu) | (n.y << 16), (n.x >> 16) | (n.y & 0xFFFF0000u),
                      (n.z & 0xFFFFu) | (n.w << 16), (n.z >> 16) | (n.w & 0xFFFF0000u));
}

__device__ __forceinline__ float dot8_int8(uint4 qp, v2u k, float acc)
{
    const CodePairs c0 = int8_pairs(k.x), c1 = int8_pairs(k.y);
    acc = __builtin_amdgcn_fdot2(c0.a, as_h2(qp.x), acc, false);
    acc = __builtin_amdgcn_fdot2(c0.b, as_h2(qp.y), acc, false);
    acc = __builtin_amdgcn_fdot2(c1.a, as_h2(qp.z), acc, false);
    acc = __builtin_amdgcn_fdot2(c1.b, as_h2(qp.w), acc, false);
    return acc;
}

// acc[e] += p * code_e for the 8 codes of one piece (dims e = 0..7)
__device__ __forceinline__ void axpy8_int8(float p, v2u v, float *acc)
{
    const CodePairs c0 = int8_pairs(v.x), c1 = int8_pairs(v.y);
    acc[0] = fmaf(p, (float)c0.a.x, acc[0]);
    acc[2] = fmaf(p, (float)c0.a.y, acc[2]);
    acc[1] = fmaf(p, (float)c0.b.x, acc[1]);
    acc[3] = fmaf(p, (float)c0.b.y, acc[3]);
    acc[4] = fmaf(p, (float)c1.a.x, acc[4]);
    acc[6] = fmaf(p, (float)c1.a.y, acc[6]);
    acc[5] = fmaf(p, (float)c1.b.x, acc[5]);
    acc[7] = fmaf(p, (float)c1.b.y, acc[7]);
}

#ifndef Q4_ATT_DEPTH
#define Q4_ATT_DEPTH 2
#endif
#ifndef Q4_ATT_WAVES
#define Q4_ATT_WAVES 4
#endif
constexpr int kWaves = Q4_ATT_WAVES;              // wavefronts per block
constexpr int kStep = 16;                         // positions per wavefront step (one page)
constexpr int kMinChunk = kStep * kWaves;         // positions per block: one step per wavefront ..
constexpr int kMaxChunk = 64 * kStep * kWaves;    // .. up to 64 pages per wavefront
#ifndef Q4_ATT_TARGET_BLOCKS
#define Q4_ATT_TARGET_BLOCKS 256
#endif
constexpr int64_t kTargetBlocks = Q4_ATT_TARGET_BLOCKS;   // blocks the chunking aims for

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

// 2^x in f32 (v_exp_f32; 2^-inf = 0).
__device__ __forceinline__ float exp2_f32(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge two online-softmax states (max m, sum l, accumulator acc; scores in
// base-2 units): the result is the state of the union of their positions.
template <int LD>
__device__ __forceinline__ void merge_state(float &m, float &l, float *acc, float mo, float lo,
                                            const float *acco)
{
    const float mn = fmaxf(m, mo);
    const float e1 = m == -INFINITY ? 0.f : exp2_f32(m - mn);
    const float e2 = mo == -INFINITY ? 0.f : exp2_f32(mo - mn);
    l = l * e1 + lo * e2;
#pragma unroll
    for (int i = 0; i < LD; ++i)
        acc[i] = acc[i] * e1 + acco[i] * e2;
    m = mn;
}

// DL = d / 32: 16-byte loads per lane per row (each lane d/4 dims).  Every
// lane keeps its own online softmax over the positions it meets (no
// cross-lane work per step beyond the 4-lane score sum); the 16 lanes of a
// dim slice merge their states once at the end.
template <int DL, bool I8>
__global__ __launch_bounds__(64 * kWaves) void attention_decode_kernel(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ cache,
    const int32_t *__restrict__ page_table, int32_t n_pages, int32_t ctx, int32_t nq,
    int32_t nkv, int32_t chunk_len, float scale, uint16_t *__restrict__ out,
    float *__restrict__ partial)
{
    constexpr int D = 32 * DL;
    constexpr int LD = 8 * DL;   // dims per lane
    constexpr int R = Q4_ATT_DEPTH;   // steps in flight
    __shared__ float wm[kWaves], wl[kWaves];
    __shared__ float wacc[kWaves][D];
    const int lane = threadIdx.x & 63;
    const float scale2 = scale * 1.44269504088896340736f;   // scores in base-2 units
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int h = blockIdx.x % nq, chunk = blockIdx.x / nq;
    const int g = h / (nq / nkv);
    const int sub = lane & 3, slot = lane >> 2;
    // bytes of the K (or V) half of a page, and of one head's part of it
    constexpr int64_t kRowBytes = I8 ? D : 2 * D;
    const int64_t head_bytes = I8 ? kv8_block_bytes(D) : 16 * kRowBytes;
    const int64_t half_page = (int64_t)nkv * head_bytes;
    // byte offsets inside a step's resource: this lane's pieces of its row in
    // the K run, the V run half a page further on, and (int8) the row scales
    constexpr int kPiece = I8 ? 8 : 16;
    const int k_off = slot * (int)kRowBytes + sub * kPiece;
    const int v_off = k_off + (int)half_page;
    const int ks_off = 16 * D + 4 * slot, vs_off = ks_off + (int)half_page;
    const int span = (int)(half_page + head_bytes);

    // lane `sub` holds the 16-byte pieces sub, sub + 4, ... of a row, so the
    // 4 lanes of a position read 64 contiguous bytes per load instruction
    uint4 qv[DL];
#pragma unroll
    for (int j = 0; j < DL; ++j) {
        qv[j] = reinterpret_cast<const uint4 *>(q + (int64_t)h * D)[4 * j + sub];
        if constexpr (I8)
            qv[j] = pair_for_int8(qv[j]);
    }

    const int t_begin = chunk * chunk_len + w * (chunk_len / kWaves);
    const int t_end = min(t_begin + chunk_len / kWaves, ctx);
    // the wavefront's page indices (at most 64), one per lane, read once: a
    // step's K/V addresses then never wait on the table
    const int npg = t_begin < t_end ? (t_end - t_begin + kStep - 1) / kStep : 0;
    const int32_t my_page = lane < npg ? page_table[(t_begin >> 4) + lane] : -1;
    struct Rows {
        uint4 k[I8 ? 1 : DL], v[I8 ? 1 : DL];   // f16 pieces
        v2u k8[I8 ? DL : 1], v8[I8 ? DL : 1];   // int8 pieces
        float ks, vs;                            // int8 row scales
        bool ok;
    };
    auto load = [&](Rows &r, int t0) {
        // t0 % 16 == 0: the step is one page (uniform over the wavefront)
        const int32_t page = t0 < t_end ? __builtin_amdgcn_readlane(my_page, (t0 - t_begin) >> 4) : -1;
        r.ok = page >= 0 && page < n_pages;
        const uint8_t *base = cache + (r.ok ? (int64_t)page * 2 * half_page + (int64_t)g * head_bytes : 0);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(base), (short)0, r.ok ? span : 0, kBufferWord3);
        if constexpr (I8) {
#pragma unroll
            for (int j = 0; j < DL; ++j) {
                r.k8[j] = __builtin_amdgcn_raw_buffer_load_b64(rs, k_off + 4 * kPiece * j, 0, 0);
                r.v8[j] = __builtin_amdgcn_raw_buffer_load_b64(rs, v_off + 4 * kPiece * j, 0, 0);
            }
            r.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, ks_off, 0, 0));
            r.vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, vs_off, 0, 0));
        } else {
#pragma unroll
            for (int j = 0; j < DL; ++j) {
                const v4u k = __builtin_amdgcn_raw_buffer_load_b128(rs, k_off + 4 * kPiece * j, 0, 0);
                const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, v_off + 4 * kPiece * j, 0, 0);
                r.k[j] = make_uint4(k.x, k.y, k.z, k.w);
                r.v[j] = make_uint4(v.x, v.y, v.z, v.w);
            }
        }
    };

    float acc[LD];
#pragma unroll
    for (int i = 0; i < LD; ++i)
        acc[i] = 0.f;
    float m = -INFINITY, l = 0.f;   // this lane's state
    Rows ring[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        load(ring[i], t_begin + i * kStep);
    for (int t0 = t_begin; t0 < t_end; t0 += R * kStep) {
        // no early exit inside: a step past the end has ok == false and
        // costs only its (zero-size) loads, and one path through the loop
        // keeps the compiler's vmcnt waits exact
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int ts = t0 + i * kStep;
            const Rows &r = ring[i];
            const int t = ts + slot;
            // slots past the context (or of an absent page) hold whatever the
            // cache holds there: they take no part
            const bool valid = r.ok && t < t_end;
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < DL; ++j) {
                if constexpr (I8)
                    s = dot8_int8(qv[j], r.k8[j], s);
                else
                    s = dot8(qv[j], r.k[j], s);
            }
            s = lanes::reduce<4>(s) * scale2;
            if constexpr (I8)
                s *= r.ks;
            if (valid) {
                const float mn = fmaxf(m, s);
                const float alpha = exp2_f32(m - mn);   // 0 while m is still -inf
                const float p = exp2_f32(s - mn);
                l = l * alpha + p;
#pragma unroll
                for (int c = 0; c < LD; ++c)
                    acc[c] *= alpha;
                if constexpr (I8) {
                    const float pv = p * r.vs;
#pragma unroll
                    for (int j = 0; j < DL; ++j)
                        axpy8_int8(pv, r.v8[j], acc + 8 * j);
                } else {
#pragma unroll
                    for (int j = 0; j < DL; ++j)
                        axpy8(p, r.v[j], acc + 8 * j);
                }
                m = mn;
            }
            // the step's registers are refilled with the step R further on
            load(ring[i], ts + R * kStep);
        }
    }
    // merge the 16 lanes of each dim slice (lanes with the same `sub`)
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) {
        float acco[LD];
#pragma unroll
        for (int c = 0; c < LD; ++c)
            acco[c] = __shfl_xor(acc[c], off);
        const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
        merge_state<LD>(m, l, acc, mo, lo, acco);
    }
    if (lane < 4) {   // acc[8 j + e] is dim (4 j + lane) * 8 + e
#pragma unroll
        for (int j = 0; j < DL; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                wacc[w][(4 * j + lane) * 8 + e] = acc[8 * j + e];
    }
    if (lane == 0) {
        wm[w] = m;
        wl[w] = l;
    }
    __syncthreads();
    float M = wm[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i)
        M = fmaxf(M, wm[i]);
    float e[kWaves], L = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        e[i] = wm[i] == -INFINITY ? 0.f : exp2_f32(wm[i] - M);
        L += wl[i] * e[i];
    }
    for (int i = threadIdx.x; i < D; i += blockDim.x) {
        float A = 0.f;
#pragma unroll
        for (int u = 0; u < kWaves; ++u)
            A += wacc[u][i] * e[u];
        if (partial == nullptr) {   // the whole context in one chunk
            out[(int64_t)h * D + i] = __builtin_bit_cast(uint16_t, (_Float16)(A / L));
        } else {
            float *rec = partial + ((int64_t)h * (gridDim.x / nq) + chunk) * (D + 2);
            rec[2 + i] = A;
            if (i == 0) {
                rec[0] = M;
                rec[1] = L;
            }
        }
    }
}

// Quantise the k and v heads of one fused QKV output (f16 [nq + 2 nkv][d],
// the k heads roped) into slot pos % 16 of page page_table[pos / 16]: one
// 64-lane block per (K|V, kv head); max |x| over the row by a wavefront max,
// scale = max / 127 and each code = rint(x / scale), both f32 divisions
// correctly rounded (the codes are decided in f32); an absent page writes
// nothing.
__global__ __launch_bounds__(64) void kv_append_int8_kernel(const uint16_t *__restrict__ qkv,
                                                            int32_t nq, int32_t nkv, int32_t d,
                                                            int32_t pos, uint8_t *__restrict__ cache8,
                                                            const int32_t *__restrict__ page_table,
                                                            int32_t n_pages)
{
    const int kv = blockIdx.x / nkv, g = blockIdx.x % nkv, lane = threadIdx.x;
    const int32_t page = page_table[pos >> 4];
    if (page < 0 || page >= n_pages)
        return;
    const uint16_t *row = qkv + ((int64_t)nq + (int64_t)kv * nkv + g) * d;
    float v[4], m = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {   // d <= 256
        const int i = lane + 64 * u;
        v[u] = i < d ? (float)__builtin_bit_cast(_Float16, row[i]) : 0.f;
        m = fmaxf(m, fabsf(v[u]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        m = fmaxf(m, __shfl_xor(m, off));
    const float sc = __fdiv_rn(m, 127.0f);
    uint8_t *blk = cache8 + (int64_t)page * 2 * nkv * kv8_block_bytes(d) +
                   ((int64_t)kv * nkv + g) * kv8_block_bytes(d);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = lane + 64 * u;
        if (i < d) {
            const float c = sc == 0.f ? 0.f : rintf(__fdiv_rn(v[u], sc));
            blk[(pos & 15) * d + i] = (uint8_t)(int8_t)c;
        }
    }
    if (lane == 0)
        *reinterpret_cast<float *>(blk + 16 * d + 4 * (pos & 15)) = sc;
}

// Combine the chunks of each head:
//   out = sum_c A_c 2^(M_c - Mx) / sum_c L_c 2^(M_c - Mx),  Mx = max_c M_c
// (maxima in base-2 units).  A thread owns one dim of one head and merges the
// chunk records online, reading 16 chunks' (M, L, A) per batch with every
// load issued before the first use, so a context of up to 16 chunks costs
// one round trip to memory.
constexpr int kCombineBatch = 16;

__global__ __launch_bounds__(64) void attention_combine_kernel(const float *__restrict__ partial,
                                                               int32_t chunks, int32_t d,
                                                               uint16_t *__restrict__ out)
{
    const int h = blockIdx.x, i = blockIdx.y * 64 + threadIdx.x;
    if (i >= d)
        return;
    const int64_t stride = d + 2;
    const float *rec = partial + (int64_t)h * chunks * stride;
    float m = -INFINITY, l = 0.f, a = 0.f;
    for (int c0 = 0; c0 < chunks; c0 += kCombineBatch) {
        float mc[kCombineBatch], lc[kCombineBatch], ac[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const float *r = rec + min(c0 + u, chunks - 1) * stride;   // in bounds; extras unused
            mc[u] = r[0];
            lc[u] = r[1];
            ac[u] = r[2 + i];
        }
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            if (c0 + u < chunks) {
                const float mn = fmaxf(m, mc[u]);
                const float e1 = m == -INFINITY ? 0.f : exp2_f32(m - mn);
                const float e2 = mc[u] == -INFINITY ? 0.f : exp2_f32(mc[u] - mn);
                l = l * e1 + lc[u] * e2;
                a = a * e1 + ac[u] * e2;
                m = mn;
            }
        }
    }
    out[(int64_t)h * d + i] = __builtin_bit_cast(uint16_t, (_Float16)(a / l));
}

// Positions per block: the longest chunk (kMinChunk times a power of two, at
// most kMaxChunk) that still gives the grid about one block per compute unit,
// but never below kMinChunk.  Longer chunks spread the block's fixed cost (query,
// page indices, the final merge, the partial record) over more rows.
int64_t chunk_len(int64_t ctx, int64_t nq)
{
    int64_t c = kMaxChunk;
    while (c > kMinChunk && nq * ((ctx + c - 1) / c) < kTargetBlocks)
        c >>= 1;
    return c;
}

template <int DL, bool I8>
hipError_t launch_dl(const uint16_t *q, const uint8_t *cache, const int32_t *pt, int32_t n_pages,
                     int32_t ctx, int32_t nq, int32_t nkv, float scale, uint16_t *out, void *ws,
                     hipStream_t stream)
{
    const int cl = (int)chunk_len(ctx, nq);
    const int chunks = (ctx + cl - 1) / cl;
    float *partial = chunks > 1 ? static_cast<float *>(ws) : nullptr;
    hipLaunchKernelGGL((attention_decode_kernel<DL, I8>), dim3((unsigned)(nq * chunks)), dim3(64 * kWaves), 0,
                       stream, q, cache, pt, n_pages, ctx, nq, nkv, cl, scale, out, partial);
    if (chunks > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(attention_combine_kernel, dim3((unsigned)nq, (unsigned)(DL + 1) / 2), dim3(64),
                           0, stream, partial, chunks, 32 * DL, out);
    }
    return hipGetLastError();
}

}  // namespace

int64_t attention_workspace_bytes(int64_t ctx, int64_t nq, int64_t d)
{
    const int64_t cl = chunk_len(ctx, nq);
    const int64_t chunks = (ctx + cl - 1) / cl;
    return chunks > 1 ? nq * chunks * (d + 2) * 4 : 0;
}

template <bool I8>
static hipError_t launch_any(const uint16_t *q, const uint8_t *cache, const int32_t *page_table,
                             int32_t n_pages, int32_t ctx, int32_t nq, int32_t nkv, int32_t d,
                             float scale, uint16_t *out, void *ws, hipStream_t stream)
{
    switch (d / 32) {
    case 1: return launch_dl<1, I8>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, ws, stream);
    case 2: return launch_dl<2, I8>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, ws, stream);
    case 3: return launch_dl<3, I8>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, ws, stream);
    case 4: return launch_dl<4, I8>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, ws, stream);
    case 5: return launch_dl<5, I8>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, ws, stream);
    case 6: return launch_dl<6, I8>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, ws, stream);
    case 7: return launch_dl<7, I8>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, ws, stream);
    case 8: return launch_dl<8, I8>(q, cache, page_table, n_pages, ctx, nq, nkv, scale, out, ws, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attention(const uint16_t *q, const uint16_t *cache, const int32_t *page_table,
                            int32_t n_pages, int32_t ctx, int32_t nq, int32_t nkv, int32_t d,
                            float scale, uint16_t *out, void *ws, hipStream_t stream)
{
    return launch_any<false>(q, reinterpret_cast<const uint8_t *>(cache), page_table, n_pages, ctx,
                             nq, nkv, d, scale, out, ws, stream);
}

hipError_t launch_attention_int8(const uint16_t *q, const uint8_t *cache8, const int32_t *page_table,
                                 int32_t n_pages, int32_t ctx, int32_t nq, int32_t nkv, int32_t d,
                                 float scale, uint16_t *out, void *ws, hipStream_t stream)
{
    return launch_any<true>(q, cache8, page_table, n_pages, ctx, nq, nkv, d, scale, out, ws, stream);
}

int64_t kv_int8_page_bytes(int64_t nkv, int64_t d) { return 2 * nkv * kv8_block_bytes(d); }

hipError_t launch_kv_append_int8(const uint16_t *qkv, int32_t nq, int32_t nkv, int32_t d, int32_t pos,
                                 uint8_t *cache8, const int32_t *page_table, int32_t n_pages,
                                 hipStream_t stream)
{
    hipLaunchKernelGGL(kv_append_int8_kernel, dim3((unsigned)(2 * nkv)), dim3(64), 0, stream, qkv, nq,
                       nkv, d, pos, cache8, page_table, n_pages);
    return hipGetLastError();
}

}  // namespace q4
