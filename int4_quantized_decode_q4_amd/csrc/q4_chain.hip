// q4_chain.hip -- a chain of int4 dequantizing GEMVs in one persistent launch.
//
// Sources: "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权"
// (zingnex.cn), section 内核融合 (fusion exists to cut the number of
// dispatches per decode step: add_norm, the fused QKV, attention, gate/up +
// SiLU) and section 技术栈对比 (the dispatch count per token is what the
// hand-written engine lowers); section 性能基准 (the int4 matmuls are where
// a decode step spends its time).
//
// On MI355X a launch costs 1-2 us beyond its memory time (ramp-up to the
// full HBM rate, the drain of the last wavefronts, and the gap to the next
// launch), which is a third of a 3072x3072 GEMV.  This kernel keeps one
// block of eight wavefronts per compute unit resident for a whole sequence
// of GEMVs (a decode layer's O-proj -> add + RMSNorm -> gate/up + SiLU ->
// down), so that
//   * the weights of the next GEMV are already streaming while the previous
//     one finishes: every wavefront requests its first tile of stage s + 1
//     as soon as it has computed its last tile of stage s, before any wait;
//   * a stage that consumes an earlier stage's output waits for exactly that
//     data, with no atomics and no cache-flushing fences: the producer writes
//     every output element as a 32-bit word (f16 value | 16-bit epoch tag)
//     with a device-coherent store, and the consumer reads the words with
//     device-coherent loads until every tag is the current launch's epoch.
//     A word is written with one store, so a reader sees the old word or the
//     new one, never a mix; the buffer only ever holds this launch's tag or
//     the previous launch's, so the epoch needs no reset;
//   * a stage that must only wait for an earlier one to finish (no data)
//     polls one completion flag per block of that stage.
// The epoch is a per-block launch counter kept in the workspace: block b of
// every launch reads and bumps its own word, so all blocks agree on it with
// no communication.  Every wait is bounded in time; a wait that runs out
// sets an error word and lets the block go on, so a launch always ends.
//
// Inside a stage each wavefront streams its tiles exactly as the block
// kernel of q4_kernels.hip does (whole tile in flight, the next tile's units
// requested as the current one's are consumed); x is staged once per block
// in LDS and paired per lane into VGPRs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "q4_device.h"
#include "q4_geometry.h"
#include "q4_internal.h"
#include "q4_lanes.h"

namespace q4 {

namespace {

constexpr int kWaves = kChainWaves;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxUnits = 8;       // 2 * CG
constexpr int kMaxCG = 4;
constexpr int kXHalves = 8192;     // largest k

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// One tile's registers for any of the chain's geometries: 2*CG code units
// and CG words of scales (two f16 each).
struct Regs {
    uint4 c[kMaxUnits];
    uint32_t s[kMaxCG];
};

template <int CG>
__device__ __forceinline__ void load_unit(Regs &r, rsrc_t rs, int lane, int i)
{
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, i * 1024, 0);
    r.c[i] = make_uint4(v.x, v.y, v.z, v.w);
}

template <int CG>
__device__ __forceinline__ void load_scales(Regs &r, rsrc_t rs, int lane)
{
#pragma unroll
    for (int j = 0; j < CG; ++j)
        r.s[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4 * CG + 4 * j, 2 * CG * 1024, 0);
}

template <int CG>
__device__ __forceinline__ void load_tile(Regs &r, rsrc_t rs, int lane)
{
    load_scales<CG>(r, rs, lane);
#pragma unroll
    for (int i = 0; i < 2 * CG; ++i)
        load_unit<CG>(r, rs, lane, i);
}

// unit i = (u, j) = (i / CG, i % CG) of a tile: rows 2s + u, group c*CG + j
template <int CG>
__device__ __forceinline__ void unit_mac(const Regs &r, int i, const uint32_t (&xp)[CG][16],
                                         float (&acc)[2], const DequantConsts &m)
{
    const int u = i / CG, j = i % CG;
    const float p = dot_unit4(r.c[i], &xp[j][0], m);
    const float sv = f16_value((uint16_t)(r.s[i >> 1] >> ((i & 1) * 16)));
    acc[u] = fmaf(sv, p, acc[u]);
}

// compute `cur`, requesting the units of `nxt` (the next tile of the same
// stage) one by one as cur's are consumed
template <int CG>
__device__ __forceinline__ void stream(const Regs &cur, Regs &nxt, rsrc_t nrs, int lane,
                                       const uint32_t (&xp)[CG][16], float (&acc)[2],
                                       const DequantConsts &m)
{
#pragma unroll
    for (int i = 0; i < 2 * CG; ++i) {
        unit_mac<CG>(cur, i, xp, acc, m);
        // issue the unit's arithmetic before the next load (otherwise the
        // compiler hoists every load to the top and the pipeline is lost)
        asm volatile("" ::"v"(acc[i / CG]) : "memory");
        if (i == 0)
            load_scales<CG>(nxt, nrs, lane);
        load_unit<CG>(nxt, nrs, lane, i);
    }
}

template <int CG>
__device__ __forceinline__ void compute(const Regs &cur, const uint32_t (&xp)[CG][16],
                                        float (&acc)[2], const DequantConsts &m)
{
#pragma unroll
    for (int i = 0; i < 2 * CG; ++i)
        unit_mac<CG>(cur, i, xp, acc, m);
}

__device__ __forceinline__ uint32_t tagged(float v, uint32_t tag)
{
    return (uint32_t)f16_bits(v) | (tag << 16);
}

// Epilogue of rows r0 (even) and r0 + 1 of a stage: y (f16), and the tagged
// copy later stages read.  F16: two rows; SILU: (gate i, up i) -> h_i.
__device__ __forceinline__ void store_pair(const ChainStageK &st, float y0, float y1, int64_t r0,
                                           uint32_t tag)
{
    if (st.epi == EPI_SILU) {
        const int64_t i = r0 >> 1;
        if (i < st.n_out) {
            const float h = y0 / (1.0f + expf(-y0)) * y1;
            st.y[i] = f16_bits(h);
            if (st.tag != nullptr)
                __hip_atomic_store(st.tag + i, tagged(h, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    if (r0 + 1 < st.rows) {
        *reinterpret_cast<uint32_t *>(st.y + r0) = (uint32_t)f16_bits(y0) | ((uint32_t)f16_bits(y1) << 16);
        if (st.tag != nullptr) {
            const uint64_t w = (uint64_t)tagged(y0, tag) | ((uint64_t)tagged(y1, tag) << 32);
            __hip_atomic_store(reinterpret_cast<uint64_t *>(st.tag + r0), w, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    } else if (r0 < st.rows) {
        st.y[r0] = f16_bits(y0);
        if (st.tag != nullptr)
            __hip_atomic_store(st.tag + r0, tagged(y0, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int L>
__device__ __forceinline__ void finish(const ChainStageK &st, const float (&acc)[2], int64_t t, int s,
                                       int c, uint32_t tag)
{
    const float y0 = lanes::reduce<L>(acc[0]);
    const float y1 = lanes::reduce<L>(acc[1]);
    if (c == 0)
        store_pair(st, y0, y1, t * (128 / L) + 2 * s, tag);
}

__device__ __forceinline__ rsrc_t tile_of(const ChainStageK &st, int64_t t, int pb)
{
    return t < st.tiles ? tile_rsrc(st.wd + t * pb, pb) : tile_rsrc(st.wd, 0);
}

// (L, CG) of each ChainGeo
template <int G>
struct GeoOf;
template <>
struct GeoOf<CHAIN_G64_1> {
    static constexpr int L = 64, CG = 1;
};
template <>
struct GeoOf<CHAIN_G32_3> {
    static constexpr int L = 32, CG = 3;
};
template <>
struct GeoOf<CHAIN_G64_2> {
    static constexpr int L = 64, CG = 2;
};
template <>
struct GeoOf<CHAIN_G64_3> {
    static constexpr int L = 64, CG = 3;
};
template <>
struct GeoOf<CHAIN_G64_4> {
    static constexpr int L = 64, CG = 4;
};

// A wavefront's LDS slot for the first tile of the next stage: the tile's
// bytes as they lie in memory (2*CG units of 1 KiB, then 256*CG bytes of
// scales), copied there by LDS-direct buffer loads, so nothing of it sits in
// VGPRs while the wavefront waits for the next stage's x.  Such a load puts
// lane i's bytes at the LDS base (M0) + i * size; an instruction offset
// would move the LDS address as well as the memory one, so the memory offset
// goes in the lane's voffset instead.
constexpr int kSlotBytes = kMaxCG * 2304;
typedef __attribute__((address_space(3))) void lds_void;

template <int G>
__device__ __forceinline__ void prefetch_g(uint8_t *slot, const ChainStageK &st, int64_t gw, int lane)
{
    constexpr int CG = GeoOf<G>::CG, PB = CG * 2304;
    const rsrc_t rs = tile_of(st, gw, PB);
    lds_void *dst = (lds_void *)slot;
    // units: 16 bytes per lane, 1 KiB per instruction
#define Q4_UNIT_DMA(i)                                                                            \
    if ((i) < 2 * CG)                                                                             \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)((uint8_t *)slot + (i) * 1024), 16, \
                                                 lane * 16 + (i) * 1024, 0, 0, 0);
    Q4_UNIT_DMA(0) Q4_UNIT_DMA(1) Q4_UNIT_DMA(2) Q4_UNIT_DMA(3)
    Q4_UNIT_DMA(4) Q4_UNIT_DMA(5) Q4_UNIT_DMA(6) Q4_UNIT_DMA(7)
#undef Q4_UNIT_DMA
    // scales: 4 bytes per lane, 256 bytes per instruction
#define Q4_SCALE_DMA(j)                                                                           \
    if ((j) < CG)                                                                                 \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)((uint8_t *)slot + 2 * CG * 1024 + (j) * 256), \
                                                 4, lane * 4 + 2 * CG * 1024 + (j) * 256, 0, 0, 0);
    Q4_SCALE_DMA(0) Q4_SCALE_DMA(1) Q4_SCALE_DMA(2) Q4_SCALE_DMA(3)
#undef Q4_SCALE_DMA
    (void)dst;
}

// Request the first tile of stage `st` for wavefront `gw` into its slot (a
// stage with no tile for it reads nothing: zero-size resource).
__device__ __forceinline__ void prefetch(uint8_t *slot, const ChainStageK *st, int64_t gw, int lane)
{
    switch (st != nullptr ? st->geo : -1) {
    case CHAIN_G64_1: prefetch_g<CHAIN_G64_1>(slot, *st, gw, lane); break;
    case CHAIN_G32_3: prefetch_g<CHAIN_G32_3>(slot, *st, gw, lane); break;
    case CHAIN_G64_2: prefetch_g<CHAIN_G64_2>(slot, *st, gw, lane); break;
    case CHAIN_G64_3: prefetch_g<CHAIN_G64_3>(slot, *st, gw, lane); break;
    case CHAIN_G64_4: prefetch_g<CHAIN_G64_4>(slot, *st, gw, lane); break;
    default: break;
    }
}

// The slot's tile into registers (the caller has waited for the copy).
template <int CG>
__device__ __forceinline__ void slot_to_regs(Regs &r, const uint8_t *slot, int lane)
{
#pragma unroll
    for (int i = 0; i < 2 * CG; ++i)
        r.c[i] = *reinterpret_cast<const uint4 *>(slot + i * 1024 + lane * 16);
#pragma unroll
    for (int j = 0; j < CG; ++j)
        r.s[j] = *reinterpret_cast<const uint32_t *>(slot + 2 * CG * 1024 + lane * 4 * CG + 4 * j);
}

// Wait until this wavefront's own stores have completed, but not the
// prefetch issued after them (vector memory operations, LDS-direct loads
// included, retire in order on this architecture): the count is that of the
// prefetch of the next stage's geometry.
__device__ __forceinline__ void wait_stores(int next_geo)
{
    switch (next_geo) {
    case CHAIN_G64_1: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;    // 2 + 1 loads
    case CHAIN_G32_3:
    case CHAIN_G64_3: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;    // 6 + 3
    case CHAIN_G64_2: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;    // 4 + 2
    case CHAIN_G64_4: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;   // 8 + 4
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// The tiles of stage st handled by wavefront gw: gw, gw + step, ...  The
// first one is in the wavefront's slot (requested earlier); the rest
// ping-pong between two register sets, each tile's loads issued while the
// one before it is computed.  After the last one, the first tile of stage
// `next` is requested into the slot.
template <int G>
__device__ __forceinline__ void run_stage(const ChainStageK &st, const ChainStageK *next, int64_t gw,
                                          int64_t step, uint8_t *slot, const uint4 *xs, uint32_t tag,
                                          int lane)
{
    constexpr int L = GeoOf<G>::L, CG = GeoOf<G>::CG, PB = CG * 2304;
    const int s = lane / L, c = lane % L;
    const int64_t G_ = st.k >> 5;
    uint32_t xp[CG][16];
#pragma unroll
    for (int j = 0; j < CG; ++j) {
        const int64_t g = (int64_t)c * CG + j;
        if (g < G_) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pair_into(&xp[j][4 * q], xs[g * 4 + q]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                xp[j][i] = 0u;
        }
    }
    const DequantConsts m = dequant_consts();
    Regs ra, rb;
    // the second tile is requested before the first (in the slot) is waited
    // for, so two tiles are in flight from the start of the stage; then the
    // slot's copy (older than those loads: vmcnt counts in order) is waited
    // for and read
    int64_t t = gw;
    load_tile<CG>(rb, tile_of(st, t + step, PB), lane);
    if constexpr (CG == 1)
        asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if constexpr (CG == 2)
        asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if constexpr (CG == 3)
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    slot_to_regs<CG>(ra, slot, lane);
    // no branch between "stream" and "compute only": the last tile's next
    // loads go to a zero-size resource (they read nothing), so the compiler
    // has no common code to hoist above a branch (which had kept a whole
    // tile's dequantised words live at once)
    if (t < st.tiles) {
        float a0[2] = {0.f, 0.f};
        compute<CG>(ra, xp, a0, m);
        finish<L>(st, a0, t, s, c, tag);
        t += step;
        while (t < st.tiles) {
            float a1[2] = {0.f, 0.f};
            stream<CG>(rb, ra, tile_of(st, t + step, PB), lane, xp, a1, m);
            finish<L>(st, a1, t, s, c, tag);
            t += step;
            if (t >= st.tiles)
                break;
            float a2[2] = {0.f, 0.f};
            stream<CG>(ra, rb, tile_of(st, t + step, PB), lane, xp, a2, m);
            finish<L>(st, a2, t, s, c, tag);
            t += step;
        }
    }
    // the slot is read (the ds_reads above completed before any of the
    // tile's arithmetic); the stores above are issued before the prefetch
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    prefetch(slot, next, gw, lane);
}

// 100 MHz device clock, for bounding waits
__device__ __forceinline__ int64_t ticks() { return (int64_t)wall_clock64(); }

__device__ __forceinline__ void raise_error(uint32_t *error)
{
    __hip_atomic_store(error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// add + RMSNorm of one staged vector in LDS (k halves at xb): h = f16(x +
// r), x' = f16(h * gamma / rms(h)), h -> h_out (block 0).  The sum of
// squares is taken in a fixed order (thread chunks, then the waves in
// order), so every block gets the same bits.  Called by every thread; ends
// with x' visible to the block.
__device__ void norm_lds(uint4 *xb, int64_t k, const uint16_t *r, const uint16_t *gamma, uint16_t *h_out,
                         float eps, float *red)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint4 *r4 = reinterpret_cast<const uint4 *>(r);
    const uint4 *g4 = reinterpret_cast<const uint4 *>(gamma);
    constexpr int kChunks = kXHalves / 8 / kThreads;   // uint4 chunks per thread, at most
    uint4 hv[kChunks];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
        const int64_t i = tid + (int64_t)q * kThreads;
        if (i < k / 8) {
            hv[q] = xb[i];
            if (r4 != nullptr)
                hv[q] = residual_add8(hv[q], r4[i]);
            ss += sumsq8(hv[q]);
            if (h_out != nullptr && blockIdx.x == 0)
                reinterpret_cast<uint4 *>(h_out)[i] = hv[q];
        }
    }
    ss = lanes::reduce<64>(ss);
    if (lane == 0)
        red[w] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
        tot += red[i];
    const float inv = inv_rms(tot, k, eps);
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
        const int64_t i = tid + (int64_t)q * kThreads;
        if (i < k / 8)
            xb[i] = norm8(hv[q], g4[i], inv);
    }
    __syncthreads();
}

// The wait of a dependent stage, and its x into LDS (xb, f16 [k]) when it
// reads an earlier stage's output: wait for the stage it must follow (one
// flag per block of it, polled by wave 0), poll the source stage's tagged
// words pair by pair until both carry this launch's tag, and apply the add +
// RMSNorm prologue.  Called by every thread of the block; ends with a block
// barrier (and the staged x visible to the whole block).
__device__ void stage_dep(const ChainArgs &a, const ChainStageK &st, uint32_t tag, uint4 *xb,
                          float *red, int nblocks)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t k = st.k;
    if (st.after >= 0 && w == 0) {
        const uint32_t *flags = a.st[st.after].flags;
        const int64_t t0 = ticks();
        for (int i = lane; i < nblocks; i += 64) {
            while (__hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag) {
                if (ticks() - t0 > a.wait_ticks) {
                    raise_error(a.error);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
    }
    if (st.src >= 0) {
        uint32_t *xw = reinterpret_cast<uint32_t *>(xb);
        const uint64_t *src = reinterpret_cast<const uint64_t *>(a.st[st.src].tag);
        const int64_t t0 = ticks();
        for (int64_t i = tid; i < k / 2; i += kThreads) {
            uint64_t v = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            while (((uint32_t)(v >> 16) & 0xFFFFu) != tag || (uint32_t)(v >> 48) != tag) {
                if (ticks() - t0 > a.wait_ticks) {
                    raise_error(a.error);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                v = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            xw[i] = (uint32_t)(v & 0xFFFFu) | (uint32_t)((v >> 16) & 0xFFFF0000u);
        }
    }
    __syncthreads();
    if (st.gamma != nullptr)
        norm_lds(xb, k, st.r, st.gamma, st.h_out, st.eps, red);
}

// Stage every given x into the staged-x area at the start of the launch:
// all of their loads are issued before any is used (up to 4 chunks of 8
// halves per thread), then the prologues run.  Thread 0 also records the
// block's launch count e (loaded before the first tile was requested) and
// publishes the launch's tag.
// x chunks of the given vectors into registers (up to 4 chunks of 8 halves
// per thread), then into the staged-x area, around the request of stage 0's
// first tile: the x loads go out first, and the wait before the LDS writes
// (in the same straight-line code as the tile request) leaves the tile's
// loads in flight.
template <int G>
__device__ __forceinline__ void given_to_lds(const ChainArgs &a, uint4 *xg, uint8_t *slot, int64_t gw,
                                             int lane, const uint4 (&v)[kChainGivenHalves / 8 / kThreads],
                                             int total)
{
    prefetch_g<G>(slot, a.st[0], gw, lane);
#pragma unroll
    for (int q = 0; q < kChainGivenHalves / 8 / kThreads; ++q) {
        const int c = threadIdx.x + q * kThreads;
        if (c < total)
            xg[c] = v[q];
    }
}

// Stage every given x at the start of the launch, request stage 0's first
// tile, record the block's launch count (e, loaded before everything else)
// and publish the launch's tag; then the prologues of given vectors run.
__device__ void stage_given(const ChainArgs &a, uint4 *xg, float *red, uint8_t *slot, int64_t gw,
                            int lane, uint32_t e_prev, uint32_t *tag_s)
{
    constexpr int kPer = kChainGivenHalves / 8 / kThreads;
    const int tid = threadIdx.x;
    // the entries' pointers and offsets, read up front (scalar loads that do
    // not depend on one another)
    const uint16_t *gx[kChainMaxStages];
    int goff[kChainMaxStages];
    const int ng = a.n_given;
#pragma unroll
    for (int g = 0; g < kChainMaxStages; ++g) {
        gx[g] = a.given[g].x;
        goff[g] = g < ng ? a.given[g].off : 0x7fffffff;
    }
    const int total = a.given[ng - 1].off + (int)(a.given[ng - 1].k / 8);
    uint4 v[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        // the vector holding chunk c, chosen per lane among the entries'
        // pointers (the kernel arguments are read with scalar loads only);
        // a lane past the end re-reads the last chunk and discards it, so
        // the load needs no branch
        const int c = min(tid + q * kThreads, total - 1);
        const uint16_t *xp = gx[0];
        int off = 0;
#pragma unroll
        for (int g = 1; g < kChainMaxStages; ++g)
            if (c >= goff[g]) {
                xp = gx[g];
                off = goff[g];
            }
        v[q] = reinterpret_cast<const uint4 *>(xp)[c - off];
    }
    switch (a.st[0].geo) {
    case CHAIN_G64_1: given_to_lds<CHAIN_G64_1>(a, xg, slot, gw, lane, v, total); break;
    case CHAIN_G32_3: given_to_lds<CHAIN_G32_3>(a, xg, slot, gw, lane, v, total); break;
    case CHAIN_G64_2: given_to_lds<CHAIN_G64_2>(a, xg, slot, gw, lane, v, total); break;
    case CHAIN_G64_3: given_to_lds<CHAIN_G64_3>(a, xg, slot, gw, lane, v, total); break;
    case CHAIN_G64_4: given_to_lds<CHAIN_G64_4>(a, xg, slot, gw, lane, v, total); break;
    default: break;
    }
    if (tid == 0) {
        const uint32_t e = e_prev + 1u;
        __hip_atomic_store(a.epochs + blockIdx.x, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *tag_s = e % 65535u + 1u;   // 1 .. 65535: never the 0 of a cleared workspace
    }
    __syncthreads();
    for (int g = 0; g < ng; ++g)
        if (a.given[g].gamma != nullptr)
            norm_lds(xg + a.given[g].off, a.given[g].k, a.given[g].r, a.given[g].gamma, a.given[g].h_out,
                     a.given[g].eps, red);
}

__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs args)
{
    // the stages are indexed by a loop counter: read them in place from the
    // kernel-argument segment (indexing the by-value parameter would copy it
    // to private memory)
    (void)args;
    const ChainArgs &a = *(const ChainArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    __shared__ uint4 xg[kChainGivenHalves / 8];   // every given x, staged once
    __shared__ uint4 xd[2][kXHalves / 8];         // the x of dependent stages, alternately
    __shared__ float red[kWaves];
    __shared__ uint32_t tag_s;
    __shared__ uint4 slots[kWaves][kSlotBytes / 16];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nblocks = gridDim.x;
    // tile t of a stage goes to block t % nblocks, wavefront (t / nblocks) % 8:
    // a small stage spreads over every compute unit (a few wavefronts each)
    // instead of filling a few of them
    const int64_t gw = (int64_t)w * nblocks + blockIdx.x;   // this wavefront's first tile of a stage
    const int64_t step = (int64_t)nblocks * kWaves;
    uint8_t *slot = reinterpret_cast<uint8_t *>(&slots[w][0]);
    // this block's launch count: every block of every launch bumps its own
    // word, so all blocks of one launch agree on it.  It, every given x and
    // stage 0's first tile are requested in that order, before anything
    // waits.
    // (every thread loads the word: no branch, so nothing waits for it
    // before it is used)
    const uint32_t e_prev = __hip_atomic_load(a.epochs + blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stage_given(a, xg, red, slot, gw, lane, e_prev, &tag_s);   // ends with a block barrier
    const uint32_t tag = tag_s;
    int dep = 0;                   // dependent stages so far: which xd buffer is next
    for (int si = 0; si < a.n; ++si) {
        const ChainStageK &st = a.st[si];
        const ChainStageK *next = si + 1 < a.n ? &a.st[si + 1] : nullptr;
        // a stage with its own x needs no block barrier: the staged x does
        // not change, and every wavefront moves on as soon as it is done.  A
        // dependent stage stages its x into the xd buffer not used by the
        // dependent stage before it (a wavefront still in that stage may be
        // reading it), and its staging ends with a block barrier.
        const uint4 *xb = xg + st.xoff;
        if (st.src >= 0 || st.after >= 0) {
            uint4 *buf = xd[dep & 1];
            stage_dep(a, st, tag, buf, red, nblocks);
            if (st.src >= 0) {
                xb = buf;
                ++dep;
            }
        }
        switch (st.geo) {
        case CHAIN_G64_1: run_stage<CHAIN_G64_1>(st, next, gw, step, slot, xb, tag, lane); break;
        case CHAIN_G32_3: run_stage<CHAIN_G32_3>(st, next, gw, step, slot, xb, tag, lane); break;
        case CHAIN_G64_2: run_stage<CHAIN_G64_2>(st, next, gw, step, slot, xb, tag, lane); break;
        case CHAIN_G64_3: run_stage<CHAIN_G64_3>(st, next, gw, step, slot, xb, tag, lane); break;
        case CHAIN_G64_4: run_stage<CHAIN_G64_4>(st, next, gw, step, slot, xb, tag, lane); break;
        default: break;
        }
        // a stage that others wait for publishes this block's completion
        // once every wavefront's stores of it are done
        if (st.flags != nullptr) {
            wait_stores(next != nullptr ? next->geo : -1);
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_store(st.flags + blockIdx.x, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

int chain_geo_of(const Geometry &geo)
{
    if (geo.P != 1)
        return -1;
    if (geo.L == 64 && geo.CG == 1)
        return CHAIN_G64_1;
    if (geo.L == 32 && geo.CG == 3)
        return CHAIN_G32_3;
    if (geo.L == 64 && geo.CG == 2)
        return CHAIN_G64_2;
    if (geo.L == 64 && geo.CG == 3)
        return CHAIN_G64_3;
    if (geo.L == 64 && geo.CG == 4)
        return CHAIN_G64_4;
    return -1;
}

hipError_t launch_chain(const ChainArgs &a, int blocks, hipStream_t stream)
{
    hipLaunchKernelGGL(chain_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace q4
