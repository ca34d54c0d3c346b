// q4_internal.h -- launchers shared by the host API (q4_api.cpp) and the
// kernels (q4_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "q4_geometry.h"

namespace q4 {

enum Epilogue {
    EPI_F16 = 0,   // y f16, rounded to nearest even
    EPI_F32 = 1,   // f32 logits, optional argmax
    EPI_SILU = 2,  // interleaved gate/up rows -> SiLU(g) * u, f16
    EPI_ROPE = 3,  // rotary-paired head rows -> RoPE on q and k, f16, KV append
};

// The fused QKV epilogue: heads of d rows, nq q heads then nkv k heads then
// nkv v heads; RoPE at position pos on q and k; k and v appended to the
// paged cache [n_pages][2][nkv][16][d] (cache may be null).
struct RopeArgs {
    int32_t d, nq, nkv, pos;
    double base;
    uint16_t *cache;
    const int32_t *page_table;
    int32_t n_pages;
};

// What the RoPE epilogue's kernels receive: RopeArgs plus the launch's
// twiddles (cos, sin of pos * base^(-2i/d), i < d/2), computed on the host
// in f64 and passed in the kernel arguments.  Other epilogues get NoRope.
constexpr int kRopeMaxHalf = 256;   // head_dim <= 512
struct RopeTab {
    int32_t d, nq, nkv, pos;
    uint16_t *cache;
    const int32_t *page_table;
    int32_t n_pages;
    float cs[kRopeMaxHalf][2];
};
struct NoRope {
};
template <int EPI>
struct RopeParam {
    using type = NoRope;
};
template <>
struct RopeParam<EPI_ROPE> {
    using type = RopeTab;
};

// Row order of a packed layout: plain, gate/up interleave, rotary pairs.
enum PackMode { PACK_ROWS = 0, PACK_GATE_UP = 1, PACK_ROPE = 2 };

// Scratch of the LM-head argmax inside the caller's workspace: 17 counters
// of 256 bytes each at the start (at the same place for every weight shape,
// zero before the first call; every call leaves them zero again), then one
// 8-byte candidate per launched block.
struct ArgmaxScratch {
    unsigned long long *partials; // one (f32 bits | index << 32) per block
    int32_t *result;              // device int32 [1]
    uint32_t *counters;           // the workspace's first kArgmaxCounterBytes
};

constexpr int64_t kArgmaxCounterBytes = 256 * 17;

// Bytes of workspace the LM-head argmax needs for a weight of this geometry.
int64_t argmax_workspace_bytes(const Geometry &geo);

hipError_t launch_pack(const uint32_t *w0, const uint16_t *s0, const uint32_t *w1,
                       const uint16_t *s1, int64_t rows, int64_t k, PackMode mode, int64_t d,
                       const Geometry &geo, void *dst, hipStream_t stream);

hipError_t launch_unpack(const void *src, int64_t rows, int64_t k, PackMode mode, int64_t d,
                         const Geometry &geo, uint32_t *words, uint16_t *scales,
                         hipStream_t stream);

// Residual add + RMSNorm applied to x inside a GEMV launch (EPI_F16 and
// EPI_SILU only): h = f16(x + r) (r may be null), the matmul sees
// f16(h * gamma / sqrt(mean(h^2) + eps)); h_out (may be null) receives h.
struct NormArgs {
    const uint16_t *r;
    const uint16_t *gamma;
    uint16_t *h_out;
    float eps;
};

hipError_t launch_gemv_family(const Geometry &geo, Epilogue epi, const void *wdata,
                              const uint16_t *x, void *out, int64_t rows, int64_t k,
                              int64_t n_out, ArgmaxScratch am, const NormArgs *norm,
                              const RopeArgs *rope, hipStream_t stream);

// int3 weights (q4_kernels.hip): repacking both ways (plain rows, or gate/up
// interleaved with a second source) and the matmuls (single pass, k <= 8192;
// f16, f32 + argmax and SiLU epilogues).
hipError_t launch_pack3(const uint32_t *w3, const uint16_t *s, const uint32_t *w3_up,
                        const uint16_t *s_up, int64_t rows, int64_t k, const Geometry &geo,
                        void *dst, hipStream_t stream);
hipError_t launch_unpack3(const void *src, int64_t rows, int64_t k, const Geometry &geo,
                          uint32_t *w3, uint16_t *s, hipStream_t stream);
hipError_t launch_gemv3(const Geometry &geo, Epilogue epi, const void *wdata, const uint16_t *x,
                        void *out, int64_t rows, int64_t k, int64_t n_out, ArgmaxScratch am,
                        hipStream_t stream);

// Paged-attention decode (q4_attention.hip): workspace bytes (0 when the
// context fits one chunk) and the launch.
int64_t attention_workspace_bytes(int64_t ctx, int64_t nq, int64_t d);
hipError_t launch_attention(const uint16_t *q, const uint16_t *cache, const int32_t *page_table,
                            int32_t n_pages, int32_t ctx, int32_t nq, int32_t nkv, int32_t d,
                            float scale, uint16_t *out, void *ws, hipStream_t stream);
// the int8 cache: page bytes, the attention over it (same workspace), and the
// quantise-and-append of one fused QKV output
int64_t kv_int8_page_bytes(int64_t nkv, int64_t d);
hipError_t launch_attention_int8(const uint16_t *q, const uint8_t *cache8, const int32_t *page_table,
                                 int32_t n_pages, int32_t ctx, int32_t nq, int32_t nkv, int32_t d,
                                 float scale, uint16_t *out, void *ws, hipStream_t stream);
hipError_t launch_kv_append_int8(const uint16_t *qkv, int32_t nq, int32_t nkv, int32_t d, int32_t pos,
                                 uint8_t *cache8, const int32_t *page_table, int32_t n_pages,
                                 hipStream_t stream);

// Compute units of the current device (hipDeviceAttributeMultiprocessorCount,
// asked once per device), or 256 -- an MI355X -- when there is no device to
// ask (host-only sizing queries).  Launch plans size their grids from it.
int device_cus();

// The plain streaming read (q4_probe.hip): blocks it launches for `bytes`
// (the sink receives one 32-bit word per block) and the launch.
int64_t read_probe_blocks(int64_t bytes, int cus);
hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, int cus,
                             hipStream_t stream);

// ------------------------------------------------------------------ chain --
// A persistent launch over a sequence of int4 GEMV stages (q4_chain.hip).
// Stage s reads x (given, or the output of an earlier stage `src`, published
// with epoch tags), optionally behind the add + RMSNorm prologue, may wait
// for an earlier stage `after` to be complete, and writes y (f16, or
// SiLU(g) * u over a gate/up weight).
constexpr int kChainMaxStages = 6;
constexpr int kChainWaves = 8;          // wavefronts per block, one block per CU
constexpr int kChainMaxBlocks = 1024;

// (L, CG) geometries the chain kernel is built for: k from 1568 to 8192.
enum ChainGeo { CHAIN_G64_1 = 0, CHAIN_G32_3 = 1, CHAIN_G64_2 = 2, CHAIN_G64_3 = 3, CHAIN_G64_4 = 4 };
int chain_geo_of(const Geometry &geo);   // -1 when the chain kernel has no path for it

struct ChainStageK {
    const uint8_t *wd;        // packed weight (single pass)
    const uint16_t *r;        // norm of a dependent x: residual (may be null)
    const uint16_t *gamma;    // norm of a dependent x: gamma; null = none
    uint16_t *h_out;          // norm of a dependent x: h = f16(x + r) (may be null)
    uint16_t *y;              // f16 output [n_out]
    uint32_t *tag;            // tagged copy of y read by later stages (null: none)
    uint32_t *flags;          // per-block completion flags of this stage (null: none)
    int64_t tiles, rows, n_out, k;
    int32_t geo, epi, src, after;
    int32_t xoff;             // given x (src < 0): its offset in the staged-x area, in 8-half chunks
    float eps;
};

// An input vector given to the chain (x of one or more stages with no src),
// staged into LDS once at the start of the launch, with its own add +
// RMSNorm prologue if it has one.
struct ChainGiven {
    const uint16_t *x, *r, *gamma;
    uint16_t *h_out;
    float eps;
    int32_t k, off;           // length; offset in the staged-x area, in 8-half chunks
};
constexpr int kChainGivenHalves = 16384;   // staged-x area

struct ChainArgs {
    ChainStageK st[kChainMaxStages];
    ChainGiven given[kChainMaxStages];
    int32_t n, n_given;
    uint32_t *epochs;         // one word per block
    uint32_t *error;          // set to 1 by a wait that timed out
    int64_t wait_ticks;       // bound of one wait, in 100 MHz ticks
};

hipError_t launch_chain(const ChainArgs &a, int blocks, hipStream_t stream);

enum GemmPath { GEMM_PATH_AUTO = 0, GEMM_PATH_VALU = 1, GEMM_PATH_MFMA = 2 };

// Whether the MFMA GEMM kernel takes weights of this geometry (single pass,
// at least 8 lanes per row); others always run the VALU kernel.
bool gemm_mfma_eligible(const Geometry &geo);

hipError_t launch_gemm(const Geometry &geo, const void *wdata, const uint16_t *X,
                       int64_t m, int64_t n, int64_t k, uint16_t *Y, int path,
                       hipStream_t stream, bool int3 = false);

}  // namespace q4
