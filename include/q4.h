/*
 * q4.h -- C ABI of libq4: the int4-dequantizing matrix multiply of LLM decode
 * on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权"
 *        (zingnex.cn forum article).
 *        - section 完整的推理流水线: the int4 dequantizing matmul is the core of
 *          the decoder, in several variants (baseline, subgroup reduction, tiled
 *          rows x4 / x8) plus an f32-output version for the LM head; decoding is
 *          a greedy argmax dispatch.
 *        - section 内核融合: gate, up and the SiLU activation fused in one pass.
 *        - section 性能基准: matmul and int4 dequant are where the cost is.
 *        - section 技术限制与诚实声明: batched-prefill shaders exist (the
 *          batched form of the matmul, q4_gemm here).
 *        - sections 技术栈对比 / 性能基准: the weights are Phi-3-mini "q4f16_1".
 *   [P4] the Zero-TVM README: repacking of weights is tested byte for byte.
 *
 * The pages name the weight format but do not define it.  Canonical form, as
 * this library defines it (host or device arrays handed to q4_pack):
 *   words  uint32 [n][k/8]: code k = 8*j + i of a row is bits 4*i..4*i+3 of
 *                            the row's word j (low nibble first), codes 0..15;
 *   scales f16    [n][k/32]: one IEEE binary16 scale per 32 consecutive k;
 *   weight w[r][k] = (code - 8) * scale;   y[r] = sum_k x[k] * w[r][k].
 * f16 values cross the ABI as uint16_t bit patterns.
 *
 * Conventions for every call:
 *   - all buffer pointers are DEVICE pointers (hipMalloc or equivalent) unless
 *     stated; the caller owns all memory; the library never allocates, frees
 *     or synchronises;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); the
 *     work is enqueued there and the call returns at once; device faults
 *     surface at the caller's next synchronisation;
 *   - every argument is validated on the host BEFORE anything is enqueued;
 *     on error nothing is launched and nothing is written;
 *   - buffers must stay alive until the stream has passed the call.
 *
 * Device layout, version 1 (what q4_pack writes; opaque to callers but
 * specified here so that it can be checked byte for byte):
 *   G = k/32 groups per row.  P = ceil(G/256) passes, Gp = ceil(G/P).
 *   (L, CG) = lanes per row L in {64,32,16,8,4,2,1} and groups per lane CG in
 *   {1,2,3,4} with L*CG >= Gp; least L*CG wins, ties go to the larger L.
 *   A tile holds TR = 2*64/L rows; tiles = ceil(rows/TR); each tile is P
 *   passes of PB = CG*2304 bytes.  Logical (row r, group g) lives at
 *     t = r / TR, s = (r % TR) / 2, u = r % 2, p = g / (L*CG),
 *     c = (g % (L*CG)) / CG, j = g % CG, lane = s*L + c, base = t*P*PB + p*PB:
 *     its 4 canonical words at base + (u*CG + j)*1024 + lane*16,
 *     its scale             at base + 2*CG*1024 + lane*4*CG + (u*CG + j)*2.
 *   Padding rows (r >= rows) and groups (g >= G): words 0x88888888, scale 0.
 *   So each 64-lane wavefront reads every 128-bit unit of a pass with one
 *   fully contiguous 1 KiB load per (u, j), and each lane's 2*CG scales with
 *   one load.  Gate/up layout: logical row 2i is gate row i, row 2i+1 is up
 *   row i, so both land in the same lane after the cross-lane reduction.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define Q4_OK             0
#define Q4_ERR_NULL      -1  /* a required pointer is NULL */
#define Q4_ERR_SHAPE     -2  /* n < 1, k < 32, k % 32 != 0, m < 1, or a size overflows */
#define Q4_ERR_ALIGN     -3  /* a pointer is not aligned as documented */
#define Q4_ERR_LAYOUT    -4  /* weight layout/version does not suit the call */
#define Q4_ERR_WORKSPACE -5  /* workspace NULL or smaller than q4_workspace_bytes */
#define Q4_ERR_ALIAS     -6  /* an output range overlaps an input range */
#define Q4_ERR_HIP       -7  /* the HIP runtime refused the launch (q4_last_hip_error) */
#define Q4_ERR_SIZE      -8  /* a destination buffer is smaller than required */

/* weight layouts */
#define Q4_LAYOUT_ROWS    1  /* plain rows: q4_gemv, q4_gemm, q4_lmhead_f32 */
#define Q4_LAYOUT_GATE_UP 2  /* interleaved gate/up rows: q4_ffn_gate_up_silu */
#define Q4_LAYOUT_ROPE    3  /* rotary-paired head rows: q4_qkv_rope_append */
#define Q4_LAYOUT_INT3    4  /* int3 rows (q4_pack_int3): q4_gemv, q4_gemm, q4_lmhead_f32 */
#define Q4_LAYOUT_INT3_GATE_UP 5  /* int3 gate/up rows (q4_pack_int3_gate_up): q4_ffn_gate_up_silu */
#define Q4_LAYOUT_VERSION 1

/* operations, for q4_workspace_bytes */
#define Q4_OP_GEMV    1
#define Q4_OP_GEMM    2
#define Q4_OP_FFN     3
#define Q4_OP_LMHEAD  4
#define Q4_OP_ATTENTION 5  /* q4_workspace_bytes(Q4_OP_ATTENTION, ctx, n_q_heads, head_dim) */

/*
 * Host-side descriptor of a packed weight, filled by q4_pack*; only `data`
 * points to device memory.  The descriptor is read on the host by every op
 * and never on the device.
 */
typedef struct q4_weight {
    int32_t n;        /* output rows (gate/up: rows of EACH half) */
    int32_t k;        /* input columns, k % 32 == 0 */
    int32_t layout;   /* Q4_LAYOUT_ROWS, Q4_LAYOUT_GATE_UP or Q4_LAYOUT_ROPE */
    int32_t version;  /* Q4_LAYOUT_VERSION */
    void   *data;     /* device, 256-byte aligned, `bytes` long */
    int64_t bytes;    /* q4_packed_bytes(n, k, layout) */
    int32_t head_dim; /* Q4_LAYOUT_ROPE: rows per head (even, divides n); else 0 */
    int32_t reserved; /* 0 */
} q4_weight;

/* Bytes of the packed layout; 0 for an invalid shape or layout. */
int64_t q4_packed_bytes(int32_t n, int32_t k, int32_t layout);

/* Bytes of device workspace an op needs (0 = none).  The LM-head argmax needs
 * one (per-block candidates), and so does q4_attention_decode over a context
 * split into chunks (per-chunk records); contents need no initialisation.
 * Two calls that share a workspace must be ordered on one stream. */
int64_t q4_workspace_bytes(int32_t op, int32_t m, int32_t n, int32_t k);

/*
 * Repack canonical weights into the device layout ([P4]: repacking is a pure
 * permutation, checked byte for byte).
 *   words  : device, uint32 [n][k/8], 16-byte aligned
 *   scales : device, f16 bits [n][k/32], 2-byte aligned
 *   dst    : device, >= q4_packed_bytes(n, k, Q4_LAYOUT_ROWS) bytes, 256-byte aligned
 *   out    : host descriptor written on success
 * Errors: NULL, SHAPE, ALIGN, SIZE (dst_bytes too small), ALIAS, HIP.
 */
int q4_pack(const uint32_t *words, const uint16_t *scales, int32_t n, int32_t k,
            void *dst, int64_t dst_bytes, q4_weight *out, void *stream);

/*
 * Repack the gate and up halves of an FFN ([P1] 内核融合) into one
 * interleaved layout for q4_ffn_gate_up_silu.  Each of gw/gs and uw/us is a
 * canonical [n][k/8] / [n][k/32] pair as in q4_pack; dst needs
 * q4_packed_bytes(n, k, Q4_LAYOUT_GATE_UP) bytes.
 */
int q4_pack_gate_up(const uint32_t *gw, const uint16_t *gs, const uint32_t *uw,
                    const uint16_t *us, int32_t n, int32_t k, void *dst,
                    int64_t dst_bytes, q4_weight *out, void *stream);

/*
 * Rotary-paired layout for the fused QKV step ([P1] 内核融合: qkv_fused
 * applies RoPE inside the projection): the n rows are heads of head_dim
 * rows; the device layout is the plain one over a row permutation that puts
 * dims i and i + head_dim/2 of a head on logical rows 2p and 2p + 1 (p =
 * head * head_dim/2 + i), so both halves of a rotation pair meet in one lane.
 * Arguments as q4_pack, plus head_dim (even, >= 2, dividing n); the
 * descriptor records it.  Errors as q4_pack.
 */
int q4_pack_rope(const uint32_t *words, const uint16_t *scales, int32_t n, int32_t k,
                 int32_t head_dim, void *dst, int64_t dst_bytes, q4_weight *out, void *stream);

/*
 * int3 weights: the int3 variant of the same matmul (the Zero-TVM README,
 * where it says where the shaders live, names one generator for an int4/int3
 * matmul family; no page defines the int3 format).  Definition: codes q in
 * 0..7, weight (q - 4) * scale, one f16 scale per 32 consecutive k; a row's
 * codes form one bit stream, LSB first over its little-endian uint32 words,
 * code k in stream bits 3k .. 3k+2 (so a group of 32 codes fills 3 words).
 *   words3 : device, uint32 [n][3k/32], 4-byte aligned
 *   scales : device, f16 bits [n][k/32], 2-byte aligned
 *   k      : a multiple of 32 (k > 8192 takes several passes, as for int4)
 *   dst    : device, >= q4_packed_bytes(n, k, Q4_LAYOUT_INT3) bytes, 256-byte
 *            aligned.  The device layout uses the tiles and passes of the int4
 *            one with 12-byte lane units (word i of a group's unit: codes 10i + m at
 *            bits 3m and 10i + 5 + m at bits 16 + 3m, m = 0..4; bit i of
 *            codes 30 and 31 at bits 15 and 31); padding is code 4, scale 0.
 * The result feeds q4_gemv, q4_gemm and q4_lmhead_f32 (and q4_unpack).  Errors as q4_pack.
 */
int q4_pack_int3(const uint32_t *words3, const uint16_t *scales, int32_t n, int32_t k,
                 void *dst, int64_t dst_bytes, q4_weight *out, void *stream);

/*
 * The gate and up halves of an FFN as int3 weights (each canonical as in
 * q4_pack_int3) in one interleaved layout (logical row 2i = gate row i, 2i+1
 * = up row i) for q4_ffn_gate_up_silu; dst needs q4_packed_bytes(n, k,
 * Q4_LAYOUT_INT3_GATE_UP) bytes.  Errors as q4_pack.
 */
int q4_pack_int3_gate_up(const uint32_t *gw3, const uint16_t *gs, const uint32_t *uw3,
                         const uint16_t *us, int32_t n, int32_t k, void *dst, int64_t dst_bytes,
                         q4_weight *out, void *stream);

/*
 * Inverse of q4_pack / q4_pack_gate_up / q4_pack_rope / q4_pack_int3 (for
 * round-trip checks): writes the canonical words [rows][k/8] (int3: words3
 * [rows][3k/32], 4-byte aligned) and scales [rows][k/32] of the packed
 * weight, rows = n (plain, rotary-paired and int3: original row order) or 2n
 * (gate/up, interleaved order: gate 0, up 0, gate 1 ...).
 */
int q4_unpack(const q4_weight *w, uint32_t *words, uint16_t *scales, void *stream);

/*
 * y = x . dequant(W)^T, batch 1 ([P1] 完整的推理流水线: the int4 dequantizing
 * matmul; the rows-per-invocation and subgroup-reduction variants there are
 * the two-rows-per-lane tiles and the cross-lane reduction here).
 *   w : Q4_LAYOUT_ROWS, or Q4_LAYOUT_INT3 (the int3 variant)
 *   x : device f16 [k], 16-byte aligned
 *   y : device f16 [n], 4-byte aligned; f32 accumulation, rounded to nearest
 *       even once at the end
 * Errors: NULL, SHAPE, ALIGN, LAYOUT, ALIAS, HIP.
 */
int q4_gemv(const q4_weight *w, const uint16_t *x, uint16_t *y, void *stream);

/*
 * Y = X . dequant(W)^T for m activation rows ([P1] 技术限制与诚实声明: the
 * batched-prefill form).  m = 1 with Y 4-byte aligned runs the q4_gemv
 * kernels (otherwise m = 1 runs a VALU kernel that reads W once per 8
 * activation rows with exact dequant); m >= 2 dequantizes W to f16
 * (q - 8) * s in registers (one rounding, relative error <= 2^-11) and
 * contracts on the matrix cores (v_mfma_f32_32x32x16_f16; for m > 128 with
 * k > 4096, v_mfma_f32_16x16x32_f16), f32 accumulation; the f32 sum of a row is
 * formed in a fixed order for a given shape (the same bits on every call).
 *   w : Q4_LAYOUT_ROWS, or Q4_LAYOUT_INT3 ((q - 4) * s on the same paths)
 *   X : device f16 [m][k] row-major, 16-byte aligned
 *   Y : device f16 [m][n] row-major, 2-byte aligned
 *   ws: unused (pass NULL, 0)
 */
int q4_gemm(const q4_weight *w, const uint16_t *X, int32_t m, uint16_t *Y,
            void *ws, int64_t ws_bytes, void *stream);

/* GEMM kernel choice for q4_gemm_path. */
#define Q4_GEMM_AUTO 0   /* what q4_gemm does: MFMA for m >= 2, m = 1: q4_gemv (VALU if Y is only 2-byte aligned) */
#define Q4_GEMM_VALU 1   /* VALU kernel for any m */
#define Q4_GEMM_MFMA 2   /* MFMA kernel for any m (falls back to VALU for
                            layouts it does not take: k > 8192 or k < 256) */

/*
 * q4_gemm with the kernel chosen by the caller (for measuring where the MFMA
 * kernel overtakes the VALU one); same arguments and results as q4_gemm up
 * to the rounding differences of the two kernels.  Errors as q4_gemm, and
 * Q4_ERR_SHAPE for an unknown path.
 */
int q4_gemm_path(const q4_weight *w, const uint16_t *X, int32_t m, uint16_t *Y, int32_t path,
                 void *stream);

/*
 * h = SiLU(x . Wg^T) * (x . Wu^T) in one kernel ([P1] 内核融合, fused_ffn),
 * SiLU(g) = g / (1 + e^-g) in f32, h rounded to f16.
 *   w : Q4_LAYOUT_GATE_UP (or Q4_LAYOUT_INT3_GATE_UP) with n rows per half;
 *       x : f16 [k]; h : f16 [n]
 */
int q4_ffn_gate_up_silu(const q4_weight *w, const uint16_t *x, uint16_t *h,
                        void *stream);

/*
 * LM head with f32 logits and greedy argmax ([P1] 完整的推理流水线: the f32
 * output variant for sampling stability, and the argmax dispatch).
 *   w      : Q4_LAYOUT_ROWS, or Q4_LAYOUT_INT3
 *   logits : device f32 [n], 8-byte aligned
 *   argmax : device int32 [1] or NULL; the lowest index holding the maximum
 *            logit (as computed in f32)
 *   ws     : >= q4_workspace_bytes(Q4_OP_LMHEAD, 1, n, k) bytes, 256-byte
 *            aligned, when argmax is not NULL: each block's candidate and a
 *            few counters by which the block that finishes last finds out it
 *            is last and combines the candidates, in the same launch.  The
 *            counters must be ZERO before the first call on a workspace (a
 *            zero-filled buffer); each call leaves them zero again, so the
 *            workspace is then left to LM-head calls (not shared with another
 *            op's workspace) and calls on it are made in stream order.
 */
int q4_lmhead_f32(const q4_weight *w, const uint16_t *x, float *logits,
                  int32_t *argmax, void *ws, int64_t ws_bytes, void *stream);

/*
 * q4_lmhead_f32 for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, kernels and results, with the argmax candidates and counters
 * kept in a static device array of the library (64 KiB per GPU, zero when
 * the library loads, held until the process ends) instead of a caller
 * workspace.  No hipMalloc, hipFree or
 * other allocation happens in the call; the first call on a device looks
 * up the array's address there (hipGetSymbolAddress).  Every call on one
 * GPU shares that GPU's array, so calls that overlap on one GPU (two
 * streams, or two host threads) race and must be ordered by the caller.
 *   w, x, logits, argmax : as q4_lmhead_f32
 * Errors: as q4_lmhead_f32; WORKSPACE when the candidates would not fit the
 * 64 KiB array (more than 8192 blocks: never on one MI355X).
 */
int q4_lmhead_f32_noalloc(const q4_weight *w, const uint16_t *x, float *logits,
                          int32_t *argmax, void *stream);

/*
 * Residual add + RMSNorm in front of the matmul, fused into its activation
 * staging ([P1] 内核融合: add_norm merges the residual connection and
 * RMSNorm; here that step also runs inside the QKV or gate/up matmul that
 * consumes it, saving its launch and its round trip through memory):
 *   h_i  = f16(x_i + residual_i)          (residual NULL: h_i = x_i)
 *   xn_i = f16(h_i * gamma_i / sqrt(mean_k(h^2) + eps))   (f32 arithmetic)
 *   y    = xn . dequant(W)^T, exactly as q4_gemv computes it from xn
 *   x, residual, gamma : device f16 [k], 16-byte aligned; residual may be NULL
 *   eps                : finite, >= 0 (the pages do not give it)
 *   residual_out       : device f16 [k], 16-byte aligned, or NULL; receives h
 *                        (the updated residual stream)
 *   y                  : device f16 [n], 4-byte aligned
 * No output may overlap an input or the other output (in particular
 * residual_out != residual: every block reads the residual).
 * Errors: NULL, SHAPE (also eps < 0 or not finite), ALIGN, LAYOUT, ALIAS, HIP.
 */
int q4_add_rmsnorm_gemv(const q4_weight *w, const uint16_t *x, const uint16_t *residual,
                        const uint16_t *gamma, float eps, uint16_t *residual_out, uint16_t *y,
                        void *stream);

/*
 * The same prologue in front of the fused gate/up + SiLU
 * (q4_ffn_gate_up_silu): h_ffn = SiLU(xn . Wg^T) * (xn . Wu^T), f16 [n],
 * 2-byte aligned; other arguments as q4_add_rmsnorm_gemv.
 */
int q4_add_rmsnorm_ffn_gate_up_silu(const q4_weight *w, const uint16_t *x,
                                    const uint16_t *residual, const uint16_t *gamma, float eps,
                                    uint16_t *residual_out, uint16_t *h, void *stream);

/*
 * The fused QKV step ([P1] 内核融合: qkv_fused merges the Q/K/V projection,
 * RoPE and the paged KV-cache append into one dispatch; 完整的推理流水线:
 * vLLM-style page table, RoPE computed in place):
 *   y = x . dequant(W)^T over rows [nq q heads | nkv k heads | nkv v heads]
 *   (each head d = w->head_dim rows, nkv = (n/d - nq) / 2); dims i and
 *   i + d/2 of every q and k head are rotated by pos * rope_base^(-2i/d)
 *   (y_i' = y_i cos - y_j sin, y_j' = y_j cos + y_i sin, angle in f64,
 *   rotation in f32); v is left as is.
 *   w          : Q4_LAYOUT_ROPE (q4_pack_rope)
 *   x          : device f16 [k], 16-byte aligned
 *   qkv        : device f16 [n], 4-byte aligned: y after RoPE
 *   kv_cache   : device f16 [n_pages][2][nkv][16][d] or NULL (no append):
 *                page, then K (0) / V (1), then head, then the 16 token
 *                slots of the page, then dim (one head's 16 rows of a page
 *                are contiguous); the k and v heads of y (k after
 *                RoPE) are written to slot pos % 16 of page
 *                page_table[pos / 16]; nothing else is written
 *   page_table : device int32, at least pos / 16 + 1 entries (needed with a
 *                cache); an entry outside [0, n_pages) appends nothing
 *   pos        : >= 0;  rope_base : finite, > 0;  head_dim <= 512
 * Errors: NULL, SHAPE (nq, pos, rope_base, n_pages out of range), ALIGN,
 * LAYOUT, ALIAS, HIP.
 */
int q4_qkv_rope_append(const q4_weight *w, const uint16_t *x, int32_t n_q_heads, int32_t pos,
                       double rope_base, uint16_t *qkv, uint16_t *kv_cache,
                       const int32_t *page_table, int32_t n_pages, void *stream);

/*
 * q4_qkv_rope_append behind the residual add + RMSNorm prologue of
 * q4_add_rmsnorm_gemv (the whole add_norm + qkv_fused pair of [P1] 内核融合
 * in one launch); arguments as the two calls.
 */
int q4_add_rmsnorm_qkv_rope_append(const q4_weight *w, const uint16_t *x,
                                   const uint16_t *residual, const uint16_t *gamma, float eps,
                                   uint16_t *residual_out, int32_t n_q_heads, int32_t pos,
                                   double rope_base, uint16_t *qkv, uint16_t *kv_cache,
                                   const int32_t *page_table, int32_t n_pages, void *stream);

/*
 * Paged-attention decode for one token ([P1] 内核融合: attention merges paged
 * attention with the page-table reads), over the cache q4_qkv_rope_append
 * fills:  for query head h (kv head g = h / (nq / nkv)) and positions
 * t = 0 .. ctx-1 (slot t % 16 of page page_table[t / 16]):
 *   s_t = scale * q_h . K_t,   p = softmax(s),   out_h = sum_t p_t V_t
 * (f32 arithmetic, f16 out).
 *   q          : device f16 [nq][d], 16-byte aligned (the roped q heads)
 *   kv_cache   : device f16 [n_pages][2][nkv][16][d], 16-byte aligned
 *   page_table : device int32, (ctx + 15) / 16 entries in [0, n_pages); an
 *                entry outside that range makes its 16 positions count as
 *                absent (a head with every position absent gives NaN)
 *   d          : 32 .. 256, a multiple of 32;  nq % nkv == 0;  ctx >= 1;
 *                one page (2 * nkv * 16 * d halves) under 2 GiB
 *   out        : device f16 [nq][d], 4-byte aligned
 *   ws         : q4_workspace_bytes(Q4_OP_ATTENTION, ctx, nq, d) bytes, 16-byte
 *                aligned (NULL when that is 0: a context short enough for
 *                one block per head needs none; a longer one is split into
 *                chunks whose f32 records a second launch merges; contents
 *                need no initialisation)
 * Errors: NULL, SHAPE, ALIGN, WORKSPACE, ALIAS, HIP.
 */
int q4_attention_decode(const uint16_t *q, const uint16_t *kv_cache, const int32_t *page_table,
                        int32_t n_pages, int32_t ctx, int32_t nq, int32_t nkv, int32_t d,
                        float scale, uint16_t *out, void *ws, int64_t ws_bytes, void *stream);

/*
 * The int8 KV cache ([P1] 完整的推理流水线: the paged KV cache has an optional
 * int8 quantisation path that halves its memory; the pages give no scheme).
 * Each (token, kv head) row of d values is stored as d int8 codes and one f32
 * scale: scale = max_i |x_i| / 127 and code_i = rint(x_i / scale) (f32,
 * correctly rounded division, ties to even; all codes 0 when the row is 0),
 * so x_i ~ code_i * scale.  Page layout: [page][K=0|V=1][kv head] blocks of
 * 16 rows of d codes (slot order) followed by the 16 rows' f32 scales, i.e.
 * q4_kv_int8_page_bytes(nkv, d) = 2 * nkv * (16 d + 64) bytes per page
 * (Phi-3-mini: 102,400 B against 196,608 B in f16).
 * Returns 0 for an invalid shape (d not in 32 .. 256 step 32, nkv < 1, or a
 * page of 2 GiB or more).
 */
int64_t q4_kv_int8_page_bytes(int32_t n_kv_heads, int32_t head_dim);

/*
 * Quantise the k and v heads of one fused QKV output into the int8 cache at
 * position pos (slot pos % 16 of page page_table[pos / 16]); run it after
 * q4_qkv_rope_append (whose own f16 append may be skipped with a NULL cache).
 *   qkv        : device f16 [(n_q_heads + 2 n_kv_heads) * head_dim], 2-byte
 *                aligned: q heads, k heads (roped), v heads
 *   cache8     : device, n_pages * q4_kv_int8_page_bytes(..) bytes, 16-byte aligned
 *   page_table : device int32, at least pos / 16 + 1 entries; an entry outside
 *                [0, n_pages) appends nothing
 * Errors: NULL, SHAPE, ALIGN, ALIAS, HIP.
 */
int q4_kv_append_int8(const uint16_t *qkv, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                      int32_t pos, void *cache8, const int32_t *page_table, int32_t n_pages,
                      void *stream);

/*
 * q4_attention_decode over the int8 cache: K_t = code * scale, V_t = code *
 * scale of each row, otherwise the same definition, arguments (cache8 as
 * above, 16-byte aligned) and workspace (q4_workspace_bytes(Q4_OP_ATTENTION,
 * ctx, nq, d)).  Errors as q4_attention_decode.
 */
int q4_attention_decode_int8(const uint16_t *q, const void *cache8, const int32_t *page_table,
                             int32_t n_pages, int32_t ctx, int32_t nq, int32_t nkv, int32_t d,
                             float scale, uint16_t *out, void *ws, int64_t ws_bytes, void *stream);

/*
 * A chain of int4 GEMVs in one launch ([P1] 内核融合: kernels are fused to cut
 * the dispatches of a decode step; 性能基准: the int4 matmuls dominate it).
 * Stage i computes, in order,
 *   xi = x (given) or the y of stage src (src < i);
 *   with gamma: h = f16(xi + residual) (residual may be NULL: h = xi),
 *               xi = f16(h * gamma / sqrt(mean(h^2) + eps)), h -> residual_out;
 *   y  = xi . dequant(W)^T (Q4_LAYOUT_ROWS, f16 [n], as q4_gemv), or
 *        SiLU(xi . Wg^T) * (xi . Wu^T) (Q4_LAYOUT_GATE_UP, f16 [n], as
 *        q4_ffn_gate_up_silu),
 * and does not start computing before stage `after` (< i) has finished.  A
 * stage waits only for what it names (src, after); stages with neither run
 * back to back with no grid-wide wait, and every stage's weights start
 * streaming while the stage before it finishes.
 *   w          : Q4_LAYOUT_ROWS or Q4_LAYOUT_GATE_UP, k from 1568 to 8192
 *                (the chain kernel's geometries; Q4_ERR_SHAPE otherwise)
 *   x          : device f16 [k], 16-byte aligned; NULL exactly when src >= 0
 *                (then stage src's n must equal this k)
 *   gamma, residual, residual_out : as q4_add_rmsnorm_gemv (16-byte aligned)
 *   y          : device f16 [n], 4-byte aligned (2-byte for GATE_UP)
 *   ws         : q4_chain_workspace_bytes(stages, n_stages) bytes, 256-byte
 *                aligned, ZERO-FILLED before its first use and then left to
 *                the library: it carries a launch counter per block from one
 *                call to the next, so every call on one workspace must be
 *                made on one stream of one device (calls on other streams
 *                race).  Word 0 (uint32) is set non-zero by the device if a
 *                wait ran out of time (2 ms; only when the GPU cannot hold
 *                all blocks of the launch at once, e.g. beside other work);
 *                the results of such a call are undefined, and the word stays
 *                set until the caller clears it.
 * The launch holds one block of 8 wavefronts per compute unit for its whole
 * duration.  Errors: NULL, SHAPE, ALIGN, LAYOUT, SIZE, WORKSPACE, ALIAS, HIP.
 */
typedef struct q4_chain_stage {
    const q4_weight *w;
    const uint16_t *x;
    int32_t src;
    int32_t after;
    const uint16_t *residual;
    const uint16_t *gamma;
    float eps;
    int32_t reserved;         /* 0 */
    uint16_t *residual_out;
    uint16_t *y;
} q4_chain_stage;

/* Workspace bytes q4_chain needs for these stages (0 if they are invalid). */
int64_t q4_chain_workspace_bytes(const q4_chain_stage *stages, int32_t n_stages);

int q4_chain(const q4_chain_stage *stages, int32_t n_stages, void *ws, int64_t ws_bytes,
             void *stream);

/*
 * Measurement aid: a plain streaming read of `bytes` bytes (a multiple of 16)
 * at `src` (device, 16-byte aligned), the ceiling against which the matmuls' HBM rates are
 * read (the Zero-TVM article, section 性能基准, keeps its protocol and raw
 * data beside each figure).  Every 64-lane wavefront reads 1 KiB per load
 * instruction, two 8 KiB chunks in flight, two blocks of four wavefronts per
 * compute unit; nothing is computed but an xor of the words read.
 *   sink       : device, 4-byte aligned, >= 8 * (compute units) bytes (8 KiB
 *                covers any MI355X partition); receives one word per block
 *   sink_bytes : its size
 * Errors: NULL, SHAPE (bytes not a positive multiple of 16), ALIGN, SIZE,
 * ALIAS, HIP.
 */
int q4_read_probe(const void *src, int64_t bytes, uint32_t *sink, int64_t sink_bytes,
                  void *stream);

/* Static text for a return code. */
const char *q4_strerror(int code);

/* hipError_t behind the last Q4_ERR_HIP returned on this thread (0 if none). */
int q4_last_hip_error(void);

/* Digest of the sources this library was built from (16 hex digits of the
 * SHA-256 over the kernel/ABI sources and this header, as computed by the
 * build script), or "unstamped".  Static text; never NULL. */
const char *q4_source_hash(void);

/* Layout geometry for a weight of `rows` logical rows: out[0..5] = L, CG, P,
 * TR, tiles, tile bytes.  Returns Q4_OK or Q4_ERR_SHAPE/Q4_ERR_NULL. */
int q4_layout_geometry(int32_t rows, int32_t k, int64_t *out);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
