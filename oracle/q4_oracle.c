/*
 * q4_oracle.c -- plain, slow, obviously correct CPU reference for the int4
 * dequantizing matrix multiply.  TEST INFRASTRUCTURE ONLY: it is loaded by the
 * tests, by the smoke check and by the CPU-baseline leg of the benchmark, and
 * never by the library.  It shares no source with the HIP path.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权"
 *        (zingnex.cn forum article).  Section 完整的推理流水线 names the int4
 *        dequantizing matmul as the core of decode, with an f32-output variant
 *        for the LM head and a greedy argmax dispatch; section 内核融合 fuses
 *        gate, up and SiLU into one pass; section 性能基准 says matmul and int4
 *        dequant are where the time goes; 技术栈对比 / 性能基准 name the weights
 *        "Phi-3-mini q4f16_1".
 *   [P4] the Zero-TVM README (abgnydn/zero-tvm): repacking is tested
 *        byte-for-byte; every kernel is tested against a plain reference.
 *
 * The pages name the weight format (q4f16_1: 4-bit codes with f16 scales) but
 * never define it bit by bit.  This library's definition, which the oracle
 * follows literally:
 *   - codes q in 0..15, packed 8 per uint32 along K; code k = 8*j + i of a row
 *     sits in bits 4*i .. 4*i+3 of that row's word j (low nibble first);
 *   - one f16 scale per group of 32 consecutive k of a row; scales [N][K/32];
 *   - weight value w = (q - 8) * scale;
 *   - y[n] = sum_k x[k] * w[n][k].
 * Everything is computed in IEEE double (f64), k ascending, one term at a time.
 * Each product x*(q-8)*s needs at most 11+4+11 = 26 significant bits, so the
 * products are exact in f64; only the running sum rounds.
 *
 * Also here: an f16 decoder and an f64->f16 round-to-nearest-even encoder of
 * its own, and an encoder of the library's device layout (layout version 1),
 * written from that layout's specification by walking the logical matrix and
 * computing each destination address.
 */
#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ f16 -- */

/* IEEE 754 binary16 bits -> double.  Normal: (1024+m) * 2^(e-25);
 * subnormal: m * 2^-24; e == 31: infinity or NaN. */
double q4o_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* round a non-negative double (< 2^52) to the nearest integer, ties to even */
static double round_half_even(double q)
{
    double f = floor(q);
    double d = q - f;            /* exact for q < 2^52 */
    if (d > 0.5)
        return f + 1.0;
    if (d < 0.5)
        return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* double -> binary16 bits, round to nearest, ties to even; overflow -> inf */
uint16_t q4o_double_to_half(double v)
{
    if (isnan(v))
        return 0x7e00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: count units of 2^-24; 1024 units is the smallest
         * normal, whose encoding 0x0400 is the same integer */
        double r = round_half_even(ldexp(a, 24));
        return sign | (uint16_t)r;
    }
    int e2;
    frexp(a, &e2);               /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;              /* 2^E <= a < 2^(E+1) */
    double r = round_half_even(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(r - 1024.0);
}

/* ------------------------------------------------------- the definition -- */

/* code of row r at position kk (K = k columns): word kk/8, nibble kk%8 */
static int code_at(const uint32_t *words, int64_t r, int64_t kk, int64_t k)
{
    uint32_t word = words[r * (k / 8) + kk / 8];
    return (int)((word >> (4 * (kk % 8))) & 15u);
}

/* dequantized weight w[r][kk] = (q - 8) * scale, exact in f64 */
static double weight_at(const uint32_t *words, const uint16_t *scales,
                        int64_t r, int64_t kk, int64_t k)
{
    int q = code_at(words, r, kk, k);
    double s = q4o_half_to_double(scales[r * (k / 32) + kk / 32]);
    return (double)(q - 8) * s;
}

/*
 * y = x . dequant(W)^T for one activation vector ([P1] 完整的推理流水线).
 * words [n][k/8], scales [n][k/32], x [k] f16 bits.
 * y[r] = sum_k x_k * w[r][k]; a[r] = sum_k |x_k * w[r][k]| (the magnitude sum
 * that sizes the tolerance).  a may be NULL.  Returns 0, or -1 on a bad shape.
 */
int q4o_gemv(const uint32_t *words, const uint16_t *scales, const uint16_t *x,
             int64_t n, int64_t k, double *y, double *a)
{
    if (n < 0 || k < 32 || k % 32 != 0)
        return -1;
    for (int64_t r = 0; r < n; ++r) {
        double sum = 0.0, asum = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            double term = q4o_half_to_double(x[kk]) *
                          weight_at(words, scales, r, kk, k);
            sum += term;
            asum += fabs(term);
        }
        y[r] = sum;
        if (a)
            a[r] = asum;
    }
    return 0;
}

/*
 * Y = X . dequant(W)^T for m activation rows (the batched form of the same
 * matmul).  X [m][k] f16 bits row-major; Y, A [m][n] row-major.
 */
int q4o_gemm(const uint32_t *words, const uint16_t *scales, const uint16_t *X,
             int64_t m, int64_t n, int64_t k, double *Y, double *A)
{
    if (m < 0 || n < 0 || k < 32 || k % 32 != 0)
        return -1;
    for (int64_t i = 0; i < m; ++i) {
        int rc = q4o_gemv(words, scales, X + i * k, n, k, Y + i * n,
                          A ? A + i * n : NULL);
        if (rc)
            return rc;
    }
    return 0;
}

/* SiLU(g) = g * sigmoid(g) = g / (1 + e^-g) */
double q4o_silu(double g)
{
    return g / (1.0 + exp(-g));
}

/* the gated product of one intermediate row: SiLU of the gate times the up */
static double gated(double g, double u)
{
    return q4o_silu(g) * u;
}

/*
 * Fused gate/up + SiLU ([P1] 内核融合, fused_ffn): h = SiLU(x.Wg^T) * (x.Wu^T),
 * elementwise over the n intermediate rows.  Also returns the gate and up
 * pre-activations and their magnitude sums (any of g, u, ag, au may be NULL).
 */
int q4o_ffn_gate_up_silu(const uint32_t *gw, const uint16_t *gs,
                         const uint32_t *uw, const uint16_t *us,
                         const uint16_t *x, int64_t n, int64_t k, double *h,
                         double *g, double *u, double *ag, double *au)
{
    if (n < 0 || k < 32 || k % 32 != 0)
        return -1;
    for (int64_t r = 0; r < n; ++r) {
        double gv, uv, agv, auv;
        q4o_gemv(gw + r * (k / 8), gs + r * (k / 32), x, 1, k, &gv, &agv);
        q4o_gemv(uw + r * (k / 8), us + r * (k / 32), x, 1, k, &uv, &auv);
        h[r] = gated(gv, uv);
        if (g)
            g[r] = gv;
        if (u)
            u[r] = uv;
        if (ag)
            ag[r] = agv;
        if (au)
            au[r] = auv;
    }
    return 0;
}

/*
 * Residual add + RMSNorm ([P1] 内核融合: add_norm merges the residual
 * connection and RMSNorm), the step in front of the QKV and gate/up matmuls.
 * The pages give neither epsilon nor where results are rounded; the reading
 * here: epsilon is a parameter, and the two vectors a separate kernel would
 * store are f16:
 *   h_i  = f16(x_i + r_i)                 (r NULL: h_i = x_i) -- new residual
 *   ms   = (1/k) * sum_i h_i^2            (f64, over the f16 values h_i)
 *   xn_i = f16(h_i * gamma_i / sqrt(ms + eps))
 * x, r, gamma, h, xn are f16 bits [k]; h may be NULL.  Returns 0, or -1 for
 * k < 1 or eps < 0.
 */
int q4o_add_rmsnorm(const uint16_t *x, const uint16_t *r, const uint16_t *gamma,
                    int64_t k, double eps, uint16_t *h, uint16_t *xn)
{
    if (k < 1 || eps < 0)
        return -1;
    double ss = 0.0;
    for (int64_t i = 0; i < k; ++i) {
        double v = q4o_half_to_double(x[i]);
        if (r)
            v += q4o_half_to_double(r[i]);   /* exact: two f16 */
        const double hv = q4o_half_to_double(q4o_double_to_half(v));
        ss += hv * hv;
    }
    const double rms = sqrt(ss / (double)k + eps);
    for (int64_t i = 0; i < k; ++i) {
        double v = q4o_half_to_double(x[i]);
        if (r)
            v += q4o_half_to_double(r[i]);
        const uint16_t hb = q4o_double_to_half(v);
        if (h)
            h[i] = hb;
        xn[i] = q4o_double_to_half(q4o_half_to_double(hb) * q4o_half_to_double(gamma[i]) / rms);
    }
    return 0;
}

/*
 * Rotary position embedding of one pair of head dims ([P1] 完整的推理流水线:
 * RoPE is computed in place inside the fused QKV kernel).  The pages give
 * neither the pairing nor the base; the reading is Phi-3's: dim i of a head
 * d wide is paired with dim i + d/2 ("rotate half"), angle
 * pos * base^(-2i/d), and
 *   out_i = y_i cos - y_j sin,   out_j = y_j cos + y_i sin   (j = i + d/2).
 */
void q4o_rope_pair(double yi, double yj, int64_t i, int64_t d, int64_t pos,
                   double base, double *oi, double *oj)
{
    const double ang = (double)pos * pow(base, -2.0 * (double)i / (double)d);
    const double c = cos(ang), s = sin(ang);
    *oi = yi * c - yj * s;
    *oj = yj * c + yi * s;
}

/*
 * The fused QKV step ([P1] 内核融合: qkv_fused merges the Q/K/V projection,
 * RoPE and the paged KV-cache append): y = x . dequant(W)^T over rows
 * [nq q heads | nkv k heads | nkv v heads], each head d rows, then RoPE on
 * the q and k heads; v is left as is.  nkv = (n/d - nq) / 2.  y, a: f64 [n];
 * a[r] is row r's magnitude sum before the rotation.  Returns 0 or -1.
 */
int q4o_qkv_rope(const uint32_t *words, const uint16_t *scales, const uint16_t *x,
                 int64_t n, int64_t k, int64_t d, int64_t nq, int64_t pos, double base,
                 double *y, double *a)
{
    if (d < 2 || d % 2 || n % d || nq < 0)
        return -1;
    const int64_t heads = n / d, nkv = (heads - nq) / 2;
    if (nkv < 0 || nq + 2 * nkv != heads)
        return -1;
    if (q4o_gemv(words, scales, x, n, k, y, a))
        return -1;
    for (int64_t h = 0; h < nq + nkv; ++h)   /* q heads, then k heads */
        for (int64_t i = 0; i < d / 2; ++i) {
            double oi, oj;
            q4o_rope_pair(y[h * d + i], y[h * d + i + d / 2], i, d, pos, base, &oi, &oj);
            y[h * d + i] = oi;
            y[h * d + i + d / 2] = oj;
        }
    return 0;
}

/*
 * Paged-attention decode for one token ([P1] 内核融合: attention merges paged
 * attention with the page-table reads; 完整的推理流水线: vLLM-style page
 * table).  Cache layout as the fused QKV step writes it:
 * cache[page][K=0|V=1][nkv heads][16 slots][d] (head-major inside a page, as
 * vLLM's blocks are), position t in slot t % 16 of page page_table[t / 16].
 * Query head h reads kv head h / (nq / nkv).
 *   s_t = scale * sum_i q[h][i] K_t[i],  p_t = e^(s_t - max s) / sum_u e^(s_u - max s)
 *   out[h][i] = sum_t p_t V_t[i],        a[h][i] = sum_t p_t |V_t[i]|
 * over t = 0 .. ctx-1.  q [nq][d], cache f16 bits; out, a f64 [nq][d].
 * Returns 0, or -1 for a bad shape or a page entry outside [0, n_pages).
 * The same definition serves the int8 cache (q4o_attention_decode_int8);
 * kv_at reads either.
 */

/* where one decode step reads its keys and values: the f16 cache, or the
 * int8 cache (the int8 KV section below) */
struct kv_source {
    const uint16_t *f16;     /* [pages][2][nkv][16][d] f16 bits, or NULL */
    const uint8_t *i8;       /* int8 pages (16 d codes + 16 f32 scales per block) */
    const int32_t *table;
    int64_t nkv, d;
};

int64_t q4o_kv8_page_bytes(int64_t nkv, int64_t d);

/* element i of the key (kv = 0) or value (kv = 1) row of kv head g at
 * position t, exact in f64 */
static double kv_at(const struct kv_source *src, int kv, int64_t g, int64_t t, int64_t i)
{
    const int64_t page = src->table[t / 16], d = src->d;
    if (src->f16)
        return q4o_half_to_double(src->f16[(((page * 2 + kv) * src->nkv + g) * 16 + t % 16) * d + i]);
    const uint8_t *blk = src->i8 + page * q4o_kv8_page_bytes(src->nkv, d) +
                         (kv * src->nkv + g) * (16 * d + 64);
    float s;
    memcpy(&s, blk + 16 * d + 4 * (t % 16), 4);
    return (double)(int8_t)blk[(t % 16) * d + i] * (double)s;
}

/* the attention definition over either cache (see q4o_attention_decode) */
static int attend(const uint16_t *q, const struct kv_source *src, int64_t n_pages, int64_t ctx,
                  int64_t nq, double scale, double *out, double *a)
{
    const int64_t nkv = src->nkv, d = src->d;
    if (ctx < 1 || nq < 1 || nkv < 1 || nq % nkv || d < 1)
        return -1;
    for (int64_t t = 0; t < ctx; ++t)
        if (src->table[t / 16] < 0 || src->table[t / 16] >= n_pages)
            return -1;
    double *sc = (double *)malloc(sizeof(double) * (size_t)ctx);
    if (!sc)
        return -1;
    for (int64_t h = 0; h < nq; ++h) {
        const int64_t g = h / (nq / nkv);
        double mx = -INFINITY;
        for (int64_t t = 0; t < ctx; ++t) {
            double dot = 0.0;
            for (int64_t i = 0; i < d; ++i)
                dot += q4o_half_to_double(q[h * d + i]) * kv_at(src, 0, g, t, i);
            sc[t] = scale * dot;
            if (sc[t] > mx)
                mx = sc[t];
        }
        double den = 0.0;
        for (int64_t t = 0; t < ctx; ++t) {
            sc[t] = exp(sc[t] - mx);
            den += sc[t];
        }
        for (int64_t i = 0; i < d; ++i) {
            double o = 0.0, m = 0.0;
            for (int64_t t = 0; t < ctx; ++t) {
                const double v = kv_at(src, 1, g, t, i);
                o += sc[t] * v;
                m += sc[t] * fabs(v);
            }
            out[h * d + i] = o / den;
            if (a)
                a[h * d + i] = m / den;
        }
    }
    free(sc);
    return 0;
}

int q4o_attention_decode(const uint16_t *q, const uint16_t *cache, const int32_t *page_table,
                         int64_t n_pages, int64_t ctx, int64_t nq, int64_t nkv, int64_t d,
                         double scale, double *out, double *a)
{
    const struct kv_source src = {cache, NULL, page_table, nkv, d};
    return attend(q, &src, n_pages, ctx, nq, scale, out, a);
}

/* greedy argmax ([P1] 完整的推理流水线, 贪婪解码采样): the lowest index that
 * holds the maximum.  Returns -1 for n < 1. */
int64_t q4o_argmax(const double *v, int64_t n)
{
    if (n < 1)
        return -1;
    int64_t best = 0;
    for (int64_t i = 1; i < n; ++i)
        if (v[i] > v[best])
            best = i;
    return best;
}

/*
 * LM head with f32 logits ([P1] 完整的推理流水线): the same matmul; the
 * oracle keeps f64 logits, and returns the greedy argmax of them.
 */
int64_t q4o_lmhead(const uint32_t *words, const uint16_t *scales,
                   const uint16_t *x, int64_t n, int64_t k, double *logits,
                   double *a)
{
    if (q4o_gemv(words, scales, x, n, k, logits, a))
        return -1;
    return q4o_argmax(logits, n);
}

/* --------------------------------------------- device layout, version 1 --
 *
 * Specification (the library's own design; no page describes one):
 *   G = k/32 groups per row.  P = ceil(G/256) passes; Gp = ceil(G/P).
 *   (L, CG): L in {64,32,16,8,4,2,1} lanes per row, CG in {1,2,3,4} groups per
 *   lane, with L*CG >= Gp; the least L*CG wins, ties go to the larger L.
 *   U = 2 rows per lane slot; RW = 64/L slots; TR = 2*RW rows per tile.
 *   Tiles T = ceil(rows / TR); pass bytes PB = CG*2304; tile bytes TB = P*PB.
 *   Logical (row r, group g) with r < T*TR and g < P*L*CG lives at
 *     t = r / TR, s = (r % TR) / 2, u = r % 2,
 *     p = g / (L*CG), c = (g % (L*CG)) / CG, j = g % CG, lane = s*L + c,
 *     codes (4 words, canonical order) at t*TB + p*PB + (u*CG + j)*1024 + lane*16,
 *     scale (f16)                      at t*TB + p*PB + 2*CG*1024 + lane*4*CG
 *                                          + (u*CG + j)*2.
 *   Rows >= rows or groups >= G are padding: words 0x88888888, scale 0x0000.
 *   Gate/up layout: logical row 2i is gate row i, row 2i+1 is up row i
 *   (2n logical rows in all), then the same placement.
 */
static void geometry(int64_t k, int *L_out, int *CG_out, int *P_out)
{
    int64_t G = k / 32;
    int64_t P = (G + 255) / 256;
    int64_t Gp = (G + P - 1) / P;
    int bestL = 0, bestCG = 0;
    int64_t bestCover = 0;
    for (int L = 64; L >= 1; L /= 2) {
        for (int CG = 1; CG <= 4; ++CG) {
            int64_t cover = (int64_t)L * CG;
            if (cover < Gp)
                continue;
            if (bestL == 0 || cover < bestCover) {
                bestL = L;
                bestCG = CG;
                bestCover = cover;
            }
        }
    }
    *L_out = bestL;
    *CG_out = bestCG;
    *P_out = (int)P;
}

/* geometry as seen by the tests: out[0..5] = L, CG, P, TR, tiles, tile bytes */
int q4o_layout_geometry(int64_t rows, int64_t k, int64_t *out)
{
    if (rows < 1 || k < 32 || k % 32 != 0)
        return -1;
    int L, CG, P;
    geometry(k, &L, &CG, &P);
    int64_t TR = 2 * (64 / L);
    out[0] = L;
    out[1] = CG;
    out[2] = P;
    out[3] = TR;
    out[4] = (rows + TR - 1) / TR;
    out[5] = (int64_t)P * CG * 2304;
    return 0;
}

/* bytes of the device layout for `rows` logical rows (gate/up: 2n) */
int64_t q4o_layout_bytes(int64_t rows, int64_t k)
{
    int64_t g[6];
    if (q4o_layout_geometry(rows, k, g))
        return 0;
    return g[4] * g[5];
}

/* byte offsets of the code unit and the scale of logical (row r, group g)
 * for lane units of UB bytes (int4: 1024 = 64 lanes x 16; int3: 768 = 64 x
 * 12): a pass is CG * (2 UB + 256) bytes, a tile P passes (TB bytes) */
static void unit_offsets(int64_t r, int64_t g, int L, int CG, int64_t TR, int64_t TB,
                         int64_t UB, int64_t *code_off, int64_t *scale_off)
{
    int64_t PB = (int64_t)CG * (2 * UB + 256);
    int64_t t = r / TR, s = (r % TR) / 2, u = r % 2;
    int64_t p = g / ((int64_t)L * CG);
    int64_t c = (g % ((int64_t)L * CG)) / CG, j = g % CG;
    int64_t lane = s * L + c;
    int64_t base = t * TB + p * PB;
    *code_off = base + (u * CG + j) * UB + lane * (UB / 64);
    *scale_off = base + (int64_t)2 * CG * UB + lane * 4 * CG + (u * CG + j) * 2;
}

/* place one logical (row, group) at its destination; src words may be NULL
 * (padding) */
static void place(uint8_t *dst, int64_t r, int64_t g, int L, int CG,
                  int64_t TR, int64_t TB, const uint32_t *src_words,
                  uint16_t src_scale)
{
    int64_t co, so;
    unit_offsets(r, g, L, CG, TR, TB, 1024, &co, &so);
    uint8_t *code_dst = dst + co;
    uint8_t *scale_dst = dst + so;
    for (int w = 0; w < 4; ++w) {
        uint32_t word = src_words ? src_words[w] : 0x88888888u;
        memcpy(code_dst + 4 * w, &word, 4); /* little-endian, as on the GPU */
    }
    memcpy(scale_dst, &src_scale, 2);
}

/* shared walk over the logical rows r of the layout; the canonical row
 * behind r: plain (mode 0), gate/up interleave (mode 1: 2i = gate i, 2i+1 =
 * up i), or rotary pairs (mode 2, heads d wide: 2p + u = dim p % (d/2) +
 * u d/2 of head p / (d/2)) */
static int encode(const uint32_t *w0, const uint16_t *s0, const uint32_t *w1,
                  const uint16_t *s1, int64_t rows, int64_t k, int interleave,
                  int64_t d, uint8_t *dst)
{
    int64_t geo[6];
    if (q4o_layout_geometry(rows, k, geo))
        return -1;
    int L = (int)geo[0], CG = (int)geo[1], P = (int)geo[2];
    int64_t TR = geo[3], T = geo[4], TB = geo[5];
    int64_t G = k / 32;
    for (int64_t r = 0; r < T * TR; ++r) {
        const uint32_t *rw = NULL;
        const uint16_t *rs = NULL;
        if (r < rows) {
            if (interleave == 1) {
                int64_t i = r / 2;
                rw = (r % 2 ? w1 : w0) + i * (k / 8);
                rs = (r % 2 ? s1 : s0) + i * G;
            } else if (interleave == 2) {
                int64_t pr = r / 2, u = r % 2;
                int64_t src = (pr / (d / 2)) * d + pr % (d / 2) + u * (d / 2);
                rw = w0 + src * (k / 8);
                rs = s0 + src * G;
            } else {
                rw = w0 + r * (k / 8);
                rs = s0 + r * G;
            }
        }
        for (int64_t g = 0; g < (int64_t)P * L * CG; ++g) {
            if (rw && g < G)
                place(dst, r, g, L, CG, TR, TB, rw + 4 * g, rs[g]);
            else
                place(dst, r, g, L, CG, TR, TB, NULL, 0);
        }
    }
    return 0;
}

/* plain row layout of words [n][k/8], scales [n][k/32] */
int q4o_encode_rows(const uint32_t *words, const uint16_t *scales, int64_t n,
                    int64_t k, uint8_t *dst)
{
    return encode(words, scales, NULL, NULL, n, k, 0, 0, dst);
}

/* gate/up interleaved layout: 2n logical rows */
int q4o_encode_gate_up(const uint32_t *gw, const uint16_t *gs,
                       const uint32_t *uw, const uint16_t *us, int64_t n,
                       int64_t k, uint8_t *dst)
{
    return encode(gw, gs, uw, us, 2 * n, k, 1, 0, dst);
}

/* rotary-pair layout of words [n][k/8], scales [n][k/32]: heads of d rows
 * (d even, n % d == 0), dims i and i + d/2 of a head on logical rows 2p, 2p+1 */
int q4o_encode_rope(const uint32_t *words, const uint16_t *scales, int64_t n,
                    int64_t k, int64_t d, uint8_t *dst)
{
    if (d < 2 || d % 2 || n % d)
        return -1;
    return encode(words, scales, NULL, NULL, n, k, 2, d, dst);
}

/* ----------------------------------------------------------------- int3 -- */

/*
 * The int3 variant of the same matmul ([P4] the Zero-TVM README, where it
 * says where the shaders live, names one generator for an int4/int3 matmul
 * family; no page gives the int3 bit layout).  This
 * library's definition, which the oracle follows literally:
 *   - codes q in 0..7; a row's codes form one bit stream, LSB first, over its
 *     little-endian uint32 words [n][3k/32]: code k sits in stream bits
 *     3k, 3k+1, 3k+2 (bit b of the stream is bit b % 32 of word b / 32), so
 *     each group of 32 codes fills exactly 3 words;
 *   - one f16 scale per group of 32 consecutive k of a row; scales [N][K/32];
 *   - weight value w = (q - 4) * scale (4 is the midpoint of 0..7);
 *   - y[n] = sum_k x[k] * w[n][k], f64, k ascending, one term at a time.
 */

/* bit b of row r's stream */
static int stream_bit(const uint32_t *words3, int64_t r, int64_t k, int64_t b)
{
    uint32_t word = words3[r * (3 * k / 32) + b / 32];
    return (int)((word >> (b % 32)) & 1u);
}

/* code of row r at position kk: stream bits 3kk (least significant) .. 3kk+2 */
static int code3_at(const uint32_t *words3, int64_t r, int64_t kk, int64_t k)
{
    int q = 0;
    for (int t = 0; t < 3; ++t)
        q |= stream_bit(words3, r, k, 3 * kk + t) << t;
    return q;
}

/* y = x . dequant3(W)^T; words3 [n][3k/32], scales [n][k/32], x [k] f16 bits;
 * a as in q4o_gemv (may be NULL).  Returns 0, or -1 on a bad shape. */
int q4o_gemv3(const uint32_t *words3, const uint16_t *scales, const uint16_t *x,
              int64_t n, int64_t k, double *y, double *a)
{
    if (n < 1 || k < 32 || k % 32 != 0)
        return -1;
    const int64_t G = k / 32;
    for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0, mag = 0.0;
        for (int64_t col = 0; col < k; ++col) {
            int q = code3_at(words3, r, col, k);
            double s = q4o_half_to_double(scales[r * G + col / 32]);
            double term = q4o_half_to_double(x[col]) * ((double)(q - 4) * s);
            acc += term;
            mag += fabs(term);
        }
        y[r] = acc;
        if (a)
            a[r] = mag;
    }
    return 0;
}

/* Y = X . dequant3(W)^T for m activation rows (the int3 form of q4o_gemm):
 * X [m][k] f16 bits, Y, A [m][n] (A may be NULL). */
int q4o_gemm3(const uint32_t *words3, const uint16_t *scales, const uint16_t *X, int64_t m,
              int64_t n, int64_t k, double *Y, double *A)
{
    if (m < 1)
        return -1;
    for (int64_t r = 0; r < m; ++r) {
        const int rc = q4o_gemv3(words3, scales, X + r * k, n, k, Y + r * n, A ? A + r * n : NULL);
        if (rc)
            return rc;
    }
    return 0;
}

/* The fused gate/up + SiLU FFN over int3 weights: q4o_ffn_gate_up_silu with
 * the int3 matmul (gate and up rows each a canonical int3 stream). */
int q4o_ffn_gate_up_silu3(const uint32_t *gw3, const uint16_t *gs, const uint32_t *uw3,
                          const uint16_t *us, const uint16_t *x, int64_t n, int64_t k, double *h,
                          double *g, double *u, double *ag, double *au)
{
    if (n < 0 || k < 32 || k % 32 != 0)
        return -1;
    for (int64_t r = 0; r < n; ++r) {
        double gv, uv, agv, auv;
        q4o_gemv3(gw3 + r * (3 * k / 32), gs + r * (k / 32), x, 1, k, &gv, &agv);
        q4o_gemv3(uw3 + r * (3 * k / 32), us + r * (k / 32), x, 1, k, &uv, &auv);
        h[r] = gated(gv, uv);
        if (g)
            g[r] = gv;
        if (u)
            u[r] = uv;
        if (ag)
            ag[r] = agv;
        if (au)
            au[r] = auv;
    }
    return 0;
}

/*
 * Device layout of an int3 weight (layout Q4_LAYOUT_INT3, version 1), from
 * its specification.  The tile geometry (L, CG, P, TR, tiles) is the int4
 * one above; a lane unit holds one group of one row in 12 bytes (3 words)
 * instead of 16, so a unit slot is 768 bytes and a pass PB3 = CG * 1792:
 *   codes (3 words) at t*TB3 + p*PB3 + (u*CG + j)*768 + lane*12,
 *   scale (f16)     at t*TB3 + p*PB3 + 2*CG*768 + lane*4*CG + (u*CG + j)*2,
 * with TB3 = P * PB3 and (t, p, u, j, lane) from (row, group) as for int4.
 * The 32 codes c0..c31 of a group sit in its 3 device words w0, w1, w2:
 *   word i, bits 3m .. 3m+2       (m = 0..4): code 10i + m,
 *   word i, bits 16+3m .. 18+3m   (m = 0..4): code 10i + 5 + m,
 *   word i, bit 15: bit i of code 30;  word i, bit 31: bit i of code 31.
 * Padding (rows >= n or groups >= G): every code 4, scale 0x0000.
 * The gate/up int3 layout (Q4_LAYOUT_INT3_GATE_UP) is the same placement over
 * 2n logical rows, row 2i = gate row i and row 2i+1 = up row i.
 */
static void place3(uint8_t *dst, int64_t r, int64_t g, int L, int CG, int64_t TR,
                   int64_t TB3, const int *codes, uint16_t scale)
{
    int64_t co, so;
    unit_offsets(r, g, L, CG, TR, TB3, 768, &co, &so);
    uint8_t *code_dst = dst + co;
    uint8_t *scale_dst = dst + so;
    for (int i = 0; i < 3; ++i) {
        uint32_t word = 0;
        for (int m = 0; m < 5; ++m) {
            word |= (uint32_t)codes[10 * i + m] << (3 * m);
            word |= (uint32_t)codes[10 * i + 5 + m] << (16 + 3 * m);
        }
        word |= (uint32_t)((codes[30] >> i) & 1) << 15;
        word |= (uint32_t)((codes[31] >> i) & 1) << 31;
        memcpy(code_dst + 4 * i, &word, 4);
    }
    memcpy(scale_dst, &scale, 2);
}

/* int3 device layout over `rows` logical rows; logical row r reads row r of
 * (w0, s0), or with a second source row r / 2 of (w0, s0) for even r and of
 * (w1, s1) for odd r (gate/up) */
static int encode3(const uint32_t *w0, const uint16_t *s0, const uint32_t *w1, const uint16_t *s1,
                   int64_t rows, int64_t k, uint8_t *dst)
{
    int64_t geo[6];
    if (q4o_layout_geometry(rows, k, geo))
        return -1;
    int L = (int)geo[0], CG = (int)geo[1], P = (int)geo[2];
    int64_t TR = geo[3], T = geo[4];
    int64_t TB3 = (int64_t)P * CG * 1792;
    int64_t G = k / 32;
    int codes[32];
    for (int64_t r = 0; r < T * TR; ++r) {
        const uint32_t *rw = w1 ? (r % 2 ? w1 : w0) : w0;
        const uint16_t *rs = w1 ? (r % 2 ? s1 : s0) : s0;
        const int64_t src = w1 ? r / 2 : r;
        for (int64_t g = 0; g < (int64_t)P * L * CG; ++g) {
            int real = r < rows && g < G;
            for (int i = 0; i < 32; ++i)
                codes[i] = real ? code3_at(rw, src, 32 * g + i, k) : 4;
            place3(dst, r, g, L, CG, TR, TB3, codes, real ? rs[src * G + g] : 0);
        }
    }
    return 0;
}

/* int3 device layout of words3 [n][3k/32], scales [n][k/32] */
int q4o_encode3(const uint32_t *words3, const uint16_t *scales, int64_t n, int64_t k,
                uint8_t *dst)
{
    return encode3(words3, scales, NULL, NULL, n, k, dst);
}

/* int3 gate/up layout: 2n logical rows, gate i on row 2i, up i on row 2i + 1 */
int q4o_encode3_gate_up(const uint32_t *gw3, const uint16_t *gs, const uint32_t *uw3,
                        const uint16_t *us, int64_t n, int64_t k, uint8_t *dst)
{
    return encode3(gw3, gs, uw3, us, 2 * n, k, dst);
}

/* bytes of the int3 device layout */
int64_t q4o_layout3_bytes(int64_t n, int64_t k)
{
    int64_t g[6];
    if (q4o_layout_geometry(n, k, g))
        return 0;
    return g[4] * g[2] * g[1] * 1792;
}

/* ------------------------------------------------------------ int8 KV -- */

/*
 * The optional int8 KV cache ([P1] 完整的推理流水线: the paged KV cache has an
 * int8 quantisation path that halves its memory; no page gives the scheme).
 * Reading: symmetric quantisation per (token, kv head) row of d values:
 *   m = max_i |x_i|  (over the f16 values, exact in f32),
 *   scale = m / 127  (f32, correctly rounded),  scale = 0 when m = 0,
 *   q_i = rint(x_i / scale)  (f32 quotient, ties to even; 0 when scale = 0),
 * so |q_i| <= 127 and x_i ~ q_i * scale.  The codes are decided in f32, the
 * kernel's precision, as the oracle must decide them the same way.
 * Cache layout: [page][K=0|V=1][kv head] blocks of 16 * d int8 codes (slot
 * major) followed by 16 f32 scales, i.e. 16 d + 64 bytes per block.
 */
void q4o_kv_quant_row(const uint16_t *x, int64_t d, int8_t *q, float *scale)
{
    float m = 0.0f;
    for (int64_t i = 0; i < d; ++i) {
        float a = (float)fabs(q4o_half_to_double(x[i]));
        if (a > m)
            m = a;
    }
    float s = m / 127.0f;   /* f32 division, rounded once */
    *scale = s;
    for (int64_t i = 0; i < d; ++i) {
        if (s == 0.0f) {
            q[i] = 0;
            continue;
        }
        float t = (float)q4o_half_to_double(x[i]) / s;
        q[i] = (int8_t)rintf(t);
    }
}

/* bytes of one int8 page: 2 * nkv blocks of 16 d codes + 16 f32 scales */
int64_t q4o_kv8_page_bytes(int64_t nkv, int64_t d)
{
    return 2 * nkv * (16 * d + 64);
}

/*
 * Append the k and v heads of a fused QKV output (f16 [nq + 2 nkv][d], k heads
 * after RoPE) at position pos: each head row quantised by q4o_kv_quant_row
 * into slot pos % 16 of page page_table[pos / 16].  An entry outside
 * [0, n_pages) appends nothing.  Returns 0, or -1 on a bad shape.
 */
int q4o_kv_append_int8(const uint16_t *qkv, int64_t nq, int64_t nkv, int64_t d, int64_t pos,
                       uint8_t *cache8, const int32_t *page_table, int64_t n_pages)
{
    if (nq < 1 || nkv < 1 || d < 1 || pos < 0)
        return -1;
    int64_t page = page_table[pos / 16];
    if (page < 0 || page >= n_pages)
        return 0;
    int64_t block = 16 * d + 64;
    for (int64_t kv = 0; kv < 2; ++kv)
        for (int64_t g = 0; g < nkv; ++g) {
            const uint16_t *row = qkv + (nq + kv * nkv + g) * d;
            uint8_t *blk = cache8 + page * q4o_kv8_page_bytes(nkv, d) + (kv * nkv + g) * block;
            float s;
            q4o_kv_quant_row(row, d, (int8_t *)(blk + (pos % 16) * d), &s);
            memcpy(blk + 16 * d + 4 * (pos % 16), &s, 4);
        }
    return 0;
}

/*
 * Paged-attention decode over the int8 cache: the definition of
 * q4o_attention_decode with K_t[i] = q * scale and V_t[i] = q * scale
 * (the dequantised values, exact in f64).
 */
int q4o_attention_decode_int8(const uint16_t *q, const uint8_t *cache8, const int32_t *page_table,
                              int64_t n_pages, int64_t ctx, int64_t nq, int64_t nkv, int64_t d,
                              double scale, double *out, double *a)
{
    const struct kv_source src = {NULL, cache8, page_table, nkv, d};
    return attend(q, &src, n_pages, ctx, nq, scale, out, a);
}
