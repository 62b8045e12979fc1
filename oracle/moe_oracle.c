/*
 * CPU oracle for the MoE W4A16 layer — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct C: fp64 arithmetic throughout, loops in the order of the
 * definitions, no blocking or fusion.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this file's library; the product path never does.  It shares no
 * code, header, table or helper with the HIP implementation.
 *
 * Sources (pages), cited by title and section:
 *   [Atlas]  "告别Python堆栈：Atlas用纯Rust重写LLM推理，在GB10上跑赢vLLM"
 *            section "编译时内核选择和W4A16 Grouped GEMM": per-expert gate_up and down projections over
 *            packed FP4 weights that are dequantized to BF16 before the matmul; a launch grid sized by
 *            max_m_tiles.  Section "KV Cache量化、MTP推测解码和调试工具链": names E2M1 as the FP4
 *            element format, and the single-precision reference-oracle debugging method.
 *   [ATOM]   "AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍"
 *            section "8.1 MoE 路径：路由、专家并行与 MORI 通信": routing, top-k selection, expert compute
 *            and the final combine.  Section "6.1 Linear：按量化类型分派 GEMM": per-1x32 MXFP4 (one scale
 *            per 32 weights along K).
 *   [RustDL] "Rust 实现深度学习推理引擎：从计算图到异构硬件加速"
 *            section "四、算子融合：性能翻倍的关键": SiLU as the activation fused after the matmul.
 *   The Atlas section "KV Cache量化、MTP推测解码和调试工具链" also names, per MoE layer, the gate
 *   input, the gate logits, the routed-only output and the shared expert output.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - E2M1 follows the OCP microscaling element definition: 1 sign, 2 exponent bits (bias 1),
 *     1 mantissa bit, exponent field 0 is subnormal (0 or 0.5).  Code 8 is -0.0.
 *   - Two codes per byte, the even K index in the low nibble; one bf16 scale per 32 K elements.
 *   - Gate rows are [0, I) of the gate_up weight, up rows are [I, 2I); h = silu(gate) * up.
 *   - Routing: softmax over all E logits, keep the k largest, renormalise over the kept k.  Softmax
 *     is strictly increasing in the logit, so the kept set is the k largest logits; equal logits are
 *     broken toward the lower expert id, and slot 0 holds the largest.  The comparison is made on
 *     the fp32 logits themselves.
 *   - Permutation: a stable counting sort of the flat slot index f = t*k + s by expert id.
 *   - Combine: y[t] = sum over slots s (ascending) of w[t,s] * o[t,s].
 *   - Gate logits: logits[t, e] = sum_h x[t, h] * w_router[e, h] with bf16 x and w_router.
 *   - Shared expert: one more SwiGLU FFN with the same W4 format, applied to every token, whose
 *     output is added to the routed output with weight 1.
 *   - MXFP4 (the ATOM page, section 6.1, lists "per-1x32 MXFP4" with an a4w4 GEMM, and section 8.2
 *     lists dynamic activation quantization as part of a format's contract): weights are E2M1
 *     codes with one E8M0 scale (2^(byte - 127)) per 32 K elements; activations are quantized on
 *     the fly to the same format before each projection (x before gate_up, h before down), by the
 *     OCP Microscaling (MX) v1.0 conversion: per block of 32, X = 2^(floor(log2(amax)) - 2) (2 = the
 *     largest E2M1 exponent), clamped to the E8M0 range, an all-zero block taking 2^-127; each
 *     element becomes the E2M1 value nearest to v / X, ties to the even code, |v / X| > 6 saturating
 *     to 6.  Each projection's output is exact sums of products of the dequantized operands.
 *   - FP8 (the ATOM page, section 6.1, lists "per-1x128 FP8" served by an a8w8 block-scale GEMM, and
 *     section 8.1 names an FP8 path of its fused MoE): weights and activations are OCP FP8 E4M3 codes
 *     (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 subnormal; S.1111.111
 *     is NaN; largest finite 448), one byte per element, with one fp32 scale per row and block of 128
 *     consecutive K elements on both operands (the literal reading of "per-1x128", applied to both).
 *     Activations are quantized on the fly before each projection (x before gate_up, h before down):
 *     per block, the values rounded to fp32, amax = max |v|, s = amax / 448 rounded to fp32, and each
 *     code the E4M3 value nearest to the fp32 quotient v / s, ties to the even code; s == 0 (an
 *     all-zero block) gives codes 0.  These decisions are taken in fp32, the precision the GPU takes
 *     them in, so that both sides reach the same codes from the same fp32 values.
 *   - W4A8 (the scaled-instruction path with 8-bit activations beside the a4w4 one): weights as in
 *     the MXFP4 layer; activations quantized on the fly to MXFP8, the OCP MX format with E4M3
 *     elements: per block of 32 K elements X = 2^(floor(log2(amax)) - 8) (8 = the largest E4M3
 *     exponent), clamped to the E8M0 range, an all-zero block taking 2^-127; each element becomes the
 *     E4M3 value nearest to v / X, ties to the even code, magnitudes beyond 448 saturating to 448.
 *     v / X is exact, so every decision is taken on exact values.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GROUP 32

/* ---- element decode ---------------------------------------------------------------------- */

/* E2M1 code -> value.  Bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent field 0: subnormal, value = 0.5 * m.  Otherwise 2^(e-1) * (1 + m/2). */
double oracle_e2m1_value(int code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* bf16 bit pattern -> value (the upper 16 bits of an IEEE binary32). */
double oracle_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Dequantized weight W[n, kk] of a row-major [N, K] matrix stored as codes q [N, K/2] and scales
 * s [N, K/32]: value(code) * scale, computed in fp32 (the product of a <=2-bit and an 8-bit
 * significand is exact in fp32) and returned widened to fp64. */
static double weight_at(const uint8_t *q, const uint16_t *s, int64_t K, int64_t n, int64_t kk)
{
    uint8_t byte = q[n * (K / 2) + kk / 2];
    int code = (kk % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    float v = (float)oracle_e2m1_value(code);
    float sc = (float)oracle_bf16_value(s[n * (K / ORACLE_GROUP) + kk / ORACLE_GROUP]);
    return (double)(v * sc);
}

/* Dense dequantization of one [N, K] weight matrix into out [N, K] (fp64). */
void oracle_dequant(const uint8_t *q, const uint16_t *s, int64_t N, int64_t K, double *out)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t kk = 0; kk < K; ++kk)
            out[n * K + kk] = weight_at(q, s, K, n, kk);
}

/* ---- routing ------------------------------------------------------------------------------ */

/* "a ranks before b" for top-k selection: larger logit first, then lower expert id. */
static int ranks_before(float la, int a, float lb, int b)
{
    if (la != lb) return la > lb;
    return a < b;
}

/* Top-k routing of T tokens over E experts: ids [T, k] (slot 0 = best), weights [T, k] in fp64.
 * Softmax over all experts, keep k, renormalise over the kept k. */
void oracle_route(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *ids, double *w)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        /* softmax over all E, in fp64 */
        double mx = -INFINITY;
        for (int64_t e = 0; e < E; ++e) if ((double)l[e] > mx) mx = (double)l[e];
        double z = 0.0;
        for (int64_t e = 0; e < E; ++e) { p[e] = exp((double)l[e] - mx); z += p[e]; }
        for (int64_t e = 0; e < E; ++e) p[e] /= z;
        /* k rounds of selection of the best remaining expert */
        memset(taken, 0, (size_t)E);
        for (int64_t s = 0; s < k; ++s) {
            int best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l[e], (int)e, l[best], best)) best = (int)e;
            }
            taken[best] = 1;
            ids[t * k + s] = best;
        }
        /* renormalise the kept probabilities */
        double sum = 0.0;
        for (int64_t s = 0; s < k; ++s) sum += p[ids[t * k + s]];
        for (int64_t s = 0; s < k; ++s) w[t * k + s] = p[ids[t * k + s]] / sum;
    }
    free(p);
    free(taken);
}

/* ---- token -> expert permutation ------------------------------------------------------------ */

/* Stable counting sort of the R = T*k flat slots by expert id.
 *   counts[E]       rows routed to each expert
 *   offsets[E+1]    exclusive prefix sum of counts (offsets[E] = R)
 *   sorted_ids[R]   flat slot f = t*k+s held at permuted row r (ascending f within an expert)
 *   inv_perm[R]     permuted row of flat slot f
 *   tiles[*,3]      (expert, first row, rows) for every block of up to block_m rows of one expert,
 *                   experts ascending, rows ascending
 * Returns the number of tiles.  The maximum number of row tiles of any one expert is
 * written to *max_m_tiles. */
int64_t oracle_align(const int32_t *ids, int64_t T, int64_t k, int64_t E, int64_t block_m,
                     int32_t *counts, int32_t *offsets, int32_t *sorted_ids, int32_t *inv_perm,
                     int32_t *tiles, int32_t *max_m_tiles)
{
    int64_t R = T * k;
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t f = 0; f < R; ++f) counts[ids[f]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int64_t e = 0; e < E; ++e) next[e] = offsets[e];
    for (int64_t f = 0; f < R; ++f) {           /* ascending f keeps the sort stable */
        int32_t r = next[ids[f]]++;
        sorted_ids[r] = (int32_t)f;
        inv_perm[f] = r;
    }
    free(next);
    int64_t nt = 0;
    int32_t mmt = 0;
    for (int64_t e = 0; e < E; ++e) {
        int32_t m_tiles = 0;
        for (int64_t r0 = offsets[e]; r0 < offsets[e + 1]; r0 += block_m) {
            int64_t rows = offsets[e + 1] - r0;
            if (rows > block_m) rows = block_m;
            if (tiles) {
                tiles[nt * 3 + 0] = (int32_t)e;
                tiles[nt * 3 + 1] = (int32_t)r0;
                tiles[nt * 3 + 2] = (int32_t)rows;
            }
            ++nt;
            ++m_tiles;
        }
        if (m_tiles > mmt) mmt = m_tiles;
    }
    if (max_m_tiles) *max_m_tiles = mmt;
    return nt;
}

/* ---- expert projections ---------------------------------------------------------------------- */

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* One expert's W4 matrix [N, K] times one activation row a [K] (fp64): out[n] = sum_kk a[kk] W[n,kk],
 * sums in ascending kk.  Each weight is the value weight_at gives (the code's E2M1 value times the
 * group's bf16 scale, in fp32); the 16 code values are looked up in a table filled from
 * oracle_e2m1_value and each group's scale is decoded once, which changes no product. */
static void expert_matvec(const uint8_t *q, const uint16_t *s, int64_t N, int64_t K,
                          const double *a, double *out)
{
    float tab[16];
    for (int c = 0; c < 16; ++c) tab[c] = (float)oracle_e2m1_value(c);
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *qr = q + n * (K / 2);
        const uint16_t *sr = s + n * (K / ORACLE_GROUP);
        double acc = 0.0;
        for (int64_t g = 0; g < K / ORACLE_GROUP; ++g) {
            const float sc = (float)oracle_bf16_value(sr[g]);
            for (int64_t i = 0; i < ORACLE_GROUP; ++i) {
                const int64_t kk = g * ORACLE_GROUP + i;
                const uint8_t byte = qr[kk / 2];
                const int code = (kk % 2 == 0) ? (byte & 0xF) : (byte >> 4);
                acc += a[kk] * (double)(tab[code] * sc);
            }
        }
        out[n] = acc;
    }
}

/* Full layer for a subset of tokens (tok == NULL: tokens 0..n_tok-1).
 *   x [T, H] bf16 bits, logits [T, E] fp32, w13_q [E, 2I, H/2], w13_s [E, 2I, H/32] bf16 bits,
 *   w2_q [E, H, I/2], w2_s [E, H, I/32] bf16 bits.
 *   y [n_tok, H] fp64.  Optional diagnostics (may be NULL): h [n_tok, k, I], o [n_tok, k, H].
 * Per token: route, then for each slot s the expert's gate_up projection, h = silu(gate) * up,
 * the down projection o = W2 h, and finally y = sum_s w_s o_s. */
void oracle_moe_ffn(const uint16_t *x, const float *logits, int64_t T, int64_t H, int64_t I,
                    int64_t E, int64_t k, const uint8_t *w13_q, const uint16_t *w13_s,
                    const uint8_t *w2_q, const uint16_t *w2_s, const int64_t *tok, int64_t n_tok,
                    double *y, double *h_out, double *o_out)
{
    (void)T;
    const int64_t sz13_q = 2 * I * (H / 2), sz13_s = 2 * I * (H / ORACLE_GROUP);
    const int64_t sz2_q = H * (I / 2), sz2_s = H * (I / ORACLE_GROUP);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < n_tok; ++j) {
        int64_t t = tok ? tok[j] : j;
        int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
        double *w = (double *)malloc(sizeof(double) * (size_t)k);
        double *xa = (double *)malloc(sizeof(double) * (size_t)H);
        double *g = (double *)malloc(sizeof(double) * (size_t)(2 * I));
        double *h = (double *)malloc(sizeof(double) * (size_t)I);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        oracle_route(logits + t * E, 1, E, k, ids, w);
        for (int64_t c = 0; c < H; ++c) xa[c] = oracle_bf16_value(x[t * H + c]);
        for (int64_t c = 0; c < H; ++c) y[j * H + c] = 0.0;
        for (int64_t s = 0; s < k; ++s) {
            int64_t e = ids[s];
            expert_matvec(w13_q + e * sz13_q, w13_s + e * sz13_s, 2 * I, H, xa, g);
            for (int64_t i = 0; i < I; ++i) h[i] = silu(g[i]) * g[I + i];
            expert_matvec(w2_q + e * sz2_q, w2_s + e * sz2_s, H, I, h, o);
            for (int64_t c = 0; c < H; ++c) y[j * H + c] += w[s] * o[c];
            if (h_out) memcpy(h_out + (j * k + s) * I, h, sizeof(double) * (size_t)I);
            if (o_out) memcpy(o_out + (j * k + s) * H, o, sizeof(double) * (size_t)H);
        }
        free(ids); free(w); free(xa); free(g); free(h); free(o);
    }
}

/* Grouped projection over permuted rows, the operation of one grouped-GEMM launch:
 * for each permuted row r of expert e (offsets[e] <= r < offsets[e+1]) with activation row
 * a_row = (a_row_of ? a_row_of[r] / a_row_div : r):
 *   C[r, n] = sum_kk A[a_row, kk] * W_e[n, kk]           (n < N),
 * A bf16 bits [*, K], Wq [E, N, K/2], Ws [E, N, K/32].  With silu_mul != 0 the output is
 *   C[r, j] = silu(G[r, j]) * G[r, N/2 + j]             (j < N/2).
 * With row_scale != NULL every output of row r is multiplied by row_scale[r].  C is fp64. */
void oracle_grouped_proj(const uint16_t *A, const int32_t *a_row_of, int64_t a_row_div,
                         const uint8_t *Wq, const uint16_t *Ws, int64_t E, int64_t N, int64_t K,
                         const int32_t *offsets, int silu_mul, const double *row_scale, double *C)
{
    const int64_t szq = N * (K / 2), szs = N * (K / ORACLE_GROUP);
    const int64_t nout = silu_mul ? N / 2 : N;
    for (int64_t e = 0; e < E; ++e) {
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r) {
            int64_t arow = a_row_of ? a_row_of[r] / a_row_div : r;
            double *a = (double *)malloc(sizeof(double) * (size_t)K);
            double *g = (double *)malloc(sizeof(double) * (size_t)N);
            for (int64_t c = 0; c < K; ++c) a[c] = oracle_bf16_value(A[arow * K + c]);
            expert_matvec(Wq + e * szq, Ws + e * szs, N, K, a, g);
            for (int64_t n = 0; n < nout; ++n) {
                double v = silu_mul ? silu(g[n]) * g[N / 2 + n] : g[n];
                if (row_scale) v *= row_scale[r];
                C[r * nout + n] = v;
            }
            free(a); free(g);
        }
    }
}

/* Routing-weighted scatter-reduce: y[t, c] = sum_{s<k} w[t, s] * O[inv_perm[t*k+s], c]
 * (O given as fp64 [R, H]). */
void oracle_combine(const double *O, const int32_t *inv_perm, const double *w, int64_t T, int64_t k,
                    int64_t H, double *y)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int64_t s = 0; s < k; ++s) acc += w[t * k + s] * O[(int64_t)inv_perm[t * k + s] * H + c];
            y[t * H + c] = acc;
        }
}

/* ---- router gate and shared expert --------------------------------------------------------------- */

/* Gate logits: logits[t, e] = sum_h x[t, h] * wr[e, h] (x [T, H] and wr [E, H] as bf16 bits, fp64
 * sums in ascending h). */
void oracle_router_logits(const uint16_t *x, const uint16_t *wr, int64_t T, int64_t H, int64_t E, double *logits)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; ++h) acc += oracle_bf16_value(x[t * H + h]) * oracle_bf16_value(wr[e * H + h]);
            logits[t * E + e] = acc;
        }
}

/* Shared expert for a subset of tokens (tok == NULL: tokens 0..n_tok-1): out[j] = W2s h with
 * h = silu(W13s[0:Is] x) * W13s[Is:2Is] x, where w13s_q [2Is, H/2], w13s_s [2Is, H/32],
 * w2s_q [H, Is/2], w2s_s [H, Is/32] (one expert of the routed weight format).  out fp64 [n_tok, H]. */
void oracle_shared_ffn(const uint16_t *x, int64_t H, int64_t Is, const uint8_t *w13s_q, const uint16_t *w13s_s,
                       const uint8_t *w2s_q, const uint16_t *w2s_s, const int64_t *tok, int64_t n_tok, double *out)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < n_tok; ++j) {
        int64_t t = tok ? tok[j] : j;
        double *xa = (double *)malloc(sizeof(double) * (size_t)H);
        double *g = (double *)malloc(sizeof(double) * (size_t)(2 * Is));
        double *h = (double *)malloc(sizeof(double) * (size_t)Is);
        for (int64_t c = 0; c < H; ++c) xa[c] = oracle_bf16_value(x[t * H + c]);
        expert_matvec(w13s_q, w13s_s, 2 * Is, H, xa, g);
        for (int64_t i = 0; i < Is; ++i) h[i] = silu(g[i]) * g[Is + i];
        expert_matvec(w2s_q, w2s_s, H, Is, h, out + j * H);
        free(xa); free(g); free(h);
    }
}

/* ---- MXFP4: E2M1 codes with E8M0 block scales on both operands ----------------------------------- */

/* E8M0 scale byte -> 2^(byte - 127); byte 255 encodes NaN. */
double oracle_e8m0_value(int byte)
{
    if (byte == 255) return NAN;
    return ldexp(1.0, byte - 127);
}

/* The E2M1 code nearest to v: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the code whose
 * mantissa bit is 0, magnitudes above 6 saturate to 6; the sign bit follows v (so -0.0 -> code 8). */
int oracle_e2m1_nearest(double v)
{
    int sign = signbit(v) ? 8 : 0;
    double a = fabs(v);
    if (a >= 6.0) return sign | 7;
    int best = 0;
    double dbest = a;
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - oracle_e2m1_value(c));
        if (d < dbest || (d == dbest && (c & 1) == 0)) { best = c; dbest = d; }
    }
    return sign | best;
}

/* MX quantization of a [rows, K] matrix (K % 32 == 0) into codes q [rows, K/2] (even K index in the
 * low nibble) and scale bytes s [rows, K/32], one block of 32 consecutive K elements at a time. */
void oracle_mx_quantize(const double *v, int64_t rows, int64_t K, uint8_t *q, uint8_t *s)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < K / ORACLE_GROUP; ++b) {
            const double *blk = v + r * K + b * ORACLE_GROUP;
            double amax = 0.0;
            for (int i = 0; i < ORACLE_GROUP; ++i) if (fabs(blk[i]) > amax) amax = fabs(blk[i]);
            int e = -127;
            if (amax > 0.0) {
                int p;
                frexp(amax, &p);  /* amax = m * 2^p, 0.5 <= m < 1: floor(log2(amax)) = p - 1 */
                e = (p - 1) - 2;
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            s[r * (K / ORACLE_GROUP) + b] = (uint8_t)(e + 127);
            for (int i = 0; i < ORACLE_GROUP; i += 2) {
                int c0 = oracle_e2m1_nearest(ldexp(blk[i], -e));
                int c1 = oracle_e2m1_nearest(ldexp(blk[i + 1], -e));
                q[r * (K / 2) + (b * ORACLE_GROUP + i) / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
}

/* Value of element kk of row n of an MX matrix stored as codes q [*, K/2] and scales s [*, K/32]. */
static double mx_at(const uint8_t *q, const uint8_t *s, int64_t K, int64_t n, int64_t kk)
{
    uint8_t byte = q[n * (K / 2) + kk / 2];
    int code = (kk % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    return oracle_e2m1_value(code) * oracle_e8m0_value(s[n * (K / ORACLE_GROUP) + kk / ORACLE_GROUP]);
}

/* Dense dequantization of an MX matrix [rows, K] into out (fp64). */
void oracle_mx_dequant(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t K, double *out)
{
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t kk = 0; kk < K; ++kk) out[n * K + kk] = mx_at(q, s, K, n, kk);
}

/* One expert's MX matrix [N, K] times one (already dequantized) activation row a [K].  Each weight
 * is the value mx_at gives (E2M1 value times the E8M0 scale, exact in fp64); the code values come
 * from a table filled from oracle_e2m1_value and each block's scale is decoded once. */
static void mx_matvec(const uint8_t *q, const uint8_t *s, int64_t N, int64_t K, const double *a, double *out)
{
    double tab[16];
    for (int c = 0; c < 16; ++c) tab[c] = oracle_e2m1_value(c);
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *qr = q + n * (K / 2);
        const uint8_t *sr = s + n * (K / ORACLE_GROUP);
        double acc = 0.0;
        for (int64_t g = 0; g < K / ORACLE_GROUP; ++g) {
            const double sc = oracle_e8m0_value(sr[g]);
            for (int64_t i = 0; i < ORACLE_GROUP; ++i) {
                const int64_t kk = g * ORACLE_GROUP + i;
                const uint8_t byte = qr[kk / 2];
                const int code = (kk % 2 == 0) ? (byte & 0xF) : (byte >> 4);
                acc += a[kk] * (tab[code] * sc);
            }
        }
        out[n] = acc;
    }
}

/* Quantize one activation row to MX and return it dequantized (in place of a). */
static void mx_roundtrip_row(double *a, int64_t K)
{
    uint8_t *q = (uint8_t *)malloc((size_t)(K / 2));
    uint8_t *sc = (uint8_t *)malloc((size_t)(K / ORACLE_GROUP));
    oracle_mx_quantize(a, 1, K, q, sc);
    for (int64_t kk = 0; kk < K; ++kk) a[kk] = mx_at(q, sc, K, 0, kk);
    free(q);
    free(sc);
}

/* Full MXFP4 (W4A4) layer for a subset of tokens (tok == NULL: tokens 0..n_tok-1).
 *   x [T, H] bf16 bits, logits [T, E] fp32, w13_q [E, 2I, H/2], w13_e [E, 2I, H/32] E8M0,
 *   w2_q [E, H, I/2], w2_e [E, H, I/32] E8M0; y [n_tok, H] fp64.
 *   Optional diagnostics (may be NULL): h [n_tok, k, I] (silu(gate) * up before its quantization).
 * Per token: route; quantize x's row to MX; for each slot s the expert's gate_up projection of the
 * quantized row, h = silu(gate) * up, h quantized to MX, the down projection, y = sum_s w_s o_s. */
void oracle_moe_ffn_mx(const uint16_t *x, const float *logits, int64_t T, int64_t H, int64_t I, int64_t E,
                       int64_t k, const uint8_t *w13_q, const uint8_t *w13_e, const uint8_t *w2_q,
                       const uint8_t *w2_e, const int64_t *tok, int64_t n_tok, double *y, double *h_out)
{
    (void)T;
    const int64_t sz13_q = 2 * I * (H / 2), sz13_e = 2 * I * (H / ORACLE_GROUP);
    const int64_t sz2_q = H * (I / 2), sz2_e = H * (I / ORACLE_GROUP);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < n_tok; ++j) {
        int64_t t = tok ? tok[j] : j;
        int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
        double *w = (double *)malloc(sizeof(double) * (size_t)k);
        double *xa = (double *)malloc(sizeof(double) * (size_t)H);
        double *g = (double *)malloc(sizeof(double) * (size_t)(2 * I));
        double *h = (double *)malloc(sizeof(double) * (size_t)I);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        oracle_route(logits + t * E, 1, E, k, ids, w);
        for (int64_t c = 0; c < H; ++c) xa[c] = oracle_bf16_value(x[t * H + c]);
        mx_roundtrip_row(xa, H);
        for (int64_t c = 0; c < H; ++c) y[j * H + c] = 0.0;
        for (int64_t s = 0; s < k; ++s) {
            int64_t e = ids[s];
            mx_matvec(w13_q + e * sz13_q, w13_e + e * sz13_e, 2 * I, H, xa, g);
            for (int64_t i = 0; i < I; ++i) h[i] = silu(g[i]) * g[I + i];
            if (h_out) memcpy(h_out + (j * k + s) * I, h, sizeof(double) * (size_t)I);
            mx_roundtrip_row(h, I);
            mx_matvec(w2_q + e * sz2_q, w2_e + e * sz2_e, H, I, h, o);
            for (int64_t c = 0; c < H; ++c) y[j * H + c] += w[s] * o[c];
        }
        free(ids); free(w); free(xa); free(g); free(h); free(o);
    }
}

/* Grouped MX projection over permuted rows (one grouped-GEMM launch of the MXFP4 path): for each
 * permuted row r of expert e with activation row a_row = (a_row_of ? a_row_of[r] / a_row_div : r),
 *   C[r, n] = sum_kk A[a_row, kk] * W_e[n, kk],  A given as MX codes Aq [*, K/2] and scales As [*, K/32],
 * W as Wq [E, N, K/2] and We [E, N, K/32].  With silu_mul != 0, C[r, j] = silu(G[r, j]) * G[r, N/2 + j]
 * (j < N/2), before any quantization.  C fp64. */
void oracle_grouped_proj_mx(const uint8_t *Aq, const uint8_t *As, const int32_t *a_row_of, int64_t a_row_div,
                            const uint8_t *Wq, const uint8_t *We, int64_t E, int64_t N, int64_t K,
                            const int32_t *offsets, int silu_mul, double *C)
{
    const int64_t szq = N * (K / 2), sze = N * (K / ORACLE_GROUP);
    const int64_t nout = silu_mul ? N / 2 : N;
    for (int64_t e = 0; e < E; ++e) {
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r) {
            int64_t arow = a_row_of ? a_row_of[r] / a_row_div : r;
            double *a = (double *)malloc(sizeof(double) * (size_t)K);
            double *g = (double *)malloc(sizeof(double) * (size_t)N);
            for (int64_t c = 0; c < K; ++c) a[c] = mx_at(Aq, As, K, arow, c);
            mx_matvec(Wq + e * szq, We + e * sze, N, K, a, g);
            for (int64_t n = 0; n < nout; ++n) C[r * nout + n] = silu_mul ? silu(g[n]) * g[N / 2 + n] : g[n];
            free(a); free(g);
        }
    }
}

/* ---- FP8: E4M3 codes with per-1x128 fp32 scales on both operands --------------------------------- */

#define ORACLE_F8_BLOCK 128

/* OCP FP8 E4M3 code -> value.  Bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.
 * Exponent field 0: subnormal, value = (m/8) * 2^-6.  Otherwise 2^(e-7) * (1 + m/8), except that
 * exponent 15 with mantissa 7 encodes NaN (the format has no infinities). */
double oracle_e4m3_value(int code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* The E4M3 code nearest to v among the finite codes (so magnitudes beyond 448 saturate to 448),
 * ties to the code whose mantissa bit 0 is clear; the sign bit follows v (-0.0 -> code 0x80). */
int oracle_e4m3_nearest(double v)
{
    int sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    int best = 0;
    double dbest = a;
    for (int c = 1; c < 0x7F; ++c) {
        double d = fabs(a - oracle_e4m3_value(c));
        if (d < dbest || (d == dbest && (c & 1) == 0)) { best = c; dbest = d; }
    }
    return sign | best;
}

/* Per-1x128 FP8 quantization of a [rows, K] matrix (K % 128 == 0) into codes q [rows, K] and fp32
 * scales s [rows, K/128].  Per block: values rounded to fp32, amax = max |v|, s = amax / 448 (fp32
 * division), code = nearest E4M3 value of the fp32 quotient v / s; s == 0 gives codes 0. */
void oracle_f8_quantize(const double *v, int64_t rows, int64_t K, uint8_t *q, float *s)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < K / ORACLE_F8_BLOCK; ++b) {
            const double *blk = v + r * K + b * ORACLE_F8_BLOCK;
            float amax = 0.0f;
            for (int i = 0; i < ORACLE_F8_BLOCK; ++i) {
                float f = fabsf((float)blk[i]);
                if (f > amax) amax = f;
            }
            float sc = amax / 448.0f;
            s[r * (K / ORACLE_F8_BLOCK) + b] = sc;
            for (int i = 0; i < ORACLE_F8_BLOCK; ++i) {
                float quot = (sc == 0.0f) ? 0.0f : (float)blk[i] / sc;
                q[r * K + b * ORACLE_F8_BLOCK + i] = (sc == 0.0f) ? 0 : (uint8_t)oracle_e4m3_nearest((double)quot);
            }
        }
}

/* Value of element kk of row n of an FP8 matrix stored as codes q [*, K] and scales s [*, K/128]
 * (fp64 product: exact). */
static double f8_at(const uint8_t *q, const float *s, int64_t K, int64_t n, int64_t kk)
{
    return oracle_e4m3_value(q[n * K + kk]) * (double)s[n * (K / ORACLE_F8_BLOCK) + kk / ORACLE_F8_BLOCK];
}

/* Dense dequantization of an FP8 matrix [rows, K] into out (fp64). */
void oracle_f8_dequant(const uint8_t *q, const float *s, int64_t rows, int64_t K, double *out)
{
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t kk = 0; kk < K; ++kk) out[n * K + kk] = f8_at(q, s, K, n, kk);
}

/* One expert's FP8 matrix [N, K] times one (already dequantized) activation row a [K].  Each weight
 * is the value f8_at gives (E4M3 value times the block's fp32 scale, exact in fp64); the 256 code
 * values come from a table filled from oracle_e4m3_value. */
static void f8_matvec(const uint8_t *q, const float *s, int64_t N, int64_t K, const double *a, double *out)
{
    double tab[256];
    for (int c = 0; c < 256; ++c) tab[c] = oracle_e4m3_value(c);
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t b = 0; b < K / ORACLE_F8_BLOCK; ++b) {
            const double sc = (double)s[n * (K / ORACLE_F8_BLOCK) + b];
            for (int64_t i = 0; i < ORACLE_F8_BLOCK; ++i) {
                const int64_t kk = b * ORACLE_F8_BLOCK + i;
                acc += a[kk] * (tab[q[n * K + kk]] * sc);
            }
        }
        out[n] = acc;
    }
}

/* Quantize one activation row to FP8 and return it dequantized (in place of a). */
static void f8_roundtrip_row(double *a, int64_t K)
{
    uint8_t *q = (uint8_t *)malloc((size_t)K);
    float *sc = (float *)malloc(sizeof(float) * (size_t)(K / ORACLE_F8_BLOCK));
    oracle_f8_quantize(a, 1, K, q, sc);
    for (int64_t kk = 0; kk < K; ++kk) a[kk] = f8_at(q, sc, K, 0, kk);
    free(q);
    free(sc);
}

/* Full FP8 (W8A8, per-1x128) layer for a subset of tokens (tok == NULL: tokens 0..n_tok-1).
 *   x [T, H] bf16 bits, logits [T, E] fp32, w13_q [E, 2I, H] E4M3, w13_s [E, 2I, H/128] fp32,
 *   w2_q [E, H, I], w2_s [E, H, I/128] fp32; y [n_tok, H] fp64.
 *   Optional diagnostics (may be NULL): h [n_tok, k, I] (silu(gate) * up before its quantization).
 * Per token: route; quantize x's row; for each slot s the expert's gate_up projection of the
 * quantized row, h = silu(gate) * up, h quantized, the down projection, y = sum_s w_s o_s. */
void oracle_moe_ffn_f8(const uint16_t *x, const float *logits, int64_t T, int64_t H, int64_t I, int64_t E,
                       int64_t k, const uint8_t *w13_q, const float *w13_s, const uint8_t *w2_q,
                       const float *w2_s, const int64_t *tok, int64_t n_tok, double *y, double *h_out)
{
    (void)T;
    const int64_t sz13_q = 2 * I * H, sz13_s = 2 * I * (H / ORACLE_F8_BLOCK);
    const int64_t sz2_q = H * I, sz2_s = H * (I / ORACLE_F8_BLOCK);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < n_tok; ++j) {
        int64_t t = tok ? tok[j] : j;
        int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
        double *w = (double *)malloc(sizeof(double) * (size_t)k);
        double *xa = (double *)malloc(sizeof(double) * (size_t)H);
        double *g = (double *)malloc(sizeof(double) * (size_t)(2 * I));
        double *h = (double *)malloc(sizeof(double) * (size_t)I);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        oracle_route(logits + t * E, 1, E, k, ids, w);
        for (int64_t c = 0; c < H; ++c) xa[c] = oracle_bf16_value(x[t * H + c]);
        f8_roundtrip_row(xa, H);
        for (int64_t c = 0; c < H; ++c) y[j * H + c] = 0.0;
        for (int64_t s = 0; s < k; ++s) {
            int64_t e = ids[s];
            f8_matvec(w13_q + e * sz13_q, w13_s + e * sz13_s, 2 * I, H, xa, g);
            for (int64_t i = 0; i < I; ++i) h[i] = silu(g[i]) * g[I + i];
            if (h_out) memcpy(h_out + (j * k + s) * I, h, sizeof(double) * (size_t)I);
            f8_roundtrip_row(h, I);
            f8_matvec(w2_q + e * sz2_q, w2_s + e * sz2_s, H, I, h, o);
            for (int64_t c = 0; c < H; ++c) y[j * H + c] += w[s] * o[c];
        }
        free(ids); free(w); free(xa); free(g); free(h); free(o);
    }
}

/* Grouped FP8 projection over permuted rows (one grouped-GEMM launch of the FP8 path): for each
 * permuted row r of expert e with activation row a_row = (a_row_of ? a_row_of[r] / a_row_div : r),
 *   C[r, n] = sum_kk A[a_row, kk] * W_e[n, kk],  A as codes Aq [*, K] and scales As [*, K/128],
 * W as Wq [E, N, K] and Ws [E, N, K/128].  With silu_mul != 0, C[r, j] = silu(G[r, j]) * G[r, N/2 + j]
 * (j < N/2), before any quantization.  C fp64. */
void oracle_grouped_proj_f8(const uint8_t *Aq, const float *As, const int32_t *a_row_of, int64_t a_row_div,
                            const uint8_t *Wq, const float *Ws, int64_t E, int64_t N, int64_t K,
                            const int32_t *offsets, int silu_mul, double *C)
{
    const int64_t szq = N * K, szs = N * (K / ORACLE_F8_BLOCK);
    const int64_t nout = silu_mul ? N / 2 : N;
    for (int64_t e = 0; e < E; ++e) {
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r) {
            int64_t arow = a_row_of ? a_row_of[r] / a_row_div : r;
            double *a = (double *)malloc(sizeof(double) * (size_t)K);
            double *g = (double *)malloc(sizeof(double) * (size_t)N);
            for (int64_t c = 0; c < K; ++c) a[c] = f8_at(Aq, As, K, arow, c);
            f8_matvec(Wq + e * szq, Ws + e * szs, N, K, a, g);
            for (int64_t n = 0; n < nout; ++n) C[r * nout + n] = silu_mul ? silu(g[n]) * g[N / 2 + n] : g[n];
            free(a); free(g);
        }
    }
}

/* ---- W4A8: MXFP8 (E4M3 + E8M0 per 32) activations, MXFP4 weights ----------------------------------- */

/* MXFP8 quantization of a [rows, K] matrix (K % 32 == 0) into codes q [rows, K] (one byte per
 * element) and scale bytes s [rows, K/32]: per block of 32, X = 2^e with e = floor(log2(amax)) - 8
 * clamped to [-127, 127] (-127 for an all-zero block), code = nearest E4M3 value of v / X. */
void oracle_mx8_quantize(const double *v, int64_t rows, int64_t K, uint8_t *q, uint8_t *s)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < K / ORACLE_GROUP; ++b) {
            const double *blk = v + r * K + b * ORACLE_GROUP;
            double amax = 0.0;
            for (int i = 0; i < ORACLE_GROUP; ++i) if (fabs(blk[i]) > amax) amax = fabs(blk[i]);
            int e = -127;
            if (amax > 0.0) {
                int p;
                frexp(amax, &p);  /* amax = m * 2^p, 0.5 <= m < 1: floor(log2(amax)) = p - 1 */
                e = (p - 1) - 8;
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            s[r * (K / ORACLE_GROUP) + b] = (uint8_t)(e + 127);
            for (int i = 0; i < ORACLE_GROUP; ++i)
                q[r * K + b * ORACLE_GROUP + i] = (uint8_t)oracle_e4m3_nearest(ldexp(blk[i], -e));
        }
}

/* Value of element kk of row n of an MXFP8 matrix stored as codes q [*, K] and scales s [*, K/32]. */
static double mx8_at(const uint8_t *q, const uint8_t *s, int64_t K, int64_t n, int64_t kk)
{
    return oracle_e4m3_value(q[n * K + kk]) * oracle_e8m0_value(s[n * (K / ORACLE_GROUP) + kk / ORACLE_GROUP]);
}

/* Dense dequantization of an MXFP8 matrix [rows, K] into out (fp64). */
void oracle_mx8_dequant(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t K, double *out)
{
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t kk = 0; kk < K; ++kk) out[n * K + kk] = mx8_at(q, s, K, n, kk);
}

/* Quantize one activation row to MXFP8 and return it dequantized (in place of a). */
static void mx8_roundtrip_row(double *a, int64_t K)
{
    uint8_t *q = (uint8_t *)malloc((size_t)K);
    uint8_t *sc = (uint8_t *)malloc((size_t)(K / ORACLE_GROUP));
    oracle_mx8_quantize(a, 1, K, q, sc);
    for (int64_t kk = 0; kk < K; ++kk) a[kk] = mx8_at(q, sc, K, 0, kk);
    free(q);
    free(sc);
}

/* Full W4A8 layer for a subset of tokens (tok == NULL: tokens 0..n_tok-1); arguments as for
 * oracle_moe_ffn_mx (the same MXFP4 weights).  Per token: route; quantize x's row to MXFP8; for each
 * slot the expert's gate_up projection of the quantized row, h = silu(gate) * up, h quantized to
 * MXFP8, the down projection, y = sum_s w_s o_s.  Optional h_out: h before its quantization. */
void oracle_moe_ffn_w4a8(const uint16_t *x, const float *logits, int64_t T, int64_t H, int64_t I, int64_t E,
                         int64_t k, const uint8_t *w13_q, const uint8_t *w13_e, const uint8_t *w2_q,
                         const uint8_t *w2_e, const int64_t *tok, int64_t n_tok, double *y, double *h_out)
{
    (void)T;
    const int64_t sz13_q = 2 * I * (H / 2), sz13_e = 2 * I * (H / ORACLE_GROUP);
    const int64_t sz2_q = H * (I / 2), sz2_e = H * (I / ORACLE_GROUP);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < n_tok; ++j) {
        int64_t t = tok ? tok[j] : j;
        int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
        double *w = (double *)malloc(sizeof(double) * (size_t)k);
        double *xa = (double *)malloc(sizeof(double) * (size_t)H);
        double *g = (double *)malloc(sizeof(double) * (size_t)(2 * I));
        double *h = (double *)malloc(sizeof(double) * (size_t)I);
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        oracle_route(logits + t * E, 1, E, k, ids, w);
        for (int64_t c = 0; c < H; ++c) xa[c] = oracle_bf16_value(x[t * H + c]);
        mx8_roundtrip_row(xa, H);
        for (int64_t c = 0; c < H; ++c) y[j * H + c] = 0.0;
        for (int64_t s = 0; s < k; ++s) {
            int64_t e = ids[s];
            mx_matvec(w13_q + e * sz13_q, w13_e + e * sz13_e, 2 * I, H, xa, g);
            for (int64_t i = 0; i < I; ++i) h[i] = silu(g[i]) * g[I + i];
            if (h_out) memcpy(h_out + (j * k + s) * I, h, sizeof(double) * (size_t)I);
            mx8_roundtrip_row(h, I);
            mx_matvec(w2_q + e * sz2_q, w2_e + e * sz2_e, H, I, h, o);
            for (int64_t c = 0; c < H; ++c) y[j * H + c] += w[s] * o[c];
        }
        free(ids); free(w); free(xa); free(g); free(h); free(o);
    }
}

/* Grouped W4A8 projection over permuted rows (one grouped-GEMM launch of the W4A8 path): as
 * oracle_grouped_proj_mx with the activations given as MXFP8 codes Aq [*, K] and scale bytes
 * As [*, K/32].  C fp64, before any quantization. */
void oracle_grouped_proj_w4a8(const uint8_t *Aq, const uint8_t *As, const int32_t *a_row_of, int64_t a_row_div,
                              const uint8_t *Wq, const uint8_t *We, int64_t E, int64_t N, int64_t K,
                              const int32_t *offsets, int silu_mul, double *C)
{
    const int64_t szq = N * (K / 2), sze = N * (K / ORACLE_GROUP);
    const int64_t nout = silu_mul ? N / 2 : N;
    for (int64_t e = 0; e < E; ++e) {
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r) {
            int64_t arow = a_row_of ? a_row_of[r] / a_row_div : r;
            double *a = (double *)malloc(sizeof(double) * (size_t)K);
            double *g = (double *)malloc(sizeof(double) * (size_t)N);
            for (int64_t c = 0; c < K; ++c) a[c] = mx8_at(Aq, As, K, arow, c);
            mx_matvec(Wq + e * szq, We + e * sze, N, K, a, g);
            for (int64_t n = 0; n < nout; ++n) C[r * nout + n] = silu_mul ? silu(g[n]) * g[N / 2 + n] : g[n];
            free(a); free(g);
        }
    }
}
