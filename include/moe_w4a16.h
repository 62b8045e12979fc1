/*
 * libmoe_w4a16 — mixture-of-experts FFN layer with 4-bit (E2M1) expert weights and bf16 activations
 * (W4A16), hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * Pages this interface follows (cited by title and section):
 *   [Atlas] "告别Python堆栈：Atlas用纯Rust重写LLM推理，在GB10上跑赢vLLM",
 *           section "编译时内核选择和W4A16 Grouped GEMM": one launch per projection covering all
 *           experts (gate_up, then down); packed FP4 weights dequantized inside the matmul with no
 *           bf16 weight write-back; a grid sized by the number of row tiles per expert (max_m_tiles).
 *           Section "KV Cache量化、MTP推测解码和调试工具链": missing zero-initialisation and a broken
 *           max_m_tiles heuristic as MoE failure modes (so outputs here never rely on the caller
 *           zeroing them, and tile counts are computed exactly on the device).
 *   [ATOM]  "AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍",
 *           section "8.1 MoE 路径：路由、专家并行与 MORI 通信": routing, top-k selection, expert
 *           compute and the final combine.  Section "8.2 量化并非单一格式，而是一套执行契约": dtype,
 *           scale shape and layout form the kernel's contract.  Section "6.1 Linear：按量化类型分派
 *           GEMM": per-1x32 scaling of 4-bit weights.
 *   [RustDL] "Rust 实现深度学习推理引擎：从计算图到异构硬件加速", section "四、算子融合：性能翻倍的关键":
 *           the activation (SiLU) fused into the producing matmul.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless stated; bf16 values are passed as their uint16_t bits.
 *   - Every device pointer must be 16-byte aligned (128-bit loads) unless stated otherwise.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls only enqueue
 *     work on it and return; there is no host<->device synchronisation.
 *   - The caller allocates and owns every buffer, workspaces included.  The library allocates
 *     nothing, frees nothing and keeps no pointer after a call returns.
 *   - Inputs are read-only.  Outputs are fully overwritten; no zero-initialisation is expected.
 *   - Arguments are validated on the host before anything is launched; a failing call returns a
 *     negative status, launches nothing and records a message for moe_last_error().
 *   - Results are deterministic: identical inputs give identical output bits (no floating-point
 *     atomics).
 *   - Calls that share a workspace or output buffer must not overlap in time.
 *
 * Weight format (the layer's contract)
 *   - Element: E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit; values 0, ±0.5, ±1, ±1.5,
 *     ±2, ±3, ±4, ±6).  Two codes per byte: byte j of a row holds element 2j in bits 0..3 and element
 *     2j+1 in bits 4..7.
 *   - Scale: one bf16 per 32 consecutive K elements of a row.  Weight value = E2M1(code) * scale.
 *   - gate_up weights: codes w13_q [E, 2I, H/2], scales w13_s [E, 2I, H/32]; rows [0, I) are the
 *     gate projection, rows [I, 2I) the up projection.
 *   - down weights: codes w2_q [E, H, I/2], scales w2_s [E, H, I/32].
 *
 * Packed layout (optional, from moe_w4_prepack; same values, same total size): for each block of
 *   16 consecutive rows and 128 consecutive K elements (blocks ordered expert, row block, K block),
 *   1024 bytes of codes in the order the kernel's 64 lanes consume them, then separately 128 bytes
 *   of scales [16 rows][4 groups].  It exists so that each wave-level load is one contiguous block
 *   (the ATOM page, 8.2, lists weight pre-rearrangement as part of a quantized format's contract).
 *   Requires N % 16 == 0 and K % 128 == 0; a gate_up tensor read with SILU_MUL also needs
 *   N % 32 == 0, so that its up rows (from N/2) start a block.  A grouped GEMM gives the same bits
 *   with either layout; the layer does too, except where the packed layout's 128-row tiles take the
 *   exact fp16 path below (canonical weights never do), which agrees within the layer tolerance.
 *
 * Numerics: E2M1 codes are exact in bf16; each 32-element group is reduced by bf16 MFMA into an
 * fp32 partial that is multiplied by the group's scale in fp32; accumulation is fp32.  h (the
 * SiLU-mul output) is stored as bf16 (round to nearest even), the down-projection output as fp16
 * with an in-band power-of-two exponent per row and 8 columns (MOE_OUT_F16E), and the combine sums the k
 * slots in fp32 in slot order before one rounding of y to bf16.  Layers whose experts average more
 * than 256 rows with packed weights (128-row tiles) run the exact fp16 path instead: x in fp16 with a
 * power-of-two exponent per row (moe_x_to_f16), weights formed exactly in fp16 as code * scale and
 * reduced by fp16 MFMA with fp32 accumulation, and h in fp16 with exponents per row and 32 columns
 * (moe_grouped_gemm_w4f16).
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;

#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)       /* NULL pointer, negative size, k > E, bad enum */
#define MOE_ERR_UNSUPPORTED_SHAPE (-2) /* size outside the supported range (see each call) */
#define MOE_ERR_MISALIGNED (-3)        /* a pointer is not 16-byte aligned */
#define MOE_ERR_WORKSPACE (-4)         /* workspace or tile buffer smaller than required */
#define MOE_ERR_HIP (-5)               /* a HIP launch failed */

#define MOE_EPI_NONE 0     /* C[r, n] = sum_k A[row(r), k] * W_e[n, k]                          */
#define MOE_EPI_SILU_MUL 1 /* C[r, j] = silu(G[r, j]) * G[r, N/2 + j], G the NONE result, j < N/2 */

#define MOE_OUT_BF16 0
#define MOE_OUT_F32 1
/* fp16 with an in-band power-of-two exponent per row and 8-column segment: a segment is 8 plain
 * fp16 values (round to nearest even) when its largest finite magnitude m is 0 or in [2^-6, 2^15) and
 * it holds no non-finite value; otherwise it is scaled by 2^-exp, exp = floor(log2 m) - 14 clamped to
 * [-110, 113] (exact), its first element is replaced by a marker, the fp16 quiet NaN
 * 0x7E00 | (exp + 256), and that element's scaled value is written to C_side[row, col / 8] (fp32).
 * Every value of a marked segment is then (fp16 or side value) * 2^exp.  No unmarked segment holds a
 * NaN.  The layer writes the down projection this way: half the bytes of fp32, 3 more significant
 * bits than bf16, and fp32's range. */
#define MOE_OUT_F16E 3
/* SiLU*mul output of moe_grouped_gemm_w4f16: h as fp16 [R_out, N/2] (round to nearest even) with a
 * signed exponent per row and block of 32 columns: row r's values in block j are fp16(h / 2^exp), exp =
 * 0 unless the row's largest finite |h| m in that block is 2^15 or more, or below 2^-6 but not 0 (then
 * exp = floor(log2 m) - 14 clamped to [-110, 113], which scales m into [2^14, 2^15) exactly).  C_aux
 * uint8 [max_tiles, ceil(N/2/32)] flags, per tile and block, whether any row of the tile has a nonzero
 * exponent there; C_aux2 int8 [R_out, ceil(N/2/32)] holds the exponents, written only for flagged
 * blocks. */
#define MOE_OUT_H16 4

#define MOE_LAYOUT_CANONICAL 0 /* the weight format above */
#define MOE_LAYOUT_PACKED 1    /* the same codes and scales re-laid out by moe_w4_prepack */

#define MOE_MAX_EXPERTS 1024

/* Version of this interface (incremented on any incompatible change). */
int32_t moe_abi_version(void);

/* Static text of a status code. */
const char* moe_status_string(moe_status_t status);

/* Text of the most recent failure on the calling host thread ("" if none).  Valid until the
 * thread's next call into the library. */
const char* moe_last_error(void);

/*
 * Top-k routing [ATOM, 8.1]: for each token t, softmax over the E router logits, keep the k
 * largest probabilities and renormalise them to sum to 1.
 *   logits    fp32 [T, E] row-major, finite values.
 *   topk_ids  int32 [T, k] out: expert ids; slot 0 holds the largest logit.  Equal logits are
 *             ordered by lower expert id; the ids of one token are distinct.
 *   topk_w    fp32 [T, k] out: renormalised weights, w_s = exp(l_s - l_0) / sum_j exp(l_j - l_0).
 * Shapes: T >= 0 (T == 0 launches nothing), 1 <= k <= E <= MOE_MAX_EXPERTS.
 * Alignment: 4 bytes suffices for all three pointers.
 */
moe_status_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                            float* topk_w, void* stream);

/*
 * Upper bound on the number of row tiles moe_align can emit: floor(T*k / block_m) + min(E, T*k).
 * Host-only, pure.  Returns -1 for invalid arguments.
 */
int32_t moe_max_tiles(int32_t T, int32_t k, int32_t E, int32_t block_m);

/* Device scratch bytes moe_align needs for these sizes (0 when it runs in one workgroup). */
size_t moe_align_workspace_bytes(int32_t T, int32_t k, int32_t E);

/*
 * Token -> expert permutation (moe_align) [Atlas, 编译时内核选择和W4A16 Grouped GEMM: per-expert
 * row tiles; KV Cache量化…调试工具链: the max_m_tiles failure mode].  A stable counting sort of the
 * R = T*k flat slots f = t*k + s by expert id topk_ids[f]:
 *   expert_counts  int32 [E]    out: rows routed to each expert.
 *   expert_offsets int32 [E+1]  out: exclusive prefix sum of the counts; offsets[E] = R.
 *   sorted_ids     int32 [R]    out: the flat slot at permuted row r; within an expert the slots
 *                               appear in ascending f, experts in ascending id.
 *   inv_perm       int32 [R]    out: permuted row of flat slot f (inverse of sorted_ids).
 *   tiles          int32 [max_tiles, 3] out: (expert, first permuted row, rows <= block_m) for each
 *                               block of up to block_m consecutive rows of one expert, experts
 *                               ascending then rows ascending.  Entries past *num_tiles are unused.
 *   num_tiles      int32 [1]    out: number of tiles written (stays on the device).
 *   workspace      device scratch of at least moe_align_workspace_bytes(T, k, E) bytes (may be
 *                  NULL when that is 0).
 * Shapes: T >= 0, 1 <= k <= E <= MOE_MAX_EXPERTS, 1 <= block_m <= 4096,
 *         max_tiles >= moe_max_tiles(T, k, E, block_m), T*k < 2^26.
 * topk_ids must hold ids in [0, E) with no repeats within a token (as moe_route_topk produces).
 */
moe_status_t moe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_ids,
                       int32_t* inv_perm, int32_t* tiles, int32_t max_tiles, int32_t* num_tiles,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Re-lay out one weight tensor from the canonical layout into the packed layout (see above).
 *   w_q [E, N, K/2], w_s [E, N, K/32] (canonical, device) -> packed_q (E*N*K/2 bytes) and packed_s
 *   (E*N*K/32 bf16), device buffers owned by the caller, not overlapping the inputs.
 * Shapes: 1 <= E <= MOE_MAX_EXPERTS, N >= 16, N % 16 == 0, K >= 128, K % 128 == 0.
 * Alignment: w_q, packed_q 16 bytes; w_s, packed_s 2 bytes (packed_s 8 bytes for use by the GEMMs).
 * Done once per weight tensor (e.g. at load time); every later call can read the packed copy.
 */
moe_status_t moe_w4_prepack(const uint8_t* w_q, const uint16_t* w_s, int32_t E, int32_t N, int32_t K,
                            uint8_t* packed_q, uint16_t* packed_s, void* stream);

/*
 * Grouped W4A16 GEMM, one launch over all experts [Atlas, 编译时内核选择和W4A16 Grouped GEMM].
 * For every tile (e, row0, rows) of `tiles` and every permuted row r in [row0, row0+rows):
 *   a(r) = a_row_of ? a_row_of[r] / a_row_div : r                (activation row)
 *   G[r, n] = sum_{kk<K} A[a(r), kk] * E2M1(Wq[e, n, kk]) * Ws[e, n, kk/32]      (n < N)
 *   MOE_EPI_NONE:     C[r, n] = G[r, n]                                  C is [R_out, N]
 *   MOE_EPI_SILU_MUL: C[r, j] = silu(G[r, j]) * G[r, N/2 + j]            C is [R_out, N/2]
 * with silu(g) = g / (1 + exp(-g)) [RustDL, 四、算子融合].  Rows of C that no tile covers are not
 * written.
 *   A          bf16 [*, K] row-major activations (gate_up: the tokens x, with a_row_of = sorted_ids
 *              and a_row_div = k; down: h in permuted order with a_row_of = NULL).
 *   Wq, Ws     [E, N, K/2] codes and [E, N, K/32] bf16 scales (the weight format above), in
 *              weight_layout MOE_LAYOUT_CANONICAL or MOE_LAYOUT_PACKED (then N % 16 == 0 -- with
 *              SILU_MUL N % 32 == 0 --, K % 128 == 0 and Ws 8-byte aligned).
 *   tiles, num_tiles  as written by moe_align with the same block_m; max_tiles is the capacity
 *              passed to moe_align (it sizes the launch; tiles past *num_tiles cost nothing).
 *   block_m    one of 16, 32, 64, 128.  With block_m 16 and max_tiles <= 32 the four waves of a
 *              workgroup split K (fp32 partial sums added in wave order), so bits can differ from a
 *              call with a larger capacity; both stay within the same error bound, and identical
 *              arguments always give identical bits.
 *   out_dtype  MOE_OUT_BF16 (round to nearest even), MOE_OUT_F32, or (NONE only) MOE_OUT_F16E:
 *              C fp16 [R_out, N] with side values C_side fp32 [R_out, ceil(N/8)] (see
 *              MOE_OUT_F16E; C_side is written only for marked segments, and is ignored for the
 *              other kinds and may then be NULL).  SILU_MUL requires BF16.
 * Shapes: 1 <= E <= MOE_MAX_EXPERTS, N >= 1 (N even for SILU_MUL), K % 32 == 0, K >= 32,
 *         N*K/2 < 4 GiB (one expert's codes).
 * Alignment: A, Wq, C 16 bytes; Ws 2 bytes.
 */
moe_status_t moe_grouped_gemm_w4a16(const uint16_t* A, const int32_t* a_row_of, int32_t a_row_div,
                                    const uint8_t* Wq, const uint16_t* Ws, int32_t weight_layout,
                                    int32_t E, int32_t N,
                                    int32_t K, const int32_t* tiles, int32_t max_tiles,
                                    const int32_t* num_tiles, int32_t block_m, int32_t epilogue,
                                    void* C, int32_t out_dtype, float* C_side, void* stream);

/*
 * Activations for the exact fp16 path of the grouped GEMM (moe_grouped_gemm_w4f16):
 *   x16[t, c] = fp16(x[t, c] * 2^-x_exp[t]) (round to nearest even), x_exp[t] = floor(log2 m) - 14
 *   where m is row t's largest finite |x| (x_exp = 0 for an all-zero row; clamped to [-110, 113]).
 * The row's largest magnitude lands in [2^14, 2^15): every value at most 2^31 below it is exact in
 * fp16; non-finite values stay non-finite.
 *   x bf16 [T, H]; x16 fp16 [T, H]; x_exp int32 [T].  Shapes: T >= 0, H % 8 == 0.
 */
moe_status_t moe_x_to_f16(const uint16_t* x, int32_t T, int32_t H, uint16_t* x16, int32_t* x_exp, void* stream);

/*
 * Grouped W4A16 GEMM, exact fp16 form [Atlas, 编译时内核选择和W4A16 Grouped GEMM: dequantization inside
 * the matmul]: the same result as moe_grouped_gemm_w4a16 with activations given in fp16 with power-
 * of-two exponents.  Each weight E2M1(code) * scale is formed in fp16, exact when the bf16 scale has
 * an exponent in [-16, 12], so every product is exact and the fp32 MFMA accumulation carries the group
 * scales with it.  A K step holding any other scale (zero, subnormal, non-finite, out of that range),
 * or h blocks with exponents, takes a general form: the scale is split into an fp16-exact part and a
 * power of two, and the fp32 accumulators are scaled by that power of two (exactly) around each group.
 *   A          fp16 [*, K]: with a_row_of (gathered rows, e.g. x16 of moe_x_to_f16) activation row a
 *              is A[a] * 2^a_row_exp[a] (a_row_exp NULL: exponents 0); with a_row_of NULL (h of the
 *              previous SILU_MUL call, with its two exponent arrays as a_blk_flag and a_row_blk_exp)
 *              row r's values in K columns [32j, 32j+32) are A * 2^a_row_blk_exp[r * ceil(K/32) + j]
 *              when a_blk_flag[i * ceil(K/32) + j] is nonzero for r's tile i, else A (a_blk_flag
 *              NULL: no exponents).
 *   block_m    64, or 128 with MOE_LAYOUT_PACKED weights (the tile list of moe_align with it).
 *   epilogue   MOE_EPI_SILU_MUL with out_dtype MOE_OUT_H16 (C fp16 [R_out, N/2], C_aux and C_aux2 the
 *              exponent flags and exponents, see MOE_OUT_H16), or MOE_EPI_NONE with MOE_OUT_F32 (C
 *              fp32) or MOE_OUT_F16E (C fp16, C_aux fp32 side values [R_out, ceil(N/8)]); C_aux2 is
 *              used by SILU_MUL only.
 * Other arguments, shapes and alignment as for moe_grouped_gemm_w4a16.
 */
moe_status_t moe_grouped_gemm_w4f16(const uint16_t* A, const int32_t* a_row_exp, const uint8_t* a_blk_flag,
                                    const uint8_t* a_row_blk_exp, const int32_t* a_row_of, int32_t a_row_div,
                                    const uint8_t* Wq, const uint16_t* Ws, int32_t weight_layout, int32_t E, int32_t N,
                                    int32_t K, const int32_t* tiles, int32_t max_tiles, const int32_t* num_tiles,
                                    int32_t block_m, int32_t epilogue, void* C, int32_t out_dtype, void* C_aux,
                                    uint8_t* C_aux2, void* stream);

/*
 * Routing-weighted scatter-reduce (combine) [ATOM, 8.1]:
 *   y[t, c] = bf16( sum_{s=0}^{k-1} topk_w[t, s] * O[inv_perm[t*k + s], c]  (+ shared[t, c]) )
 * summed in fp32 in ascending slot order, then the shared term (if any) added, rounded once to bf16.
 *   O          expert outputs in permuted row order, [T*k, H]: o_dtype MOE_OUT_F32 (fp32, O_side
 *              ignored) or MOE_OUT_F16E (fp16 with in-band exponents and side values O_side fp32
 *              [T*k, H/8], the down projection's output kind in the layer; each value decodes
 *              exactly to fp32);
 *   inv_perm int32 [T*k]; topk_w fp32 [T, k]; shared fp32 [T, H] or NULL (the shared-expert output
 *   of moe_dense_ffn_w4a16, added with weight 1 [Atlas, KV Cache量化、MTP推测解码和调试工具链]);
 *   y bf16 [T, H] out.
 * Shapes: T >= 0, k >= 1, H % 8 == 0.
 */
moe_status_t moe_combine(const void* O, int32_t o_dtype, const float* O_side, const int32_t* inv_perm,
                         const float* topk_w, const float* shared, int32_t T, int32_t k, int32_t H, uint16_t* y,
                         void* stream);

/*
 * Router gate logits [Atlas, KV Cache量化、MTP推测解码和调试工具链: the gate input and the gate logits
 * of each MoE layer; ATOM, 8.1: the logits the top-k routing reads]:
 *   logits[t, e] = sum_h x[t, h] * w_router[e, h], bf16 products accumulated in fp32 (MFMA order,
 *   so not bit-identical to another summation order).
 *   x bf16 [T, H]; w_router bf16 [E, H]; logits fp32 [T, E] out (4-byte aligned).
 * Shapes: 0 <= T < 2^26 (T == 0 launches nothing), 1 <= E <= MOE_MAX_EXPERTS, H % 32 == 0, H >= 32.
 */
moe_status_t moe_router_logits(const uint16_t* x, const uint16_t* w_router, int32_t T, int32_t H, int32_t E,
                               float* logits, void* stream);

/* Workspace bytes moe_dense_ffn_w4a16 needs (host-only, pure; 0 on invalid sizes). */
size_t moe_dense_ffn_workspace_bytes(int32_t T, int32_t H, int32_t I);

/*
 * Dense W4A16 SwiGLU FFN: one expert applied to every token (the shared expert of an MoE block
 * [Atlas, KV Cache量化、MTP推测解码和调试工具链]), on the same grouped-GEMM kernels with every row in
 * one group:
 *   out[t] = W2 ( silu(W1 x[t]) * (W3 x[t]) ), h rounded to bf16 between the projections.
 *   x bf16 [T, H]; w13_q [2I, H/2], w13_s [2I, H/32], w2_q [H, I/2], w2_s [H, I/32] in the weight
 *   format above (one expert, E = 1), all in weight_layout; out fp32 [T, H].
 *   workspace: device scratch of at least moe_dense_ffn_workspace_bytes(T, H, I) bytes (holds h).
 * Shapes: T >= 0 (T == 0 launches nothing), H and I positive multiples of 32 (of 128 when packed),
 *         T < 2^26.
 */
moe_status_t moe_dense_ffn_w4a16(const uint16_t* x, int32_t T, int32_t H, int32_t I, const uint8_t* w13_q,
                                 const uint16_t* w13_s, const uint8_t* w2_q, const uint16_t* w2_s,
                                 int32_t weight_layout, float* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Row-tile height (block_m) moe_ffn_forward uses for these sizes and weight layout (host-only,
 * pure; -1 on invalid sizes or layout).  Lets a caller run the same launch configuration through
 * the separate entry points.  moe_ffn_workspace_bytes covers every layout's choice. */
int32_t moe_ffn_block_m(int32_t T, int32_t E, int32_t k, int32_t weight_layout);

/* Workspace bytes moe_ffn_forward needs for these sizes (host-only, pure; 0 on invalid sizes). */
size_t moe_ffn_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);

/*
 * The whole MoE FFN layer [ATOM, 8.1; Atlas, 编译时内核选择和W4A16 Grouped GEMM]:
 *   route (moe_route_topk) -> permute (moe_align) -> gate_up grouped GEMM with SiLU*mul fused
 *   -> down grouped GEMM -> combine, all enqueued on `stream`:
 *   y[t] = sum_s w[t,s] * W2_e(s) ( silu(W1_e(s) x[t]) * (W3_e(s) x[t]) ),  e(s) = topk_ids[t, s].
 *   x bf16 [T, H]; router_logits fp32 [T, E]; weights in the format above, all four tensors in
 *   weight_layout (MOE_LAYOUT_PACKED needs H % 128 == 0 and I % 128 == 0); y bf16 [T, H] out.
 *   topk_ids_out int32 [T, k], topk_w_out fp32 [T, k]: optional copies of the routing (NULL = skip).
 *   workspace: device scratch of at least moe_ffn_workspace_bytes(T, H, I, E, k) bytes.
 * Shapes: T >= 0 (T == 0 launches nothing), 1 <= k <= E <= MOE_MAX_EXPERTS, H % 32 == 0,
 *         I % 32 == 0, H >= 32, I >= 32, T*k < 2^26, H*I < 4 GiB (one expert's gate_up codes).
 * Diagnostics: with MOE_DUMP=1 in the environment (read on every call), the call then synchronises
 *   `stream` and prints one line to stderr: shape, tile height and count, rows per expert (least,
 *   most, experts without rows), most tiles of one expert, the ten largest logits of token 0 and
 *   the L2 norms of x and y [Atlas, KV Cache量化、MTP推测解码和调试工具链: per-layer expert-id dump].
 *   Results are unchanged; nothing is printed for a stream under graph capture; a failing copy
 *   returns MOE_ERR_HIP.  moe_ffn_block_forward does the same; moe_ffn_forward_noalloc never dumps.
 */
moe_status_t moe_ffn_forward(const uint16_t* x, const float* router_logits, int32_t T, int32_t H,
                             int32_t I, int32_t E, int32_t k, const uint8_t* w13_q,
                             const uint16_t* w13_s, const uint8_t* w2_q, const uint16_t* w2_s,
                             int32_t weight_layout, uint16_t* y, int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch array that moe_ffn_forward_noalloc works in (64 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t moe_ffn_noalloc_scratch_bytes(void);

/*
 * moe_ffn_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments, layouts, results and
 * errors as moe_ffn_forward minus the workspace: the intermediate buffers (routing, permutation,
 * tile list, h, O) live in one static device array of MOE_NOALLOC_SCRATCH_BYTES inside the library.
 * The call allocates nothing (no hipMalloc, no allocating library routine) and launches exactly the
 * kernels moe_ffn_forward launches, so its outputs are bit-identical to moe_ffn_forward's.
 *   - Limit: sizes whose moe_ffn_workspace_bytes exceeds MOE_NOALLOC_SCRATCH_BYTES are rejected with
 *     MOE_ERR_WORKSPACE before anything touches the device (the 800-token, 256-expert, H = 2048,
 *     I = 512 layer needs about 39 MB; every decode batch of a few hundred tokens fits).
 *   - Each GPU holds its own copy of the array from the first call on that device (the calling
 *     thread's current device, which `stream` must belong to) until the process ends.
 *   - All calls on one GPU share that GPU's array: calls that overlap in time on one GPU (two streams,
 *     two host threads) race and must be serialised by the caller.
 */
moe_status_t moe_ffn_forward_noalloc(const uint16_t* x, const float* router_logits, int32_t T, int32_t H, int32_t I,
                                     int32_t E, int32_t k, const uint8_t* w13_q, const uint16_t* w13_s,
                                     const uint8_t* w2_q, const uint16_t* w2_s, int32_t weight_layout, uint16_t* y,
                                     int32_t* topk_ids_out, float* topk_w_out, void* stream);

/* Workspace bytes moe_ffn_block_forward needs (host-only, pure; 0 on invalid sizes).  Is = 0 means
 * no shared expert. */
size_t moe_ffn_block_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t Is);

/*
 * The whole MoE block from the hidden states [Atlas, KV Cache量化、MTP推测解码和调试工具链: gate input,
 * gate logits, routed output and shared-expert output of a layer]:
 *   logits = moe_router_logits(x, w_router); (when Is > 0) s = moe_dense_ffn_w4a16(x, shared weights);
 *   y = moe_ffn_forward(x, logits, ...) with s added in the combine (weight 1).
 *   w_router bf16 [E, H]; the routed weights as for moe_ffn_forward; Is = shared-expert intermediate
 *   size (0 = none, the four shared pointers are then ignored), shared weights w13s_q [2Is, H/2],
 *   w13s_s [2Is, H/32], w2s_q [H, Is/2], w2s_s [H, Is/32] in weight_layout.
 *   logits_out fp32 [T, E], topk_ids_out int32 [T, k], topk_w_out fp32 [T, k]: optional copies
 *   (NULL = skip).  workspace: at least moe_ffn_block_workspace_bytes(T, H, I, E, k, Is) bytes.
 * Shapes: those of moe_ffn_forward; Is >= 0, and Is > 0 follows the rules for I.
 */
moe_status_t moe_ffn_block_forward(const uint16_t* x, const uint16_t* w_router, int32_t T, int32_t H, int32_t I,
                                   int32_t E, int32_t k, const uint8_t* w13_q, const uint16_t* w13_s,
                                   const uint8_t* w2_q, const uint16_t* w2_s, int32_t Is, const uint8_t* w13s_q,
                                   const uint16_t* w13s_s, const uint8_t* w2s_q, const uint16_t* w2s_s,
                                   int32_t weight_layout, uint16_t* y, float* logits_out, int32_t* topk_ids_out,
                                   float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ---- MXFP4 (W4A4) variant ------------------------------------------------------------------------
 * [ATOM, 6.1: per-1x32 MXFP4 served by an a4w4 GEMM; ATOM, 8.2: dynamic activation quantization is
 * part of a format's contract.]  Weights and activations are E2M1 codes (as above) with one E8M0
 * scale byte per 32 consecutive K elements: value = E2M1(code) * 2^(byte - 127) (byte 255 = NaN is
 * not accepted in weights).  Activations are quantized on the fly, per row and block of 32, by the
 * OCP MX conversion: X = 2^(floor(log2(max |v|)) - 2) clamped to [2^-127, 2^127] (an all-zero block
 * takes byte 0), code = nearest E2M1 value of v / X, ties to the even code, saturating at +-6.
 * Products run on the gfx950 scaled FP4 matrix instruction with fp32 accumulation.
 */

/* x bf16 [rows, K] -> codes q [rows, K/2] and scale bytes s [rows, K/32] (MX conversion above).
 * Shapes: 0 <= rows < 2^26, K a positive multiple of 32.  x and q 16-byte aligned. */
moe_status_t moe_mx_quantize(const uint16_t* x, int32_t rows, int32_t K, uint8_t* q, uint8_t* s, void* stream);

/* Activation layouts of the MXFP4 GEMM. */
#define MOE_ACT_ROWS 0   /* row-major [*, K/2] codes and [*, K/32] scales, rows gathered through a_row_of */
#define MOE_ACT_TILED 1  /* tile-blocked: the tile list's rows, tile by tile, in the packed block order */

/*
 * Packed MXFP4 weight layout (same bytes, MFMA lane order): the [E, N, K] matrix cut into blocks of
 * 16 rows x 128 K elements ordered (expert, row block, K block), K fastest; per block 1024 bytes of
 * codes (bytes [16l, 16l+16) = row l % 16, K elements [32 (l / 16), +32)) and, separately, 64 scale
 * bytes (byte l = the same row and 32-block).  w_q [E, N, K/2], w_e [E, N, K/32] canonical in,
 * packed_q / packed_e of the same sizes out.  Needs N % 16 == 0, K % 128 == 0 [ATOM, 8.2: weight
 * pre-rearrangement is part of a quantized format's contract].
 */
moe_status_t moe_mx_prepack(const uint8_t* w_q, const uint8_t* w_e, int32_t E, int32_t N, int32_t K, uint8_t* packed_q,
                            uint8_t* packed_e, void* stream);

/*
 * x quantized (as moe_mx_quantize) and gathered into the tile-blocked activation layout of a tile
 * list: tile t's rows r = tiles[t].row0 + i (i < tiles[t].rows), source row a_row_of[r] / a_row_div
 * (or r), padded to block_m rows; blocks of 16 rows x 128 K ordered (tile, 16-row group, K block) with
 * K fastest, each 1024 code bytes in the packed lane order plus 64 scale bytes.  Padding rows and
 * tiles past *num_tiles are left unwritten.  q: max_tiles * block_m * K/2 bytes, s: max_tiles *
 * block_m * K/32 bytes.  Needs K % 128 == 0, block_m 16, 32 or 64.
 */
moe_status_t moe_mx_quantize_tiles(const uint16_t* x, int32_t T, int32_t K, const int32_t* a_row_of,
                                  int32_t a_row_div, const int32_t* tiles, int32_t max_tiles, const int32_t* num_tiles,
                                  int32_t block_m, uint8_t* q, uint8_t* s, void* stream);

/*
 * Grouped MXFP4 GEMM over the tile list of moe_align [Atlas, 编译时内核选择和W4A16 Grouped GEMM: one
 * launch over all experts]: for each permuted row r of expert e, activation row
 * a = (a_row_of ? a_row_of[r] / a_row_div : r):
 *   G[r, n] = sum_k A[a, k] * W_e[n, k],  A = (Aq [*, K/2], As [*, K/32]), W = (Wq [E, N, K/2], We [E, N, K/32]).
 *   epilogue NONE:     C [rows, N] fp32 or bf16 (out_dtype); Cs unused.
 *   epilogue SILU_MUL: h[r, j] = silu(G[r, j]) * G[r, N/2 + j] in fp32, then quantized per 32 columns:
 *                      C = codes [rows, N/4], Cs = scale bytes [rows, N/64] (out_dtype ignored).
 * weight_layout: MOE_LAYOUT_CANONICAL or MOE_LAYOUT_PACKED (moe_mx_prepack; needs N % 16 == 0 and
 * K % 128 == 0).  act_layout: MOE_ACT_ROWS, or MOE_ACT_TILED (packed weights only; A from
 * moe_mx_quantize_tiles or a previous SILU_MUL output, a_row_of unused; a SILU_MUL output is then
 * written tile-blocked too, for K = N/2 of the next projection, which needs N/2 % 128 == 0).
 * Results are bit-identical across layouts.  block_m 16, 32, 64 or 128 (the tile height moe_align
 * used); 128 runs a 128 x 256 LDS-staged kernel (bit-identical to the others) that needs
 * K % 128 == 0, MOE_ACT_ROWS and 4-byte aligned As and We.  K % 32 == 0; SILU_MUL needs N % 64 == 0.
 */
moe_status_t moe_grouped_gemm_mxfp4(const uint8_t* Aq, const uint8_t* As, const int32_t* a_row_of, int32_t a_row_div,
                                    const uint8_t* Wq, const uint8_t* We, int32_t weight_layout, int32_t act_layout,
                                    int32_t E, int32_t N, int32_t K,
                                    const int32_t* tiles, int32_t max_tiles, const int32_t* num_tiles, int32_t block_m,
                                    int32_t epilogue, void* C, uint8_t* Cs, int32_t out_dtype, void* stream);

/* Row-tile height and workspace bytes of moe_ffn_forward_mxfp4 (host-only, pure; -1 / 0 on invalid sizes). */
int32_t moe_ffn_mxfp4_block_m(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);
size_t moe_ffn_mxfp4_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);

/*
 * The whole MXFP4 (W4A4) layer [ATOM, 6.1 and 8.1-8.2]: route -> permute -> x quantized -> gate_up
 * (SiLU*mul, h quantized in the epilogue) -> down (fp32) -> combine, all enqueued on `stream`:
 *   y[t] = sum_s w[t,s] * W2_e(s) Q( silu(W1_e(s) Q(x[t])) * (W3_e(s) Q(x[t])) ),  Q = MX quantization.
 *   x bf16 [T, H]; router_logits fp32 [T, E]; w13_q [E, 2I, H/2], w13_e [E, 2I, H/32],
 *   w2_q [E, H, I/2], w2_e [E, H, I/32], all four in weight_layout (MOE_LAYOUT_PACKED from
 *   moe_mx_prepack needs H % 128 == 0 and I % 128 == 0; the quantized activations are then kept in
 *   the same blocked order internally; results are bit-identical to the canonical layout);
 *   y bf16 [T, H].  Optional routing copies as for moe_ffn_forward.  With experts of more than 128
 *   rows on average (and H, I multiples of 128) the 128-row kernel runs, on row-major activations,
 *   and the scale arrays need 4-byte alignment.
 *   workspace: at least moe_ffn_mxfp4_workspace_bytes(T, H, I, E, k) bytes (either layout).
 * Shapes: as moe_ffn_forward (H, I positive multiples of 32).
 */
moe_status_t moe_ffn_forward_mxfp4(const uint16_t* x, const float* router_logits, int32_t T, int32_t H, int32_t I,
                                   int32_t E, int32_t k, const uint8_t* w13_q, const uint8_t* w13_e,
                                   const uint8_t* w2_q, const uint8_t* w2_e, int32_t weight_layout, uint16_t* y,
                                   int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * ---- W4A8 variant (MXFP8 activations on the MXFP4 weights) -----------------------------------------
 * [ATOM, 6.1: the MX formats served by the scaled-instruction GEMMs; ATOM, 8.2: dynamic activation
 * quantization is part of a format's contract.]  Weights exactly as the MXFP4 variant (either layout,
 * the same moe_mx_prepack).  Activations are MXFP8: OCP FP8 E4M3 codes (one byte per element; 1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, largest finite 448) with one E8M0 scale byte per 32
 * consecutive K elements: value = E4M3(code) * 2^(byte - 127).  Quantization per row and block of 32:
 * X = 2^(floor(log2(max |v|)) - 8) clamped to [2^-127, 2^127] (an all-zero block takes byte 0), code =
 * nearest E4M3 value of v / X, ties to the even code, saturating at +-448.  Products run on the gfx950
 * scaled matrix instruction with E4M3 x E2M1 operands and fp32 accumulation.
 */

/* x bf16 [rows, K] -> codes q [rows, K] and scale bytes s [rows, K/32] (MXFP8 conversion above).
 * Shapes: 0 <= rows < 2^26, K a positive multiple of 32.  x and q 16-byte aligned. */
moe_status_t moe_mx8_quantize(const uint16_t* x, int32_t rows, int32_t K, uint8_t* q, uint8_t* s, void* stream);

/*
 * x quantized to MXFP8 (as moe_mx8_quantize) and gathered into the tile-blocked layout of a tile list
 * (rows as for moe_mx_quantize_tiles): blocks of 16 rows x 128 K ordered (tile, 16-row group, K block),
 * K fastest, each 2048 code bytes in the instruction's 8-bit lane order with the halves apart: bytes
 * [16l, 16l+16) = row l % 16, K [16 (l / 16), +16) of the block; bytes [1024 + 16l, +16) = the same row,
 * K [64 + 16 (l / 16), +16); and, separately, 64 scale bytes (byte l = row l % 16, 32-block l / 16).
 * Padding rows and tiles past *num_tiles are left unwritten.  q: max_tiles * block_m * K bytes, s:
 * max_tiles * block_m * K/32 bytes.  Needs K % 128 == 0, block_m 16, 32 or 64.
 */
moe_status_t moe_mx8_quantize_tiles(const uint16_t* x, int32_t T, int32_t K, const int32_t* a_row_of,
                                   int32_t a_row_div, const int32_t* tiles, int32_t max_tiles, const int32_t* num_tiles,
                                   int32_t block_m, uint8_t* q, uint8_t* s, void* stream);

/*
 * Grouped W4A8 GEMM over the tile list of moe_align (as moe_grouped_gemm_mxfp4): for each permuted
 * row r of expert e, activation row a = (a_row_of ? a_row_of[r] / a_row_div : r):
 *   G[r, n] = sum_k A[a, k] * W_e[n, k],  A = (Aq [*, K] E4M3 codes, As [*, K/32]), W = (Wq [E, N, K/2], We [E, N, K/32]).
 *   epilogue NONE:     C [rows, N] fp32 or bf16 (out_dtype); Cs unused.
 *   epilogue SILU_MUL: h[r, j] = silu(G[r, j]) * G[r, N/2 + j] in fp32, then quantized to MXFP8 per 32
 *                      columns: C = codes [rows, N/2], Cs = scale bytes [rows, N/64] (out_dtype ignored).
 * weight_layout: MOE_LAYOUT_CANONICAL or MOE_LAYOUT_PACKED (moe_mx_prepack; needs N % 16 == 0 and
 * K % 128 == 0).  act_layout: MOE_ACT_ROWS, or MOE_ACT_TILED (packed weights and block_m <= 64; A from
 * moe_mx8_quantize_tiles or a previous SILU_MUL output, a_row_of unused; a SILU_MUL output is then
 * written tile-blocked too, which needs N/2 % 128 == 0).  Results are bit-identical across layouts.
 * block_m 16, 32, 64 or 128 (the tile height moe_align used); 128 runs a 128 x 256 LDS-staged kernel
 * (bit-identical to the others) that needs K % 128 == 0, MOE_ACT_ROWS and 4-byte aligned As and We.
 * K % 32 == 0; SILU_MUL needs N % 64 == 0.  Aq, Wq and C 16-byte aligned.
 */
moe_status_t moe_grouped_gemm_w4a8(const uint8_t* Aq, const uint8_t* As, const int32_t* a_row_of, int32_t a_row_div,
                                   const uint8_t* Wq, const uint8_t* We, int32_t weight_layout, int32_t act_layout,
                                   int32_t E, int32_t N, int32_t K, const int32_t* tiles, int32_t max_tiles,
                                   const int32_t* num_tiles, int32_t block_m, int32_t epilogue, void* C, uint8_t* Cs,
                                   int32_t out_dtype, void* stream);

/* Row-tile height and workspace bytes of moe_ffn_forward_w4a8 (host-only, pure; -1 / 0 on invalid sizes):
 * the MXFP4 layer's choice (128 for experts averaging more than 128 rows with H, I multiples of 128). */
int32_t moe_ffn_w4a8_block_m(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);
size_t moe_ffn_w4a8_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);

/*
 * The whole W4A8 layer [ATOM, 6.1 and 8.1-8.2]: route -> permute -> x quantized to MXFP8 -> gate_up
 * (SiLU*mul, h quantized to MXFP8 in the epilogue) -> down (fp32) -> combine, all enqueued on `stream`:
 *   y[t] = sum_s w[t,s] * W2_e(s) Q8( silu(W1_e(s) Q8(x[t])) * (W3_e(s) Q8(x[t])) ),  Q8 = MXFP8 quantization.
 *   Arguments as moe_ffn_forward_mxfp4 (the same MXFP4 weights in either layout; packed needs
 *   H % 128 == 0 and I % 128 == 0, results bit-identical to the canonical layout); y bf16 [T, H].
 *   With packed weights the quantized activations are kept tile-blocked internally.  With experts of
 *   more than 128 rows on average (and H, I multiples of 128) the 128-row kernel runs, on row-major
 *   activations, and the scale arrays need 4-byte alignment.
 *   workspace: at least moe_ffn_w4a8_workspace_bytes(T, H, I, E, k) bytes.
 * Shapes: as moe_ffn_forward (H, I positive multiples of 32).
 */
moe_status_t moe_ffn_forward_w4a8(const uint16_t* x, const float* router_logits, int32_t T, int32_t H, int32_t I,
                                  int32_t E, int32_t k, const uint8_t* w13_q, const uint8_t* w13_e,
                                  const uint8_t* w2_q, const uint8_t* w2_e, int32_t weight_layout, uint16_t* y,
                                  int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * ---- FP8 (W8A8, per-1x128) variant ----------------------------------------------------------------
 * [ATOM, 6.1: per-1x128 FP8 served by an a8w8 block-scale GEMM; ATOM, 8.1: the FP8 path of the fused
 * MoE; ATOM, 8.2: dynamic activation quantization is part of a format's contract.]  Weights and
 * activations are OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent
 * field 0 subnormal; largest finite 448; the NaN codes 0x7F / 0xFF are not accepted in weights), one
 * byte per element, rows K-contiguous, with one fp32 scale per row and block of 128 consecutive K
 * elements: value = E4M3(code) * scale.  Activations are quantized on the fly, per row and block:
 * s = max |v| / 448 (fp32 division), code = the E4M3 value nearest to the fp32 quotient v / s, ties to
 * the even code; an all-zero block gets s = 0 and codes 0.  Products run on the gfx950 FP8 matrix
 * instruction, one 128-element K block per instruction, whose fp32 partial is multiplied by the two
 * block scales in fp32; accumulation is fp32.
 */
#define MOE_IN_BF16 0
#define MOE_IN_F32 1
#define MOE_OUT_F8 2  /* SILU_MUL output of moe_grouped_gemm_f8 quantized per 1x128 (codes + fp32 scales) */

/* x [rows, K] (bf16 bits, or fp32 with in_dtype MOE_IN_F32) -> codes q [rows, K] and fp32 scales
 * s [rows, K/128] (the conversion above).  Shapes: 0 <= rows < 2^26, K a positive multiple of 128.
 * Alignment: x and q 16 bytes, s 4 bytes. */
moe_status_t moe_f8_quantize(const void* x, int32_t in_dtype, int32_t rows, int32_t K, uint8_t* q, float* s,
                             void* stream);

/*
 * Grouped FP8 GEMM over the tile list of moe_align [Atlas, 编译时内核选择和W4A16 Grouped GEMM: one
 * launch over all experts]: for each permuted row r of expert e, activation row
 * a = (a_row_of ? a_row_of[r] / a_row_div : r):
 *   G[r, n] = sum_k A[a, k] * W_e[n, k],  A = (Aq [*, K], As [*, K/128]), W = (Wq [E, N, K], Ws [E, N, K/128]).
 *   epilogue NONE:     C [rows, N], fp32 or bf16 (out_dtype).
 *   epilogue SILU_MUL: h[r, j] = silu(G[r, j]) * G[r, N/2 + j] in fp32, stored as
 *                      out_dtype MOE_OUT_F32: C [rows, N/2] fp32 (moe_f8_quantize then quantizes it), or
 *                      out_dtype MOE_OUT_F8: quantized in the epilogue exactly as moe_f8_quantize would,
 *                      C = codes [rows, N/2], Cs = fp32 scales [rows, N/256]; needs block_m 128 and
 *                      N/2 % 128 == 0.  Cs is unused (may be NULL) for the other output types.
 * Rows of C that no tile covers are not written.  block_m 16, 32, 64 or 128 (the tile height
 * moe_align used).  With block_m 16 or 32 the waves of a workgroup split K (four ways when block_m
 * is 16 and max_tiles <= 32, else two) and add their fp32 partials in wave order, so bits can
 * differ between tile heights and capacities; identical arguments always give identical bits.
 * 128 runs a 128 x 256 LDS-staged kernel, bit-identical to the 64-row one.
 * Shapes: 1 <= E <= MOE_MAX_EXPERTS, N >= 1 (N even for SILU_MUL), K a positive multiple of 128,
 *         K <= 32768.  Alignment: Aq, Wq, C 16 bytes; As, Ws 4 bytes.
 */
moe_status_t moe_grouped_gemm_f8(const uint8_t* Aq, const float* As, const int32_t* a_row_of, int32_t a_row_div,
                                 const uint8_t* Wq, const float* Ws, int32_t E, int32_t N, int32_t K,
                                 const int32_t* tiles, int32_t max_tiles, const int32_t* num_tiles, int32_t block_m,
                                 int32_t epilogue, void* C, float* Cs, int32_t out_dtype, void* stream);

/* Row-tile height and workspace bytes of moe_ffn_forward_f8 (host-only, pure; -1 / 0 on invalid sizes). */
int32_t moe_ffn_f8_block_m(int32_t T, int32_t E, int32_t k);
size_t moe_ffn_f8_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);

/*
 * The whole FP8 (W8A8, per-1x128) layer [ATOM, 6.1 and 8.1-8.2]: route -> permute -> x quantized ->
 * gate_up (SiLU*mul, h in fp32) -> h quantized (in the gate_up epilogue with 128-row tiles) -> down
 * (fp32) -> combine, all enqueued on `stream`:
 *   y[t] = sum_s w[t,s] * W2_e(s) Q( silu(W1_e(s) Q(x[t])) * (W3_e(s) Q(x[t])) ),  Q = FP8 quantization.
 *   x bf16 [T, H]; router_logits fp32 [T, E]; w13_q [E, 2I, H], w13_s [E, 2I, H/128] fp32,
 *   w2_q [E, H, I], w2_s [E, H, I/128] fp32; y bf16 [T, H].  Optional routing copies as for
 *   moe_ffn_forward.  workspace: at least moe_ffn_f8_workspace_bytes(T, H, I, E, k) bytes.
 * Shapes: as moe_ffn_forward, with H and I positive multiples of 128, H and I <= 32768.
 */
moe_status_t moe_ffn_forward_f8(const uint16_t* x, const float* router_logits, int32_t T, int32_t H, int32_t I,
                                int32_t E, int32_t k, const uint8_t* w13_q, const float* w13_s, const uint8_t* w2_q,
                                const float* w2_s, uint16_t* y, int32_t* topk_ids_out, float* topk_w_out,
                                void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
