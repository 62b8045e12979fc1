// Internal host-side launchers (one per kernel family).  Each enqueues on `stream` and returns the
// launch status; argument validation happens in the C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_w4a16.h"

namespace moe {

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, int T, int H, int E, float* logits,
                                hipStream_t stream);
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t stream);

// Single-workgroup permutation: up to kAlignSingleMaxR slots and kAlignSingleMaxE experts (static
// LDS: 16 per-wave count rows, the staged permutation and 16 per-wave peer tables).
constexpr int kAlignSingleMaxR = 8192;
constexpr int kAlignSingleMaxE = 512;
inline bool align_single_fits(int R, int E) { return R <= kAlignSingleMaxR && E <= kAlignSingleMaxE; }
// Routing and permutation of a small batch in one single-workgroup launch: up to 16 tokens (one
// wave each), k <= kFusedMaxK, T * k <= kFusedMaxR, E <= kAlignSingleMaxE.
constexpr int kFusedMaxT = 16;
constexpr int kFusedMaxK = 64;
constexpr int kFusedMaxR = 1024;
inline bool route_align_fused_fits(int T, int E, int k) {
  return T >= 1 && T <= kFusedMaxT && k <= kFusedMaxK && T * k <= kFusedMaxR && E <= kAlignSingleMaxE;
}
hipError_t launch_route_align_small(const float* logits, int T, int E, int k, int block_m, int32_t* topk_ids,
                                   float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                                   int32_t* inv_perm, int32_t* tiles, int max_tiles, int32_t* num_tiles,
                                   hipStream_t stream);
// Flat slots per workgroup in the multi-workgroup permutation.
constexpr int kAlignChunk = 4096;
size_t align_workspace_bytes(int R, int E);
hipError_t launch_align(const int32_t* ids, int R, int E, int block_m, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_ids, int32_t* inv_perm, int32_t* tiles,
                        int max_tiles, int32_t* num_tiles, void* workspace, hipStream_t stream);

struct GemmArgs {
  const uint16_t* A;       // bf16 activations [*, K]
  const int32_t* a_row_of; // permuted row -> flat index (NULL = identity)
  int a_row_div;           // activation row = a_row_of[r] / a_row_div
  const uint8_t* Wq;       // [E, N, K/2]
  const uint16_t* Ws;      // [E, N, K/32]
  int N, K;
  const int32_t* tiles;    // [max_tiles, 3]; NULL = dense mode (one expert, rows 0..dense_rows)
  const int32_t* num_tiles;
  int max_tiles;
  int dense_rows;          // dense mode: tile i covers rows [i * BM, min((i + 1) * BM, dense_rows)) of expert 0
  void* C;
  int epilogue;            // MOE_EPI_*
  int out_f32;             // NONE epilogue: 0 bf16, 1 fp32, 2 fp16 with in-band exponents (C_side)
  int packed;              // weights in the prepacked kernel layout (prepack.hip)
  // Shared expert run in the same launch (NULL = none): one more expert with weights [N, K/2] and
  // [N, K/32] (same layout as Wq / Ws), applied to shared_rows rows whose output rows start at
  // shared_row0.  Its tiles follow the routed ones.  Its activation rows are the output rows
  // themselves when a_row_of is NULL, else the token index (output row - shared_row0).
  const uint8_t* Wq_sh;
  const uint16_t* Ws_sh;
  int shared_rows;
  int shared_row0;
  int a_row_sub;           // per-tile view only (set by the kernels; callers leave it 0)
  // Routing prologue (SiLU*mul launch with 16-row tiles, route_prologue_fits; route_logits NULL = off):
  // every workgroup routes the batch from the router logits and builds its own tile list entry and
  // row gather in LDS instead of reading tiles / num_tiles / a_row_of; it writes what the later
  // launches read: the tile list and its length, the permutation (sorted_ids, inv_perm) and the
  // routing (ids, weights).  Expert counts and offsets are not written.
  const float* route_logits;  // [T, E]
  int route_T, route_E, route_k;
  int32_t* route_ids;         // [T, k]
  float* route_w;             // [T, k]
  int32_t* route_tiles;       // [max_tiles, 3]
  int32_t* route_num_tiles;
  int32_t* route_sorted;      // [T * k]
  int32_t* route_inv;         // [T * k]
  // out_f32 == 2: fp32 values of the marked elements, [rows, ceil(N / 8)] (see kOutF16Exp)
  float* C_side;
  // The exact fp16 path (64- and 128-row tile kernels; a_f16 != 0): A holds fp16 values.
  //  * Gathered rows (a_row_of set, or the shared expert's token rows): activation row a is
  //    A[a] * 2^a_row_exp[a] (launch_x_to_f16); the row sums are multiplied by that power of two.
  //  * Identity rows (h), in blocks of 32 columns of K: a_blk_flag[tile * a_blk_stride + kk / 32]
  //    says whether any row of the tile carries an exponent in that block; if so, row r's values
  //    there are A * 2^a_row_blk_exp[r * a_blk_stride + kk / 32].
  //  * SILU_MUL output (out_f32 == 3): h as fp16 [rows, N/2]; per row and 32 columns the values are
  //    divided by 2^exp first, exp = 0 unless the row's largest finite |h| there reached 2^15; the
  //    flags c_blk_flag [tiles, c_blk_stride] are always written, the exponents c_row_blk_exp
  //    [rows, c_blk_stride] only for flagged blocks.
  int a_f16;
  const int32_t* a_row_exp;
  const uint8_t* a_blk_flag;
  const uint8_t* a_row_blk_exp;
  int a_blk_stride;
  uint8_t* c_blk_flag;
  uint8_t* c_row_blk_exp;
  int c_blk_stride;
};
// Batches the routing prologue serves: at most 16 tokens (so every expert fits one 16-row tile),
// k <= 16, E <= 512.
constexpr int kRouteMaxT = 16, kRouteMaxK = 16;
inline bool route_prologue_fits(int T, int E, int k) {
  return T >= 1 && T <= kRouteMaxT && k <= kRouteMaxK && E <= kAlignSingleMaxE;
}
hipError_t launch_grouped_gemm(const GemmArgs& a, int block_m, hipStream_t stream);
// bf16 x [T, H] -> fp16 x16 [T, H] and row exponents xexp [T]: x16 = fp16(x * 2^-xexp) (convert.hip).
hipError_t launch_x_to_f16(const uint16_t* x, int T, int H, uint16_t* x16, int32_t* xexp, hipStream_t stream);

// MXFP4 (W4A4) grouped GEMM: activations and weights as E2M1 codes with E8M0 scale bytes per 32 K.
struct MxGemmArgs {
  const uint8_t* Aq;        // activation codes [*, K/2]
  const uint8_t* As;        // activation scale bytes [*, K/32]
  const int32_t* a_row_of;  // permuted row -> flat index (NULL = identity)
  int a_row_div;            // activation row = a_row_of[r] / a_row_div
  const uint8_t* Wq;        // [E, N, K/2]
  const uint8_t* We;        // [E, N, K/32]
  int N, K;
  const int32_t* tiles;     // [max_tiles, 3]
  const int32_t* num_tiles;
  int max_tiles;
  void* C;                  // NONE: fp32 or bf16 [rows, N]; SILU_MUL: h codes [rows, N/4]
  uint8_t* Cs;              // SILU_MUL: h scale bytes [rows, N/64]
  int epilogue;             // MOE_EPI_*
  int out_f32;
  // 0: row-major activations (gathered through a_row_of), canonical weights, row-major output;
  // 1: as 0 with packed weights (moe_mx_prepack);
  // 2: tile-blocked activations (mx_tiled_* below), packed weights; a SILU_MUL output (h) is
  //    written tile-blocked for the next projection, a NONE output row-major.  Needs K % 128 == 0.
  int mode;
  // W4A8 (nonzero): activations are MXFP8 (E4M3 codes, one byte per element, and scale bytes):
  // row-major [*, K] and [*, K/32] (mode 0 or 1, or 128-row tiles) or tile-blocked (mode 2, blocks of
  // 2048 code bytes and 64 scale bytes, see mx8_quant_tiles_kernel); a SILU_MUL output is MXFP8 h in the
  // same arrangement (row-major codes [rows, N/2], scale bytes [rows, N/64]).
  int act_e4m3;
  // out_f32 == 2 (fp16 C with in-band exponents, kOutF16Exp; E2M1 activations only): fp32 values of
  // the marked elements, [rows, ceil(N / 8)]
  float* C_side;
};
hipError_t launch_grouped_gemm_mx(const MxGemmArgs& a, int block_m, hipStream_t stream);
hipError_t launch_mx_quant(const uint16_t* x, long long rows, int K, uint8_t* q, uint8_t* s, hipStream_t stream);
// bf16 x [rows, K] -> MXFP8 codes [rows, K] and scale bytes [rows, K/32].
hipError_t launch_mx8_quant(const uint16_t* x, long long rows, int K, uint8_t* q, uint8_t* s, hipStream_t stream);
// x rows quantized to MXFP8 and gathered into the tile-blocked layout of a tile list (block height bm).
hipError_t launch_mx8_quant_tiles(const uint16_t* x, int K, const int32_t* a_row_of, int a_row_div,
                                  const int32_t* tiles, const int32_t* num_tiles, int max_tiles, int bm, uint8_t* q,
                                  uint8_t* s, hipStream_t stream);
// x rows quantized and gathered into the tile-blocked layout of a tile list (block height bm).
hipError_t launch_mx_quant_tiles(const uint16_t* x, int K, const int32_t* a_row_of, int a_row_div,
                                 const int32_t* tiles, const int32_t* num_tiles, int max_tiles, int bm, uint8_t* q,
                                 uint8_t* s, hipStream_t stream);
hipError_t launch_mx_prepack(const uint8_t* wq, const uint8_t* we, int E, int N, int K, uint8_t* pq, uint8_t* pe,
                             hipStream_t stream);

// FP8 (W8A8, per-1x128) grouped GEMM: E4M3 codes with one fp32 scale per row and 128 K elements.
struct F8GemmArgs {
  const uint8_t* Aq;        // activation codes [*, K]
  const float* As;          // activation scales [*, K/128]
  const int32_t* a_row_of;  // permuted row -> flat index (NULL = identity)
  int a_row_div;            // activation row = a_row_of[r] / a_row_div
  const uint8_t* Wq;        // [E, N, K]
  const float* Ws;          // [E, N, K/128]
  int N, K;
  const int32_t* tiles;     // [max_tiles, 3]
  const int32_t* num_tiles;
  int max_tiles;
  void* C;                  // NONE: fp32 or bf16 [rows, N]; SILU_MUL: fp32 h [rows, N/2] or h codes
  int epilogue;             // MOE_EPI_*
  int out_f32;              // 0 bf16, 1 fp32, 2 (SILU_MUL, 128-row tiles) h quantized per 1x128,
                            // 3 (NONE, 128-row tiles) fp16 with in-band exponents (kOutF16Exp's format)
  float* Cs;                // out_f32 == 2: h scales [rows, N/256]
  float* C_side;            // out_f32 == 3: fp32 values of the marked elements, [rows, ceil(N / 8)]
};
hipError_t launch_grouped_gemm_f8(const F8GemmArgs& a, int block_m, hipStream_t stream);
// x (bf16, or fp32 when in_f32) [rows, K] -> codes [rows, K] and scales [rows, K/128].
hipError_t launch_f8_quant(const void* x, bool in_f32, long long rows, int K, uint8_t* q, float* s,
                           hipStream_t stream);

hipError_t launch_prepack(const uint8_t* wq, const uint16_t* ws, int E, int N, int K, uint8_t* pq, uint16_t* ps,
                          hipStream_t stream);

// O: fp32 [R, H] (O_side NULL) or the down projection's fp16 output [R, H] with its side values
// O_side [R, H / 8] (MOE_OUT_F16E).  Shared term: row shared_o_row0 + t of O when
// shared_o_row0 >= 0, else the fp32 rows `shared` (or none when NULL).
hipError_t launch_combine(const void* O, const float* O_side, const int32_t* inv_perm, const float* w,
                          const float* shared, int shared_o_row0, int T, int k, int H, uint16_t* y,
                          hipStream_t stream);

}  // namespace moe
