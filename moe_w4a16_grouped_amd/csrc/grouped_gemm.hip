// Grouped W4A16 GEMM over all experts in one launch, with the SiLU*mul epilogue fused.
//
// Prior art on the pages: the Atlas page ("告别Python堆栈：Atlas用纯Rust重写LLM推理，在GB10上跑赢vLLM"),
// section "编译时内核选择和W4A16 Grouped GEMM", runs gate_up and down as one launch each over a
// (N tiles, max_m_tiles, experts) grid and dequantizes FP4 to BF16 inside the kernel (no BF16 weight
// write-back); the Kortex page ("Rust 从零写的 LLM 推理引擎 Kortex：20GB 显卡跑 70B 模型"), section
// "架构与实现要点", dequantizes in registers and reads each expert's weights once for all tokens routed
// to it; the engine page ("Rust 实现深度学习推理引擎：从计算图到异构硬件加速"), section
// "四、算子融合：性能翻倍的关键", fuses the activation into the matmul.
//
// gfx950 design shared by both kernels below:
//  * Work list instead of a 3D grid: each workgroup maps its index to an entry of the device-side
//    tile list written by moe_align (exact, never a host guess) and an N block; slots past
//    num_tiles are skipped.
//  * v_mfma_f32_16x16x32_bf16: one MFMA spans exactly one 32-element scale group.  Codes are
//    converted to exact bf16 (hardware FP4 converter, unit scale); the MFMA produces the group's
//    fp32 partial, which is multiplied by the bf16 group scale and added to the fp32 accumulator.
//    (Rounding code*scale to bf16 instead would not keep the layer inside its error bound.)  That
//    scale FMA is issued a few MFMAs after its partial's MFMA, so it never waits on the matrix core.
//  * The exact fp16 form (F16, activations in fp16 with power-of-two exponents): code*scale is
//    formed in fp16, exact for scales with an exponent in [-16, 12], and v_mfma_f32_16x16x32_f16
//    accumulates every group in place, with no fp32 scale work per group.
//  * Weights go HBM -> registers (tiled kernels) or LDS (the direct-load kernel).  Canonical layout: one 16-byte load per lane per 4 groups (row n,
//    group q of the K step) followed by a 4x4 cross-quarter transpose (permlane32/16 swaps) into
//    MFMA B-operand order.  Packed layout (prepack.hip): the same registers come from one linear
//    1 KB load per wave, and the 16 rows x 4 group scales from one 128-byte load.
//  * Loads are never behind a branch: addresses are clamped into range and out-of-range data is
//    neutralised where it is consumed, so each step waits only for its own loads.
#include "launch.h"
#include "moe_common.h"
#include "topk.h"

namespace moe {

constexpr int kBK = 128;  // K elements per step: 4 scale groups

enum Layout { kCanonGeneric = 0, kCanonFull = 1, kPacked = 2 };

// Weight-row block of one lane: canonical pointers or packed block base.
struct WBase {
  const uint8_t* q;   // the expert's codes (N x K/2 bytes in either layout)
  const uint16_t* s;  // the expert's scales (N x K/32 in either layout)
};
// A lane's weight row as 32-bit offsets within its expert (the launcher checks that an expert's codes
// stay below 4 GiB), so that a row costs two registers next to the wave-uniform expert base.
struct WRow {
  uint32_t q;  // canonical: row start (+ lane offset); packed: block (nb, ks=0) + lane * 16  (bytes)
  uint32_t s;  // canonical: scale row start; packed: scale block (nb, ks=0) + (lane % 16) * 4 (elements)
};

__device__ __forceinline__ WBase wbase_of(const GemmArgs& p, int e) {
  const size_t nk = (size_t)p.N * (size_t)p.K;
  const size_t eu = (size_t)__builtin_amdgcn_readfirstlane(e);
  return WBase{p.Wq + eu * (nk / 2), p.Ws + eu * (nk / kGroup)};
}

template <int LAYOUT>
__device__ __forceinline__ WRow wrow_of(const GemmArgs& p, int n, int q, int lane) {
  const uint32_t K = (uint32_t)p.K;
  WRow w;
  if (LAYOUT == kPacked) {
    const uint32_t blk = (uint32_t)(n / 16) * (K / kBK);
    w.q = blk * 1024u + (uint32_t)lane * 16u;
    w.s = blk * 64u + (uint32_t)(lane & 15) * 4u;
  } else {
    w.q = (uint32_t)n * (K / 2) + (LAYOUT == kCanonFull ? (uint32_t)q * 16u : 0u);
    w.s = (uint32_t)n * (K / kGroup);
  }
  return w;
}

// Load the codes and scales of K step ks (groups 4ks..4ks+3) for one lane.
// sq: kCanonGeneric -> one bf16 per entry; otherwise [0], [1] = raw bf16 pairs.
template <int LAYOUT>
__device__ __forceinline__ void load_w(const WBase& wb, const WRow& w, int ks, int q, int kgroups, u32x4& b,
                                       uint32_t (&sq)[4]) {
  if (LAYOUT == kPacked) {
    b = *reinterpret_cast<const u32x4*>(wb.q + (w.q + (uint32_t)ks * 1024u));
    const u32x2 v = *reinterpret_cast<const u32x2*>(wb.s + (w.s + (uint32_t)ks * 64u));
    sq[0] = v[0];
    sq[1] = v[1];
  } else if (LAYOUT == kCanonFull) {
    b = *reinterpret_cast<const u32x4*>(wb.q + (w.q + (uint32_t)ks * 64u));
    const u32x2 v = *reinterpret_cast<const u32x2*>(wb.s + (w.s + (uint32_t)ks * 4u));
    sq[0] = v[0];
    sq[1] = v[1];
  } else {
    const int gq = min(ks * 4 + q, kgroups - 1);
    b = *reinterpret_cast<const u32x4*>(wb.q + (w.q + (uint32_t)gq * 16u));
#pragma unroll
    for (int g = 0; g < 4; ++g) sq[g] = wb.s[w.s + (uint32_t)min(ks * 4 + g, kgroups - 1)];
  }
}

// B operand registers of the 4 groups of a step (transposed into MFMA order for canonical layouts).
template <int LAYOUT>
__device__ __forceinline__ u32x4 b_operands(const u32x4& b) {
  return LAYOUT == kPacked ? b : quarter_transpose(b);
}

template <int LAYOUT>
__device__ __forceinline__ float scale_of(const uint32_t (&sq)[4], int g) {
  if (LAYOUT == kCanonGeneric) return bf16_bits_to_f32(sq[g]);
  return __uint_as_float((g & 1) ? (sq[g >> 1] & 0xFFFF0000u) : (sq[g >> 1] << 16));
}

// The bf16 bits of group g's scale (for the fp16 path's exactness test).
template <int LAYOUT>
__device__ __forceinline__ uint32_t scale_bits_of(const uint32_t (&sq)[4], int g) {
  if (LAYOUT == kCanonGeneric) return sq[g] & 0xFFFFu;
  return (g & 1) ? (sq[g >> 1] >> 16) : (sq[g >> 1] & 0xFFFFu);
}

// Column bookkeeping for one 16-column block of the output tile.  For SiLU*mul the first NI/2
// blocks are gate rows j and the last NI/2 the matching up rows N/2 + j.
template <int EPI, int NI>
__device__ __forceinline__ void column_of(const GemmArgs& p, int col0, int ni, int l16, int& n, int& ncol,
                                          bool& valid) {
  if (EPI == MOE_EPI_SILU_MUL) {
    const int half = NI / 2;
    const int j = col0 + (ni % half) * 16 + l16;
    valid = j < p.N / 2;
    ncol = j;
    n = ni < half ? j : p.N / 2 + j;
  } else {
    n = col0 + ni * 16 + l16;
    valid = n < p.N;
    ncol = n;
  }
  if (!valid) n = 0;
}

template <int EPI, int OUT, int MI, int NI>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const f32x4 (&acc)[MI][NI], int row_base, int row0,
                                           int rows, int q, const int (&ncol)[NI], const bool (&nvalid)[NI]) {
  const int N = p.N;
  if constexpr (EPI != MOE_EPI_SILU_MUL && OUT == kOutF16Exp) {
    store_f16e<MI, NI, false>(static_cast<uint16_t*>(p.C), p.C_side, N, acc, row_base, row0, rows, q, ncol, nvalid);
    return;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row_base + mi * 16 + q * 4 + r;
      if (row >= rows) continue;
      const size_t orow = (size_t)(row0 + row);
      if (EPI == MOE_EPI_SILU_MUL) {
        uint16_t* C = static_cast<uint16_t*>(p.C);
#pragma unroll
        for (int ni = 0; ni < NI / 2; ++ni) {
          if (!nvalid[ni]) continue;
          const float g = acc[mi][ni][r], u = acc[mi][ni + NI / 2][r];
          C[orow * (N / 2) + ncol[ni]] = f32_to_bf16_bits(silu_f32(g) * u);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          if (!nvalid[ni]) continue;
          if (OUT == kOutF32) static_cast<float*>(p.C)[orow * N + ncol[ni]] = acc[mi][ni][r];
          else static_cast<uint16_t*>(p.C)[orow * N + ncol[ni]] = f32_to_bf16_bits(acc[mi][ni][r]);
        }
      }
    }
  }
}

// SiLU*mul output of the fp16 path (GemmArgs::out_f32 == kOutH16): h as fp16 with a signed exponent
// per row and 32 columns (one wave's gate columns).  The gate and up row sums are first multiplied by
// the row's power of two (gathered fp16 activations).  A row whose largest finite |h| in the block is
// 2^15 or more, or below 2^-6 (but not 0), is divided there by 2^exp (f16_seg_exponent; exact
// scaling into [2^14, 2^15)); other rows keep exp 0.
// Per tile and block the flag c_blk_flag says whether any row of the block has a nonzero exponent; only
// then are the block's row exponents written.  With WAVES_M > 1 the waves sharing a block (waves
// wn, wn + 4, ...) combine their flags through sAny (one barrier; every wave calls this).
constexpr int kOutH16 = 3;
constexpr int kHBlock = 32;

template <int MI, int NI, int WAVES_M>
__device__ __forceinline__ void store_tile_h16(const GemmArgs& p, const f32x4 (&acc)[MI][NI], const float (&rowf)[MI][4],
                                               int row_base, int row0, int rows, int q, const int (&ncol)[NI],
                                               const bool (&nvalid)[NI], int tile, int col0_wave, int* sAny) {
  static_assert(NI == 4, "a wave's gate columns form one 32-column block");
  const int N2 = p.N / 2;
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const int blk = col0_wave / kHBlock;
  float hv[MI][2][4];
  int ex[MI][4];
  bool any = false;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float m = 0.f;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const float g = acc[mi][ni][r] * rowf[mi][r], u = acc[mi][ni + 2][r] * rowf[mi][r];
        const float h = silu_f32(g) * u;
        hv[mi][ni][r] = h;
        if (nvalid[ni] && fabsf(h) <= 3.4e38f) m = fmaxf(m, fabsf(h));
      }
      // the row's 32 columns live in the 16 lanes of this quarter (two columns each)
      m = row16_max(m);
      ex[mi][r] = f16_seg_exponent(m);
      any |= ex[mi][r] != 0 && row_base + mi * 16 + q * 4 + r < rows;
    }
  bool flagged = __ballot(any) != 0ull;
  if constexpr (WAVES_M > 1) {
    const int wave = threadIdx.x >> 6;
    if (lane == 0) sAny[wave] = flagged;
    __syncthreads();
    flagged = false;
#pragma unroll
    for (int j = 0; j < WAVES_M; ++j) flagged |= sAny[(wave & 3) + 4 * j] != 0;
  }
  const bool blk_ok = blk * kHBlock < N2;
  if (lane == 0 && blk_ok && (WAVES_M == 1 || (threadIdx.x >> 6) < 4))
    p.c_blk_flag[(size_t)tile * p.c_blk_stride + blk] = flagged ? 1 : 0;
  uint16_t* C = static_cast<uint16_t*>(p.C);
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row_base + mi * 16 + q * 4 + r;
      if (row >= rows) continue;
      const float f = pow2f(-ex[mi][r]);
      if (flagged && l16 == 0 && blk_ok)
        p.c_row_blk_exp[(size_t)(row0 + row) * p.c_blk_stride + blk] = (uint8_t)(int8_t)ex[mi][r];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        if (nvalid[ni]) C[(size_t)(row0 + row) * N2 + ncol[ni]] = f32_to_f16_bits(hv[mi][ni][r] * f);
    }
}

// Whether any 32-column block of this tile's fp16 A (identity rows) carries row exponents, from the
// flags a_blk_flag: computed by the whole workgroup, published through sFlag[wave] by the caller's
// next barrier.
__device__ __forceinline__ void tile_blk_exp_flag(const GemmArgs& p, int tile, int* sFlag) {
  bool any = false;
  if (p.a_f16 && p.a_blk_flag)
    for (int i = threadIdx.x; i < p.a_blk_stride; i += blockDim.x) any |= p.a_blk_flag[(size_t)tile * p.a_blk_stride + i] != 0;
  const uint64_t b = __ballot(any);
  if ((threadIdx.x & 63) == 0) sFlag[threadIdx.x >> 6] = b != 0ull;
}

// Row factors 2^exp of gathered fp16 activation rows (a_row_exp, per activation row; 1 without it)
// for this lane's output rows row_base + mi*16 + q*4 + r of the tile, read at the epilogue.
template <int MI, int BM>
__device__ __forceinline__ void gathered_row_factors(const GemmArgs& p, const int32_t (&sRow)[BM], int row_base, int q,
                                                     float (&f)[MI][4]) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) f[mi][r] = p.a_row_exp ? pow2f(p.a_row_exp[sRow[row_base + mi * 16 + q * 4 + r]]) : 1.f;
}

// Row factors 2^exp of block kb (32 columns of K) for this lane's output rows (base + mi*16 + q*4 + r
// of the tile starting at row0; rows past `rows` read row 0's), 1 when the block is not flagged.
// Whether any of the K step's four 32-column blocks of this tile's fp16 A carries row exponents.
__device__ __forceinline__ bool step_blk_flagged(const GemmArgs& p, int tile, int s) {
  bool f = false;
#pragma unroll
  for (int g = 0; g < kBK / kHBlock; ++g) {
    const int kb = s * (kBK / kHBlock) + g;
    if (kb < p.a_blk_stride) f |= p.a_blk_flag[(size_t)tile * p.a_blk_stride + kb] != 0;
  }
  return f;
}

// Row exponents of block kb for the four output rows q*4 .. q*4+3 of a 16-row block starting at tile
// row rbase (rows past the tile repeat row 0); 0 for an unflagged block.
__device__ __forceinline__ void blk_row_exps4(const GemmArgs& p, int tile, int kb, int rbase, int row0, int rows, int q,
                                              int (&ex)[4]) {
  const bool flagged = kb < p.a_blk_stride && p.a_blk_flag[(size_t)tile * p.a_blk_stride + kb] != 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int row = rbase + q * 4 + r;
    if (row >= rows) row = 0;
    ex[r] = flagged ? (int)(int8_t)p.a_row_blk_exp[(size_t)(row0 + row) * p.a_blk_stride + kb] : 0;
  }
}

// General form of one K group of the fp16 path.  The group's partial products are exact in fp16 only
// at a common power of two per output element: 2^(rex[row] + d[col]) with rex the A row's block
// exponent (identity rows with block exponents, else 0) and d the shift of the column's scale
// (scale_f16_shift).  The accumulators are brought to that power before the group's MFMAs (sign -1)
// and back after them (sign +1); both are exact power-of-two scalings (ldexp), so the group's
// contribution is rounded once, in the MFMA's fp32 accumulation.  The exponents are re-derived on
// each call rather than kept across the MFMAs, which keeps the fast form's registers free.
// scale_at(ni) gives the group scale of column block ni, rex_at(mi, rex) the row exponents of the
// lane's four rows of 16-row block mi.
template <int MI, int NI, class ScaleAt, class RexAt>
__device__ __forceinline__ void general_rescale(f32x4 (&acc)[MI][NI], ScaleAt scale_at, RexAt rex_at, int sign) {
  // (a compiler-only memory barrier: the exponents are derived again rather than carried over)
  asm volatile("" ::: "memory");
  int d[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) d[ni] = sign * scale_f16_shift(scale_at(ni));
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    int rex[4];
    rex_at(mi, rex);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mi][ni][r] = ldexpf(acc[mi][ni][r], sign * rex[r] + d[ni]);
  }
}

// Tile list lookups.  In dense mode (no tile list: the shared expert) tile i is rows
// [i * BM, min((i + 1) * BM, dense_rows)) of expert 0.
__device__ __forceinline__ int routed_tile_count(const GemmArgs& p, int bm) {
  return p.tiles ? *p.num_tiles : (p.dense_rows + bm - 1) / bm;
}

// Tiles of one launch: the routed (or dense) tiles, then those of the shared expert.
__device__ __forceinline__ int tile_count(const GemmArgs& p, int bm) {
  return routed_tile_count(p, bm) + (p.Wq_sh ? (p.shared_rows + bm - 1) / bm : 0);
}

// The arguments as seen by one tile, with its expert, first output row and row count.  Routed
// tiles come from the tile list (dense mode: rows [i * bm, min((i + 1) * bm, dense_rows)) of expert
// 0).  Shared-expert tiles read the shared weights, and gather no rows: output row r reads
// activation row r, or token r - shared_row0 when the routed rows are gathered.
__device__ __forceinline__ GemmArgs tile_view(const GemmArgs& p, int tile, int bm, int& e, int& row0, int& rows) {
  GemmArgs v = p;
  const int nr = routed_tile_count(p, bm);
  if (tile < nr) {
    if (p.tiles) {
      e = p.tiles[3 * tile];
      row0 = p.tiles[3 * tile + 1];
      rows = p.tiles[3 * tile + 2];
    } else {
      e = 0;
      row0 = tile * bm;
      rows = min(bm, p.dense_rows - row0);
    }
  } else {
    const int j = tile - nr;
    e = 0;
    row0 = p.shared_row0 + j * bm;
    rows = min(bm, p.shared_rows - j * bm);
    v.Wq = p.Wq_sh;
    v.Ws = p.Ws_sh;
    if (p.a_row_of) {
      v.a_row_of = nullptr;
      v.a_row_sub = p.shared_row0;
    }
  }
  return v;
}

// Activation row of output row r.
__device__ __forceinline__ int a_row(const GemmArgs& p, int r) {
  return p.a_row_of ? p.a_row_of[r] / p.a_row_div : r - p.a_row_sub;
}

// ---------------------------------------------------------------------------------------------------
// Routing prologue of the gate_up launch for small batches (GemmArgs::route_logits).  The ATOM page
// ("AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍", section "8.1 MoE 路径：路由、
// 专家并行与 MORI 通信") routes each token to its top-k experts and groups the slots by expert; at a
// few tokens those steps are a chain of dependent memory round trips, so instead of a launch of
// their own every workgroup of this launch repeats them in LDS (a few hundred slots at most) and
// derives its own tile.  The result is the permutation moe_align builds: experts in ascending order,
// each expert's slots in ascending flat order (token * k + slot), one 16-row tile per touched expert
// (a batch of at most 16 tokens gives every expert at most 16 rows), tile j = j-th touched expert.
// Workgroup 0 writes the routing and the tile count, the workgroup with N block 0 of each tile writes
// that tile's list entry and its part of the permutation, for the launches that follow.
struct __attribute__((aligned(16))) RouteLds {
  uint64_t kept[4][2 * kRouteMaxK];
  int32_t ids[kRouteMaxT * kRouteMaxK];
  int32_t cnt[kAlignSingleMaxE];
  int32_t wsum[4];
  int32_t wmatch[4];
  int32_t tile_e, tile_row0, tile_rows;
  int32_t tok[16];  // token of each row of this workgroup's tile
};

// Runs the routing prologue in a 256-thread workgroup and maps the workgroup (linear index b) to its
// tile and N block as xcd_tile does over the routed tiles plus `shared_tiles`.  Returns false when the
// workgroup has no tile.  For a routed tile (tile < nr) sets e, row0 (first permuted row), rows and
// L.tok; shared tiles are left to the caller.
template <int NJ>
__device__ bool route_prologue(const GemmArgs& p, RouteLds& L, int nbn, int shared_tiles, int& tile, int& nb,
                               int& nr, int& e, int& row0, int& rows) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = p.route_T, E = p.route_E, k = p.route_k, R = T * k;
  const long long b = linear_block();
  const bool writer = b == 0;
  for (int i = tid; i < E; i += 256) L.cnt[i] = 0;
  if constexpr (NJ <= 2) {
    // every logits load of this wave's tokens (at most 4) first, so that they share one round trip
    constexpr int TPW = kRouteMaxT / 4;
    uint32_t u[TPW][NJ];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
      if (wave + 4 * j < T) route_keys_load<NJ>(p.route_logits + (size_t)(wave + 4 * j) * E, E, u[j]);
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = wave + 4 * j;
      if (t >= T) break;
      route_token_keys<NJ>(u[j], E, k, L.kept[wave], L.kept[wave] + k, writer ? p.route_ids + (size_t)t * k : nullptr,
                           writer ? p.route_w + (size_t)t * k : nullptr, L.ids + t * k);
    }
  } else {
    for (int t = wave; t < T; t += 4) {
      const float* lg = p.route_logits + (size_t)t * E;
      int32_t* io = writer ? p.route_ids + (size_t)t * k : nullptr;
      float* wo = writer ? p.route_w + (size_t)t * k : nullptr;
      route_token<NJ>(lg, E, k, L.kept[wave], L.kept[wave] + k, io, wo, L.ids + t * k);
    }
  }
  __syncthreads();
  for (int i = tid; i < R; i += 256) atomicAdd(&L.cnt[L.ids[i]], 1);
  __syncthreads();
  // Exclusive scan over experts of (rows << 16 | touched): thread tid owns experts 2 tid, 2 tid + 1
  // (R <= 256 rows and E <= 512 experts both fit 16 bits).
  const int e0 = 2 * tid, e1 = e0 + 1;
  const int c0 = e0 < E ? L.cnt[e0] : 0, c1 = e1 < E ? L.cnt[e1] : 0;
  const int v = ((c0 + c1) << 16) | ((c0 > 0) + (c1 > 0));
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) L.wsum[wave] = incl;
  __syncthreads();
  int excl = incl - v;
  for (int w = 0; w < wave; ++w) excl += L.wsum[w];
  nr = (L.wsum[0] + L.wsum[1] + L.wsum[2] + L.wsum[3]) & 0xFFFF;
  if (writer && tid == 0) *p.route_num_tiles = nr;
  if (!xcd_tile(b, nbn, nr + shared_tiles, tile, nb)) return false;
  if (tile >= nr) return true;
  const int j0 = excl & 0xFFFF, r0 = excl >> 16;
  int te = -1, trow = 0, trows = 0;
  if (c0 > 0 && j0 == tile) te = e0, trow = r0, trows = c0;
  if (c1 > 0 && j0 + (c0 > 0) == tile) te = e1, trow = r0 + c0, trows = c1;
  if (te >= 0) {
    L.tile_e = te;
    L.tile_row0 = trow;
    L.tile_rows = trows;
    if (nb == 0) {
      p.route_tiles[3 * tile] = te;
      p.route_tiles[3 * tile + 1] = trow;
      p.route_tiles[3 * tile + 2] = trows;
    }
  }
  __syncthreads();
  e = L.tile_e;
  row0 = L.tile_row0;
  rows = L.tile_rows;
  // rows of the tile: slot i (thread i, R <= 256) ranks among the slots routed to e
  const bool m = tid < R && L.ids[tid] == e;
  const uint64_t bal = __ballot(m);
  if (lane == 0) L.wmatch[wave] = __popcll(bal);
  __syncthreads();
  int rank = __popcll(bal & ((1ull << lane) - 1ull));
  for (int w = 0; w < wave; ++w) rank += L.wmatch[w];
  if (m) {
    L.tok[rank] = tid / k;
    if (nb == 0) {
      p.route_sorted[row0 + rank] = tid;
      p.route_inv[tid] = row0 + rank;
    }
  }
  __syncthreads();
  return true;
}

// The view of a shared-expert tile (tile index j past the routed ones), as tile_view gives it.
__device__ __forceinline__ GemmArgs shared_view(const GemmArgs& p, int j, int bm, int& e, int& row0, int& rows) {
  GemmArgs v = p;
  e = 0;
  row0 = p.shared_row0 + j * bm;
  rows = min(bm, p.shared_rows - j * bm);
  v.Wq = p.Wq_sh;
  v.Ws = p.Ws_sh;
  v.a_row_of = nullptr;
  v.a_row_sub = p.shared_row0;
  return v;
}

// ---------------------------------------------------------------------------------------------------
// Tiled kernel: BM x BN tile per 256-thread workgroup, waves split it WAVES_M x WAVES_N; the
// activation tile of each K step is staged once in LDS (double buffer, one barrier per step) and
// shared by the waves.  PF = K steps in flight ahead of the one computed (ring of PF+1 slots).
constexpr int kLDA = kBK + 8;  // padded LDS activation row of the tiled kernel (bf16 elements)

// One BM x BN output tile (expert e, permuted rows [row0, row0 + rows), N block nb) of the tiled
// kernel; p is the tile's view of the arguments and sRow already holds the activation row of each
// tile row (padding rows repeat row 0); it is published by the barrier before the first K step.
// F16: the exact fp16 path (GemmArgs::a_f16): fp16 activations, weights dequantized to fp16 as
// code * scale (exact when the step's scales pass scales_f16_ok, checked per wave and K step), one
// MFMA per group accumulating in place.  A step whose scales fail the test, or whose A blocks carry
// row exponents, takes the general form (general_rescale around the same MFMAs).
template <int BM, int BN, int WAVES_M, int PF, int EPI, int OUT_F32, int LAYOUT, bool F16 = false>
__device__ __forceinline__ void tiled_tile(const GemmArgs& p, int tile, int e, int row0, int rows, int nb,
                                           uint16_t (&sA)[2][BM * kLDA], const int32_t (&sRow)[BM]) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int LDA = kLDA;
  constexpr int ACH = BM * (kBK / 8) / 256;  // 16-byte activation chunks per thread per step
  constexpr int NS = PF + 1;
  static_assert(MI >= 1 && NI >= 1 && ACH >= 1, "tile shape");
  static_assert(EPI != MOE_EPI_SILU_MUL || NI % 2 == 0, "SiLU*mul pairs gate and up blocks");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int l16 = lane & 15, q = lane >> 4;
  const int K = p.K;
  const int kgroups = K / kGroup;
  const int nks = (K + kBK - 1) / kBK;

  const WBase wb = wbase_of(p, e);
  WRow wr[NI];
  const int col0 = EPI == MOE_EPI_SILU_MUL ? nb * (BN / 2) + wn * (WN / 2) : nb * BN + wn * WN;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int n, nc;
    bool nv;
    column_of<EPI, NI>(p, col0, ni, l16, n, nc, nv);
    wr[ni] = wrow_of<LAYOUT>(p, n, q, lane);
  }
  __shared__ int sFlag[4];
  // row exponents of the K step's four A blocks (tiles whose A blocks carry exponents), per LDS buffer
  __shared__ int8_t sRex[F16 ? 2 : 1][F16 ? BM * 4 : 1];
  if (F16) tile_blk_exp_flag(p, tile, sFlag);
  __syncthreads();
  // (gathered activations carry row exponents only: the block form is for identity rows, never SiLU*mul)
  // (read through readfirstlane: the branches on it are uniform, which keeps them out of exec masking)
  const bool hblk = F16 && EPI != MOE_EPI_SILU_MUL &&
                    __builtin_amdgcn_readfirstlane(sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3]) != 0;

  // thread tid stages chunk column acol of rows tid / 16 + 16 i (256 threads cover 16 rows of 16 chunks)
  static_assert(kBK / 8 == 16, "16 chunks per activation row of a K step");
  const int acol = (tid % 16) * 8;
  const int alds0 = (tid / 16) * LDA + acol;
  const uint16_t* arow[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) arow[i] = p.A + (size_t)sRow[tid / 16 + 16 * i] * K;

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  // bf16 form: the partial waiting for its scale, and the scale of a partial of the previous group
  // (the pipeline starts with zero partials and scales: 0 * 0 added to a zero accumulator)
  f32x4 pend[NI];
  float psc[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    pend[ni] = f32x4{0.f, 0.f, 0.f, 0.f};
    psc[ni] = 0.f;
  }

  u32x4 areg[NS][ACH];
  u32x4 breg[NS][NI];
  uint32_t sreg[NS][NI][4];

  auto load_step = [&](int s, int u) {
    s = min(s, nks - 1);  // prefetches past the end re-read the last step (never used)
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      areg[u][i] = *reinterpret_cast<const u32x4*>(arow[i] + min(s * kBK + acol, K - 8));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) load_w<LAYOUT>(wb, wr[ni], s, q, kgroups, breg[u][ni], sreg[u][ni]);
  };

  auto compute_step = [&](const uint16_t* a_lds, int u, int s) {
    u32x4 bt[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) bt[ni] = b_operands<LAYOUT>(breg[u][ni]);
    if constexpr (F16) {
      // the step's scales as bf16 pairs: sd[2 ni + h] holds groups 2h (low half) and 2h + 1
      uint32_t sd[2 * NI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        sd[2 * ni] = scale_bits_of<LAYOUT>(sreg[u][ni], 0) | (scale_bits_of<LAYOUT>(sreg[u][ni], 1) << 16);
        sd[2 * ni + 1] = scale_bits_of<LAYOUT>(sreg[u][ni], 2) | (scale_bits_of<LAYOUT>(sreg[u][ni], 3) << 16);
      }
      const bool general = __builtin_amdgcn_readfirstlane(
                               __ballot(!scales_f16_ok(sd)) != 0ull || (hblk && step_blk_flagged(p, tile, s))) != 0;
      // one pass in the fast form, one pass per group in the general form (as in mm_tile)
      const int npass = general ? 4 : 1;
      for (int pass = 0; pass < npass; ++pass) {
        uint32_t sw[2 * NI];
        auto sc_p = [&](int ni) {
          const uint32_t d = sd[2 * ni + (pass >> 1)];
          return __uint_as_float((pass & 1) ? (d & 0xFFFF0000u) : (d << 16));
        };
        auto rex_p = [&](int mi, int (&rex)[4]) {
#pragma unroll
          for (int r = 0; r < 4; ++r) rex[r] = hblk ? (int)sRex[s & 1][(wm * WM + mi * 16 + q * 4 + r) * 4 + pass] : 0;
        };
        if (general) {
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const uint32_t m = scale_f16_mantissa_bits(sc_p(ni)) << (16 * (pass & 1));
            sw[2 * ni] = (pass >> 1) == 0 ? m : 0u;
            sw[2 * ni + 1] = (pass >> 1) == 1 ? m : 0u;
          }
          general_rescale<MI, NI>(acc, sc_p, rex_p, -1);
        } else {
#pragma unroll
          for (int i = 0; i < 2 * NI; ++i) sw[i] = sd[i];
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f16x8 bf[NI];
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const uint32_t d = sw[2 * ni + (g >> 1)];
            bf[ni] = e2m1x8_to_f16(bt[ni][g], (_Float16)__uint_as_float((g & 1) ? (d & 0xFFFF0000u) : (d << 16)));
          }
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) {
            const f16x8 af =
                *reinterpret_cast<const f16x8*>(&a_lds[(wm * WM + mi * 16 + l16) * LDA + g * 32 + q * 8]);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma16x16x32_f16(af, bf[ni], acc[mi][ni]);
          }
        }
        if (general) general_rescale<MI, NI>(acc, sc_p, rex_p, 1);
      }
    } else {
      // the partial of MFMA (mi, ni) is scaled into its accumulator NI MFMAs later (pend, psc: as in
      // mm_tile), so no FMA waits on the MFMA just issued; each accumulator still takes its groups in
      // K order
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x8 bf[NI];
        float sc[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          bf[ni] = e2m1x8_to_bf16(bt[ni][g]);
          sc[ni] = scale_of<LAYOUT>(sreg[u][ni], g);
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const bf16x8 af =
              *reinterpret_cast<const bf16x8*>(&a_lds[(wm * WM + mi * 16 + l16) * LDA + g * 32 + q * 8]);
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const f32x4 part = mfma16x16x32(af, bf[ni], f32x4{0.f, 0.f, 0.f, 0.f});
            if (mi == 0) acc[MI - 1][ni] += psc[ni] * pend[ni];
            else acc[mi - 1][ni] += sc[ni] * pend[ni];
            pend[ni] = part;
          }
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) psc[ni] = sc[ni];
      }
    }
  };

  // One K step: stage A(s) from ring slot u into LDS buffer s&1, sync, optionally prefetch step
  // s+PF into the slot freed by step s-1, then compute step s.  Activation chunks past K are zeroed
  // here, which makes the matching partial products exactly zero whatever the clamped codes hold.
  auto step = [&](int s, int u, bool prefetch) {
    // keep the scheduler from hoisting work on later steps' registers into this step, which would
    // make this step wait for their loads and shorten the prefetch distance
    __builtin_amdgcn_sched_barrier(0);
    uint16_t* a_lds = sA[s & 1];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      u32x4 v = areg[u][i];
      if (LAYOUT == kCanonGeneric && s * kBK + acol >= K) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&a_lds[alds0 + 16 * i * LDA]) = v;
    }
    if constexpr (F16 && EPI != MOE_EPI_SILU_MUL) {
      if (hblk) {
        // thread i < BM * 4: row i / 4 of the tile, block 4 s + i % 4 (rows past the tile read row 0)
        for (int i = tid; i < BM * 4; i += 256) {
          const int row = i / 4 < rows ? i / 4 : 0, kb = s * (kBK / kHBlock) + i % 4;
          const bool f = kb < p.a_blk_stride && p.a_blk_flag[(size_t)tile * p.a_blk_stride + kb] != 0;
          sRex[s & 1][i] = f ? (int8_t)p.a_row_blk_exp[(size_t)(row0 + row) * p.a_blk_stride + kb] : (int8_t)0;
        }
      }
    }
    __syncthreads();
    if (prefetch) load_step(s + PF, (u + PF) % NS);
    compute_step(a_lds, u, s);
  };

#pragma unroll
  for (int u = 0; u < PF; ++u) load_step(u, u);
  int s0 = 0;
  for (; s0 + NS <= nks; s0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) step(s0 + u, u, true);
  }
#pragma unroll
  for (int u = 0; u < NS - 1; ++u)
    if (s0 + u < nks) step(s0 + u, u, false);
  if constexpr (!F16) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[MI - 1][ni] += psc[ni] * pend[ni];
  }

  int ncol[NI];
  bool nvalid[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int n;
    column_of<EPI, NI>(p, col0, ni, l16, n, ncol[ni], nvalid[ni]);
  }
  if constexpr (F16 && EPI == MOE_EPI_SILU_MUL) {
    static_assert(WAVES_M == 1, "one wave per 32-column block of h");
    float rowf[MI][4];
    gathered_row_factors<MI>(p, sRow, wm * WM, q, rowf);
    store_tile_h16<MI, NI, 1>(p, acc, rowf, wm * WM, row0, rows, q, ncol, nvalid, tile, col0, nullptr);
  } else {
    store_tile<EPI, OUT_F32, MI, NI>(p, acc, wm * WM, row0, rows, q, ncol, nvalid);
  }
}

// RNJ > 0: the launch runs the routing prologue (route_token over 64 * RNJ experts per lane group).
// The fp16 path with packed weights (fp16 h or fp16 O) is held to two workgroups per CU (its register need
// is just above that budget otherwise, which would halve the CU's waves).
template <int BM, int BN, int WAVES_M, int PF, int EPI, int OUT_F32, int LAYOUT, int RNJ = 0, bool F16 = false>
__global__ __launch_bounds__(256, (F16 && LAYOUT == kPacked && OUT_F32 != kOutF32) ? 2 : 1) void gemm_w4a16_tiled(GemmArgs p0) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kLDA];
  __shared__ int32_t sRow[BM];
  const int nbn = EPI == MOE_EPI_SILU_MUL ? (p0.N / 2 + BN / 2 - 1) / (BN / 2) : (p0.N + BN - 1) / BN;
  int tile, nb, e, row0, rows;
  GemmArgs p;
  if constexpr (RNJ > 0) {
    static_assert(BM == 16, "the routing prologue builds 16-row tiles");
    __shared__ RouteLds rl;
    int nr;
    const int sh = p0.Wq_sh ? (p0.shared_rows + BM - 1) / BM : 0;
    if (!route_prologue<RNJ>(p0, rl, nbn, sh, tile, nb, nr, e, row0, rows)) return;
    if (tile < nr) {
      p = p0;
      for (int i = threadIdx.x; i < BM; i += 256) sRow[i] = rl.tok[i < rows ? i : 0];
    } else {
      p = shared_view(p0, tile - nr, BM, e, row0, rows);
      for (int i = threadIdx.x; i < BM; i += 256) sRow[i] = a_row(p, row0 + (i < rows ? i : 0));
    }
  } else {
    if (!xcd_tile(linear_block(), nbn, tile_count(p0, BM), tile, nb)) return;
    p = tile_view(p0, tile, BM, e, row0, rows);
    for (int i = threadIdx.x; i < BM; i += 256) sRow[i] = a_row(p, row0 + (i < rows ? i : 0));
  }
  tiled_tile<BM, BN, WAVES_M, PF, EPI, OUT_F32, LAYOUT, F16>(p, tile, e, row0, rows, nb, sA, sRow);
}

// ---------------------------------------------------------------------------------------------------
// Split-K kernel for a handful of small tiles (single-token decode), where too few workgroups exist
// to keep the weight stream busy with the tiled kernel.  The KW waves split K into contiguous
// ranges; each wave loads its weights straight into a PF-deep register ring (issued before its
// activation fragments, whose addresses wait on the permutation) and its own activation fragments
// (16-byte loads, rows gathered through a_row_of; padding rows repeat the tile's first row, which
// the load coalescer merges), so the main loop has no LDS traffic and no barrier.  The KW partial
// sums are reduced through LDS once per tile, in wave order.
template <int BM, int BN, int PF, int EPI, int OUT_F32, int LAYOUT, int KW = 4, int RNJ = 0>
__global__ __launch_bounds__(64 * KW) void gemm_w4a16_sk(GemmArgs p0) {
  constexpr int MI = BM / 16, NI = BN / 16;
  static_assert(MI >= 1 && MI <= 2 && NI >= 1, "tile shape");
  static_assert(EPI != MOE_EPI_SILU_MUL || NI % 2 == 0, "SiLU*mul pairs gate and up blocks");
  constexpr int NS = PF + 1;

  __shared__ __attribute__((aligned(16))) float red[(KW - 1) * 64 * MI * NI * 4];

  const int nbn = EPI == MOE_EPI_SILU_MUL ? (p0.N / 2 + BN / 2 - 1) / (BN / 2) : (p0.N + BN - 1) / BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int l16 = lane & 15, q = lane >> 4;
  int tile, nb, e, row0, rows;
  GemmArgs p;
  int arow_of[MI];  // activation row of each of this lane's tile rows (padding rows repeat row 0)
  if constexpr (RNJ > 0) {
    static_assert(BM == 16 && KW == 4, "the routing prologue builds 16-row tiles in 256-thread workgroups");
    __shared__ RouteLds rl;
    int nr;
    const int sh = p0.Wq_sh ? (p0.shared_rows + BM - 1) / BM : 0;
    if (!route_prologue<RNJ>(p0, rl, nbn, sh, tile, nb, nr, e, row0, rows)) return;
    if (tile < nr) {
      p = p0;
      arow_of[0] = rl.tok[l16 < rows ? l16 : 0];
    } else {
      p = shared_view(p0, tile - nr, BM, e, row0, rows);
      arow_of[0] = a_row(p, row0 + (l16 < rows ? l16 : 0));
    }
  } else {
    if (!xcd_tile(linear_block(), nbn, tile_count(p0, BM), tile, nb)) return;
    p = tile_view(p0, tile, BM, e, row0, rows);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int i = mi * 16 + l16;
      arow_of[mi] = a_row(p, row0 + (i < rows ? i : 0));
    }
  }
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K;
  const int kgroups = K / kGroup;
  const int nks = (K + kBK - 1) / kBK;
  const int per = (nks + KW - 1) / KW;  // steps per wave (contiguous K ranges)
  const int s_begin = min(nks, wk * per), s_end = min(nks, s_begin + per);
  const bool m1 = MI > 1 && rows > 16;  // second 16-row block present (wave-uniform)

  const uint16_t* arow[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) arow[mi] = p.A + (size_t)arow_of[mi] * K + q * 8;
  const WBase wb = wbase_of(p, e);
  WRow wr[NI];
  int ncol[NI];
  bool nvalid[NI];
  const int col0 = nb * (EPI == MOE_EPI_SILU_MUL ? BN / 2 : BN);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int n;
    column_of<EPI, NI>(p, col0, ni, l16, n, ncol[ni], nvalid[ni]);
    wr[ni] = wrow_of<LAYOUT>(p, n, q, lane);
  }

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[NS][MI][4];
  u32x4 breg[NS][NI];
  uint32_t sreg[NS][NI][4];

  auto load_step = [&](int s, int u) {
    s = min(s, s_end - 1);  // prefetches past this wave's range re-read its last step (unused)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) load_w<LAYOUT>(wb, wr[ni], s, q, kgroups, breg[u][ni], sreg[u][ni]);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        areg[u][mi][g] = *reinterpret_cast<const u32x4*>(arow[mi] + min(s * kBK + g * 32, K - 32));
  };

  auto compute_step = [&](int s, int u) {
    u32x4 bt[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) bt[ni] = b_operands<LAYOUT>(breg[u][ni]);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (LAYOUT == kCanonGeneric && s * 4 + g >= kgroups) break;  // K tail (wave-uniform)
      bf16x8 bf[NI];
      float sc[NI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        bf[ni] = e2m1x8_to_bf16(bt[ni][g]);
        sc[ni] = scale_of<LAYOUT>(sreg[u][ni], g);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if (mi == 1 && !m1) break;
        const bf16x8 af = __builtin_bit_cast(bf16x8, areg[u][mi][g]);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const f32x4 part = mfma16x16x32(af, bf[ni], f32x4{0.f, 0.f, 0.f, 0.f});
          acc[mi][ni] += sc[ni] * part;
        }
      }
    }
  };

  if (s_end > s_begin) {
#pragma unroll
    for (int u = 0; u < PF; ++u) load_step(s_begin + u, u);
    int s0 = s_begin;
    for (; s0 + NS <= s_end; s0 += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        load_step(s0 + u + PF, (u + PF) % NS);
        compute_step(s0 + u, u);
      }
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (s0 + u < s_end) compute_step(s0 + u, u);
  }

  // K-slice reduction in wave order: waves 1..KW-1 park their sums, wave 0 adds them.
  constexpr int PER = MI * NI * 4;
  if (wk > 0) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wk - 1) * 64 + lane) * PER + (mi * NI + ni) * 4 + r] = acc[mi][ni][r];
  }
  __syncthreads();
  if (wk > 0) return;
#pragma unroll
  for (int w = 0; w < KW - 1; ++w)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][ni][r] += red[(w * 64 + lane) * PER + (mi * NI + ni) * 4 + r];
  store_tile<EPI, OUT_F32, MI, NI>(p, acc, 0, row0, rows, q, ncol, nvalid);
}

// ---------------------------------------------------------------------------------------------------
// Large-tile kernel for MFMA-bound shapes (hundreds of rows per expert), packed weights only.
// 128 x 256 output tile per 512-thread workgroup: 8 waves (2 along M x 4 along N), 64 x 64 each, so
// two waves share every SIMD and one's scale FMAs can overlap the other's MFMAs.  Activations (gathered
// rows) and packed weight codes/scales reach LDS through direct global->LDS 16-byte loads
// (global_load_lds_dwordx4: lane l of an instruction fills LDS bytes [16l, 16l+16) after a
// wave-uniform base), so staging costs no registers.  NSTAGE LDS stages, one barrier per K step:
// the loads of step s+NSTAGE-1 are issued right after the barrier of step s, into the stage computed
// at step s-1.  Activation rows are 256-byte LDS rows whose 16-byte chunks are XOR-swizzled by
// (row % 16), which makes the fragment reads conflict-free.
// Work order is XCD-aware (mm_work): workgroup b runs on XCD b % 8 (round-robin dispatch); with at
// least 8 N blocks each XCD walks one row tile across its N blocks before the next tile, so the tile's
// activations are fetched into that XCD's L2 once and reused by all of its N blocks; with fewer N
// blocks the XCDs take contiguous shares of the tile list instead, so that none idles.

// Shape of a direct-load tile kernel: BM x BN output tile per workgroup of WAVES_M x WAVES_N waves,
// NSTAGE LDS stages of activations and codes.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NSTAGE_>
struct MmCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NSTAGE = NSTAGE_;
  static constexpr int NW = WAVES_M * WAVES_N, THREADS = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, MI = WM / 16, NI = WN / 16;
  static constexpr int CB = BN / 16;      // 16-row code blocks per stage
  static constexpr int AI = BM / 4 / NW;  // activation loads per wave and step (4 rows of 256 bytes each)
  static constexpr int BI = CB / NW;      // code block loads per wave and step
  static constexpr int SI = CB / 8;       // scale loads per step (1 KiB each, waves 0 .. SI-1)
  static constexpr int A_BYTES = BM * 256, STAGE = A_BYTES + CB * 1024;
  // Scales travel one K step ahead of activations and codes, in a ring of their own: at step s the
  // slots of steps s (computed), s + 1 (tested meanwhile by the fp16 path, or in flight) up to
  // s + NSTAGE (issued at step s) are live, NSTAGE + 1 slots.
  static constexpr int SCALE_SLOT = CB * 128, SCALE_SLOTS = NSTAGE + 1;
  static constexpr int LDS = NSTAGE * STAGE + SCALE_SLOTS * SCALE_SLOT;
  static_assert(MI >= 1 && NI >= 2 && NI % 2 == 0 && AI >= 1 && BI >= 1 && SI >= 1 && SI <= NW, "tile shape");
  static_assert(AI * NW * 4 == BM && BI * NW == CB && SI * 8 == CB, "loads cover the stage");
  static_assert(NSTAGE >= 3 && NSTAGE <= 5, "stages");
};
// 128 x 256 tiles, 8 waves, for MFMA-bound shapes.  (32 x 128 tiles in this form, 4 waves with 3 or 4
// stages, were measured on MI355X at 800 tokens over 256 experts: gate_up 90.2 / 95.5 us against
// 87.7 us for the register-staged tiled kernel.)
using MmLarge = MmCfg<128, 256, 2, 4, 3>;

// s_waitcnt for `later` K steps' loads still in flight (at most MAXL), X loads per step.
template <int X, int MAXL>
__device__ __forceinline__ void wait_steps(int later) {
  if constexpr (MAXL == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= MAXL) wait_vmcnt<X * MAXL>();
    else wait_steps<X, MAXL - 1>(later);
  }
}

// One BM x BN output tile (tile list entry `tile`, N block `nb`) of a direct-load tile kernel.
// F16: the exact fp16 path as in tiled_tile (fp16 activations in the same LDS layout, weights
// dequantized to fp16 as code * scale, one MFMA per group accumulating in place, the general form for
// steps whose scales fail the exactness test or whose A blocks carry row exponents).
template <class Cfg, int EPI, int OUT_F32, bool F16 = false>
__device__ __forceinline__ void mm_tile(const GemmArgs& p0, int tile, int nb, uint8_t (&smem)[Cfg::LDS],
                                        int32_t (&sRow)[Cfg::BM]) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, MI = Cfg::MI, NI = Cfg::NI, NW = Cfg::NW, NSTAGE = Cfg::NSTAGE;
  constexpr int WM = Cfg::WM, WN = Cfg::WN, CB = Cfg::CB, AI = Cfg::AI, BI = Cfg::BI, SI = Cfg::SI;
  constexpr int A_BYTES = Cfg::A_BYTES, STAGE = Cfg::STAGE;
  static_assert(!F16 || (NI == 4 && Cfg::WAVES_M == 2), "the fp16 path's h blocks: one wave's 32 gate columns");
  int e, row0, rows;
  const GemmArgs p = tile_view(p0, tile, BM, e, row0, rows);
  const int N = p.N, K = p.K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int l16 = lane & 15, q = lane >> 4;
  const int nks = K / kBK;
  const int NB16 = N / 16;

  auto block_row = [&](int blk) -> int {  // packed row-block index of LDS block blk (clamped)
    int rb, first;
    if (EPI == MOE_EPI_SILU_MUL) {
      first = nb * (BN / 2) + (blk % (CB / 2)) * 16;
      rb = (blk < CB / 2 ? first : N / 2 + first) / 16;
      if (first >= N / 2) rb = 0;
    } else {
      first = nb * BN + blk * 16;
      rb = first / 16;
      if (first >= N) rb = 0;
    }
    return rb;
  };

  // fp16 path: the tile's scales over the whole of K are tested once, here (CB row blocks of nks * 128
  // contiguous bytes each); their loads overlap those of the permutation below
  constexpr int kScanUnroll = 8;
  bool scales_ok = true;
  if constexpr (F16) {
    const int per_blk = nks * 8;  // 16-byte chunks of one row block's scales
    const int total = CB * per_blk;
    const uint8_t* ws = reinterpret_cast<const uint8_t*>(p.Ws);
    for (int i0 = tid; i0 < total; i0 += kScanUnroll * Cfg::THREADS) {
      u32x4 v[kScanUnroll];
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        const int i = min(i0 + u * Cfg::THREADS, total - 1);
        const int b = i / per_blk;
        v[u] = *reinterpret_cast<const u32x4*>(ws + ((size_t)e * NB16 + block_row(b)) * (size_t)nks * 128 +
                                               (size_t)(i - b * per_blk) * 16);
      }
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        const uint32_t d[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
        scales_ok &= scales_f16_ok(d);
      }
    }
  }
  for (int i = tid; i < BM; i += Cfg::THREADS) {
    const int r = row0 + (i < rows ? i : 0);
    sRow[i] = a_row(p, r);
  }
  __shared__ int sFlag[NW];
  __shared__ int sGen[NW];
  if constexpr (F16) {
    tile_blk_exp_flag(p, tile, sFlag);
    const uint64_t bad = __ballot(!scales_ok);
    if (lane == 0) sGen[wave] = bad != 0ull;
  }
  __syncthreads();
  int any_flag = 0, any_bad = 0;
  if constexpr (F16) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      any_flag |= sFlag[w];
      any_bad |= sGen[w];
    }
  }
  const bool hblk = F16 && EPI != MOE_EPI_SILU_MUL && __builtin_amdgcn_readfirstlane(any_flag) != 0;
  // every K step of the tile takes the general form when one scale of the tile fails the test or an
  // A block carries row exponents (wave-uniform)
  const bool general = F16 && (hblk || __builtin_amdgcn_readfirstlane(any_bad) != 0);

  // global sources of this wave's direct loads
  const uint16_t* a_src[AI];  // activation instructions i = AI*wave + t: rows 4i .. 4i+3
#pragma unroll
  for (int t = 0; t < AI; ++t) {
    const int r = 4 * (AI * wave + t) + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    a_src[t] = p.A + (size_t)sRow[r] * K + c * 8;
  }
  const uint8_t* b_src[BI];
#pragma unroll
  for (int t = 0; t < BI; ++t)
    b_src[t] = p.Wq + ((size_t)e * NB16 + block_row(BI * wave + t)) * (size_t)nks * 1024 + lane * 16;
  const uint8_t* s_src = reinterpret_cast<const uint8_t*>(p.Ws) +
                         ((size_t)e * NB16 + block_row(8 * (wave % SI) + (lane >> 3))) * (size_t)nks * 128 +
                         (lane & 7) * 16;

  // LDS blocks of this wave's column blocks (SiLU*mul: NI/2 gate blocks, then the matching up blocks)
  int blk[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    blk[ni] = EPI == MOE_EPI_SILU_MUL ? (ni < NI / 2 ? wn * (NI / 2) + ni : CB / 2 + wn * (NI / 2) + (ni - NI / 2))
                                      : wn * NI + ni;

  uint8_t* const sring = smem + NSTAGE * STAGE;
  auto issue_scales = [&](int ks) {
    if (wave < SI)
      g2lds16(s_src + (size_t)ks * 128, sring + (ks % Cfg::SCALE_SLOTS) * Cfg::SCALE_SLOT + wave * 1024);
  };
  // A and codes of step ks into stage `stage`, and the scales of step ks + 1
  auto issue = [&](int ks, int stage) {
    uint8_t* st = smem + stage * STAGE;
#pragma unroll
    for (int t = 0; t < AI; ++t) g2lds16(a_src[t] + (size_t)ks * kBK, st + (AI * wave + t) * 1024);
#pragma unroll
    for (int t = 0; t < BI; ++t) g2lds16(b_src[t] + (size_t)ks * 1024, st + A_BYTES + (BI * wave + t) * 1024);
    if (ks + 1 < nks) issue_scales(ks + 1);
  };
  auto scales_of = [&](int s, int ni) -> u32x2 {
    return *reinterpret_cast<const u32x2*>(sring + (s % Cfg::SCALE_SLOTS) * Cfg::SCALE_SLOT + blk[ni] * 128 + l16 * 8);
  };
  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over the MFMA sequence (g, mi, ni), carried across K steps: the partial of
  // MFMA (mi, ni) waits in pend[ni] and is scaled into its accumulator four MFMAs later, right after
  // MFMA (mi + 1, ni) is issued; the scale of a partial from the previous group is in psc.  So an MFMA
  // result is never read right after it is produced, and the scale FMAs fill the MFMA shadow.  The
  // accumulators still receive their groups in K order; the pipeline starts with zero partials and
  // zero scales (adding 0 * 0 to a zero accumulator).
  f32x4 pend[NI];
  float psc[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    psc[ni] = 0.f;
    pend[ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](int stage, int s) {
    const uint8_t* st = smem + stage * STAGE;
    u32x4 braw[NI];
    u32x2 sraw[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      braw[ni] = *reinterpret_cast<const u32x4*>(st + A_BYTES + blk[ni] * 1024 + lane * 16);
      sraw[ni] = scales_of(s, ni);
    }
    if constexpr (F16) {
      uint32_t sd[2 * NI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        sd[2 * ni] = sraw[ni][0];
        sd[2 * ni + 1] = sraw[ni][1];
      }
      // One pass over the step's four groups in the fast form; in the general form one pass per group
      // (the other groups' scales zeroed), with the accumulators rescaled around the pass.  The MFMA
      // sequence is the same straight-line block either way.
      const int npass = general ? 4 : 1;
      for (int pass = 0; pass < npass; ++pass) {
        uint32_t sw[2 * NI];
        auto sc_p = [&](int ni) {
          const uint32_t d = sd[2 * ni + (pass >> 1)];
          return __uint_as_float((pass & 1) ? (d & 0xFFFF0000u) : (d << 16));
        };
        auto rex_p = [&](int mi, int (&rex)[4]) {
          if (hblk) {
            blk_row_exps4(p, tile, s * (kBK / kHBlock) + pass, wm * WM + mi * 16, row0, rows, q, rex);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) rex[r] = 0;
          }
        };
        if (general) {
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const uint32_t m = scale_f16_mantissa_bits(sc_p(ni)) << (16 * (pass & 1));
            sw[2 * ni] = (pass >> 1) == 0 ? m : 0u;
            sw[2 * ni + 1] = (pass >> 1) == 1 ? m : 0u;
          }
          general_rescale<MI, NI>(acc, sc_p, rex_p, -1);
        } else {
#pragma unroll
          for (int i = 0; i < 2 * NI; ++i) sw[i] = sd[i];
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f16x8 af[MI], bf[NI];
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) {
            const int r = wm * WM + mi * 16 + l16;  // r % 16 == l16
            af[mi] = *reinterpret_cast<const f16x8*>(st + r * 256 + (((g * 4 + q) ^ l16) * 16));
          }
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const uint32_t d = sw[2 * ni + (g >> 1)];
            bf[ni] = e2m1x8_to_f16(braw[ni][g], (_Float16)__uint_as_float((g & 1) ? (d & 0xFFFF0000u) : (d << 16)));
          }
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma16x16x32_f16(af[mi], bf[ni], acc[mi][ni]);
        }
        if (general) general_rescale<MI, NI>(acc, sc_p, rex_p, 1);
      }
      return;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x8 af[MI], bf[NI];
      float sc[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wm * WM + mi * 16 + l16;  // r % 16 == l16
        af[mi] = *reinterpret_cast<const bf16x8*>(st + r * 256 + (((g * 4 + q) ^ l16) * 16));
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        bf[ni] = e2m1x8_to_bf16(braw[ni][g]);
        sc[ni] = __uint_as_float((g & 1) ? (sraw[ni][g >> 1] & 0xFFFF0000u) : (sraw[ni][g >> 1] << 16));
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const f32x4 part = mfma16x16x32(af[mi], bf[ni], f32x4{0.f, 0.f, 0.f, 0.f});
          if (mi == 0) acc[MI - 1][ni] += psc[ni] * pend[ni];
          else acc[mi - 1][ni] += sc[ni] * pend[ni];
          pend[ni] = part;
        }
#pragma unroll
      for (int i = 0; i < MI * NI; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // then four VALU instructions
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) psc[ni] = sc[ni];
    }
  };

  // Per-step direct loads of each wave: AI + BI, one more for the waves that load scales.  Step s
  // lives in stage s % NSTAGE, its scales in slot s % 4, loaded with the previous step; steps
  // s+1 .. s+NSTAGE-2 are in flight while step s is computed.  The waits are explicit: a stage is read
  // after this wave's loads for it (and for the next step's scales) have landed (only later steps'
  // loads still in flight) and after the barrier that publishes everyone's.
  issue_scales(0);
#pragma unroll
  for (int u = 0; u < NSTAGE - 1; ++u)
    if (u < nks) issue(u, u);
  for (int s = 0; s < nks; ++s) {
    wait_steps<AI + BI, NSTAGE - 2>(min(NSTAGE - 2, nks - 1 - s));
    __syncthreads();
    if (s + NSTAGE - 1 < nks) issue(s + NSTAGE - 1, (s + NSTAGE - 1) % NSTAGE);
    compute(s % NSTAGE, s);
  }
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) acc[MI - 1][ni] += psc[ni] * pend[ni];

  int ncol[NI];
  bool nvalid[NI];
  const int col0 = EPI == MOE_EPI_SILU_MUL ? nb * (BN / 2) + wn * (WN / 2) : nb * BN + wn * WN;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int n;
    column_of<EPI, NI>(p, col0, ni, l16, n, ncol[ni], nvalid[ni]);
  }
  if constexpr (F16 && EPI == MOE_EPI_SILU_MUL) {
    float rowf[MI][4];
    gathered_row_factors<MI>(p, sRow, wm * WM, q, rowf);
    store_tile_h16<MI, NI, Cfg::WAVES_M>(p, acc, rowf, wm * WM, row0, rows, q, ncol, nvalid, tile, col0, sFlag);
  } else {
    store_tile<EPI, OUT_F32, MI, NI>(p, acc, wm * WM, row0, rows, q, ncol, nvalid);
  }
}

template <class Cfg, int EPI, int OUT_F32, bool F16 = false>
__global__ __launch_bounds__(Cfg::THREADS) void gemm_w4a16_mm(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::LDS];
  __shared__ int32_t sRow[Cfg::BM];
  const int ncols = EPI == MOE_EPI_SILU_MUL ? p.N / 2 : p.N;
  const int bcols = EPI == MOE_EPI_SILU_MUL ? Cfg::BN / 2 : Cfg::BN;
  const int nbn = (ncols + bcols - 1) / bcols;
  int tile, nb;
  if (!mm_work(linear_block(), nbn, tile_count(p, Cfg::BM), tile, nb)) return;
  mm_tile<Cfg, EPI, OUT_F32, F16>(p, tile, nb, smem, sRow);
}

// ---------------------------------------------------------------------------------------------------
// Launch configuration.

static int layout_of(const GemmArgs& a) {
  if (a.packed) return kPacked;
  return ((a.K % kBK) == 0 && (reinterpret_cast<uintptr_t>(a.Ws) % 8) == 0) ? kCanonFull : kCanonGeneric;
}

static dim3 grid_of(const GemmArgs& a, int bn) {
  const int ncols = a.epilogue == MOE_EPI_SILU_MUL ? a.N / 2 : a.N;
  const int bcols = a.epilogue == MOE_EPI_SILU_MUL ? bn / 2 : bn;
  const long long nbn = (ncols + bcols - 1) / bcols;
  return grid2d(8LL * ((a.max_tiles + 7) / 8) * nbn);
}

template <int BM, int BN, int WAVES_M, int PF>
struct Tiled {
  template <int EPI, int F32, int LAYOUT, int RNJ = 0, bool F16 = false>
  static hipError_t run(const GemmArgs& a, hipStream_t s) {
    gemm_w4a16_tiled<BM, BN, WAVES_M, PF, EPI, F32, LAYOUT, RNJ, F16><<<grid_of(a, BN), 256, 0, s>>>(a);
    return hipGetLastError();
  }
};

template <int BM, int BN, int PF, int KW = 4>
struct SplitK {
  template <int EPI, int F32, int LAYOUT, int RNJ = 0>
  static hipError_t run(const GemmArgs& a, hipStream_t s) {
    gemm_w4a16_sk<BM, BN, PF, EPI, F32, LAYOUT, KW, RNJ><<<grid_of(a, BN), 64 * KW, 0, s>>>(a);
    return hipGetLastError();
  }
};

// Tile lists of at most this capacity (16-row tiles) use the split-K kernel: measured on MI355X at
// one token with 128 experts top-8, 8 tiles (weights streamed from HBM), gate_up takes 6.5 us with
// K split 8 ways against 9.1 us for the tiled kernel, down 4.1 us against 5.1 us.  Swept again with
// HIP events at 1 and 3 tokens: 32-column blocks with K split 4 ways take 9.1 / 14.8 us for gate_up
// against 10.4 / 19.7 us for 64-column blocks split 8 ways.
constexpr int kSplitKMaxTiles = 32;

template <class Cfg, int EPI, int F32>
static hipError_t by_layout(const GemmArgs& a, hipStream_t s) {
  switch (layout_of(a)) {
    case kPacked: return Cfg::template run<EPI, F32, kPacked>(a, s);
    case kCanonFull: return Cfg::template run<EPI, F32, kCanonFull>(a, s);
    default: return Cfg::template run<EPI, F32, kCanonGeneric>(a, s);
  }
}

// The SiLU*mul launch with the routing prologue (16-row tiles): experts per lane group 128 or 512.
template <class Cfg>
static hipError_t routed(const GemmArgs& a, hipStream_t s) {
  constexpr int EPI = MOE_EPI_SILU_MUL;
  const bool small = a.route_E <= 128;
  switch (layout_of(a)) {
    case kPacked:
      return small ? Cfg::template run<EPI, false, kPacked, 2>(a, s) : Cfg::template run<EPI, false, kPacked, 8>(a, s);
    case kCanonFull:
      return small ? Cfg::template run<EPI, false, kCanonFull, 2>(a, s)
                   : Cfg::template run<EPI, false, kCanonFull, 8>(a, s);
    default:
      return small ? Cfg::template run<EPI, false, kCanonGeneric, 2>(a, s)
                   : Cfg::template run<EPI, false, kCanonGeneric, 8>(a, s);
  }
}

// The fp16 path (a.a_f16) of a tiled configuration: SiLU*mul writes fp16 h with block exponents.
template <class Cfg, int EPI, int F32>
static hipError_t by_layout_f16(const GemmArgs& a, hipStream_t s) {
  switch (layout_of(a)) {
    case kPacked: return Cfg::template run<EPI, F32, kPacked, 0, true>(a, s);
    case kCanonFull: return Cfg::template run<EPI, F32, kCanonFull, 0, true>(a, s);
    default: return Cfg::template run<EPI, F32, kCanonGeneric, 0, true>(a, s);
  }
}

template <class Cfg>
static hipError_t by_variant_f16(const GemmArgs& a, hipStream_t s) {
  if (a.epilogue == MOE_EPI_SILU_MUL) return by_layout_f16<Cfg, MOE_EPI_SILU_MUL, kOutH16>(a, s);
  if (a.out_f32 == kOutF16Exp) return by_layout_f16<Cfg, MOE_EPI_NONE, kOutF16Exp>(a, s);
  return by_layout_f16<Cfg, MOE_EPI_NONE, kOutF32>(a, s);
}

template <class Cfg>
static hipError_t by_variant(const GemmArgs& a, hipStream_t s) {
  if (a.epilogue == MOE_EPI_SILU_MUL) return by_layout<Cfg, MOE_EPI_SILU_MUL, kOutBf16>(a, s);
  if (a.out_f32 == kOutF16Exp) return by_layout<Cfg, MOE_EPI_NONE, kOutF16Exp>(a, s);
  if (a.out_f32 == kOutF32) return by_layout<Cfg, MOE_EPI_NONE, kOutF32>(a, s);
  return by_layout<Cfg, MOE_EPI_NONE, kOutBf16>(a, s);
}

// The NONE epilogue (the down projection) of a tiled configuration.
template <class Cfg>
static hipError_t by_variant_none(const GemmArgs& a, hipStream_t s) {
  if (a.out_f32 == kOutF16Exp) return by_layout<Cfg, MOE_EPI_NONE, kOutF16Exp>(a, s);
  if (a.out_f32 == kOutF32) return by_layout<Cfg, MOE_EPI_NONE, kOutF32>(a, s);
  return by_layout<Cfg, MOE_EPI_NONE, kOutBf16>(a, s);
}

template <class Cfg, int EPI, int F32, bool F16 = false>
static hipError_t launch_mm(const GemmArgs& a, hipStream_t s) {
  const int ncols = EPI == MOE_EPI_SILU_MUL ? a.N / 2 : a.N;
  const int bcols = EPI == MOE_EPI_SILU_MUL ? Cfg::BN / 2 : Cfg::BN;
  const int nbn = (ncols + bcols - 1) / bcols;
  gemm_w4a16_mm<Cfg, EPI, F32, F16><<<mm_grid(nbn, a.max_tiles), Cfg::THREADS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs& a, int block_m, hipStream_t stream) {
  if (a.max_tiles <= 0) return hipSuccess;
  // weight rows are addressed by 32-bit offsets within an expert (WRow)
  if ((size_t)a.N * (size_t)a.K / 2 > 0xFFFFF000ull) return hipErrorInvalidValue;
  if (a.a_f16) {
    // the exact fp16 path: 128-row tiles (packed weights) or 64-row tiles (checked by the caller)
    if (block_m == 128) {
      if (a.epilogue == MOE_EPI_SILU_MUL) return launch_mm<MmLarge, MOE_EPI_SILU_MUL, kOutH16, true>(a, stream);
      if (a.out_f32 == kOutF16Exp) return launch_mm<MmLarge, MOE_EPI_NONE, kOutF16Exp, true>(a, stream);
      return launch_mm<MmLarge, MOE_EPI_NONE, kOutF32, true>(a, stream);
    }
    return by_variant_f16<Tiled<64, 256, 1, 1>>(a, stream);
  }
  // (packed SiLU*mul needs N % 32 == 0, checked by the caller: up rows start a 16-row block)
  if (block_m == 128 && a.packed) {
    if (a.epilogue == MOE_EPI_SILU_MUL) return launch_mm<MmLarge, MOE_EPI_SILU_MUL, kOutBf16>(a, stream);
    if (a.out_f32 == kOutF16Exp) return launch_mm<MmLarge, MOE_EPI_NONE, kOutF16Exp>(a, stream);
    if (a.out_f32 == kOutF32) return launch_mm<MmLarge, MOE_EPI_NONE, kOutF32>(a, stream);
    return launch_mm<MmLarge, MOE_EPI_NONE, kOutBf16>(a, stream);
  }
  switch (block_m) {
    case 16:
      // (the routing prologue, a.route_logits, comes with the SiLU*mul epilogue and 16-row tiles only)
      if (a.max_tiles <= kSplitKMaxTiles) {
        if (a.route_logits) return routed<SplitK<16, 32, 2, 4>>(a, stream);
        return by_variant<SplitK<16, 32, 2, 4>>(a, stream);
      }
      // SiLU*mul: 256-column blocks once the grid holds three workgroups per CU (768) with them:
      // measured on MI355X with 128 experts top-8, 32 and 64 tokens: gate_up 39.8 / 41.3 us against
      // 40.4 / 44.0 us for 128-column blocks; at 8 tokens (408 workgroups) 128-column blocks are
      // faster, and with one K step in flight rather than two (22.0 against 23.5 us).  The down
      // projection (K = 768) is fastest with 128-column blocks one step ahead at 8, 32 and 64 tokens:
      // 11.6 / 23.5 / 25.0 us against 13.2 / 24.1 / 26.7 us with 256-column blocks.
      if (a.epilogue == MOE_EPI_SILU_MUL && 8LL * ((a.max_tiles + 7) / 8) * ((a.N / 2 + 127) / 128) >= 768) {
        if (a.route_logits) return routed<Tiled<16, 256, 1, 1>>(a, stream);
        return by_variant<Tiled<16, 256, 1, 1>>(a, stream);
      }
      if (a.route_logits) return routed<Tiled<16, 128, 1, 1>>(a, stream);
      return by_variant<Tiled<16, 128, 1, 1>>(a, stream);
    case 32:
      // 800 tokens, 256 experts top-8 (H 2048, I 512), four runs on one MI355X: gate_up 70.4-71.2 us one
      // K step ahead against 72.1-73.1 us two steps ahead; down 47.2-48.1 us two steps ahead against
      // 47.9-48.9 us one step ahead.  With canonical weights the other way round: the layer took
      // 173.2-174.1 against 176.6-177.4 us.
      if (a.epilogue == MOE_EPI_SILU_MUL) {
        if (!a.packed) return by_variant<Tiled<32, 128, 1, 2>>(a, stream);
        return by_variant<Tiled<32, 128, 1, 1>>(a, stream);
      }
      if (!a.packed) return by_variant_none<Tiled<32, 128, 1, 1>>(a, stream);
      return by_variant_none<Tiled<32, 128, 1, 2>>(a, stream);
    case 64:
      // The down projection in 128-column blocks two K steps ahead (164-168 VGPRs, three workgroups per
      // CU, against 256 VGPRs and two for 64 x 256): measured on MI355X, 8192 tokens over 512 experts
      // top-10 (K = 512) 291 against 307 us, and 4096 tokens over 8 experts top-2 with canonical
      // weights (K = 14336) 1423-1427 against 1887-1892 us.  gate_up keeps 256-column blocks (8192
      // tokens: 379-386 against 410-412 us with 128-column blocks) when the weights are packed; with
      // canonical weights (whose loads take a cross-lane transpose) 128-column blocks two steps ahead
      // are faster there too: 8192 skewed tokens 474-487 against 585 us, 4096 tokens 3144-3151
      // against 3387-3463 us.
      if (a.epilogue != MOE_EPI_SILU_MUL) return by_variant_none<Tiled<64, 128, 1, 2>>(a, stream);
      if (!a.packed) return by_variant<Tiled<64, 128, 1, 2>>(a, stream);
      return by_variant<Tiled<64, 256, 1, 1>>(a, stream);
    default: return by_variant<Tiled<128, 128, 2, 1>>(a, stream);
  }
}

}  // namespace moe
