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
//  * Work list instead of a 3D grid: blockIdx.y indexes the device-side tile list written by
//    moe_align (exact, never a host guess); blockIdx.x is the N block.  Slots past num_tiles exit.
//  * v_mfma_f32_16x16x32_bf16: one MFMA spans exactly one 32-element scale group.  Codes are
//    converted to exact bf16 (hardware FP4 converter, unit scale); the MFMA produces the group's
//    fp32 partial, which is multiplied by the bf16 group scale and added to the fp32 accumulator.
//    (Rounding code*scale to bf16 instead would not keep the layer inside its error bound.)
//  * Weights go HBM -> registers.  Canonical layout: one 16-byte load per lane per 4 groups (row n,
//    group q of the K step) followed by a 4x4 cross-quarter transpose (permlane32/16 swaps) into
//    MFMA B-operand order.  Packed layout (prepack.hip): the same registers come from one linear
//    1 KB load per wave, and the 16 rows x 4 group scales from one 128-byte load.
//  * Loads are never behind a branch: addresses are clamped into range and out-of-range data is
//    neutralised where it is consumed, so each step waits only for its own loads.
#include "launch.h"
#include "moe_common.h"

namespace moe {

constexpr int kBK = 128;  // K elements per step: 4 scale groups

enum Layout { kCanonGeneric = 0, kCanonFull = 1, kPacked = 2 };

// Weight-row block of one lane: canonical pointers or packed block base.
struct WRow {
  const uint8_t* q;   // canonical: row start (+ lane offset); packed: block (e, nb, ks=0) + lane * 16
  const uint16_t* s;  // canonical: scale row start; packed: scale block (e, nb, ks=0) + (lane % 16) * 4
};

template <int LAYOUT>
__device__ __forceinline__ WRow wrow_of(const GemmArgs& p, int e, int n, int q, int lane) {
  const int N = p.N, K = p.K;
  WRow w;
  if (LAYOUT == kPacked) {
    const size_t blk = ((size_t)e * (N / 16) + n / 16) * (size_t)(K / kBK);
    w.q = p.Wq + blk * 1024 + lane * 16;
    w.s = p.Ws + blk * 64 + (lane & 15) * 4;
  } else {
    w.q = p.Wq + ((size_t)e * N + n) * (size_t)(K / 2) + (LAYOUT == kCanonFull ? q * 16 : 0);
    w.s = p.Ws + ((size_t)e * N + n) * (size_t)(K / kGroup);
  }
  return w;
}

// Load the codes and scales of K step ks (groups 4ks..4ks+3) for one lane.
// sq: kCanonGeneric -> one bf16 per entry; otherwise [0], [1] = raw bf16 pairs.
template <int LAYOUT>
__device__ __forceinline__ void load_w(const WRow& w, int ks, int q, int kgroups, u32x4& b, uint32_t (&sq)[4]) {
  if (LAYOUT == kPacked) {
    b = *reinterpret_cast<const u32x4*>(w.q + (size_t)ks * 1024);
    const u32x2 v = *reinterpret_cast<const u32x2*>(w.s + (size_t)ks * 64);
    sq[0] = v[0];
    sq[1] = v[1];
  } else if (LAYOUT == kCanonFull) {
    b = *reinterpret_cast<const u32x4*>(w.q + (size_t)ks * 64);
    const u32x2 v = *reinterpret_cast<const u32x2*>(w.s + (size_t)ks * 4);
    sq[0] = v[0];
    sq[1] = v[1];
  } else {
    const int gq = min(ks * 4 + q, kgroups - 1);
    b = *reinterpret_cast<const u32x4*>(w.q + (size_t)gq * 16);
#pragma unroll
    for (int g = 0; g < 4; ++g) sq[g] = w.s[min(ks * 4 + g, kgroups - 1)];
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

template <int EPI, bool OUT_F32, int MI, int NI>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const f32x4 (&acc)[MI][NI], int row_base, int row0,
                                           int rows, int q, const int (&ncol)[NI], const bool (&nvalid)[NI]) {
  const int N = p.N;
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
          if (OUT_F32) static_cast<float*>(p.C)[orow * N + ncol[ni]] = acc[mi][ni][r];
          else static_cast<uint16_t*>(p.C)[orow * N + ncol[ni]] = f32_to_bf16_bits(acc[mi][ni][r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------------
// Tiled kernel: BM x BN tile per 256-thread workgroup, waves split it WAVES_M x WAVES_N; the
// activation tile of each K step is staged once in LDS (double buffer, one barrier per step) and
// shared by the waves.  PF = K steps in flight ahead of the one computed (ring of PF+1 slots).
template <int BM, int BN, int WAVES_M, int PF, int EPI, bool OUT_F32, int LAYOUT>
__global__ __launch_bounds__(256) void gemm_w4a16_tiled(GemmArgs p) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int LDA = kBK + 8;               // padded LDS row (bf16 elements)
  constexpr int ACH = BM * (kBK / 8) / 256;  // 16-byte activation chunks per thread per step
  constexpr int NS = PF + 1;
  static_assert(MI >= 1 && NI >= 1 && ACH >= 1, "tile shape");
  static_assert(EPI != MOE_EPI_SILU_MUL || NI % 2 == 0, "SiLU*mul pairs gate and up blocks");

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDA];
  __shared__ int32_t sRow[BM];

  const int tile = blockIdx.y;
  if (tile >= *p.num_tiles) return;
  const int e = p.tiles[3 * tile], row0 = p.tiles[3 * tile + 1], rows = p.tiles[3 * tile + 2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int l16 = lane & 15, q = lane >> 4;
  const int K = p.K;
  const int kgroups = K / kGroup;
  const int nks = (K + kBK - 1) / kBK;

  for (int i = tid; i < BM; i += 256) {
    const int r = row0 + (i < rows ? i : 0);
    sRow[i] = p.a_row_of ? p.a_row_of[r] / p.a_row_div : r;
  }
  WRow wr[NI];
  int ncol[NI];
  bool nvalid[NI];
  const int col0 = EPI == MOE_EPI_SILU_MUL ? blockIdx.x * (BN / 2) + wn * (WN / 2) : blockIdx.x * BN + wn * WN;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int n;
    column_of<EPI, NI>(p, col0, ni, l16, n, ncol[ni], nvalid[ni]);
    wr[ni] = wrow_of<LAYOUT>(p, e, n, q, lane);
  }
  __syncthreads();

  const uint16_t* arow[ACH];
  int acol[ACH], alds[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + 256 * i;
    const int row = c / (kBK / 8);
    acol[i] = (c % (kBK / 8)) * 8;
    alds[i] = row * LDA + acol[i];
    arow[i] = p.A + (size_t)sRow[row] * K;
  }

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[NS][ACH];
  u32x4 breg[NS][NI];
  uint32_t sreg[NS][NI][4];

  auto load_step = [&](int s, int u) {
    s = min(s, nks - 1);  // prefetches past the end re-read the last step (never used)
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      areg[u][i] = *reinterpret_cast<const u32x4*>(arow[i] + min(s * kBK + acol[i], K - 8));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) load_w<LAYOUT>(wr[ni], s, q, kgroups, breg[u][ni], sreg[u][ni]);
  };

  auto compute_step = [&](const uint16_t* a_lds, int u) {
    u32x4 bt[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) bt[ni] = b_operands<LAYOUT>(breg[u][ni]);
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
          acc[mi][ni] += sc[ni] * part;
        }
      }
    }
  };

  // One K step: stage A(s) from ring slot u into LDS buffer s&1, sync, optionally prefetch step
  // s+PF into the slot freed by step s-1, then compute step s.  Activation chunks past K are zeroed
  // here, which makes the matching partial products exactly zero whatever the clamped codes hold.
  auto step = [&](int s, int u, bool prefetch) {
    uint16_t* a_lds = sA[s & 1];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      u32x4 v = areg[u][i];
      if (LAYOUT == kCanonGeneric && s * kBK + acol[i] >= K) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&a_lds[alds[i]]) = v;
    }
    __syncthreads();
    if (prefetch) load_step(s + PF, (u + PF) % NS);
    compute_step(a_lds, u);
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

  store_tile<EPI, OUT_F32, MI, NI>(p, acc, wm * WM, row0, rows, q, ncol, nvalid);
}

// ---------------------------------------------------------------------------------------------------
// Streaming kernel for tiles of at most 32 rows (decode and few-rows-per-expert prefill), where the
// weight stream from HBM is the bound.  The four waves split K into contiguous ranges; each wave
// loads its own activation fragments (16-byte loads, rows gathered through a_row_of; padding rows
// repeat the tile's first row, which the load coalescer merges) and its weights straight into a
// PF-deep register ring, so the main loop has no LDS traffic and no barrier.  The four partial sums
// are reduced through LDS once per tile, in wave order.
template <int BM, int BN, int PF, int EPI, bool OUT_F32, int LAYOUT>
__global__ __launch_bounds__(256) void gemm_w4a16_sk(GemmArgs p) {
  constexpr int MI = BM / 16, NI = BN / 16;
  static_assert(MI >= 1 && MI <= 2 && NI >= 1, "tile shape");
  static_assert(EPI != MOE_EPI_SILU_MUL || NI % 2 == 0, "SiLU*mul pairs gate and up blocks");
  constexpr int NS = PF + 1;

  __shared__ __attribute__((aligned(16))) float red[3 * 64 * MI * NI * 4];

  const int tile = blockIdx.y;
  if (tile >= *p.num_tiles) return;
  const int e = p.tiles[3 * tile], row0 = p.tiles[3 * tile + 1], rows = p.tiles[3 * tile + 2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
  const int K = p.K;
  const int kgroups = K / kGroup;
  const int nks = (K + kBK - 1) / kBK;
  const int per = (nks + 3) / 4;  // steps per wave (contiguous K ranges)
  const int s_begin = min(nks, wk * per), s_end = min(nks, s_begin + per);
  const bool m1 = MI > 1 && rows > 16;  // second 16-row block present (wave-uniform)

  const uint16_t* arow[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int i = mi * 16 + l16;
    const int r = row0 + (i < rows ? i : 0);
    arow[mi] = p.A + (size_t)(p.a_row_of ? p.a_row_of[r] / p.a_row_div : r) * K + q * 8;
  }
  WRow wr[NI];
  int ncol[NI];
  bool nvalid[NI];
  const int col0 = blockIdx.x * (EPI == MOE_EPI_SILU_MUL ? BN / 2 : BN);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int n;
    column_of<EPI, NI>(p, col0, ni, l16, n, ncol[ni], nvalid[ni]);
    wr[ni] = wrow_of<LAYOUT>(p, e, n, q, lane);
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
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        areg[u][mi][g] = *reinterpret_cast<const u32x4*>(arow[mi] + min(s * kBK + g * 32, K - 32));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) load_w<LAYOUT>(wr[ni], s, q, kgroups, breg[u][ni], sreg[u][ni]);
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
        load_step(s0 + u + PF, (u + PF) % NS);
        compute_step(s0 + u, u);
      }
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (s0 + u < s_end) compute_step(s0 + u, u);
  }

  // K-slice reduction in wave order: waves 1..3 park their sums, wave 0 adds them.
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
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][ni][r] += red[(w * 64 + lane) * PER + (mi * NI + ni) * 4 + r];
  store_tile<EPI, OUT_F32, MI, NI>(p, acc, 0, row0, rows, q, ncol, nvalid);
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
  return dim3((ncols + bcols - 1) / bcols, a.max_tiles);
}

template <int BM, int BN, int WAVES_M, int PF>
struct Tiled {
  template <int EPI, bool F32, int LAYOUT>
  static hipError_t run(const GemmArgs& a, hipStream_t s) {
    gemm_w4a16_tiled<BM, BN, WAVES_M, PF, EPI, F32, LAYOUT><<<grid_of(a, BN), 256, 0, s>>>(a);
    return hipGetLastError();
  }
};

template <int BM, int BN, int PF>
struct Streaming {
  template <int EPI, bool F32, int LAYOUT>
  static hipError_t run(const GemmArgs& a, hipStream_t s) {
    gemm_w4a16_sk<BM, BN, PF, EPI, F32, LAYOUT><<<grid_of(a, BN), 256, 0, s>>>(a);
    return hipGetLastError();
  }
};

template <class Cfg, int EPI, bool F32>
static hipError_t by_layout(const GemmArgs& a, hipStream_t s) {
  switch (layout_of(a)) {
    case kPacked: return Cfg::template run<EPI, F32, kPacked>(a, s);
    case kCanonFull: return Cfg::template run<EPI, F32, kCanonFull>(a, s);
    default: return Cfg::template run<EPI, F32, kCanonGeneric>(a, s);
  }
}

template <class Cfg>
static hipError_t by_variant(const GemmArgs& a, hipStream_t s) {
  if (a.epilogue == MOE_EPI_SILU_MUL) return by_layout<Cfg, MOE_EPI_SILU_MUL, false>(a, s);
  if (a.out_f32) return by_layout<Cfg, MOE_EPI_NONE, true>(a, s);
  return by_layout<Cfg, MOE_EPI_NONE, false>(a, s);
}

hipError_t launch_grouped_gemm(const GemmArgs& a, int block_m, hipStream_t stream) {
  if (a.max_tiles <= 0) return hipSuccess;
  switch (block_m) {
    case 16: return by_variant<Tiled<16, 128, 1, 3>>(a, stream);
    case 32: return by_variant<Tiled<32, 128, 1, 3>>(a, stream);
    case 64: return by_variant<Tiled<64, 128, 1, 2>>(a, stream);
    default: return by_variant<Tiled<128, 128, 2, 1>>(a, stream);
  }
}

}  // namespace moe
