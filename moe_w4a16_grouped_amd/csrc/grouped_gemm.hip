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
// gfx950 design:
//  * Work list instead of a 3D grid: blockIdx.y indexes the device-side tile list written by
//    moe_align (exact, never a host guess); blockIdx.x is the N block.  Slots past num_tiles exit.
//  * v_mfma_f32_16x16x32_bf16: one MFMA spans exactly one 32-element scale group.  Codes are
//    converted to exact bf16 (hardware FP4 converter, unit scale); the MFMA produces the group's
//    fp32 partial, which is multiplied by the bf16 group scale and added to the fp32 accumulator.
//    (Rounding code*scale to bf16 instead would not keep the layer inside its error bound.)
//  * Weights go HBM -> registers with one 16-byte load per lane per 4 groups (row n, group q of the
//    K step) and a 4x4 cross-quarter transpose (permlane32/16 swaps) into MFMA B-operand order.
//  * Activations (gathered rows for gate_up) are staged through LDS with 16-byte loads and shared by
//    the four waves; the next K step is prefetched into registers while the current one computes.
#include "launch.h"
#include "moe_common.h"

namespace moe {

constexpr int kBK = 128;  // K elements per step: 4 scale groups, 64 bytes of codes per weight row

template <int BM, int BN, int WAVES_M, int EPI, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_w4a16_tiled(GemmArgs p) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int LDA = kBK + 8;  // padded LDS row, bf16 elements
  constexpr int ACH = BM * (kBK / 8) / 256;  // 16-byte A chunks per thread per K step
  static_assert(MI >= 1 && NI >= 1 && ACH >= 1, "tile shape");
  static_assert(EPI != 1 || NI % 2 == 0, "SiLU*mul pairs gate and up blocks");

  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * LDA];
  __shared__ int32_t sRow[BM];

  const int tile = blockIdx.y;
  if (tile >= *p.num_tiles) return;
  const int e = p.tiles[3 * tile], row0 = p.tiles[3 * tile + 1], rows = p.tiles[3 * tile + 2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int l16 = lane & 15, q = lane >> 4;
  const int N = p.N, K = p.K;

  for (int i = tid; i < BM; i += 256) {
    const int r = row0 + (i < rows ? i : 0);
    sRow[i] = p.a_row_of ? p.a_row_of[r] / p.a_row_div : r;
  }

  // Weight rows handled by this lane (one per 16-column block).  For SiLU*mul the first NI/2
  // blocks are gate rows j and the last NI/2 the matching up rows N/2 + j.
  const uint8_t* wp[NI];
  const uint16_t* sp[NI];
  int ncol[NI];
  bool nvalid[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int n;
    if (EPI == MOE_EPI_SILU_MUL) {
      const int half = NI / 2;
      const int j = blockIdx.x * (BN / 2) + wn * (WN / 2) + (ni % half) * 16 + l16;
      nvalid[ni] = j < N / 2;
      ncol[ni] = j;
      n = ni < half ? j : N / 2 + j;
    } else {
      n = blockIdx.x * BN + wn * WN + ni * 16 + l16;
      nvalid[ni] = n < N;
      ncol[ni] = n;
    }
    const int nn = nvalid[ni] ? n : 0;
    wp[ni] = p.Wq + ((size_t)e * N + nn) * (size_t)(K / 2) + q * 16;
    sp[ni] = p.Ws + ((size_t)e * N + nn) * (size_t)(K / kGroup);
  }
  __syncthreads();

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[ACH];
  u32x4 breg[NI];
  uint32_t sreg[NI][4];
  const int nks = (K + kBK - 1) / kBK;
  const int kgroups = K / kGroup;

  auto load_step = [&](int ks) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 4, col = (c & 15) * 8;
      const int kk = ks * kBK + col;
      areg[i] = kk < K ? *reinterpret_cast<const u32x4*>(p.A + (size_t)sRow[row] * K + kk)
                       : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      breg[ni] = (ks * 4 + q) < kgroups ? *reinterpret_cast<const u32x4*>(wp[ni] + (size_t)ks * 64)
                                        : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int g = 0; g < 4; ++g) sreg[ni][g] = (ks * 4 + g) < kgroups ? sp[ni][ks * 4 + g] : 0u;
    }
  };

  load_step(0);
  for (int ks = 0; ks < nks; ++ks) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&sA[(c >> 4) * LDA + (c & 15) * 8]) = areg[i];
    }
    u32x4 bcur[NI];
    uint32_t scur[NI][4];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      bcur[ni] = breg[ni];
#pragma unroll
      for (int g = 0; g < 4; ++g) scur[ni][g] = sreg[ni][g];
    }
    __syncthreads();
    if (ks + 1 < nks) load_step(ks + 1);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) bcur[ni] = quarter_transpose(bcur[ni]);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x8 bf[NI];
      float sc[NI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        bf[ni] = e2m1x8_to_bf16(bcur[ni][g]);
        sc[ni] = bf16_bits_to_f32(scur[ni][g]);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const bf16x8 af =
            *reinterpret_cast<const bf16x8*>(&sA[(wm * WM + mi * 16 + l16) * LDA + g * 32 + q * 8]);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const f32x4 part = mfma16x16x32(af, bf[ni], f32x4{0.f, 0.f, 0.f, 0.f});
          acc[mi][ni] += sc[ni] * part;
        }
      }
    }
    __syncthreads();
  }

  // Epilogue: lane holds rows wm*WM + mi*16 + 4q + r of column ncol[ni].
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * WM + mi * 16 + q * 4 + r;
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

template <int BM, int BN, int WAVES_M, int EPI, bool OUT_F32>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t stream) {
  const int ncols = EPI == MOE_EPI_SILU_MUL ? a.N / 2 : a.N;
  const int bcols = EPI == MOE_EPI_SILU_MUL ? BN / 2 : BN;
  const dim3 grid((ncols + bcols - 1) / bcols, a.max_tiles);
  gemm_w4a16_tiled<BM, BN, WAVES_M, EPI, OUT_F32><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

template <int BM, int BN, int WAVES_M>
static hipError_t dispatch_epi(const GemmArgs& a, hipStream_t stream) {
  if (a.epilogue == MOE_EPI_SILU_MUL) return launch_tiled<BM, BN, WAVES_M, MOE_EPI_SILU_MUL, false>(a, stream);
  if (a.out_f32) return launch_tiled<BM, BN, WAVES_M, MOE_EPI_NONE, true>(a, stream);
  return launch_tiled<BM, BN, WAVES_M, MOE_EPI_NONE, false>(a, stream);
}

hipError_t launch_grouped_gemm(const GemmArgs& a, int block_m, hipStream_t stream) {
  if (a.max_tiles <= 0) return hipSuccess;
  switch (block_m) {
    case 16: return dispatch_epi<16, 128, 1>(a, stream);
    case 32: return dispatch_epi<32, 128, 1>(a, stream);
    case 64: return dispatch_epi<64, 128, 2>(a, stream);
    default: return dispatch_epi<128, 128, 2>(a, stream);
  }
}

}  // namespace moe
