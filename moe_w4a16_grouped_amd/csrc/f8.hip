// FP8 (W8A8, per-1x128) variant of the layer on gfx950's FP8 matrix cores.
//
// Format (the ATOM page "AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍", section
// "6.1 Linear：按量化类型分派 GEMM", lists per-1x128 FP8 served by an a8w8 block-scale GEMM; section
// "8.1 MoE 路径：路由、专家并行与 MORI 通信" names an FP8 path of the fused MoE; section "8.2 量化并非单一
// 格式，而是一套执行契约" lists dynamic activation quantization as part of a format's contract): weights
// and activations are OCP FP8 E4M3 codes, one byte per element, K-contiguous rows, with one fp32
// scale per row and block of 128 consecutive K elements on both operands.  Activations are quantized
// on the fly, per block: s = amax / 448 (fp32), code = nearest E4M3 value of the fp32 quotient v / s
// (ties to even); s == 0 gives codes 0.
//
// Products: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E4M3 (format 0) and unit E8M0
// scales covers one 128-element K block of a 16 x 16 output block per instruction; its fp32 partial
// is multiplied by the two block scales (activation row, weight row) in fp32 and added to the fp32
// accumulator, so one K step is one scale block.  Each lane supplies 32 bytes of each operand, row
// l % 16, K bytes [16 (l / 16), +16) and [64 + 16 (l / 16), +16) of the block: two 16-byte loads per
// lane that each read 64 contiguous bytes of a row per 16-lane quarter.  A and B fragments use the
// same K assignment, so the dot product is the same whichever K order the instruction uses inside.
#include "launch.h"
#include "moe_common.h"

namespace moe {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kF8Block = 128;   // K elements per scale (and per K step)
constexpr float kE4M3Max = 448.0f;

// Inclusive max over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1 within the row).
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(o));
}
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_max<0x128>(v);  // row_ror:8
  v = dpp_max<0x124>(v);  // row_ror:4
  v = dpp_max<0x122>(v);  // row_ror:2
  v = dpp_max<0x121>(v);  // row_ror:1
  return v;
}

// Four E4M3 codes of v[j] / s, j < 4 (correctly rounded fp32 quotient, clamped to +-448, then the
// hardware conversion: round to nearest even).
__device__ __forceinline__ uint32_t f8_encode4(const float* v, float s) {
  float q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = fminf(fmaxf(v[j] / s, -kE4M3Max), kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
  return (uint32_t)w;
}

// ---------------------------------------------------------------------------------------------------
// Activation quantization: 16 threads (one DPP row) per 128-element block, 8 elements each; the
// block maximum is reduced across the row.  IN_F32: fp32 input, else bf16.
template <bool IN_F32>
__global__ __launch_bounds__(256) void f8_quant_kernel(const void* __restrict__ x, long long nblocks, int K,
                                                       uint8_t* __restrict__ q, float* __restrict__ s) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long blk = gid >> 4;
  const int part = (int)(gid & 15);
  const bool live = blk < nblocks;  // whole rows of 16 lanes are live or not
  const long long b = live ? blk : 0;
  const int kb = K / kF8Block;
  const long long row = b / kb;
  const size_t e0 = (size_t)row * K + (size_t)(b % kb) * kF8Block + part * 8;
  float v[8];
  if (IN_F32) {
    const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + e0);
    const f32x4 a = src[0], c = src[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[4 + j] = c[j]; }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + e0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = row16_max(amax);
  const float sc = amax / kE4M3Max;
  u32x2 out = {0u, 0u};
  if (sc != 0.f) {
    out[0] = f8_encode4(v, sc);
    out[1] = f8_encode4(v + 4, sc);
  }
  if (!live) return;
  *reinterpret_cast<u32x2*>(q + e0) = out;
  if (part == 0) s[b] = sc;
}

hipError_t launch_f8_quant(const void* x, bool in_f32, long long rows, int K, uint8_t* q, float* s,
                           hipStream_t stream) {
  const long long nblocks = rows * (K / kF8Block);
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)((nblocks * 16 + 255) / 256));
  if (in_f32) f8_quant_kernel<true><<<grid, 256, 0, stream>>>(x, nblocks, K, q, s);
  else f8_quant_kernel<false><<<grid, 256, 0, stream>>>(x, nblocks, K, q, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------
// Grouped FP8 GEMM over the device-side tile list (the list moe_align writes).  A workgroup of four
// waves computes a BM x BN tile; the waves split K KW ways and N 4/KW ways.  Each wave loads its
// operand fragments straight into a register ring PF K steps deep (activation rows gathered through
// a_row_of; padding rows repeat the tile's first row), so the main loop has no barrier.  The tile's
// activation scales are staged once in LDS as [K step][row], so that the four row scales a lane's
// outputs need come from one 16-byte LDS read per step; the weight row scales travel with the
// weight fragments.  K-split partials are added in LDS in wave order.
// Epilogues: NONE stores fp32 or bf16 [rows, N]; SILU_MUL stores h = silu(gate) * up in fp32
// [rows, N/2] (gate rows [0, N/2) of the weight, up rows [N/2, N)), which the next projection
// quantizes.
template <int BM, int BN, int KW, int PF, int EPI, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_f8_kernel(F8GemmArgs p) {
  constexpr int WNS = 4 / KW;   // waves along N
  constexpr int WN = BN / WNS;  // columns per wave
  constexpr int MI = BM / 16, NI = WN / 16;
  constexpr int NS = PF + 1;
  static_assert(KW * WNS == 4 && NI >= 1 && MI >= 1, "tile shape");
  static_assert(EPI != MOE_EPI_SILU_MUL || NI % 2 == 0, "SiLU*mul pairs gate and up blocks");
  __shared__ __attribute__((aligned(16))) float red[KW > 1 ? WNS * (KW - 1) * 64 * MI * NI * 4 : 1];
  extern __shared__ __attribute__((aligned(16))) float sa_lds[];  // [nks][BM] activation scales

  const int N = p.N, K = p.K;
  const int nks = K / kF8Block;
  const int nbn = EPI == MOE_EPI_SILU_MUL ? (N / 2 + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  int tile, nb;
  if (!xcd_tile(linear_block(), nbn, *p.num_tiles, tile, nb)) return;
  const int e = p.tiles[3 * tile], row0 = p.tiles[3 * tile + 1], rows = p.tiles[3 * tile + 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave % KW, wn = wave / KW;
  const int l16 = lane & 15, q = lane >> 4;
  const int per = (nks + KW - 1) / KW;
  const int s_begin = min(nks, wk * per), s_end = min(nks, s_begin + per);

  // activation scales of the tile's rows, [K step][row]
  for (int i = tid; i < BM * nks; i += 256) {
    const int row = i % BM, ks = i / BM;
    const int r = row0 + (row < rows ? row : 0);
    const int ar = p.a_row_of ? p.a_row_of[r] / p.a_row_div : r;
    sa_lds[i] = p.As[(size_t)ar * nks + ks];
  }
  // activation fragments: row mi * 16 + l16 of the tile
  const uint8_t* aq[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int i = mi * 16 + l16;
    const int r = row0 + (i < rows ? i : 0);
    const int ar = p.a_row_of ? p.a_row_of[r] / p.a_row_div : r;
    aq[mi] = p.Aq + (size_t)ar * K + 16 * q;
  }
  // weight fragments: SILU_MUL pairs gate block j with up block j (rows N/2 + j)
  const uint8_t* wq[NI];
  const float* ws[NI];
  int ncol[NI];
  bool nvalid[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int n;
    if (EPI == MOE_EPI_SILU_MUL) {
      const int j = nb * (BN / 2) + wn * (WN / 2) + (ni % (NI / 2)) * 16 + l16;
      nvalid[ni] = j < N / 2;
      ncol[ni] = j;
      n = ni < NI / 2 ? j : N / 2 + j;
    } else {
      n = nb * BN + wn * WN + ni * 16 + l16;
      nvalid[ni] = n < N;
      ncol[ni] = n;
    }
    if (!nvalid[ni]) n = 0;
    wq[ni] = p.Wq + ((size_t)e * N + n) * K + 16 * q;
    ws[ni] = p.Ws + ((size_t)e * N + n) * nks;
  }
  __syncthreads();

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[NS][MI][2], breg[NS][NI][2];
  float bsc[NS][NI];
  auto load_step = [&](int s, int u) {
    s = min(s, s_end - 1);  // prefetches past this wave's range re-read its last step (unused)
    const size_t off = (size_t)s * kF8Block;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      breg[u][ni][0] = *reinterpret_cast<const u32x4*>(wq[ni] + off);
      breg[u][ni][1] = *reinterpret_cast<const u32x4*>(wq[ni] + off + 64);
      bsc[u][ni] = ws[ni][s];
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      areg[u][mi][0] = *reinterpret_cast<const u32x4*>(aq[mi] + off);
      areg[u][mi][1] = *reinterpret_cast<const u32x4*>(aq[mi] + off + 64);
    }
  };
  auto compute_step = [&](int s, int u) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const u32x4 a0 = areg[u][mi][0], a1 = areg[u][mi][1];
      const i32x8 a8 = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      const f32x4 sa = *reinterpret_cast<const f32x4*>(&sa_lds[s * BM + mi * 16 + 4 * q]);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const u32x4 b0 = breg[u][ni][0], b1 = breg[u][ni][1];
        const i32x8 b8 = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
        const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                            127, 0, 127);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][ni][r] = fmaf(sa[r] * bsc[u][ni], part[r], acc[mi][ni][r]);
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

  // K-split partials, added in wave order by the first wave of each N group
  constexpr int PER = MI * NI * 4;
  if constexpr (KW > 1) {
    if (wk > 0) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[(((wn * (KW - 1) + wk - 1) * 64) + lane) * PER + (mi * NI + ni) * 4 + r] = acc[mi][ni][r];
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
          for (int r = 0; r < 4; ++r)
            acc[mi][ni][r] += red[(((wn * (KW - 1) + w) * 64) + lane) * PER + (mi * NI + ni) * 4 + r];
  }

#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mi * 16 + 4 * q + r;
      if (row >= rows) continue;
      const size_t orow = (size_t)(row0 + row);
      if constexpr (EPI == MOE_EPI_SILU_MUL) {
#pragma unroll
        for (int ni = 0; ni < NI / 2; ++ni) {
          if (!nvalid[ni]) continue;
          const float g = acc[mi][ni][r], u = acc[mi][ni + NI / 2][r];
          static_cast<float*>(p.C)[orow * (N / 2) + ncol[ni]] = silu_f32(g) * u;
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

template <int BM, int BN, int KW, int PF>
static hipError_t launch_f8_cfg(const F8GemmArgs& a, hipStream_t s) {
  const int ncols = a.epilogue == MOE_EPI_SILU_MUL ? a.N / 2 : a.N;
  const int bcols = a.epilogue == MOE_EPI_SILU_MUL ? BN / 2 : BN;
  const dim3 grid = grid2d(8LL * ((a.max_tiles + 7) / 8) * ((ncols + bcols - 1) / bcols));
  const size_t lds = (size_t)BM * (a.K / kF8Block) * sizeof(float);
  if (a.epilogue == MOE_EPI_SILU_MUL) gemm_f8_kernel<BM, BN, KW, PF, MOE_EPI_SILU_MUL, true><<<grid, 256, lds, s>>>(a);
  else if (a.out_f32) gemm_f8_kernel<BM, BN, KW, PF, MOE_EPI_NONE, true><<<grid, 256, lds, s>>>(a);
  else gemm_f8_kernel<BM, BN, KW, PF, MOE_EPI_NONE, false><<<grid, 256, lds, s>>>(a);
  return hipGetLastError();
}

// Tile lists of at most this capacity (16-row tiles) split K four ways (decode).
constexpr int kF8SplitKMaxTiles = 32;

hipError_t launch_grouped_gemm_f8(const F8GemmArgs& a, int block_m, hipStream_t stream) {
  if (a.max_tiles <= 0) return hipSuccess;
  switch (block_m) {
    case 16:
      if (a.max_tiles <= kF8SplitKMaxTiles) return launch_f8_cfg<16, 64, 4, 2>(a, stream);
      return launch_f8_cfg<16, 128, 1, 2>(a, stream);
    case 32: return launch_f8_cfg<32, 128, 1, 2>(a, stream);
    default: return launch_f8_cfg<64, 128, 1, 1>(a, stream);
  }
}

}  // namespace moe
