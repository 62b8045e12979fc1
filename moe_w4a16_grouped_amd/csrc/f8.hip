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

// ---------------------------------------------------------------------------------------------------
// Large-tile FP8 kernel for MFMA-bound shapes (hundreds of rows per expert).  A 128 x 256 output tile
// per 512-thread workgroup: 8 waves (2 along M x 4 along N), 64 x 64 each, two waves per SIMD so one's
// scale arithmetic can overlap the other's matrix instructions.  Per K step the tile's activation
// codes (128 rows x 128 B, gathered rows), weight codes (256 rows x 128 B) and both operands' row
// scales reach LDS by direct global->LDS loads, through three stages with one barrier per step.  Code
// rows are 128 B with their 16-byte chunks XOR-swizzled by (row / 2) % 8, so the sixteen rows a
// fragment read touches fall in sixteen distinct bank groups.  Same products, scale arithmetic and K
// order as gemm_f8_kernel, so the results are bit-identical to it.
// SILU_MUL with OUT == 2 quantizes h in the epilogue: a workgroup holds 128 h columns of each of its
// rows, exactly one 1x128 block, so h goes through LDS once and one DPP row of 16 lanes per row takes
// the block maximum and writes the E4M3 codes and the scale, with the arithmetic of f8_quant_kernel
// (bit-identical to storing fp32 h and quantizing it there).
constexpr int kF8MmBM = 128, kF8MmBN = 256;
constexpr int kF8MmHLD = kF8MmBN / 2 + 4;  // padded LDS row of the h tile (floats)
constexpr int kF8MmA = kF8MmBM * 128, kF8MmB = kF8MmBN * 128;  // code bytes per stage
constexpr int kF8MmStage = kF8MmA + kF8MmB + (kF8MmBM + kF8MmBN) * 4;

// Direct global->LDS 4-byte load (lane l writes LDS bytes [4l, 4l+4) after the wave-uniform base).
__device__ __forceinline__ void g2lds4(const void* g, void* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  asm volatile("global_load_lds_dword %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ int f8_swz(int row) { return (row >> 1) & 7; }

// The NONE epilogue of gemm_f8_mm with fp16 output and in-band exponents (OUT 3), one 16-row block at a
// time (fewer live registers); padding rows are left out of the exponent test.
template <int MI, int NI>
__device__ __forceinline__ void f8_mm_store_f16e(const F8GemmArgs& p, const f32x4 (&acc)[MI][NI], int nb, int wm,
                                                 int wn, int row0, int rows, int q, int l16) {
  int ncol[NI];
  bool nvalid[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    ncol[ni] = nb * kF8MmBN + wn * 64 + ni * 16 + l16;
    nvalid[ni] = ncol[ni] < p.N;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
    store_f16e<1, NI, true>(static_cast<uint16_t*>(p.C), p.C_side, p.N,
                            reinterpret_cast<const f32x4(&)[1][NI]>(acc[mi]), wm * 64 + mi * 16, row0, rows, q, ncol,
                            nvalid);
}

template <int EPI, int OUT, int NSTAGE>
__global__ __launch_bounds__(512) void gemm_f8_mm(F8GemmArgs p) {
  constexpr int MI = 4, NI = 4;
  constexpr bool OUT_F32 = OUT == 1;
  static_assert(OUT != 2 || EPI == MOE_EPI_SILU_MUL, "quantized output is h");
  static_assert(NSTAGE * kF8MmStage >= kF8MmBM * kF8MmHLD * 4, "stages also hold the h tile");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NSTAGE * kF8MmStage];
  __shared__ int32_t sRow[kF8MmBM];
  const int N = p.N, K = p.K;
  const int ncols = EPI == MOE_EPI_SILU_MUL ? N / 2 : N;
  const int bcols = EPI == MOE_EPI_SILU_MUL ? kF8MmBN / 2 : kF8MmBN;
  const int nbn = (ncols + bcols - 1) / bcols;
  int tile, nb;
  if (!mm_work(linear_block(), nbn, *p.num_tiles, tile, nb)) return;
  const int e = p.tiles[3 * tile], row0 = p.tiles[3 * tile + 1], rows = p.tiles[3 * tile + 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int l16 = lane & 15, q = lane >> 4;
  const int nks = K / kF8Block;

  for (int i = tid; i < kF8MmBM; i += 512) {
    const int r = row0 + (i < rows ? i : 0);
    sRow[i] = p.a_row_of ? p.a_row_of[r] / p.a_row_div : r;
  }
  __syncthreads();

  // weight row of tile column nt (0..255): SILU_MUL puts the 128 gate rows first, then their up rows
  auto wrow = [&](int nt) -> int {
    int n;
    if (EPI == MOE_EPI_SILU_MUL) {
      const int j = nb * (kF8MmBN / 2) + (nt & 127);
      n = j < N / 2 ? (nt < 128 ? j : N / 2 + j) : 0;
    } else {
      n = nb * kF8MmBN + nt;
      if (n >= N) n = 0;
    }
    return n;
  };
  // sources of this wave's direct loads: code instructions cover 8 rows each (lane l: row l / 8,
  // LDS chunk l % 8, which holds the row's global chunk (l % 8) ^ swizzle)
  const uint8_t* a_src[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 8 * (2 * wave + t) + (lane >> 3);
    a_src[t] = p.Aq + (size_t)sRow[r] * K + 16 * ((lane & 7) ^ f8_swz(r));
  }
  const uint8_t* b_src[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int nt = 8 * (4 * wave + t) + (lane >> 3);
    b_src[t] = p.Wq + ((size_t)e * N + wrow(nt)) * K + 16 * ((lane & 7) ^ f8_swz(nt));
  }
  // scales: waves 0, 1 the 128 activation rows, waves 2..5 the 256 weight rows (one float per lane)
  const float* s_src = nullptr;
  if (wave < 2) s_src = p.As + (size_t)sRow[64 * wave + lane] * nks;
  else if (wave < 6) s_src = p.Ws + ((size_t)e * N + wrow(64 * (wave - 2) + lane)) * nks;

  auto issue = [&](int ks, int stage) {
    uint8_t* st = smem + stage * kF8MmStage;
#pragma unroll
    for (int t = 0; t < 2; ++t) g2lds16(a_src[t] + (size_t)ks * 128, st + (2 * wave + t) * 1024);
#pragma unroll
    for (int t = 0; t < 4; ++t) g2lds16(b_src[t] + (size_t)ks * 128, st + kF8MmA + (4 * wave + t) * 1024);
    if (wave < 2) g2lds4(s_src + ks, st + kF8MmA + kF8MmB + wave * 256);
    else if (wave < 6) g2lds4(s_src + ks, st + kF8MmA + kF8MmB + kF8MmBM * 4 + (wave - 2) * 256);
  };

  // tile columns of this wave's four 16-column blocks
  int ntile[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    ntile[ni] = EPI == MOE_EPI_SILU_MUL ? (ni < 2 ? wn * 32 + ni * 16 : 128 + wn * 32 + (ni - 2) * 16) + l16
                                        : wn * 64 + ni * 16 + l16;

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto frag = [&](const uint8_t* base, int row) -> i32x8 {
    const int sw = f8_swz(row);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + row * 128 + 16 * (q ^ sw));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + row * 128 + 16 * ((4 + q) ^ sw));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  auto compute = [&](int stage) {
    const uint8_t* st = smem + stage * kF8MmStage;
    const float* sa = reinterpret_cast<const float*>(st + kF8MmA + kF8MmB);
    const float* sb = sa + kF8MmBM;
    i32x8 bf[NI];
    float sw[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      bf[ni] = frag(st + kF8MmA, ntile[ni]);
      sw[ni] = sb[ntile[ni]];
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int r = wm * 64 + mi * 16;
      const i32x8 af = frag(st, r + l16);
      const f32x4 sa4 = *reinterpret_cast<const f32x4*>(&sa[r + 4 * q]);
      f32x4 part[NI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        part[ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[ni], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                     127, 0, 127);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[mi][ni][rr] = fmaf(sa4[rr] * sw[ni], part[ni][rr], acc[mi][ni][rr]);
    }
  };

  // Per-step direct loads of each wave: 7 (waves 0..5) or 6 (waves 6, 7).  Step s lives in stage
  // s % NSTAGE.  A stage is read after this wave's loads for it have landed (at most the next step's
  // loads still in flight) and after the barrier that publishes everyone's.
  issue(0, 0);
  if (nks > 1) issue(1, 1);
  for (int s = 0; s < nks; ++s) {
    if (s + 1 < nks) wait_vmcnt<6>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (s + 2 < nks) issue(s + 2, (s + 2) % NSTAGE);
    compute(s % NSTAGE);
  }

  if constexpr (OUT == 2) {
    // h tile in LDS (the stages are free once every wave has passed this barrier)
    float* htile = reinterpret_cast<float*>(smem);
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          htile[(wm * 64 + mi * 16 + 4 * q + rr) * kF8MmHLD + wn * 32 + ni * 16 + l16] =
              silu_f32(acc[mi][ni][rr]) * acc[mi][ni + 2][rr];
    __syncthreads();
    // one DPP row (16 lanes, 8 columns each) per h row: 32 rows per pass over the 512 threads
    const int hcol = nb * (kF8MmBN / 2);
    const int part = lane & 15;
#pragma unroll
    for (int pass = 0; pass < kF8MmBM / 32; ++pass) {
      const int row = pass * 32 + (tid >> 4);  // wave-uniform per 16-lane row
      const float* src = htile + row * kF8MmHLD + part * 8;
      float v[8];
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[j] = src[j];
        amax = fmaxf(amax, fabsf(v[j]));
      }
      amax = row16_max(amax);
      const float sc = amax / kE4M3Max;
      u32x2 out = {0u, 0u};
      if (sc != 0.f) {
        out[0] = f8_encode4(v, sc);
        out[1] = f8_encode4(v + 4, sc);
      }
      if (row < rows && hcol < N / 2) {
        const size_t orow = (size_t)(row0 + row);
        *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(p.C) + orow * (N / 2) + hcol + part * 8) = out;
        if (part == 0) p.Cs[orow * (N / 256) + nb] = sc;
      }
    }
    return;
  }
  if constexpr (EPI == MOE_EPI_NONE && OUT == 3) {
    f8_mm_store_f16e<MI, NI>(p, acc, nb, wm, wn, row0, rows, q, l16);
    return;
  }

#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = wm * 64 + mi * 16 + 4 * q + rr;
      if (row >= rows) continue;
      const size_t orow = (size_t)(row0 + row);
      if constexpr (EPI == MOE_EPI_SILU_MUL) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int j = nb * (kF8MmBN / 2) + wn * 32 + ni * 16 + l16;
          if (j >= N / 2) continue;
          static_cast<float*>(p.C)[orow * (N / 2) + j] = silu_f32(acc[mi][ni][rr]) * acc[mi][ni + 2][rr];
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int n = nb * kF8MmBN + wn * 64 + ni * 16 + l16;
          if (n >= N) continue;
          if (OUT_F32) static_cast<float*>(p.C)[orow * N + n] = acc[mi][ni][rr];
          else static_cast<uint16_t*>(p.C)[orow * N + n] = f32_to_bf16_bits(acc[mi][ni][rr]);
        }
      }
    }
}


template <int EPI, int OUT>
static hipError_t launch_f8_mm(const F8GemmArgs& a, hipStream_t s) {
  const int ncols = EPI == MOE_EPI_SILU_MUL ? a.N / 2 : a.N;
  const int bcols = EPI == MOE_EPI_SILU_MUL ? kF8MmBN / 2 : kF8MmBN;
  const int nbn = (ncols + bcols - 1) / bcols;
  gemm_f8_mm<EPI, OUT, 3><<<mm_grid(nbn, a.max_tiles), 512, 0, s>>>(a);
  return hipGetLastError();
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
  if (block_m == 128) {
    if (a.epilogue == MOE_EPI_SILU_MUL)
      return a.out_f32 == 2 ? launch_f8_mm<MOE_EPI_SILU_MUL, 2>(a, stream) : launch_f8_mm<MOE_EPI_SILU_MUL, 1>(a, stream);
    if (a.out_f32 == 3) return a.C_side ? launch_f8_mm<MOE_EPI_NONE, 3>(a, stream) : hipErrorInvalidValue;
    if (a.out_f32) return launch_f8_mm<MOE_EPI_NONE, 1>(a, stream);
    return launch_f8_mm<MOE_EPI_NONE, 0>(a, stream);
  }
  if (a.out_f32 == 3) return hipErrorInvalidValue;  // fp16 output with exponents: 128-row tiles only
  // Configurations from sweeps on MI355X (HIP events, weights streamed from HBM): with 128 experts
  // top-8 at 8 and 64 tokens, gate_up takes 36 / 86 us with <16,64,KW2> against 43 / 90 us for
  // <16,128,KW1>, down 21 / 44 us with <16,256,KW2> against 21 / 52 us; at 800 tokens and 256
  // experts <32,128,KW2> takes 151 / 85 us (gate_up / down) against 174 / 91 us for <32,128,KW1>;
  // 64-row tiles run 148 us with 256 columns against 182 us with 128.
  switch (block_m) {
    case 16:
      if (a.max_tiles <= kF8SplitKMaxTiles) return launch_f8_cfg<16, 64, 4, 2>(a, stream);
      if (a.epilogue == MOE_EPI_SILU_MUL) return launch_f8_cfg<16, 64, 2, 2>(a, stream);
      return launch_f8_cfg<16, 256, 2, 1>(a, stream);
    case 32: return launch_f8_cfg<32, 128, 2, 2>(a, stream);
    default: return launch_f8_cfg<64, 256, 1, 1>(a, stream);
  }
}

}  // namespace moe
