// MXFP4 (W4A4) variant of the layer on gfx950's scaled matrix cores.
//
// Format (the ATOM page "AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍", section
// "6.1 Linear：按量化类型分派 GEMM", lists per-1x32 MXFP4 with an a4w4 GEMM; section "8.2 量化并非单一
// 格式，而是一套执行契约" lists dynamic activation quantization as part of a format's contract): weights
// and activations are E2M1 codes, two per byte with the even K index in the low nibble, with one
// E8M0 scale byte (2^(byte - 127)) per 32 consecutive K elements.  Activations are quantized on the
// fly by the OCP MX conversion: per block, X = 2^(floor(log2(amax)) - 2) clamped to E8M0's range
// (an all-zero block takes 2^-127), elements rounded to the nearest E2M1 value of v / X, ties to
// even, saturating at 6.
//
// The Atlas page ("告别Python堆栈：Atlas用纯Rust重写LLM推理，在GB10上跑赢vLLM", section "编译时内核选择
// 和W4A16 Grouped GEMM") runs W4A16 because GB10 has no native FP4 matrix instruction; gfx950 has
// one: v_mfma_scale_f32_16x16x128_f8f6f4 multiplies 16 x 128 by 128 x 16 E2M1 operands and applies
// one E8M0 scale per lane and 32-element K block in hardware.  Lane l supplies row l % 16 and the
// 32 K elements [32 (l / 16), +32) (16 bytes) of each operand plus that block's scale byte; the
// result has the 16 x 16 fp32 layout of the bf16 instruction (checked exactly on the GPU).  So a K
// step of 128 is one instruction per 16 x 16 block, with no dequantization and no scale arithmetic
// in software.
//
// W4A8: the same instruction takes E4M3 activations (format 0) against the E2M1 weights.  Activations
// are then MXFP8: E4M3 codes, one byte per element, with one E8M0 scale per 32 K elements, X =
// 2^(floor(log2(amax)) - 8) (8 = the largest E4M3 exponent) and elements rounded to the nearest E4M3
// value of v / X, ties to even, saturating at 448.  An 8-bit operand is laid out differently from a
// 4-bit one: lane l supplies 32 bytes, K elements [16 (l / 16), +16) in its first four dwords and
// [64 + 16 (l / 16), +16) in the last four (measured with one-hot operands on the GPU), while its
// scale byte still belongs to the 32-element block [32 (l / 16), +32), as for the E2M1 operand.  h
// leaves the gate_up epilogue as MXFP8.
#include "launch.h"
#include "moe_common.h"

namespace moe {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// Shared exponent of a block from its largest magnitude: floor(log2(amax)) - 2, clamped to E8M0's
// range; zero and subnormal maxima give -127.
__device__ __forceinline__ int mx_block_exp(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  if (ef == 0) return -127;
  return max(-127, min(127, ef - 129));
}

// Four E2M1 codes of v / 2^e into byte J of w (hardware conversion: nearest, ties to even,
// saturating; scaling by a power of two is exact).
template <int J>
__device__ __forceinline__ uint32_t mx_pack2(uint32_t w, float a, float b, int e) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, ldexpf(a, -e), ldexpf(b, -e), 1.0f, J);
}

// 32 values -> 16 bytes of codes (given the block exponent).
__device__ __forceinline__ u32x4 mx_encode32(const float (&v)[32], int e) {
  u32x4 c;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w = 0;
    w = mx_pack2<0>(w, v[8 * d + 0], v[8 * d + 1], e);
    w = mx_pack2<1>(w, v[8 * d + 2], v[8 * d + 3], e);
    w = mx_pack2<2>(w, v[8 * d + 4], v[8 * d + 5], e);
    w = mx_pack2<3>(w, v[8 * d + 6], v[8 * d + 7], e);
    c[d] = w;
  }
  return c;
}

// MXFP8 (W4A8 activations): shared exponent floor(log2(amax)) - 8, clamped to E8M0's range; zero and
// subnormal maxima give -127.
__device__ __forceinline__ int mx8_block_exp(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  if (ef == 0) return -127;
  return max(-127, min(127, ef - 135));
}

// 32 values -> 32 E4M3 codes of v / 2^e (exact power-of-two scaling, clamped to +-448, then the
// hardware conversion: nearest, ties to even), element j at byte j.
__device__ __forceinline__ void mx8_encode32(const float (&v)[32], int e, u32x4& c0, u32x4& c1) {
  uint32_t w[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    float a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = fminf(fmaxf(ldexpf(v[4 * d + j], -e), -448.0f), 448.0f);
    int t = __builtin_amdgcn_cvt_pk_fp8_f32(a[0], a[1], 0, false);
    t = __builtin_amdgcn_cvt_pk_fp8_f32(a[2], a[3], t, true);
    w[d] = (uint32_t)t;
  }
  c0 = u32x4{w[0], w[1], w[2], w[3]};
  c1 = u32x4{w[4], w[5], w[6], w[7]};
}

// ---------------------------------------------------------------------------------------------------
// Activation quantization: one thread per 32-element block of a row-major bf16 matrix whose rows
// are whole blocks, so block i sits at element 32 i of x, byte 16 i of the codes and byte i of the
// scales.  Four 16-byte loads and one 16-byte store per thread.
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t* __restrict__ x, long long nblocks,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + i * 32);
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32x4 w = src[d];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * d + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * d + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      amax = fmaxf(amax, fmaxf(fabsf(v[8 * d + 2 * j]), fabsf(v[8 * d + 2 * j + 1])));
    }
  }
  const int e = mx_block_exp(amax);
  *reinterpret_cast<u32x4*>(q + i * 16) = mx_encode32(v, e);
  s[i] = (uint8_t)(e + 127);
}

// MXFP8 quantization, same decomposition: 32 code bytes (two 16-byte stores) and one scale byte per
// thread.
__global__ __launch_bounds__(256) void mx8_quant_kernel(const uint16_t* __restrict__ x, long long nblocks,
                                                        uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + i * 32);
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32x4 w = src[d];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * d + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * d + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      amax = fmaxf(amax, fmaxf(fabsf(v[8 * d + 2 * j]), fabsf(v[8 * d + 2 * j + 1])));
    }
  }
  const int e = mx8_block_exp(amax);
  u32x4 c0, c1;
  mx8_encode32(v, e, c0, c1);
  *reinterpret_cast<u32x4*>(q + i * 32) = c0;
  *reinterpret_cast<u32x4*>(q + i * 32 + 16) = c1;
  s[i] = (uint8_t)(e + 127);
}

hipError_t launch_mx8_quant(const uint16_t* x, long long rows, int K, uint8_t* q, uint8_t* s, hipStream_t stream) {
  const long long nblocks = rows * (K / 32);
  if (nblocks <= 0) return hipSuccess;
  mx8_quant_kernel<<<dim3((unsigned)((nblocks + 255) / 256)), 256, 0, stream>>>(x, nblocks, q, s);
  return hipGetLastError();
}

hipError_t launch_mx_quant(const uint16_t* x, long long rows, int K, uint8_t* q, uint8_t* s, hipStream_t stream) {
  const long long nblocks = rows * (K / 32);
  if (nblocks <= 0) return hipSuccess;
  mx_quant_kernel<<<dim3((unsigned)((nblocks + 255) / 256)), 256, 0, stream>>>(x, nblocks, q, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------
// Operand layouts in MFMA lane order, so that every wave-level load is one contiguous block.
//  * Packed weights (moe_mx_prepack): the [E, N, K] matrix cut into blocks of 16 rows x 128 K
//    elements, ordered (expert, row block, K block) with K fastest; a block is 1024 bytes of codes
//    (bytes [16l, 16l+16) = lane l: row l % 16, K elements [32 (l / 16), +32)) and, in a separate
//    array, 64 scale bytes (byte l = lane l's block).  Needs N % 16 == 0 and K % 128 == 0.
//  * Tile-blocked activations: the rows of a tile list, tile by tile, each tile padded to bm rows,
//    in the same blocks (tile, 16-row group, K block).  Written by the quantizers below and by the
//    gate_up epilogue, read by the grouped GEMM with no gather.
__device__ __forceinline__ size_t mx_block(long long group, int s, int nks) { return (size_t)group * nks + s; }

// Tile, row and 32-K block of this thread of a tile-list quantization launch (one thread per
// (tile, row, block), 256 per workgroup); false past the end.  Below 2^31 threads the index
// arithmetic is 32-bit (the 64-bit divisions would otherwise precede every load).
__device__ __forceinline__ bool quant_tile_index(long long total, int kb, int bm, int& t, int& i, int& b) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return false;
  if (total < (1LL << 31)) {
    const uint32_t id = (uint32_t)idx, rest = id / (uint32_t)kb;
    b = (int)(id - rest * (uint32_t)kb);
    t = (int)(rest / (uint32_t)bm);
    i = (int)(rest - (uint32_t)t * (uint32_t)bm);
  } else {
    const long long rest = idx / kb;
    b = (int)(idx - rest * kb);
    t = (int)(rest / bm);
    i = (int)(rest - (long long)t * bm);
  }
  return true;
}

// x rows of a tile list quantized into the tile-blocked layout: one thread per (tile, row, 32-K
// block); tiles past num_tiles and padding rows are not written (the GEMM never stores them).
__global__ __launch_bounds__(256) void mx_quant_tiles_kernel(const uint16_t* __restrict__ x, int K,
                                                             const int32_t* __restrict__ a_row_of, int a_row_div,
                                                             const int32_t* __restrict__ tiles,
                                                             const int32_t* __restrict__ num_tiles, int bm,
                                                             long long total, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ s) {
  const int kb = K / 32;
  int t, i, b;
  if (!quant_tile_index(total, kb, bm, t, i, b)) return;
  // the tile count and the tile's entry in one round trip (t < max_tiles: the entry is in bounds;
  // past num_tiles it is not used): one condition over all three, without short-circuit, so that
  // the loads are issued together
  const int nt = *num_tiles, row0 = tiles[3 * t + 1], rows = tiles[3 * t + 2];
  if ((t >= nt) | (i >= rows) | (row0 < 0)) return;
  const int r = row0 + i;
  const int src = a_row_of ? a_row_of[r] / a_row_div : r;
  const u32x4* in = reinterpret_cast<const u32x4*>(x + (size_t)src * K + 32 * b);
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32x4 w = in[d];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * d + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * d + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      amax = fmaxf(amax, fmaxf(fabsf(v[8 * d + 2 * j]), fabsf(v[8 * d + 2 * j + 1])));
    }
  }
  const int e = mx_block_exp(amax);
  const int lane = (b & 3) * 16 + (i & 15);
  const size_t blk = mx_block((long long)t * (bm / 16) + (i >> 4), b >> 2, K / 128);
  *reinterpret_cast<u32x4*>(q + blk * 1024 + lane * 16) = mx_encode32(v, e);
  s[blk * 64 + lane] = (uint8_t)(e + 127);
}

hipError_t launch_mx_quant_tiles(const uint16_t* x, int K, const int32_t* a_row_of, int a_row_div,
                                 const int32_t* tiles, const int32_t* num_tiles, int max_tiles, int bm, uint8_t* q,
                                 uint8_t* s, hipStream_t stream) {
  const long long total = (long long)max_tiles * bm * (K / 32);
  if (total <= 0) return hipSuccess;
  mx_quant_tiles_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, stream>>>(x, K, a_row_of, a_row_div, tiles,
                                                                                  num_tiles, bm, total, q, s);
  return hipGetLastError();
}

// Tile-blocked MXFP8 activations (W4A8 with packed weights): blocks of 16 rows x 128 K ordered (tile,
// 16-row group, K block) as above, each 2048 code bytes in the 8-bit lane layout, halves first: bytes
// [16l, 16l+16) = lane l's first half (row l % 16, K [16 (l / 16), +16) of the step), bytes
// [1024 + 16l, +16) = its second half (K [64 + 16 (l / 16), +16)); so each half is one contiguous 1 KB
// wave load.  64 scale bytes per block as for MXFP4 (byte l: row l % 16, 32-block l / 16).
// Byte position of the 16 codes at K offset o (a multiple of 16 within the step) of tile row i.
__device__ __forceinline__ size_t mx8_tiled_pos(size_t blk, int o, int i) {
  const int half = o >= 64, qq = (o - 64 * half) >> 4;
  return blk * 2048 + half * 1024 + (size_t)(qq * 16 + (i & 15)) * 16;
}

// x rows of a tile list quantized to MXFP8 in the tile-blocked layout: one thread per (tile, row,
// 32-K block); tiles past num_tiles and padding rows are not written.
__global__ __launch_bounds__(256) void mx8_quant_tiles_kernel(const uint16_t* __restrict__ x, int K,
                                                              const int32_t* __restrict__ a_row_of, int a_row_div,
                                                              const int32_t* __restrict__ tiles,
                                                              const int32_t* __restrict__ num_tiles, int bm,
                                                              long long total, uint8_t* __restrict__ q,
                                                              uint8_t* __restrict__ s) {
  const int kb = K / 32;
  int t, i, b;
  if (!quant_tile_index(total, kb, bm, t, i, b)) return;
  // the tile count and the tile's entry in one round trip (t < max_tiles: the entry is in bounds;
  // past num_tiles it is not used): one condition over all three, without short-circuit, so that
  // the loads are issued together
  const int nt = *num_tiles, row0 = tiles[3 * t + 1], rows = tiles[3 * t + 2];
  if ((t >= nt) | (i >= rows) | (row0 < 0)) return;
  const int r = row0 + i;
  const int src = a_row_of ? a_row_of[r] / a_row_div : r;
  const u32x4* in = reinterpret_cast<const u32x4*>(x + (size_t)src * K + 32 * b);
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32x4 w = in[d];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * d + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * d + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      amax = fmaxf(amax, fmaxf(fabsf(v[8 * d + 2 * j]), fabsf(v[8 * d + 2 * j + 1])));
    }
  }
  const int e = mx8_block_exp(amax);
  u32x4 c0, c1;
  mx8_encode32(v, e, c0, c1);
  const size_t blk = mx_block((long long)t * (bm / 16) + (i >> 4), b >> 2, K / 128);
  const int o = 32 * (b & 3);
  *reinterpret_cast<u32x4*>(q + mx8_tiled_pos(blk, o, i)) = c0;
  *reinterpret_cast<u32x4*>(q + mx8_tiled_pos(blk, o + 16, i)) = c1;
  s[blk * 64 + (b & 3) * 16 + (i & 15)] = (uint8_t)(e + 127);
}

hipError_t launch_mx8_quant_tiles(const uint16_t* x, int K, const int32_t* a_row_of, int a_row_div,
                                  const int32_t* tiles, const int32_t* num_tiles, int max_tiles, int bm, uint8_t* q,
                                  uint8_t* s, hipStream_t stream) {
  const long long total = (long long)max_tiles * bm * (K / 32);
  if (total <= 0) return hipSuccess;
  mx8_quant_tiles_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, stream>>>(x, K, a_row_of, a_row_div, tiles,
                                                                                   num_tiles, bm, total, q, s);
  return hipGetLastError();
}

// Canonical MXFP4 weights -> packed layout: one thread per 16-byte lane slot of a block.
__global__ __launch_bounds__(256) void mx_prepack_kernel(const uint8_t* __restrict__ wq, const uint8_t* __restrict__ we,
                                                         int N, int K, long long total, uint8_t* __restrict__ pq,
                                                         uint8_t* __restrict__ pe) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int nks = K / 128, nbn = N / 16;
  const int lane = (int)(idx & 63);
  const long long blk = idx >> 6;
  const int st = (int)(blk % nks);
  const long long rb = blk / nks;  // expert * nbn + row block
  const long long e = rb / nbn;
  const int n = (int)(rb % nbn) * 16 + (lane & 15), qd = lane >> 4;
  const size_t row = (size_t)e * N + n;
  *reinterpret_cast<u32x4*>(pq + idx * 16) =
      *reinterpret_cast<const u32x4*>(wq + row * (K / 2) + (size_t)st * 64 + qd * 16);
  pe[idx] = we[row * (K / 32) + st * 4 + qd];
}

hipError_t launch_mx_prepack(const uint8_t* wq, const uint8_t* we, int E, int N, int K, uint8_t* pq, uint8_t* pe,
                             hipStream_t stream) {
  const long long total = (long long)E * (N / 16) * (K / 128) * 64;
  if (total <= 0) return hipSuccess;
  mx_prepack_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, stream>>>(wq, we, N, K, total, pq, pe);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------
// Grouped MX GEMM over the device-side tile list (the same list as the W4A16 path).  A workgroup of
// four waves computes a BM x BN tile; the waves split K KW ways and N 4/KW ways.  Every wave loads
// its operand fragments straight into a register ring PF K steps deep (16 bytes of codes and one
// scale byte per lane and 16-row block), so the main loop has no LDS traffic and no barrier; K-split
// partials are added in LDS in wave order.  With row-major activations (gathered through a_row_of)
// and canonical weights each load touches 16 rows per 16-lane quarter; the packed weights and the
// tile-blocked activations (MODE 1, 2) turn every wave-level load into one contiguous 1 KB block.
// Epilogues: NONE stores fp32 or bf16 rows; SILU_MUL forms h = silu(gate) * up in fp32 (gate rows
// [0, N/2), up rows [N/2, N) of the weight), gathers the tile's h in LDS and quantizes each
// 32-column block of each row to MXFP4 (codes [rows, N/4], scale bytes [rows, N/64]) for the next
// projection.  AF = 0 (W4A8): MXFP8 activations (32 code bytes per lane and K step in the 8-bit operand
// layout above; MODE 2: the tile-blocked MXFP8 layout, two contiguous 1 KB loads per wave), the
// instruction's A format E4M3, and h quantized to MXFP8 (row-major: codes [rows, N/2], scale bytes
// [rows, N/64]; MODE 2: tile-blocked).
template <int BM, int BN, int KW, int PF, int EPI, int OUT, int MODE, int AF = 4>
__global__ __launch_bounds__(256) void gemm_mx_kernel(MxGemmArgs p) {
  constexpr bool ATB = MODE == 2, WPK = MODE >= 1;  // tile-blocked activations, packed weights
  constexpr bool A8 = AF == 0;                       // E4M3 activations
  static_assert(AF == 0 || AF == 4, "activation format");
  constexpr int WNS = 4 / KW;             // waves along N
  constexpr int WN = BN / WNS;            // columns per wave
  constexpr int MI = BM / 16, NI = WN / 16;
  constexpr int NS = PF + 1;
  constexpr int HC = BN / 2;              // h columns of a SILU_MUL tile
  constexpr int HLD = HC + 4;             // padded LDS row of the h tile (floats)
  static_assert(KW * WNS == 4 && NI >= 1 && MI >= 1, "tile shape");
  static_assert(EPI != MOE_EPI_SILU_MUL || (NI % 2 == 0 && HC % 32 == 0), "SiLU*mul tile shape");
  __shared__ __attribute__((aligned(16))) float red[KW > 1 ? WNS * (KW - 1) * 64 * MI * NI * 4 : 1];
  __shared__ __attribute__((aligned(16))) float htile[EPI == MOE_EPI_SILU_MUL ? BM * HLD : 1];

  const int N = p.N, K = p.K;
  const int nbn = EPI == MOE_EPI_SILU_MUL ? (N / 2 + HC - 1) / HC : (N + BN - 1) / BN;
  int tile, nb;
  if (!xcd_tile(linear_block(), nbn, *p.num_tiles, tile, nb)) return;
  const int e = p.tiles[3 * tile], row0 = p.tiles[3 * tile + 1], rows = p.tiles[3 * tile + 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave % KW, wn = wave / KW;
  const int l16 = lane & 15, q = lane >> 4;
  const int nks = (K + 127) / 128;
  const int per = (nks + KW - 1) / KW;
  const int s_begin = min(nks, wk * per), s_end = min(nks, s_begin + per);
  const int KB = K / 2, KS = K / 32;  // bytes of codes and of scales per row
  const int KBA = A8 ? K : KB;        // bytes of activation codes per row

  // activation fragments: row mi * 16 + l16 of the tile (row-major: padding rows read the first row)
  const uint8_t* aq[MI];
  const uint8_t* as[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    if (ATB) {
      const size_t blk = mx_block((long long)tile * MI + mi, 0, nks);
      aq[mi] = p.Aq + blk * (A8 ? 2048 : 1024) + lane * 16;
      as[mi] = p.As + blk * 64 + lane;
    } else {
      const int i = mi * 16 + l16;
      const int r = row0 + (i < rows ? i : 0);
      const int ar = p.a_row_of ? p.a_row_of[r] / p.a_row_div : r;
      aq[mi] = p.Aq + (size_t)ar * KBA + (A8 ? 0 : q * 16);
      as[mi] = p.As + (size_t)ar * KS + q;
    }
  }
  // weight fragments: SILU_MUL pairs gate block j with up block j (rows N/2 + j)
  const uint8_t* wq[NI];
  const uint8_t* ws[NI];
  int ncol[NI];
  bool nvalid[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int n;
    if (EPI == MOE_EPI_SILU_MUL) {
      const int j = nb * HC + wn * (WN / 2) + (ni % (NI / 2)) * 16 + l16;
      nvalid[ni] = j < N / 2;
      ncol[ni] = j;
      n = ni < NI / 2 ? j : N / 2 + j;
    } else {
      n = nb * BN + wn * WN + ni * 16 + l16;
      nvalid[ni] = n < N;
      ncol[ni] = n;
    }
    if (!nvalid[ni]) n = 0;
    if (WPK) {
      const size_t blk = mx_block((long long)e * (N / 16) + (n >> 4), 0, nks);
      wq[ni] = p.Wq + blk * 1024 + lane * 16;
      ws[ni] = p.We + blk * 64 + lane;
    } else {
      wq[ni] = p.Wq + ((size_t)e * N + n) * KB + q * 16;
      ws[ni] = p.We + ((size_t)e * N + n) * KS + q;
    }
  }

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[NS][MI], areg2[NS][MI], breg[NS][NI];  // areg2: second half of an E4M3 fragment
  uint32_t asc[NS][MI], bsc[NS][NI];
  auto load_step = [&](int s, int u) {
    s = min(s, s_end - 1);  // prefetches past this wave's range re-read its last step (unused)
    // K tail (row-major, canonical): a quarter past K reads the row's last block and its activation
    // codes are zeroed.  The blocked layouts need K % 128 == 0.
    const bool qv = WPK || s * 128 + 32 * q < K;
    const int cb = qv ? s * 64 : (K - 32 - 32 * q) / 2;  // code byte offset of this lane's block
    const int sb = qv ? s * 4 : (K / 32 - 1 - q);        // scale byte offset
    // E4M3 activations: this lane's two 16-byte halves lie in blocks q / 2 and 2 + q / 2 of the step;
    // a half past K reads the row's first bytes and is zeroed
    const bool v0 = WPK || s * 4 + (q >> 1) < K / 32, v1 = WPK || s * 4 + 2 + (q >> 1) < K / 32;
    const int o0 = v0 ? s * 128 + 16 * q : 0, o1 = v1 ? s * 128 + 64 + 16 * q : 0;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      breg[u][ni] = *reinterpret_cast<const u32x4*>(wq[ni] + (WPK ? (size_t)s * 1024 : (size_t)cb));
      bsc[u][ni] = ws[ni][WPK ? s * 64 : sb];
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (A8) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(aq[mi] + (ATB ? (size_t)s * 2048 : (size_t)o0));
        const u32x4 a2 = *reinterpret_cast<const u32x4*>(aq[mi] + (ATB ? (size_t)s * 2048 + 1024 : (size_t)o1));
        areg[u][mi] = v0 ? a : u32x4{0u, 0u, 0u, 0u};
        areg2[u][mi] = v1 ? a2 : u32x4{0u, 0u, 0u, 0u};
      } else {
        const u32x4 a = *reinterpret_cast<const u32x4*>(aq[mi] + (ATB ? (size_t)s * 1024 : (size_t)cb));
        areg[u][mi] = qv ? a : u32x4{0u, 0u, 0u, 0u};
      }
      asc[u][mi] = as[mi][ATB ? s * 64 : sb];
    }
  };
  auto compute_step = [&](int u) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const u32x4 a = areg[u][mi];
      const u32x4 a2 = A8 ? areg2[u][mi] : u32x4{0u, 0u, 0u, 0u};
      const i32x8 a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)a2[0], (int)a2[1], (int)a2[2], (int)a2[3]};
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const u32x4 b = breg[u][ni];
        const i32x8 b8 = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[mi][ni], AF, 4, 0, (int)asc[u][mi],
                                                                        0, (int)bsc[u][ni]);
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
        compute_step(u);
      }
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (s0 + u < s_end) compute_step(u);
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
    if (wk == 0) {
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
  }
  const bool owner = KW == 1 || wk == 0;

  if constexpr (EPI == MOE_EPI_SILU_MUL) {
    if (owner) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int ni = 0; ni < NI / 2; ++ni) {
            const float g = acc[mi][ni][r], u = acc[mi][ni + NI / 2][r];
            htile[(mi * 16 + 4 * q + r) * HLD + wn * (WN / 2) + ni * 16 + l16] = silu_f32(g) * u;
          }
    }
    __syncthreads();
    // one thread per (row, 32-column block) of h
    constexpr int NB = HC / 32;
    for (int t = tid; t < BM * NB; t += 256) {
      const int row = t / NB, blk = t % NB;
      const int hcol = nb * HC + blk * 32;
      if (row >= rows || hcol >= N / 2) continue;
      float v[32];
      float amax = 0.f;
      const float4* src = reinterpret_cast<const float4*>(htile + row * HLD + blk * 32);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float4 f = src[d];
        v[4 * d] = f.x;
        v[4 * d + 1] = f.y;
        v[4 * d + 2] = f.z;
        v[4 * d + 3] = f.w;
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
      }
      uint8_t* C = static_cast<uint8_t*>(p.C);
      if (A8 && ATB) {
        // MXFP8 h, tile-blocked for the next projection (K = N/2 there)
        const int ex = mx8_block_exp(amax);
        u32x4 c0, c1;
        mx8_encode32(v, ex, c0, c1);
        const int b = hcol / 32;
        const size_t blk = mx_block((long long)tile * MI + (row >> 4), b >> 2, (N / 2) / 128);
        *reinterpret_cast<u32x4*>(C + mx8_tiled_pos(blk, 32 * (b & 3), row)) = c0;
        *reinterpret_cast<u32x4*>(C + mx8_tiled_pos(blk, 32 * (b & 3) + 16, row)) = c1;
        p.Cs[blk * 64 + (b & 3) * 16 + (row & 15)] = (uint8_t)(ex + 127);
        continue;
      }
      if (A8) {
        // MXFP8 h, row-major (codes [rows, N/2], scale bytes [rows, N/64])
        const int ex = mx8_block_exp(amax);
        u32x4 c0, c1;
        mx8_encode32(v, ex, c0, c1);
        const size_t orow = (size_t)(row0 + row);
        uint8_t* dst = C + orow * (N / 2) + hcol;
        *reinterpret_cast<u32x4*>(dst) = c0;
        *reinterpret_cast<u32x4*>(dst + 16) = c1;
        p.Cs[orow * (N / 64) + hcol / 32] = (uint8_t)(ex + 127);
        continue;
      }
      const int ex = mx_block_exp(amax);
      if (ATB) {
        // tile-blocked for the next projection (K = N/2 there)
        const int b = hcol / 32, ln = (b & 3) * 16 + (row & 15);
        const size_t blk = mx_block((long long)tile * MI + (row >> 4), b >> 2, (N / 2) / 128);
        *reinterpret_cast<u32x4*>(C + blk * 1024 + ln * 16) = mx_encode32(v, ex);
        p.Cs[blk * 64 + ln] = (uint8_t)(ex + 127);
      } else {
        const size_t orow = (size_t)(row0 + row);
        *reinterpret_cast<u32x4*>(C + orow * (N / 4) + hcol / 2) = mx_encode32(v, ex);
        p.Cs[orow * (N / 64) + hcol / 32] = (uint8_t)(ex + 127);
      }
    }
  } else {
    if (!owner) return;
    if constexpr (OUT == kOutF16Exp) {
      store_f16e<MI, NI, true>(static_cast<uint16_t*>(p.C), p.C_side, N, acc, 0, row0, rows, q, ncol, nvalid);
      return;
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mi * 16 + 4 * q + r;
        if (row >= rows) continue;
        const size_t orow = (size_t)(row0 + row);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          if (!nvalid[ni]) continue;
          if (OUT == kOutF32) static_cast<float*>(p.C)[orow * N + ncol[ni]] = acc[mi][ni][r];
          else static_cast<uint16_t*>(p.C)[orow * N + ncol[ni]] = f32_to_bf16_bits(acc[mi][ni][r]);
        }
      }
  }
}

// ---------------------------------------------------------------------------------------------------
// Large-tile MXFP4 kernel for MFMA-bound shapes (hundreds of rows per expert), row-major activations
// (gathered rows) with canonical (MODE 0) or packed (MODE 1) weights, K % 128 == 0.  A 128 x 256
// output tile per 512-thread workgroup: 8 waves (2 along M x 4 along N), 64 x 64 each.  Per K step of
// 128 the tile's activation codes (128 rows x 64 B), weight codes (256 rows x 64 B) and both operands'
// E8M0 scale bytes reach LDS by direct global->LDS loads, through NSTAGE stages with one barrier per
// step.  Code rows are 64 B with their 16-byte chunks XOR-swizzled by (row / 4) % 4, so the sixteen rows
// a fragment read touches fall in sixteen distinct bank groups.  The scaled instruction applies both
// scales and accumulates into the fp32 accumulators itself, so the loop holds no vector ALU work.
// Same instruction sequence per output as gemm_mx_kernel (one K step after another into the same
// accumulator), so the results are bit-identical to it.  SILU_MUL stages h in LDS and one thread per
// (row, 32-column block) quantizes it into row-major codes and scale bytes.
constexpr int kMxMmBM = 128, kMxMmBN = 256;
constexpr int kMxMmA = kMxMmBM * 64, kMxMmB = kMxMmBN * 64;  // code bytes per stage
constexpr int kMxMmA8 = kMxMmBM * 128;                        // E4M3 activation bytes per stage (W4A8)
constexpr int kMxMmHLD = kMxMmBN / 2 + 4;                     // padded LDS row of the h tile (floats)

// Direct global->LDS 4-byte load (lane l writes LDS bytes [4l, 4l+4) after the wave-uniform base).
__device__ __forceinline__ void g2lds4_mx(const void* g, void* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  asm volatile("global_load_lds_dword %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ int mx_swz(int row) { return (row >> 2) & 3; }
// E4M3 activation rows (128 bytes per K step): chunks swizzled by (row / 2) % 8.
__device__ __forceinline__ int mx8_swz(int row) { return (row >> 1) & 7; }

// s_waitcnt vmcnt(n) for a run-time n in [0, 8].
__device__ __forceinline__ void wait_vmcnt_upto8(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    default: wait_vmcnt<8>(); break;
  }
}

// AF = 0 (W4A8): E4M3 activations, 128-byte code rows per K step copied by two direct loads per wave
// and read in the 8-bit operand layout (two 16-byte halves per lane); h leaves as MXFP8.
template <int EPI, int OUT, int MODE, int NSTAGE, int AF = 4>
__global__ __launch_bounds__(512) void gemm_mx_mm(MxGemmArgs p) {
  constexpr int MI = 4, NI = 4;
  constexpr bool WPK = MODE == 1;
  constexpr bool A8 = AF == 0;
  constexpr int ABYTES = A8 ? kMxMmA8 : kMxMmA;                      // activation code bytes per stage
  constexpr int STAGE = ABYTES + kMxMmB + (kMxMmBM + kMxMmBN) * 4;
  static_assert(NSTAGE >= 3 && NSTAGE * STAGE >= kMxMmBM * kMxMmHLD * 4, "stages also hold the h tile");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NSTAGE * STAGE];
  __shared__ int32_t sRow[kMxMmBM];
  const int N = p.N, K = p.K;
  const int ncols = EPI == MOE_EPI_SILU_MUL ? N / 2 : N;
  const int bcols = EPI == MOE_EPI_SILU_MUL ? kMxMmBN / 2 : kMxMmBN;
  const int nbn = (ncols + bcols - 1) / bcols;
  int tile, nb;
  if (!mm_work(linear_block(), nbn, *p.num_tiles, tile, nb)) return;
  const int e = p.tiles[3 * tile], row0 = p.tiles[3 * tile + 1], rows = p.tiles[3 * tile + 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int l16 = lane & 15, q = lane >> 4;
  const int nks = K / 128;
  const int KB = K / 2, KS = K / 32;  // code and scale bytes per row
  const int KBA = A8 ? K : KB;        // activation code bytes per row

  for (int i = tid; i < kMxMmBM; i += 512) {
    const int r = row0 + (i < rows ? i : 0);
    sRow[i] = p.a_row_of ? p.a_row_of[r] / p.a_row_div : r;
  }
  __syncthreads();

  // weight row of tile column nt (0..255): SILU_MUL puts the 128 gate rows first, then their up rows
  auto wrow = [&](int nt) -> int {
    int n;
    if (EPI == MOE_EPI_SILU_MUL) {
      const int j = nb * (kMxMmBN / 2) + (nt & 127);
      n = j < N / 2 ? (nt < 128 ? j : N / 2 + j) : 0;
    } else {
      n = nb * kMxMmBN + nt;
      if (n >= N) n = 0;
    }
    return n;
  };
  // code sources: one instruction covers 16 rows (lane l: row l / 4, LDS chunk l % 4, which holds the
  // row's global chunk (l % 4) ^ swizzle, i.e. K elements [32 c, 32 c + 32) of the step)
  // (E4M3: two instructions of 8 rows each, lane l: row l / 8, LDS chunk l % 8 holding the row's
  // global chunk (l % 8) ^ swizzle)
  const uint8_t* a_src[A8 ? 2 : 1];
  if (A8) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 16 * wave + 8 * t + (lane >> 3);
      a_src[t] = p.Aq + (size_t)sRow[r] * KBA + 16 * ((lane & 7) ^ mx8_swz(r));
    }
  } else {
    const int r = 16 * wave + (lane >> 2);
    a_src[0] = p.Aq + (size_t)sRow[r] * KB + 16 * ((lane & 3) ^ mx_swz(r));
  }
  const uint8_t* b_src[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int nt = 16 * (2 * wave + t) + (lane >> 2);
    const int c = (lane & 3) ^ mx_swz(nt);
    const int n = wrow(nt);
    if (WPK) b_src[t] = p.Wq + ((size_t)e * (N / 16) + n / 16) * (size_t)nks * 1024 + 16 * (c * 16 + n % 16);
    else b_src[t] = p.Wq + ((size_t)e * N + n) * KB + 16 * c;
  }
  // scale sources: waves 0, 1 the 128 activation rows (4 bytes = the step's four blocks of a row);
  // waves 2..5 the weights: canonical 4 bytes per row, packed the 64-byte scale blocks of 16 rows
  const uint8_t* s_src = nullptr;
  if (wave < 2) {
    s_src = p.As + (size_t)sRow[64 * wave + lane] * KS;
  } else if (wave < 6) {
    if (WPK) {
      const int rb = 4 * (wave - 2) + (lane >> 4);
      const int n0 = wrow(16 * rb);
      s_src = p.We + ((size_t)e * (N / 16) + n0 / 16) * (size_t)nks * 64 + 4 * (lane & 15);
    } else {
      s_src = p.We + ((size_t)e * N + wrow(64 * (wave - 2) + lane)) * KS;
    }
  }

  auto issue = [&](int ks, int stage) {
    uint8_t* st = smem + stage * STAGE;
    if (A8) {
#pragma unroll
      for (int t = 0; t < 2; ++t) g2lds16(a_src[t] + (size_t)ks * 128, st + wave * 2048 + t * 1024);
    } else {
      g2lds16(a_src[0] + (size_t)ks * 64, st + wave * 1024);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
      g2lds16(b_src[t] + (size_t)ks * (WPK ? 1024 : 64), st + ABYTES + (2 * wave + t) * 1024);
    if (wave < 2) g2lds4_mx(s_src + (size_t)ks * 4, st + ABYTES + kMxMmB + wave * 256);
    else if (wave < 6)
      g2lds4_mx(s_src + (size_t)ks * (WPK ? 64 : 4), st + ABYTES + kMxMmB + kMxMmBM * 4 + (wave - 2) * 256);
  };

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
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + row * 64 + 16 * (q ^ mx_swz(row)));
    return i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
  };

  // E4M3 fragment of LDS row `row`: K bytes [16q, +16) and [64 + 16q, +16) of the step
  auto frag8 = [&](const uint8_t* base, int row) -> i32x8 {
    const int sw = mx8_swz(row);
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(base + row * 128 + 16 * (q ^ sw));
    const u32x4 v1 = *reinterpret_cast<const u32x4*>(base + row * 128 + 16 * ((4 + q) ^ sw));
    return i32x8{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3], (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
  };

  auto compute = [&](int stage) {
    const uint8_t* st = smem + stage * STAGE;
    const uint8_t* sa = st + ABYTES + kMxMmB;
    const uint8_t* sb = sa + kMxMmBM * 4;
    i32x8 bf[NI];
    int bs[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int nt = ntile[ni];
      bf[ni] = frag(st + ABYTES, nt);
      bs[ni] = WPK ? sb[(nt >> 4) * 64 + 16 * q + (nt & 15)] : sb[nt * 4 + q];
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int r = wm * 64 + mi * 16 + l16;
      const i32x8 af = A8 ? frag8(st, r) : frag(st, r);
      const int as = sa[r * 4 + q];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[ni], acc[mi][ni], AF, 4, 0, as, 0, bs[ni]);
    }
  };

  // Per-step direct loads of each wave: 4 (waves 0..5) or 3 (waves 6, 7), one more with E4M3
  // activations.  Step s lives in stage s % NSTAGE; before reading it a wave waits until only the
  // loads of the steps after s that it has already issued are outstanding, then the barrier publishes
  // everyone's.
  const int per_step = (wave < 6 ? 4 : 3) + (A8 ? 1 : 0);
#pragma unroll
  for (int u = 0; u < NSTAGE - 1; ++u)
    if (u < nks) issue(u, u);
  for (int s = 0; s < nks; ++s) {
    wait_vmcnt_upto8(min(nks - 1 - s, NSTAGE - 2) * per_step);
    __syncthreads();
    if (s + NSTAGE - 1 < nks) issue(s + NSTAGE - 1, (s + NSTAGE - 1) % NSTAGE);
    compute(s % NSTAGE);
  }

  if constexpr (EPI == MOE_EPI_SILU_MUL) {
    float* htile = reinterpret_cast<float*>(smem);
    __syncthreads();  // every wave is done with the stages
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          htile[(wm * 64 + mi * 16 + 4 * q + rr) * kMxMmHLD + wn * 32 + ni * 16 + l16] =
              silu_f32(acc[mi][ni][rr]) * acc[mi][ni + 2][rr];
    __syncthreads();
    const int row = tid >> 2, blk = tid & 3;
    const int hcol = nb * (kMxMmBN / 2) + blk * 32;
    if (row < rows && hcol < N / 2) {
      float v[32];
      float amax = 0.f;
      const float4* src = reinterpret_cast<const float4*>(htile + row * kMxMmHLD + blk * 32);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float4 f = src[d];
        v[4 * d] = f.x;
        v[4 * d + 1] = f.y;
        v[4 * d + 2] = f.z;
        v[4 * d + 3] = f.w;
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
      }
      const size_t orow = (size_t)(row0 + row);
      if (A8) {  // MXFP8 h, row-major
        const int ex = mx8_block_exp(amax);
        u32x4 c0, c1;
        mx8_encode32(v, ex, c0, c1);
        uint8_t* dst = static_cast<uint8_t*>(p.C) + orow * (N / 2) + hcol;
        *reinterpret_cast<u32x4*>(dst) = c0;
        *reinterpret_cast<u32x4*>(dst + 16) = c1;
        p.Cs[orow * (N / 64) + hcol / 32] = (uint8_t)(ex + 127);
      } else {
        const int ex = mx_block_exp(amax);
        *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p.C) + orow * (N / 4) + hcol / 2) = mx_encode32(v, ex);
        p.Cs[orow * (N / 64) + hcol / 32] = (uint8_t)(ex + 127);
      }
    }
  } else {
    if constexpr (OUT == kOutF16Exp) {
      int ncol[NI];
      bool nvalid[NI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        ncol[ni] = nb * kMxMmBN + wn * 64 + ni * 16 + l16;
        nvalid[ni] = ncol[ni] < N;
      }
      // one 16-row block at a time: fewer live registers (the E2M1 form stays at 119 VGPRs, 4 waves per SIMD)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        store_f16e<1, NI, true>(static_cast<uint16_t*>(p.C), p.C_side, N,
                                reinterpret_cast<const f32x4(&)[1][NI]>(acc[mi]), wm * 64 + mi * 16, row0, rows, q,
                                ncol, nvalid);
      return;
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = wm * 64 + mi * 16 + 4 * q + rr;
        if (row >= rows) continue;
        const size_t orow = (size_t)(row0 + row);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int n = nb * kMxMmBN + wn * 64 + ni * 16 + l16;
          if (n >= N) continue;
          if (OUT == kOutF32) static_cast<float*>(p.C)[orow * N + n] = acc[mi][ni][rr];
          else static_cast<uint16_t*>(p.C)[orow * N + n] = f32_to_bf16_bits(acc[mi][ni][rr]);
        }
      }
  }
}

template <int MODE, int AF = 4>
static hipError_t launch_mx_mm(const MxGemmArgs& a, hipStream_t s) {
  const int ncols = a.epilogue == MOE_EPI_SILU_MUL ? a.N / 2 : a.N;
  const int bcols = a.epilogue == MOE_EPI_SILU_MUL ? kMxMmBN / 2 : kMxMmBN;
  const int nbn = (ncols + bcols - 1) / bcols;
  const dim3 grid = mm_grid(nbn, a.max_tiles);
  if (a.epilogue == MOE_EPI_SILU_MUL) gemm_mx_mm<MOE_EPI_SILU_MUL, kOutBf16, MODE, 3, AF><<<grid, 512, 0, s>>>(a);
  else if (a.out_f32 == kOutF16Exp) gemm_mx_mm<MOE_EPI_NONE, kOutF16Exp, MODE, 3, AF><<<grid, 512, 0, s>>>(a);
  else if (a.out_f32) gemm_mx_mm<MOE_EPI_NONE, kOutF32, MODE, 3, AF><<<grid, 512, 0, s>>>(a);
  else gemm_mx_mm<MOE_EPI_NONE, kOutBf16, MODE, 3, AF><<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

template <int BM, int BN, int KW, int PF, int MODE, int AF = 4>
static void launch_mx_mode(const MxGemmArgs& a, dim3 grid, hipStream_t s) {
  if (a.epilogue == MOE_EPI_SILU_MUL)
    gemm_mx_kernel<BM, BN, KW, PF, MOE_EPI_SILU_MUL, kOutBf16, MODE, AF><<<grid, 256, 0, s>>>(a);
  else if (a.out_f32 == kOutF16Exp)
    gemm_mx_kernel<BM, BN, KW, PF, MOE_EPI_NONE, kOutF16Exp, MODE, AF><<<grid, 256, 0, s>>>(a);
  else if (a.out_f32) gemm_mx_kernel<BM, BN, KW, PF, MOE_EPI_NONE, kOutF32, MODE, AF><<<grid, 256, 0, s>>>(a);
  else gemm_mx_kernel<BM, BN, KW, PF, MOE_EPI_NONE, kOutBf16, MODE, AF><<<grid, 256, 0, s>>>(a);
}

template <int BM, int BN, int KW, int PF>
static hipError_t launch_mx_cfg(const MxGemmArgs& a, hipStream_t s) {
  const int ncols = a.epilogue == MOE_EPI_SILU_MUL ? a.N / 2 : a.N;
  const int bcols = a.epilogue == MOE_EPI_SILU_MUL ? BN / 2 : BN;
  const dim3 grid = grid2d(8LL * ((a.max_tiles + 7) / 8) * ((ncols + bcols - 1) / bcols));
  if (a.act_e4m3) {  // W4A8
    switch (a.mode) {
      case 2: launch_mx_mode<BM, BN, KW, PF, 2, 0>(a, grid, s); break;
      case 1: launch_mx_mode<BM, BN, KW, PF, 1, 0>(a, grid, s); break;
      default: launch_mx_mode<BM, BN, KW, PF, 0, 0>(a, grid, s); break;
    }
    return hipGetLastError();
  }
  switch (a.mode) {
    case 2: launch_mx_mode<BM, BN, KW, PF, 2>(a, grid, s); break;
    case 1: launch_mx_mode<BM, BN, KW, PF, 1>(a, grid, s); break;
    default: launch_mx_mode<BM, BN, KW, PF, 0>(a, grid, s); break;
  }
  return hipGetLastError();
}

// Tile lists of at most this capacity (16-row tiles) split K four ways for down (decode).
constexpr int kMxSplitKMaxTiles = 32;

hipError_t launch_grouped_gemm_mx(const MxGemmArgs& a, int block_m, hipStream_t stream) {
  if (a.max_tiles <= 0) return hipSuccess;
  // fp16 output with in-band exponents: NONE epilogue, with its side array
  if (a.out_f32 == kOutF16Exp && (a.epilogue != MOE_EPI_NONE || !a.C_side)) return hipErrorInvalidValue;
  if (block_m == 128) {
    if (a.act_e4m3) return a.mode == 1 ? launch_mx_mm<1, 0>(a, stream) : launch_mx_mm<0, 0>(a, stream);
    return a.mode == 1 ? launch_mx_mm<1>(a, stream) : launch_mx_mm<0>(a, stream);
  }
  // Configurations from sweeps on MI355X (HIP events, weights streamed from HBM, packed weights and
  // tile-blocked activations), 128 experts top-8: gate_up at 1 / 8 / 64 tokens takes 7.7 / 18.8 /
  // 38.9 us as <16,64,KW2> against 10.3 / 21.3 / 39.7 us before; down at 8 tokens 10.3 us with a
  // 3-deep prefetch; at 800 tokens and 256 experts down takes 38.9 us as <32,128,KW2> against 46.3 us.
  const bool silu = a.epilogue == MOE_EPI_SILU_MUL;
  switch (block_m) {
    case 16:
      if (silu) return launch_mx_cfg<16, 64, 2, 2>(a, stream);
      if (a.max_tiles <= kMxSplitKMaxTiles) return launch_mx_cfg<16, 64, 4, 2>(a, stream);
      return launch_mx_cfg<16, 128, 1, 3>(a, stream);
    case 32:
      if (silu) return launch_mx_cfg<32, 128, 1, 2>(a, stream);
      return launch_mx_cfg<32, 128, 2, 2>(a, stream);
    default: return launch_mx_cfg<64, 128, 1, 2>(a, stream);
  }
}

}  // namespace moe
