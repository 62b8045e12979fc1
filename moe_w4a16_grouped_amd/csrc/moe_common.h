// Device-side helpers shared by the kernels of libmoe_w4a16 (gfx950 / CDNA4 only).
//
// Weight format (the execution contract of the layer, following the ATOM page
// "AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍", section "8.2 量化并非单一格式，
// 而是一套执行契约": dtype, scale shape and layout are part of the kernel's contract):
//   * E2M1 4-bit codes, two per byte, the even K index in the low nibble;
//   * one bf16 scale per 32 consecutive K elements of a weight row (per-1x32 grouping, ATOM page,
//     section "6.1 Linear：按量化类型分派 GEMM");
//   * rows are K-contiguous: gate_up [E, 2I, H] (gate rows [0, I), up rows [I, 2I)), down [E, H, I].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 32;    // K elements per scale
constexpr int kWave = 64;     // CDNA wavefront

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Eight E2M1 codes (one dword, element 0 in the low nibble) -> eight exact bf16 values.
// The hardware FP4 converter is used with a unit scale, so every code lands exactly on its E2M1
// value (0, ±0.5, ±1, ±1.5, ±2, ±3, ±4, ±6); the group scale is applied later in fp32.
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16(uint32_t w) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// ---- fp16 operands (the exact fp16 path of the 64- and 128-row tile kernels) ---------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// A bf16 group scale whose products with every E2M1 value are exact in fp16 has an exponent in
// [-16, 12] (then the scale is exact in fp16, 6 * scale stays below fp16's largest finite value and
// 0.5 * scale keeps its lowest bit at or above 2^-24).  For a positive scale that is the bit range
// [0x3780, 0x4600).  Whether all scales of the given dwords (two bf16 scales each) pass: the bits
// minus 0x3780 as unsigned 16-bit lanes, largest below 0x0E80.  Zero, negative, subnormal and
// non-finite scales fail (the general form handles them).
template <int N>
__device__ __forceinline__ bool scales_f16_ok(const uint32_t (&v)[N]) {
  u16x2 worst = u16x2{0, 0};
#pragma unroll
  for (int i = 0; i < N; ++i)
    worst = __builtin_elementwise_max(worst, __builtin_bit_cast(u16x2, v[i]) - u16x2{0x3780, 0x3780});
  return worst[0] < 0x0E80 && worst[1] < 0x0E80;
}

// The general form's split of a scale into m * 2^d with m's exponent in [-16, 12] (so code * m is
// exact in fp16); d = 0 for scales already in range and for zero and non-finite scales.
__device__ __forceinline__ int scale_f16_shift(float sc) {
  const int e = __builtin_amdgcn_frexp_expf(sc) - 1;  // |sc| in [2^e, 2^(e+1)); 0 -> -1, inf/nan -> -1
  return e > 12 ? e - 12 : (e < -16 ? e + 16 : 0);
}

// bf16 bits of m = sc * 2^-scale_f16_shift(sc) (exact: m keeps sc's eight significant bits).
__device__ __forceinline__ uint32_t scale_f16_mantissa_bits(float sc) {
  return __float_as_uint(ldexpf(sc, -scale_f16_shift(sc))) >> 16;
}

// Eight E2M1 codes -> eight fp16 values code * scale: the hardware converter at unit scale gives the
// exact E2M1 values (it applies only the exponent of a scale operand, so the scale is not given to
// it), then one packed fp16 multiply by the scale per pair, exact for scales with an exponent in
// [-16, 12].
__device__ __forceinline__ f16x8 e2m1x8_to_f16(uint32_t w, _Float16 sc) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  const f16x2 s2 = f16x2{sc, sc};
  p0 *= s2;
  p1 *= s2;
  p2 *= s2;
  p3 *= s2;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ f32x4 mfma16x16x32_f16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 2^e as fp32 for -126 <= e <= 127 (exact).
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// 4x4 transpose of dwords across the four 16-lane quarters of a wave.
// Before: quarter q, register j holds dword j of K-group q (one 16-byte load per lane).
// After:  register g, quarter q holds dword q of K-group g, which is the B-operand layout of
//         v_mfma_f32_16x16x32_bf16 for group g (quarter q supplies K elements 8q..8q+7).
__device__ __forceinline__ u32x4 quarter_transpose(u32x4 v) {
  auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  return u32x4{c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// silu(g) = g / (1 + e^-g); the quotient uses the fast reciprocal (the result is rounded to bf16).
__device__ __forceinline__ float silu_f32(float g) { return __fdividef(g, 1.0f + __expf(-g)); }

// s_waitcnt: vector-memory counter <= N, others not waited on (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Direct global->LDS 16-byte load (lane l writes LDS bytes [16l, 16l+16) after the wave-uniform
// base).  Issued through inline assembly so that the compiler does not fence every later LDS read
// behind it; the kernel orders these loads itself with explicit vmcnt waits and barriers.
__device__ __forceinline__ void g2lds16(const void* g, void* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}


// Output kinds of the NONE epilogue (GemmArgs::out_f32): 0 bf16, 1 fp32, 2 fp16 (kOutF16Exp) with
// an exponent per row and 8-column segment that is carried in band.  A segment is stored plainly
// (8 fp16 values, exponent 0) when its largest finite magnitude m is 0 or in [2^-6, 2^15) and it
// holds no non-finite value; otherwise it is scaled by 2^-exp, exp = floor(log2 m) - 14 (exact; m then
// lies in [2^14, 2^15)), its first element is replaced by a marker (an fp16 NaN whose low 9 bits are
// exp + 256) and that element's scaled value goes to C_side[row, col / 8] in fp32.  fp16 keeps 11
// significant bits where bf16 keeps 8; the exponent keeps any fp32 range representable (tiny segments
// included), and in the common case nothing but the fp16 values is written.
constexpr int kOutBf16 = 0, kOutF32 = 1, kOutF16Exp = 2;
constexpr uint16_t kF16Marker = 0x7E00;  // quiet NaN; low 9 bits: the segment's exponent + 256
constexpr float kF16Small = 0.015625f;   // 2^-6: smaller maxima are scaled up

// Exponent of a row segment (or of a row's 32 columns of h) with largest finite magnitude m: 0 when m
// is 0 or in [2^-6, 2^15), else floor(log2 m) - 14 clamped to [-110, 113].
__device__ __forceinline__ int f16_seg_exponent(float m) {
  if (m == 0.f || (m >= kF16Small && m < 32768.f)) return 0;
  const int e = ilogbf(m) - 14;
  return e < -110 ? -110 : (e > 113 ? 113 : e);
}

// OR of v over the 8 lanes of each aligned group of 8 (a segment), by DPP lane moves within a row of
// 16: quad_perm [1,0,3,2], quad_perm [2,3,0,1], then row_half_mirror (lane i of a half-row takes
// lane 7 - i), after which every lane holds its segment's OR.
__device__ __forceinline__ uint32_t seg8_or(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true);
  return v;
}

// Largest value of m over each row of 16 lanes (a quarter of the wave), by DPP lane moves: the
// two quad swaps and the half-row mirror of seg8_or, then row_mirror (lane i <-> 15 - i).  (fmaxf
// ignores a NaN operand, so the order of the moves does not change the result.)
__device__ __forceinline__ float row16_max(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, true)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, true)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x141, 0xF, 0xF, true)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x140, 0xF, 0xF, true)));
  return m;
}

// The 8 columns of a segment live in 8 lanes of a quarter (one lane per column, l16 = 8j .. 8j+7):
// the largest finite magnitude over them, and whether any is non-finite.
__device__ __forceinline__ float seg8_max_finite(float v, bool& nonfinite) {
  const bool nf = !(fabsf(v) <= 3.4e38f);
  float m = nf ? 0.f : fabsf(v);
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, true)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, true)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x141, 0xF, 0xF, true)));
  int f = nf;
  f = (int)seg8_or((uint32_t)f);
  nonfinite = f != 0;
  return m;
}

// A wave's MI x NI blocks of 16 x 16 fp32 results stored as kOutF16Exp: lane (q, l16) holds rows
// row_base + mi*16 + q*4 + r (r < 4) of the tile starting at row0, at columns ncol[ni] (l16 the column
// within the block, so an 8-column segment is 8 lanes of a quarter).  C fp16 [rows, N], C_side fp32
// [rows, ceil(N / 8)]; rows at or past `rows` and columns with nvalid false are not written.  When no
// segment of the wave needs an exponent (the common case) each value is just rounded to fp16.
// PAD_ROWS: the tile's padding rows may hold anything (zeros, stale data) and are left out of that
// test; without it they are taken to be copies of a real row, whose values are representative.
template <int MI, int NI, bool PAD_ROWS>
__device__ __forceinline__ void store_f16e(uint16_t* C, float* C_side, int N, const f32x4 (&acc)[MI][NI], int row_base,
                                           int row0, int rows, int q, const int (&ncol)[NI], const bool (&nvalid)[NI]) {
  // some segment of this wave may need an exponent (a magnitude of 2^15 or more, a non-finite value,
  // or all eight below 2^-6; an invalid column counts as below).  With PAD_ROWS a padding row's
  // segments count as neither.  Bit j of `keep` says that value j of this lane is not below 2^-6;
  // OR-ed over the 8 lanes of each segment (lanes differing in their three low bits), a clear bit
  // marks a segment whose values are all below.
  constexpr int NV = MI * NI * 4;
  static_assert(NV <= 64, "a lane holds at most 64 values");
  bool big = false;
  uint32_t keep_lo = 0u, keep_hi = 0u;
  const int row_lim = rows - row_base - q * 4;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool live = !PAD_ROWS || mi * 16 + r < row_lim;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int j = (mi * 4 + r) * NI + ni;
        const float a = !live ? 1.f : (nvalid[ni] ? fabsf(acc[mi][ni][r]) : 0.f);
        big |= !(a < 32768.f);
        const uint32_t bit = a < kF16Small ? 0u : 1u;
        if (j < 32) keep_lo |= bit << j;
        else keep_hi |= bit << (j - 32);
      }
    }
  // the OR over a segment's 8 lanes by row-local lane moves: swap neighbours, swap pairs, then
  // mirror each half-row of 8 (lane i <-> 7 - i)
  keep_lo = seg8_or(keep_lo);
  if constexpr (NV > 32) keep_hi = seg8_or(keep_hi);
  constexpr uint32_t kFullLo = NV >= 32 ? 0xFFFFFFFFu : ((1u << (NV & 31)) - 1u);
  constexpr uint32_t kFullHi = NV >= 64 ? 0xFFFFFFFFu : (NV > 32 ? ((1u << ((NV - 32) & 31)) - 1u) : 0u);
  const bool tiny_here = keep_lo != kFullLo || keep_hi != kFullHi;
  const bool scaled = __ballot(big || tiny_here) != 0ull;
  if (!scaled) {
    // the common case: every value just rounded to fp16, row by row
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row_base + mi * 16 + q * 4 + r;
        if (row >= rows) continue;
        uint16_t* crow = C + (size_t)(row0 + row) * N;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          if (nvalid[ni]) crow[ncol[ni]] = f32_to_f16_bits(acc[mi][ni][r]);
      }
    return;
  }
  const int l16 = threadIdx.x & 15;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row_base + mi * 16 + q * 4 + r;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        float v = nvalid[ni] ? acc[mi][ni][r] : 0.f;
        // every lane takes part in the segment reductions, whatever its row
        bool nonfinite;
        const float m = seg8_max_finite(v, nonfinite);
        const int ex = f16_seg_exponent(m);
        v *= pow2f(-ex);  // exact
        uint16_t bits = f32_to_f16_bits(v);
        if ((ex != 0 || nonfinite) && (l16 & 7) == 0) {
          bits = (uint16_t)(kF16Marker | (ex + 256));
          if (row < rows && nvalid[ni]) C_side[(size_t)(row0 + row) * (size_t)((N + 7) / 8) + ncol[ni] / 8] = v;
        }
        if (row < rows && nvalid[ni]) C[(size_t)(row0 + row) * N + ncol[ni]] = bits;
      }
    }
}

// Launch grids are 2-D: x holds at most kGridX workgroups (a multiple of 8, so with linear index
// b = y * gridDim.x + x, b % 8 still names the XCD) and y as many rows as the work list needs.
constexpr unsigned kGridX = 8u << 16;

__device__ __forceinline__ long long linear_block() {
  return (long long)blockIdx.y * gridDim.x + blockIdx.x;
}

// Work order of the grouped GEMMs' tile lists.  Workgroup b runs on XCD b % 8 (workgroups are dispatched
// round-robin over the 8 XCDs, each with its own L2).  XCD x takes the contiguous share
// [x*n/8, (x+1)*n/8) of the n tiles and runs all N blocks of one tile before the next, so a tile's
// gathered activation rows are fetched into that XCD's L2 once, and consecutive tiles of one expert
// find its weights there.  The work list holds 8 * ceil(max_tiles / 8) * nbn slots; slots past the
// XCD's share are skipped.
__device__ __forceinline__ bool xcd_tile(long long b, int nbn, int num_tiles, int& tile, int& nb) {
  const int xcd = (int)(b & 7);
  const long long j = b >> 3;
  const int lt = (int)(j / nbn);
  nb = (int)(j - (long long)lt * nbn);
  const int t0 = (xcd * num_tiles) >> 3, t1 = ((xcd + 1) * num_tiles) >> 3;
  tile = t0 + lt;
  return tile < t1;
}

// Host side: the 2-D grid for `total` workgroups.
static inline dim3 grid2d(long long total) {
  if (total <= (long long)kGridX) return dim3((unsigned)total, 1);
  return dim3(kGridX, (unsigned)((total + kGridX - 1) / kGridX));
}

// Work order of the large-tile (LDS-staged) kernels.  With at least 8 N blocks, XCD x takes the N
// blocks nb = x, x + 8, ... of every tile, tile after tile: a tile's activations are fetched once
// per XCD and each XCD's L2 keeps its own share of an expert's weight columns across the expert's
// tiles.  With fewer N blocks that order would leave XCDs idle, so the XCDs take contiguous shares of
// the tile list instead (xcd_tile).  The grid comes from mm_grid.
__device__ __forceinline__ bool mm_work(long long b, int nbn, int num_tiles, int& tile, int& nb) {
  if (nbn >= 8) {
    const int nbx = (nbn + 7) / 8;
    const long long j = b >> 3;
    tile = (int)(j / nbx);
    nb = (int)(b & 7) + 8 * (int)(j % nbx);
    return nb < nbn && tile < num_tiles;
  }
  return xcd_tile(b, nbn, num_tiles, tile, nb);
}

static inline dim3 mm_grid(int nbn, int max_tiles) {
  if (nbn >= 8) return grid2d(8LL * ((nbn + 7) / 8) * max_tiles);
  return grid2d(8LL * ((max_tiles + 7) / 8) * nbn);
}

}  // namespace moe
