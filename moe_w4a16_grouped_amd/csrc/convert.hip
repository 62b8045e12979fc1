// bf16 activations -> fp16 with one power-of-two exponent per row, the activation operand of the exact
// fp16 path of the grouped GEMM (64- and 128-row tile kernels).
//
// The weights of that path are E2M1 code * bf16 scale formed exactly in fp16 (at most 2 + 8
// significant bits), so the products with fp16 activations are exact in the fp32 MFMA accumulation,
// like the bf16 path's; the group scale then needs no separate fp32 multiply per output.  A bf16 row
// has 8 significant bits per value but bf16's exponent range; fp16 has 11 bits and a narrow range.
// Each row is therefore scaled by 2^-e with e = floor(log2 max|x|) - 14, which puts its largest finite
// magnitude in [2^14, 2^15): every value at most 2^31 below the row's maximum converts exactly, the
// rest round to fp16's subnormal spacing.  The grouped GEMM multiplies its fp32 row sums by 2^e
// (exact).  Non-finite values stay non-finite; an all-zero row takes e = 0.
#include "launch.h"
#include "moe_common.h"

namespace moe {

// Row exponent from the largest finite bf16 magnitude (as its 15-bit pattern; 0 = all zero).
__device__ __forceinline__ int row_exponent(uint32_t maxbits) {
  if (maxbits == 0u) return 0;
  const int e = ilogbf(bf16_bits_to_f32(maxbits)) - 14;
  return e < -110 ? -110 : (e > 113 ? 113 : e);
}

// One wave per row: the largest finite magnitude (an integer maximum of the 15-bit patterns, which
// order like the values), then every 8-element chunk scaled by 2^-e and rounded to fp16 (to nearest
// even).  H % 8 == 0.
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                       uint16_t* __restrict__ x16, int32_t* __restrict__ xexp) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)t * H);
  const int nc = H / 8;
  uint32_t m = 0;
  for (int c = lane; c < nc; c += 64) {
    const u32x4 v = src[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = v[i] & 0x7FFFu, hi = (v[i] >> 16) & 0x7FFFu;
      if (lo < 0x7F80u) m = max(m, lo);
      if (hi < 0x7F80u) m = max(m, hi);
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d));
  const int e = row_exponent(m);
  const float f = pow2f(-e);
  if (lane == 0) xexp[t] = e;
  u32x4* dst = reinterpret_cast<u32x4*>(x16 + (size_t)t * H);
  for (int c = lane; c < nc; c += 64) {
    const u32x4 v = src[c];
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_bits_to_f32(v[i] & 0xFFFFu) * f, b = bf16_bits_to_f32(v[i] >> 16) * f;
      o[i] = (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(b) << 16);
    }
    dst[c] = o;
  }
}

hipError_t launch_x_to_f16(const uint16_t* x, int T, int H, uint16_t* x16, int32_t* xexp, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  x_to_f16_kernel<<<(T + 3) / 4, 256, 0, stream>>>(x, T, H, x16, xexp);
  return hipGetLastError();
}

}  // namespace moe
