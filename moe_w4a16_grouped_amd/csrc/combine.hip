// Routing-weighted scatter-reduce ("combine"): y[t] = sum_s w[t,s] * O[inv_perm[t*k+s]].
// The ATOM page ("AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍"), section
// "8.1 MoE 路径：路由、专家并行与 MORI 通信", names the final combine that gathers each token's expert
// outputs back.  Slots are summed in fp32 in ascending order (deterministic, no atomics), then the
// shared expert's output is added if given (the Atlas page, section "KV Cache量化、MTP推测解码和调试
// 工具链", lists a shared expert output beside the routed output), and y is rounded to bf16 once;
// every element of y is written.  O is the down projection's output, fp32 or fp16 with an
// in-band power-of-two exponent per row and 8 columns (the layer's own launches use the latter).
#include "launch.h"
#include "moe_common.h"

namespace moe {

// One slot row's 8 values at column block v as loaded: fp32 O (two 16-byte halves), or the fp16
// segment (one 16-byte load).
struct RowRaw {
  u32x4 a, b;
};

template <bool O16>
__device__ __forceinline__ RowRaw load_row(const void* O, int r, int H, int v) {
  RowRaw x;
  if (O16) {
    x.a = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(O) + (size_t)r * H)[v];
    x.b = u32x4{0u, 0u, 0u, 0u};
  } else {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const float*>(O) + (size_t)r * H) + 2 * v;
    x.a = src[0];
    x.b = src[1];
  }
  return x;
}

// The 8 values in fp32.  An fp16 segment whose first element is the marker (an fp16 NaN carrying the
// segment's exponent + 256 in its low 9 bits) is scaled: every value is fp16 * 2^exp and the first one
// is O_side[r, v] * 2^exp; both products are exact in fp32.  (No unmarked segment holds a NaN.)
template <bool O16>
__device__ __forceinline__ void row_values(const RowRaw& x, const float* O_side, int r, int H, int v, float (&o)[8]) {
  if (O16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = f16_bits_to_f32(x.a[i] & 0xFFFFu);
      o[2 * i + 1] = f16_bits_to_f32(x.a[i] >> 16);
    }
    const uint32_t first = x.a[0] & 0xFFFFu;
    if ((first & 0x7E00u) == 0x7E00u) {
      const float f = pow2f((int)(first & 0x1FFu) - 256);  // 2^exp, -110 <= exp <= 113
      o[0] = O_side[(size_t)r * (H / 8) + v];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = __uint_as_float(x.a[i]);
      o[4 + i] = __uint_as_float(x.b[i]);
    }
  }
}

template <bool O16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ O, const float* __restrict__ O_side,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ shared, int shared_o_row0, int T,
                                                      int k, int H, uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  const int nvec = H / 8;
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // whole chunks of 8 slots: every row index and weight of the chunk, then every row, are loaded
    // before its first FMA, so a chunk costs two dependent round trips instead of two per slot; the
    // remaining slots one by one.  The FMAs run in ascending slot order either way.
    int s = 0;
    for (; s + 8 <= k; s += 8) {
      int r[8];
      float ws[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        r[j] = inv_perm[(size_t)t * k + s + j];
        ws[j] = w[(size_t)t * k + s + j];
      }
      RowRaw x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = load_row<O16>(O, r[j], H, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float o[8];
        row_values<O16>(x[j], O_side, r[j], H, v, o);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(ws[j], o[i], acc[i]);
      }
    }
    for (; s < k; ++s) {
      const int r = inv_perm[(size_t)t * k + s];
      const float ws = w[(size_t)t * k + s];
      const RowRaw x = load_row<O16>(O, r, H, v);
      float o[8];
      row_values<O16>(x, O_side, r, H, v, o);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(ws, o[i], acc[i]);
    }
    if (shared_o_row0 >= 0) {  // the shared expert's output is row shared_o_row0 + t of O
      const RowRaw x = load_row<O16>(O, shared_o_row0 + t, H, v);
      float o[8];
      row_values<O16>(x, O_side, shared_o_row0 + t, H, v, o);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += o[i];
    } else if (shared) {
      const f32x4* src = reinterpret_cast<const f32x4*>(shared + (size_t)t * H) + 2 * v;
      const f32x4 a = src[0], b = src[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += a[i];
        acc[4 + i] += b[i];
      }
    }
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[i] = (uint32_t)f32_to_bf16_bits(acc[2 * i]) | ((uint32_t)f32_to_bf16_bits(acc[2 * i + 1]) << 16);
    reinterpret_cast<u32x4*>(y + (size_t)t * H)[v] = out;
  }
}

hipError_t launch_combine(const void* O, const float* O_side, const int32_t* inv_perm, const float* w,
                          const float* shared, int shared_o_row0, int T, int k, int H, uint16_t* y,
                          hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int threads = H / 8 >= 256 ? 256 : ((H / 8 + 63) / 64) * 64;
  if (O_side)
    combine_kernel<true><<<T, threads, 0, stream>>>(O, O_side, inv_perm, w, shared, shared_o_row0, T, k, H, y);
  else
    combine_kernel<false><<<T, threads, 0, stream>>>(O, O_side, inv_perm, w, shared, shared_o_row0, T, k, H, y);
  return hipGetLastError();
}

}  // namespace moe
