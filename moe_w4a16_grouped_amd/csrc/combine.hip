// Routing-weighted scatter-reduce ("combine"): y[t] = sum_s w[t,s] * O[inv_perm[t*k+s]].
// The ATOM page ("AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍"), section
// "8.1 MoE 路径：路由、专家并行与 MORI 通信", names the final combine that gathers each token's expert
// outputs back.  Slots are summed in fp32 in ascending order (deterministic, no atomics), then the
// shared expert's output is added if given (the Atlas page, section "KV Cache量化、MTP推测解码和调试
// 工具链", lists a shared expert output beside the routed output), and y is rounded to bf16 once;
// every element of y is written.  O is the down projection's output, fp32 or fp16 with a
// power-of-two exponent per row and 16 columns (the layer's own launches use the latter).
#include "launch.h"
#include "moe_common.h"

namespace moe {

// One slot row's 8 values at column block v as loaded: fp32 O (two 16-byte halves), or fp16 O
// (one 16-byte load) and its exponent byte.
struct RowRaw {
  u32x4 a, b;
  uint32_t ex;
};

template <bool O16>
__device__ __forceinline__ RowRaw load_row(const void* O, const uint8_t* O_exp, int r, int H, int v) {
  RowRaw x;
  if (O16) {
    x.a = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(O) + (size_t)r * H)[v];
    x.b = u32x4{0u, 0u, 0u, 0u};
    x.ex = O_exp[(size_t)r * (H / 16) + v / 2];
  } else {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const float*>(O) + (size_t)r * H) + 2 * v;
    x.a = src[0];
    x.b = src[1];
    x.ex = 0;
  }
  return x;
}

// The 8 values in fp32: fp16 * 2^exp is exact in fp32.
template <bool O16>
__device__ __forceinline__ void row_values(const RowRaw& x, float (&o)[8]) {
  if (O16) {
    const float f = __uint_as_float((127u + x.ex) << 23);  // 2^ex, ex <= 113
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = f16_bits_to_f32(x.a[i] & 0xFFFFu) * f;
      o[2 * i + 1] = f16_bits_to_f32(x.a[i] >> 16) * f;
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
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ O, const uint8_t* __restrict__ O_exp,
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
      for (int j = 0; j < 8; ++j) x[j] = load_row<O16>(O, O_exp, r[j], H, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float o[8];
        row_values<O16>(x[j], o);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(ws[j], o[i], acc[i]);
      }
    }
    for (; s < k; ++s) {
      const int r = inv_perm[(size_t)t * k + s];
      const float ws = w[(size_t)t * k + s];
      const RowRaw x = load_row<O16>(O, O_exp, r, H, v);
      float o[8];
      row_values<O16>(x, o);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(ws, o[i], acc[i]);
    }
    if (shared_o_row0 >= 0) {  // the shared expert's output is row shared_o_row0 + t of O
      const RowRaw x = load_row<O16>(O, O_exp, shared_o_row0 + t, H, v);
      float o[8];
      row_values<O16>(x, o);
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

hipError_t launch_combine(const void* O, const uint8_t* O_exp, const int32_t* inv_perm, const float* w,
                          const float* shared, int shared_o_row0, int T, int k, int H, uint16_t* y,
                          hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int threads = H / 8 >= 256 ? 256 : ((H / 8 + 63) / 64) * 64;
  if (O_exp)
    combine_kernel<true><<<T, threads, 0, stream>>>(O, O_exp, inv_perm, w, shared, shared_o_row0, T, k, H, y);
  else
    combine_kernel<false><<<T, threads, 0, stream>>>(O, O_exp, inv_perm, w, shared, shared_o_row0, T, k, H, y);
  return hipGetLastError();
}

}  // namespace moe
