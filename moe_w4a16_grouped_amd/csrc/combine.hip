// Routing-weighted scatter-reduce ("combine"): y[t] = sum_s w[t,s] * O[inv_perm[t*k+s]].
// The ATOM page ("AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍"), section
// "8.1 MoE 路径：路由、专家并行与 MORI 通信", names the final combine that gathers each token's expert
// outputs back.  Slots are summed in fp32 in ascending order (deterministic, no atomics), then the
// shared expert's output is added if given (the Atlas page, section "KV Cache量化、MTP推测解码和调试
// 工具链", lists a shared expert output beside the routed output), and y is rounded to bf16 once;
// every element of y is written.
#include "launch.h"
#include "moe_common.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ O,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ shared, int T, int k, int H,
                                                      uint16_t* __restrict__ y) {
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
      f32x4 a[8], b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4* src = reinterpret_cast<const f32x4*>(O + (size_t)r[j] * H) + 2 * v;
        a[j] = src[0];
        b[j] = src[1];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] = fmaf(ws[j], a[j][i], acc[i]);
          acc[4 + i] = fmaf(ws[j], b[j][i], acc[4 + i]);
        }
    }
    for (; s < k; ++s) {
      const int r = inv_perm[(size_t)t * k + s];
      const float ws = w[(size_t)t * k + s];
      const f32x4* src = reinterpret_cast<const f32x4*>(O + (size_t)r * H) + 2 * v;
      const f32x4 a = src[0], b = src[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] = fmaf(ws, a[i], acc[i]);
        acc[4 + i] = fmaf(ws, b[i], acc[4 + i]);
      }
    }
    if (shared) {
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

hipError_t launch_combine(const float* O, const int32_t* inv_perm, const float* w, const float* shared, int T,
                          int k, int H, uint16_t* y, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int threads = H / 8 >= 256 ? 256 : ((H / 8 + 63) / 64) * 64;
  combine_kernel<<<T, threads, 0, stream>>>(O, inv_perm, w, shared, T, k, H, y);
  return hipGetLastError();
}

}  // namespace moe
