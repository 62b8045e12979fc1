// Top-k router: softmax over E logits, keep the k largest, renormalise over the kept k.
// Follows the ATOM page ("AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍"),
// section "8.1 MoE 路径：路由、专家并行与 MORI 通信" (routing and top-k selection).
//
// One wave64 per token (the selection itself is in topk.h).
#include "launch.h"
#include "topk.h"

namespace moe {

template <int NJ>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  extern __shared__ uint64_t route_lds[];  // per wave: k compacted pairs, then k ranked pairs
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  uint64_t* kept = route_lds + (size_t)wv * 2 * k;
  route_token<NJ>(logits + (size_t)t * E, E, k, kept, kept + k, ids + (size_t)t * k, w + (size_t)t * k, nullptr);
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t stream) {
  const dim3 grid((T + 3) / 4), block(256);
  const size_t lds = 4 * 2 * (size_t)k * sizeof(uint64_t);
  const int nj = (E + 63) / 64;
  if (nj <= 1) route_topk_kernel<1><<<grid, block, lds, stream>>>(logits, T, E, k, ids, w);
  else if (nj <= 2) route_topk_kernel<2><<<grid, block, lds, stream>>>(logits, T, E, k, ids, w);
  else if (nj <= 4) route_topk_kernel<4><<<grid, block, lds, stream>>>(logits, T, E, k, ids, w);
  else if (nj <= 8) route_topk_kernel<8><<<grid, block, lds, stream>>>(logits, T, E, k, ids, w);
  else route_topk_kernel<16><<<grid, block, lds, stream>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
