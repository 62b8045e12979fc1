// Top-k router: softmax over E logits, keep the k largest, renormalise over the kept k.
// Follows the ATOM page ("AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍"),
// section "8.1 MoE 路径：路由、专家并行与 MORI 通信" (routing and top-k selection).
//
// One wave64 per token.  Each lane holds ceil(E/64) logits as 64-bit keys
// (order-preserving fp32 bits << 32 | ~expert_id), so one unsigned max picks the largest logit and,
// among equal logits, the lower expert id.  k rounds of a wave-wide max (DPP row operations)
// select the experts in order; the weights exp(l_s - l_0) / sum_j exp(l_j - l_0) are the softmax
// restricted to the kept experts, which equals softmax-then-renormalise.
#include "launch.h"
#include "moe_common.h"

namespace moe {

__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 compares equal to +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// Max of a 64-bit key over the wave with DPP row operations (xor 1, xor 2 in quads, half-row and
// row mirrors, then the row broadcasts 15 and 31), leaving the result in lane 63; read back as a
// wave-uniform value.  Lanes that a DPP step does not feed keep their own key (max with 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

template <int NJ>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? ((uint64_t)ordered_bits(l[e]) << 32) | (uint32_t)(~(uint32_t)e) : 0ull;
  }
  // slot s is owned by lane s % 64 (register j = s / 64): id and exp(l_s - l_0)
  constexpr int MAXK = 16;  // slots kept per lane: k <= 64 * MAXK
  int my_id[MAXK];
  float my_p[MAXK];
  float top = 0.f, sum = 0.f;
  for (int s = 0; s < k; ++s) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int j = 0; j < NJ; ++j) key[j] = key[j] == best ? 0ull : key[j];
    const int e = (int)(~(uint32_t)best);
    const float v = from_ordered_bits((uint32_t)(best >> 32));
    if (s == 0) top = v;
    const float p = expf(v - top);
    sum += p;
#pragma unroll
    for (int j = 0; j < MAXK; ++j)
      if (s == 64 * j + lane) { my_id[j] = e; my_p[j] = p; }
  }
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    const int s = 64 * j + lane;
    if (s < k) {
      ids[(size_t)t * k + s] = my_id[j];
      w[(size_t)t * k + s] = my_p[j] / sum;
    }
  }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t stream) {
  const dim3 grid((T + 3) / 4), block(256);
  const int nj = (E + 63) / 64;
  if (nj <= 1) route_topk_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w);
  else if (nj <= 2) route_topk_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w);
  else if (nj <= 4) route_topk_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w);
  else if (nj <= 8) route_topk_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w);
  else route_topk_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
