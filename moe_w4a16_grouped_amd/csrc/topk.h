// Top-k routing of one token by one wave (device code shared by the router and the fused small-batch
// router + permutation).  Follows the ATOM page ("AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍"),
// section "8.1 MoE 路径：路由、专家并行与 MORI 通信" (routing and top-k selection).
//
// Lane l holds the logits of experts l, l + 64, ... as order-preserving 32-bit keys.  Selection by
// radix select: up to 32 ballot-count rounds find the k-th largest key value T (the largest value
// with at least k keys >= it), stopping early once a prefix separates exactly k keys; every key
// above T is kept, and among keys equal to T the lowest expert ids fill the remaining places, which
// is the (logit desc, id asc) order.  The k kept (key, id) pairs are compacted in LDS, ranked there
// by that order (slot 0 = largest), and the weights exp(l_s - l_0) / sum_j exp(l_j - l_0) are formed
// in slot order: the softmax restricted to the kept experts, which equals softmax-then-renormalise.
#pragma once
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

// The keys of lane l's experts l, l + 64, ... (0 for absent experts).
template <int NJ>
__device__ __forceinline__ void route_keys_load(const float* __restrict__ l, int E, uint32_t (&u)[NJ]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    u[j] = e < E ? ordered_bits(l[e]) : 0u;
  }
}

// Top-k of one token by one wave from its keys (route_keys_load).  kept and ranked are this wave's
// LDS scratch (k entries each); ids_out / w_out (NULL: not written, and no weights are formed)
// receive the token's k slots; ids_lds (may be NULL) receives a copy of the ids.
template <int NJ>
__device__ __forceinline__ void route_token_keys(const uint32_t (&u)[NJ], int E, int k, uint64_t* kept,
                                                 uint64_t* ranked, int32_t* __restrict__ ids_out,
                                                 float* __restrict__ w_out, int32_t* ids_lds) {
  const int lane = threadIdx.x & 63;
  bool valid[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) valid[j] = lane + 64 * j < E;
  // k-th largest key value: the largest p with #{keys >= p} >= k (k <= E, so p = 0 qualifies).
  // Every candidate is >= 1 and absent experts hold key 0, so they are never counted.  Once exactly
  // k keys are >= the accepted prefix, those k keys are the selection whatever the lower bits hold,
  // so the rounds stop there (p then stays below the k-th largest key, and the tie rule below keeps
  // all k: need equals the number of keys equal to p).
  uint32_t p = 0;
#pragma unroll 4
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = p | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) cnt += __popcll(__ballot(u[j] >= c));
    if (cnt >= k) {
      p = c;
      if (cnt == k) break;
    }
  }
  // keep every key above p and, in ascending id order, as many keys equal to p as places remain
  int need = k;
#pragma unroll
  for (int j = 0; j < NJ; ++j) need -= __popcll(__ballot(valid[j] && u[j] > p));
  const uint64_t below = (1ull << lane) - 1ull;
  int eq_before = 0, kept_before = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const bool eq = valid[j] && u[j] == p;
    const uint64_t eq_mask = __ballot(eq);
    const bool keep = valid[j] && (u[j] > p || (eq && eq_before + __popcll(eq_mask & below) < need));
    eq_before += __popcll(eq_mask);
    const uint64_t keep_mask = __ballot(keep);
    if (keep) kept[kept_before + __popcll(keep_mask & below)] = ((uint64_t)u[j] << 32) | (uint32_t)(~(uint32_t)(lane + 64 * j));
    kept_before += __popcll(keep_mask);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // rank of each kept pair among the kept pairs (keys are distinct: the low word is ~id)
  for (int c = lane; c < k; c += 64) {
    const uint64_t key = kept[c];
    int rank = 0;
    for (int c2 = 0; c2 < k; ++c2) rank += kept[c2] > key;
    ranked[rank] = key;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  if (!ids_out) {
    if (ids_lds)
      for (int s2 = lane; s2 < k; s2 += 64) ids_lds[s2] = (int)(~(uint32_t)ranked[s2]);
    return;
  }
  const float top = from_ordered_bits((uint32_t)(ranked[0] >> 32));
  float sum = 0.f;
  for (int s2 = 0; s2 < k; ++s2) sum += expf(from_ordered_bits((uint32_t)(ranked[s2] >> 32)) - top);
  for (int s2 = lane; s2 < k; s2 += 64) {
    const uint64_t key = ranked[s2];
    const int e = (int)(~(uint32_t)key);
    ids_out[s2] = e;
    w_out[s2] = expf(from_ordered_bits((uint32_t)(key >> 32)) - top) / sum;
    if (ids_lds) ids_lds[s2] = e;
  }
}

// route_token_keys with its own loads.
template <int NJ>
__device__ __forceinline__ void route_token(const float* __restrict__ l, int E, int k, uint64_t* kept,
                                            uint64_t* ranked, int32_t* __restrict__ ids_out,
                                            float* __restrict__ w_out, int32_t* ids_lds) {
  uint32_t u[NJ];
  route_keys_load<NJ>(l, E, u);
  route_token_keys<NJ>(u, E, k, kept, ranked, ids_out, w_out, ids_lds);
}

}  // namespace moe
