// Router gate: logits[t, e] = sum_h x[t, h] * w_router[e, h], bf16 inputs, fp32 result.
// The Atlas page ("告别Python堆栈：Atlas用纯Rust重写LLM推理，在GB10上跑赢vLLM"), section
// "KV Cache量化、MTP推测解码和调试工具链", names the gate input and the gate logits among the
// per-layer MoE quantities; the logits then feed the top-k routing.
//
// A small dense GEMM on MFMA: each workgroup computes 32 tokens x 64 experts with four waves
// (2 x 2), each wave 16 tokens x 32 experts as two v_mfma_f32_16x16x32_bf16 blocks accumulated in
// fp32.  Fragments come straight from global memory (16-byte loads; lane l reads 8 consecutive K
// elements of token / expert row l % 16 at K offset 8 * (l / 16)), through a register ring
// kDepth K steps deep, so a wave keeps that many steps of loads in flight.  Rows past T or E
// re-read the last valid row and are not stored.
#include "launch.h"
#include "moe_common.h"

namespace moe {

constexpr int kRouterDepth = 8;

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr, int T, int H,
                                                            int E, float* __restrict__ logits) {
  constexpr int D = kRouterDepth;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 32 + wm * 16, e0 = blockIdx.y * 64 + wn * 32;
  const uint16_t* xa = x + (size_t)min(t0 + l16, T - 1) * H + q * 8;
  const uint16_t* w0 = wr + (size_t)min(e0 + l16, E - 1) * H + q * 8;
  const uint16_t* w1 = wr + (size_t)min(e0 + 16 + l16, E - 1) * H + q * 8;
  const int nsteps = H / 32;

  bf16x8 ra[D], rb0[D], rb1[D];
  auto load = [&](int s, int u) {
    const size_t off = (size_t)min(s, nsteps - 1) * 32;  // past the end: re-read the last step (unused)
    ra[u] = *reinterpret_cast<const bf16x8*>(xa + off);
    rb0[u] = *reinterpret_cast<const bf16x8*>(w0 + off);
    rb1[u] = *reinterpret_cast<const bf16x8*>(w1 + off);
  };
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, u);
  for (int s0 = 0; s0 < nsteps; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      if (s0 + u < nsteps) {
        acc0 = mfma16x16x32(ra[u], rb0[u], acc0);
        acc1 = mfma16x16x32(ra[u], rb1[u], acc1);
      }
      load(s0 + u + D, u);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + 4 * q + r;
    if (t >= T) continue;
    if (e0 + l16 < E) logits[(size_t)t * E + e0 + l16] = acc0[r];
    if (e0 + 16 + l16 < E) logits[(size_t)t * E + e0 + 16 + l16] = acc1[r];
  }
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, int T, int H, int E, float* logits,
                                hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((T + 31) / 32, (E + 63) / 64);  // tokens along x: no 65535 limit on T
  router_logits_kernel<<<grid, 256, 0, stream>>>(x, w_router, T, H, E, logits);
  return hipGetLastError();
}

}  // namespace moe
