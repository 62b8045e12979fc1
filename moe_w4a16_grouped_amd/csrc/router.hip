// Router gate: logits[t, e] = sum_h x[t, h] * w_router[e, h], bf16 inputs, fp32 result.
// The Atlas page ("告别Python堆栈：Atlas用纯Rust重写LLM推理，在GB10上跑赢vLLM"), section
// "KV Cache量化、MTP推测解码和调试工具链", names the gate input and the gate logits among the
// per-layer MoE quantities; the logits then feed the top-k routing.
//
// A small dense GEMM (K = hidden size, long; M = tokens and N = experts, short) on MFMA.  A
// workgroup of MW * NW * KW waves computes a (16 MW) x (16 NW) block of logits; the waves split the
// K range KW ways, each accumulating a 16 x 16 block with v_mfma_f32_16x16x32_bf16, and the KW
// partial sums are added in LDS in ascending K order (so results do not depend on timing).
// Fragments come straight from global memory: lane l reads 8 consecutive K elements of token /
// expert row l % 16 at K offset 8 * (l / 16) with one 16-byte load, through a register ring D steps
// deep, so each wave keeps D K steps of loads in flight.  Splitting K keeps the serial chain per
// wave short, which is what bounds this kernel at decode sizes.  Rows past T or E re-read the last
// valid row and are not stored.
#include "launch.h"
#include "moe_common.h"

namespace moe {

template <int MW, int NW, int KW, int D>
__global__ __launch_bounds__(64 * MW * NW * KW) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                          const uint16_t* __restrict__ wr, int T,
                                                                          int H, int E, float* __restrict__ logits) {
  __shared__ f32x4 part[KW > 1 ? MW * NW * KW * 64 : 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wk = wave % KW, wn = (wave / KW) % NW, wm = wave / (KW * NW);
  const int l16 = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * (16 * MW) + wm * 16, e0 = blockIdx.y * (16 * NW) + wn * 16;
  const int nsteps = H / 32;
  const int s_begin = (wk * nsteps) / KW, s_end = ((wk + 1) * nsteps) / KW;
  const uint16_t* xa = x + (size_t)min(t0 + l16, T - 1) * H + q * 8;
  const uint16_t* wb = wr + (size_t)min(e0 + l16, E - 1) * H + q * 8;

  bf16x8 ra[D], rb[D];
  auto load = [&](int s, int u) {
    ra[u] = *reinterpret_cast<const bf16x8*>(xa + (size_t)s * 32);
    rb[u] = *reinterpret_cast<const bf16x8*>(wb + (size_t)s * 32);
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (s_begin < s_end) {
#pragma unroll
    for (int u = 0; u < D; ++u) load(min(s_begin + u, s_end - 1), u);
    for (int s0 = s_begin; s0 < s_end; s0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        if (s0 + u < s_end) acc = mfma16x16x32(ra[u], rb[u], acc);
        if (s0 + u + D < s_end) load(s0 + u + D, u);
      }
    }
  }
  if constexpr (KW > 1) {
    part[wave * 64 + lane] = acc;
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int j = 1; j < KW; ++j) {
      const f32x4 o = part[(wave + j) * 64 + lane];
      acc[0] += o[0];
      acc[1] += o[1];
      acc[2] += o[2];
      acc[3] += o[3];
    }
  }
  const int e = e0 + l16;
  if (e >= E) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + 4 * q + r;
    if (t < T) logits[(size_t)t * E + e] = acc[r];
  }
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, int T, int H, int E, float* logits,
                                hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  // 32 x 32 blocks (K split 2 ways) once they alone give at least one workgroup per CU; otherwise
  // 16 x 16 blocks with K split 8 ways, which multiplies the waves in flight at decode sizes.
  // Tokens go along grid x (no 65535 limit on T).
  const long long big = (long long)((T + 31) / 32) * ((E + 31) / 32);
  if (big >= 256) {
    const dim3 grid((T + 31) / 32, (E + 31) / 32);
    router_logits_kernel<2, 2, 2, 8><<<grid, 512, 0, stream>>>(x, w_router, T, H, E, logits);
  } else {
    const dim3 grid((T + 15) / 16, (E + 15) / 16);
    router_logits_kernel<1, 1, 8, 8><<<grid, 512, 0, stream>>>(x, w_router, T, H, E, logits);
  }
  return hipGetLastError();
}

}  // namespace moe
