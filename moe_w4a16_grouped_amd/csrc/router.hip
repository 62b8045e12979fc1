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
//
// Work order: workgroup b runs on XCD b % 8 (round-robin dispatch; each XCD has its own L2).  The
// (token block, expert block) pairs are numbered token-major and XCD x takes the contiguous share
// [x * P / 8, (x + 1) * P / 8) of the P pairs, so each XCD reads about 1/8 of x and the router
// weight once into its L2, instead of every XCD streaming all of both.
#include "launch.h"
#include "moe_common.h"

namespace moe {

template <int MW, int NW, int KW, int D>
__global__ __launch_bounds__(64 * MW * NW * KW) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                          const uint16_t* __restrict__ wr, int T,
                                                                          int H, int E, float* __restrict__ logits) {
  __shared__ f32x4 part[KW > 1 ? MW * NW * KW * 64 : 1];
  const int neb = (E + 16 * NW - 1) / (16 * NW);
  const long long P = (long long)((T + 16 * MW - 1) / (16 * MW)) * neb;
  const int xcd = blockIdx.x & 7;
  const long long pr = (xcd * P) / 8 + (blockIdx.x >> 3);
  if (pr >= ((xcd + 1) * P) / 8) return;  // past this XCD's share (whole workgroup)
  const int tb = (int)(pr / neb), eb = (int)(pr - (long long)tb * neb);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wk = wave % KW, wn = (wave / KW) % NW, wm = wave / (KW * NW);
  const int l16 = lane & 15, q = lane >> 4;
  const int t0 = tb * (16 * MW) + wm * 16, e0 = eb * (16 * NW) + wn * 16;
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

// ---------------------------------------------------------------------------------------------------
// LDS-staged kernel for larger batches.  Loading MFMA fragments straight from global memory (above)
// makes every 16-lane quarter of a load touch 16 rows, which caps the load path far below what the
// MFMA needs once the batch is large.  Here each stage of 64 K elements of the BM token rows and BN
// expert rows (128 bytes per row) is copied into LDS with direct global->LDS loads, eight rows of
// 128 contiguous bytes per wave instruction.  The 16-byte chunks of row r sit at chunk ^ ((r / 2) % 8),
// which keeps both the copies and the fragment reads free of LDS bank conflicts.  KG groups of four
// waves split K; each group keeps NST stages in flight in its own ring (loads of stage i + NST - 1 are
// issued right after the barrier of stage i, into the slot computed at stage i - 1), and its four
// waves (2 x 2) each compute a (BM/2) x (BN/2) block.  The groups' partial sums are added in LDS in
// group order.  Needs H % 64 == 0.
template <int PER, int NST>
__device__ __forceinline__ void wait_newer_stages(int newer) {
  if constexpr (NST >= 4) {
    if (newer >= 2) {
      wait_vmcnt<2 * PER>();
      return;
    }
  }
  if (newer >= 1) wait_vmcnt<PER>();
  else wait_vmcnt<0>();
}

template <int BM, int BN, int KG, int NST>
__global__ __launch_bounds__(256 * KG) void router_logits_lds_kernel(const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ wr, int T, int H,
                                                                     int E, float* __restrict__ logits) {
  constexpr int ROWS = BM + BN;   // LDS rows of one stage: BM token rows, then BN expert rows
  constexpr int STAGE = ROWS * 128;
  constexpr int PER = ROWS / 32;  // direct loads per wave per stage (8 rows each, 4 waves)
  constexpr int MI = BM / 32, NI = BN / 32;
  static_assert(BM % 32 == 0 && BN % 32 == 0 && NST >= 2 && NST <= 4, "tile shape");
  static_assert(KG == 1 || (KG - 1) * 4 * MI * NI * 64 * 16 <= KG * NST * STAGE, "reduction space");
  __shared__ __attribute__((aligned(16))) uint8_t smem[KG * NST * STAGE];

  const int neb = (E + BN - 1) / BN;
  const long long P = (long long)((T + BM - 1) / BM) * neb;
  const int xcd = blockIdx.x & 7;
  const long long pr = (xcd * P) / 8 + (blockIdx.x >> 3);
  if (pr >= ((xcd + 1) * P) / 8) return;  // past this XCD's share (whole workgroup)
  const int tb = (int)(pr / neb), eb = (int)(pr - (long long)tb * neb);
  const int t0 = tb * BM, e0 = eb * BN;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = wave >> 2, wg = wave & 3;
  const int wm = wg >> 1, wn = wg & 1;
  const int l16 = lane & 15, q = lane >> 4;
  const int nst = H / 64;
  const int st_begin = (g * nst) / KG, cnt = ((g + 1) * nst) / KG - st_begin;
  const int iters = (nst + KG - 1) / KG;  // the same for every group: barriers are workgroup-wide
  uint8_t* gsm = smem + g * NST * STAGE;

  const uint16_t* src[PER];  // load j of a stage: rows 8 * (wg + 4j) .. + 7, 8 lanes per row
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int row = 8 * (wg + 4 * j) + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    const uint16_t* base = row < BM ? x + (size_t)min(t0 + row, T - 1) * H
                                    : wr + (size_t)min(e0 + row - BM, E - 1) * H;
    src[j] = base + chunk * 8;
  }
  auto issue = [&](int st, int slot) {
    uint8_t* dst = gsm + slot * STAGE;
#pragma unroll
    for (int j = 0; j < PER; ++j) g2lds16(src[j] + (size_t)st * 64, dst + (wg + 4 * j) * 1024);
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int slot) {
    const uint8_t* b = gsm + slot * STAGE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = h * 4 + q;
      bf16x8 af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wm * (BM / 2) + mi * 16 + l16;
        af[mi] = *reinterpret_cast<const bf16x8*>(b + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int r = BM + wn * (BN / 2) + ni * 16 + l16;
        bfr[ni] = *reinterpret_cast<const bf16x8*>(b + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma16x16x32(af[mi], bfr[ni], acc[mi][ni]);
    }
  };

#pragma unroll
  for (int u = 0; u < NST - 1; ++u)
    if (u < cnt) issue(st_begin + u, u);
  for (int i = 0; i < iters; ++i) {
    if (i < cnt) wait_newer_stages<PER, NST>(min(NST - 2, cnt - 1 - i));
    __syncthreads();
    if (i + NST - 1 < cnt) issue(st_begin + i + NST - 1, (i + NST - 1) % NST);
    if (i < cnt) compute(i % NST);
  }

  if constexpr (KG > 1) {
    __syncthreads();  // every group is done with its stages: reuse LDS for the partial sums
    f32x4* red = reinterpret_cast<f32x4*>(smem);
    if (g > 0) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) red[((((g - 1) * 4 + wg) * MI + mi) * NI + ni) * 64 + lane] = acc[mi][ni];
    }
    __syncthreads();
    if (g != 0) return;
#pragma unroll
    for (int gg = 1; gg < KG; ++gg)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const f32x4 o = red[((((gg - 1) * 4 + wg) * MI + mi) * NI + ni) * 64 + lane];
          acc[mi][ni][0] += o[0];
          acc[mi][ni][1] += o[1];
          acc[mi][ni][2] += o[2];
          acc[mi][ni][3] += o[3];
        }
  }
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int e = e0 + wn * (BN / 2) + ni * 16 + l16;
    if (e >= E) continue;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wm * (BM / 2) + mi * 16 + 4 * q + r;
        if (t < T) logits[(size_t)t * E + e] = acc[mi][ni][r];
      }
  }
}

// Workgroups for P (token block, expert block) pairs: 8 XCD shares of at most ceil(P / 8).
static unsigned router_grid(int T, int E, int bm, int bn) {
  const long long P = (long long)((T + bm - 1) / bm) * ((E + bn - 1) / bn);
  return (unsigned)(8 * ((P + 7) / 8));
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, int T, int H, int E, float* logits,
                                hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  auto pairs = [&](int bm, int bn) { return (long long)((T + bm - 1) / bm) * ((E + bn - 1) / bn); };
  // Decode sizes (and H % 64 != 0): the direct kernel, whose eight-way K split keeps the few
  // workgroups short.  Otherwise the largest LDS-staged tile that still gives two workgroups per CU,
  // down to 32 x 32 with K split four ways.
  if (T <= 64 || H % 64 != 0 || pairs(32, 32) < 128) {
    router_logits_kernel<1, 1, 8, 8><<<router_grid(T, E, 16, 16), 512, 0, stream>>>(x, w_router, T, H, E, logits);
  } else if (pairs(128, 64) >= 512) {
    router_logits_lds_kernel<128, 64, 1, 3><<<router_grid(T, E, 128, 64), 256, 0, stream>>>(x, w_router, T, H, E,
                                                                                            logits);
  } else if (pairs(64, 64) >= 512) {
    router_logits_lds_kernel<64, 64, 1, 4><<<router_grid(T, E, 64, 64), 256, 0, stream>>>(x, w_router, T, H, E,
                                                                                          logits);
  } else {
    router_logits_lds_kernel<32, 32, 4, 3><<<router_grid(T, E, 32, 32), 1024, 0, stream>>>(x, w_router, T, H, E,
                                                                                           logits);
  }
  return hipGetLastError();
}

}  // namespace moe
