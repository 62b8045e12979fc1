// One-time weight re-layout ("preshuffle") from the canonical W4 layout into the kernel layout.
//
// The ATOM page ("AMD ATOM推理引擎：如何用分页KV缓存和分段编译实现大模型推理性能翻倍"), section
// "8.2 量化并非单一格式，而是一套执行契约", lists whether weights are pre-rearranged as part of a
// quantized format's execution contract.  Here the re-layout makes every wave-level load of the
// grouped GEMM one contiguous block:
//
//   block (e, nb, ks) = 16 weight rows n = 16*nb .. 16*nb+15 and 128 K elements k = 128*ks .. +127
//   codes:  1024 bytes; bytes [16*l, 16*l+16) belong to lane l = (n % 16) + 16*q (q = 0..3) and hold
//           dword j (j = 0..3) = the 8 codes of row n, K elements 32*(4*ks+j) + 8*q .. +7, i.e. the
//           MFMA B operand of group 4*ks+j for that lane, low nibble first as in the canonical layout.
//   scales: 128 bytes; bf16 [n % 16][j] = scale of row n, group 4*ks+j.
//   blocks are ordered (e, nb, ks) with ks fastest.
// Requires N % 16 == 0 and K % 128 == 0.  The total size equals the canonical size.
#include "launch.h"
#include "moe_common.h"

namespace moe {

__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                      int E, int N, int K, uint8_t* __restrict__ pq,
                                                      uint16_t* __restrict__ ps) {
  const int NB = N / 16, KS = K / 128;
  const size_t nblocks = (size_t)E * NB * KS;
  // one wave per block: lane l writes its 16 code bytes; lanes 0..63 also write one scale each
  const size_t blk = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;
  const int l = threadIdx.x & 63;
  const int ks = (int)(blk % KS);
  const size_t rb = blk / KS;  // e * NB + nb
  const int nb = (int)(rb % NB);
  const int e = (int)(rb / NB);
  const int n = nb * 16 + (l & 15), q = l >> 4;
  const uint8_t* row = wq + ((size_t)e * N + n) * (size_t)(K / 2);
  u32x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const uint32_t*>(row + 16 * (4 * ks + j) + 4 * q);
  reinterpret_cast<u32x4*>(pq + blk * 1024)[l] = v;
  // scales: lane l -> row (l / 4), group j = l % 4
  const int sn = nb * 16 + (l >> 2), sj = l & 3;
  ps[blk * 64 + l] = ws[((size_t)e * N + sn) * (size_t)(K / kGroup) + 4 * ks + sj];
}

hipError_t launch_prepack(const uint8_t* wq, const uint16_t* ws, int E, int N, int K, uint8_t* pq, uint16_t* ps,
                          hipStream_t stream) {
  const size_t nblocks = (size_t)E * (N / 16) * (K / 128);
  if (nblocks == 0) return hipSuccess;
  prepack_kernel<<<(unsigned)((nblocks + 3) / 4), 256, 0, stream>>>(wq, ws, E, N, K, pq, ps);
  return hipGetLastError();
}

}  // namespace moe
