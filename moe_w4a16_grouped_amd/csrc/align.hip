// moe_align: stable counting sort of the R = T*k flat routing slots by expert id, plus the per-expert
// row-tile list that sizes the grouped GEMM launches.
//
// The Atlas page ("告别Python堆栈：Atlas用纯Rust重写LLM推理，在GB10上跑赢vLLM"), section
// "编译时内核选择和W4A16 Grouped GEMM", launches its grouped GEMM over (N tiles, max_m_tiles, experts);
// section "KV Cache量化、MTP推测解码和调试工具链" reports a broken max_m_tiles heuristic and a missing
// zero-init as real bugs.  Here the exact tile list and its length are produced on the device, and
// every output is written in full (no output relies on prior zeroing).
//
// Counting uses LDS atomic adds (order-independent).  Ranking within a wave: the lanes holding the
// same expert id ("peers") are found through a per-wave LDS table: each lane clears its id's entry,
// ORs in its own lane bit and reads the entry back, which yields the exact peer set whatever order
// the OR operations land in.  A lane's rank among its peers is the popcount of the peers below it,
// so the order is ascending flat index (stable) and deterministic.  Across waves and workgroups,
// per-segment counts are turned into per-segment base offsets by a prefix sum in (segment, expert)
// order.
#include "launch.h"
#include "moe_common.h"
#include "topk.h"

namespace moe {

// Peer set of each lane: lanes of this wave holding the same expert id.  tbl is this wave's table of
// E 64-bit entries; a wave's LDS operations complete in issue order, so the clear, the ORs and the
// read-back of one call are ordered, and only entries of ids present in the call are touched.
__device__ __forceinline__ uint64_t lds_peers(uint64_t* tbl, int id, bool valid) {
  const int lane = threadIdx.x & 63;
  if (valid) tbl[id] = 0ull;
  if (valid) atomicOr(reinterpret_cast<unsigned long long*>(tbl + id), 1ull << lane);
  return valid ? tbl[id] : 0ull;
}

// Inclusive prefix sum over the 64 lanes with DPP: shifts by 1, 2, 4, 8 within each row of 16,
// then the last lane of row 0 is added to row 1 (and of row 2 to row 3), then lane 31 to rows 2, 3.
// Lanes without a DPP source add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_add(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v = dpp_add<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add<0x118, 0xF>(v);  // row_shr:8
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Exclusive scan of (a, b) over the threads of a 1024-thread block; also returns the totals.
// scratch: 32 ints of LDS.
__device__ void block_exclusive_scan2(int a, int b, int& ea, int& eb, int& ta, int& tb, int* scratch) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ia = wave_inclusive_scan(a), ib = wave_inclusive_scan(b);
  if (lane == 63) { scratch[wave] = ia; scratch[16 + wave] = ib; }
  __syncthreads();
  if (wave == 0) {
    const int va = lane < 16 ? scratch[lane] : 0, vb = lane < 16 ? scratch[16 + lane] : 0;
    const int sa = wave_inclusive_scan(va), sb = wave_inclusive_scan(vb);
    if (lane < 16) { scratch[lane] = sa - va; scratch[16 + lane] = sb - vb; }
    if (lane == 15) { scratch[32] = sa; scratch[33] = sb; }
  }
  __syncthreads();
  ea = scratch[wave] + ia - a;
  eb = scratch[16 + wave] + ib - b;
  ta = scratch[32];
  tb = scratch[33];
}

// Multi-workgroup epilogue: thread e owns expert e (s_toff, s_off, s_cnt: E + 1, E, E ints of LDS).
// seg_cnt holds per-segment counts for expert e at seg_cnt[s * E + e]; they are replaced by the
// expert-local exclusive prefix (the permuted row of a segment's first slot of expert e is
// offsets[e] + seg_cnt[s * E + e]).
__device__ void finish_expert(int e, int E, int nseg, int bm, int32_t* seg_cnt, int32_t* counts,
                              int32_t* offsets, int32_t* tiles, int max_tiles, int32_t* num_tiles,
                              int* scratch, int32_t* s_toff, int32_t* s_off, int32_t* s_cnt) {
  int c = 0;
  if (e < E) {
    // segment counts are read 32 at a time so the loads are in flight together (80 segments of the
    // 81920-slot skewed batch: three round trips)
    constexpr int kBatch = 32;
    for (int s0 = 0; s0 < nseg; s0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = s0 + j < nseg ? seg_cnt[(s0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (s0 + j < nseg) {
          seg_cnt[(s0 + j) * E + e] = c;
          c += v[j];
        }
    }
  }
  const int nt = (c + bm - 1) / bm;
  int off, toff, total_c, total_t;
  block_exclusive_scan2(c, nt, off, toff, total_c, total_t, scratch);
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    s_toff[e] = toff;
    s_off[e] = off;
    s_cnt[e] = c;
  }
  if (threadIdx.x == 0) {
    offsets[E] = total_c;
    num_tiles[0] = total_t;
    s_toff[E] = total_t;
  }
  __syncthreads();
  // tile i belongs to the expert e with s_toff[e] <= i < s_toff[e + 1] (the last such e: experts without
  // rows have no tiles), so the whole workgroup writes the list, a hot expert's tiles included
  const int nw = min(total_t, max_tiles);
  for (int i = threadIdx.x; i < nw; i += blockDim.x) {
    int lo = 0, hi = E;  // s_toff[lo] <= i < s_toff[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_toff[mid] <= i) lo = mid;
      else hi = mid;
    }
    const int j = i - s_toff[lo];
    int32_t* t = tiles + 3 * (size_t)i;
    t[0] = lo;
    t[1] = s_off[lo] + j * bm;
    t[2] = min(bm, s_cnt[lo] - j * bm);
  }
}

// Single-workgroup epilogue: thread e owns expert e; cnt[w * E + e] (16 waves) holds the counts of
// wave w and is replaced by the absolute permuted row of wave w's first slot of expert e.
__device__ void finish_expert_single(int e, int E, int bm, int32_t* cnt, int32_t* counts, int32_t* offsets,
                                     int32_t* tiles, int max_tiles, int32_t* num_tiles, int* scratch) {
  int v[16];
  int c = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    v[w] = e < E ? cnt[w * E + e] : 0;
    c += v[w];
  }
  const int nt = (c + bm - 1) / bm;
  int off, toff, total_c, total_t;
  block_exclusive_scan2(c, nt, off, toff, total_c, total_t, scratch);
  if (e < E) {
    int run = off;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      cnt[w * E + e] = run;
      run += v[w];
    }
    counts[e] = c;
    offsets[e] = off;
    for (int i = 0; i < nt && toff + i < max_tiles; ++i) {
      int32_t* t = tiles + 3 * (size_t)(toff + i);
      t[0] = e;
      t[1] = off + i * bm;
      t[2] = min(bm, c - i * bm);
    }
  }
  if (threadIdx.x == 0) {
    offsets[E] = total_c;
    num_tiles[0] = total_t;
  }
}

// Per-wave segments hold at most 64 * kSegRegs slots; their ids are loaded once, in one burst, into
// registers (lane l holds slots f0 + 64*j + l) and used by both the counting and the scatter pass.
constexpr int kSegRegs = 16;

__device__ __forceinline__ void load_segment(const int32_t* ids, int f0, int f1, int (&id)[kSegRegs]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kSegRegs; ++j) {
    const int f = f0 + 64 * j + lane;
    id[j] = f < f1 ? ids[f] : -1;
  }
}

// Count segment [f0, f1) of one wave into cnt[id] (LDS atomic adds).
__device__ __forceinline__ void wave_count(const int (&id)[kSegRegs], int f0, int f1, int32_t* cnt) {
#pragma unroll
  for (int j = 0; j < kSegRegs; ++j) {
    if (f0 + 64 * j >= f1) break;
    if (id[j] >= 0) atomicAdd(cnt + id[j], 1);
  }
}

// Scatter segment [f0, f1) of one wave; off[id] + base[id] (base[id] alone when off is NULL) is the
// next free permuted row of expert id (base is advanced here), tbl this wave's peer table.
// sorted_ids may point to LDS (staging) or global memory.
__device__ __forceinline__ void wave_scatter(const int (&id)[kSegRegs], int f0, int f1, int32_t* base,
                                             const int32_t* off, uint64_t* tbl, int32_t* sorted_ids,
                                             int32_t* inv_perm) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < kSegRegs; ++j) {
    if (f0 + 64 * j >= f1) break;
    const int f = f0 + 64 * j + lane;
    const bool v = id[j] >= 0;
    const int e = v ? id[j] : 0;
    const int b = v ? base[e] : 0;
    const int o = (v && off) ? off[e] : 0;
    const uint64_t peers = lds_peers(tbl, e, v);
    if (v) {
      const int r = o + b + __popcll(peers & below);
      sorted_ids[r] = f;
      inv_perm[f] = r;
    }
    // the highest peer advances the expert's base; every peer has read it above
    if (v && (peers >> lane) == 1ull) base[e] = b + __popcll(peers);
  }
}

// Whole permutation of the R slots ids[0..R) (global or LDS) by one 1024-thread workgroup.  cnt
// (16 * E ints, zeroed by the caller before a barrier), tbl (16 * E) and sorted_lds (R) are LDS.
// sorted_ids is staged in LDS (the scatter is random) and written out with coalesced stores.
__device__ __forceinline__ void align_block(const int32_t* ids, int R, int E, int bm, int32_t* counts,
                                            int32_t* offsets, int32_t* sorted_ids, int32_t* inv_perm,
                                            int32_t* tiles, int max_tiles, int32_t* num_tiles, int32_t* cnt,
                                            int* scratch, int32_t* sorted_lds, uint64_t* tbl) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const int seg = (((R + 15) / 16) + 63) & ~63;
  const int f0 = min(R, wave * seg), f1 = min(R, f0 + seg);
  int id[kSegRegs];
  load_segment(ids, f0, f1, id);
  __syncthreads();
  wave_count(id, f0, f1, cnt + wave * E);
  __syncthreads();
  finish_expert_single(tid, E, bm, cnt, counts, offsets, tiles, max_tiles, num_tiles, scratch);
  __syncthreads();
  wave_scatter(id, f0, f1, cnt + wave * E, nullptr, tbl + wave * E, sorted_lds, inv_perm);
  __syncthreads();
  for (int r = tid; r < R; r += 1024) sorted_ids[r] = sorted_lds[r];
}

// Whole permutation in one 1024-thread workgroup (align_single_fits(R, E)).
__global__ __launch_bounds__(1024) void align_single_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                            int bm, int32_t* counts, int32_t* offsets,
                                                            int32_t* sorted_ids, int32_t* inv_perm,
                                                            int32_t* tiles, int max_tiles, int32_t* num_tiles) {
  __shared__ int32_t cnt[16 * kAlignSingleMaxE];
  __shared__ int scratch[64];
  __shared__ int32_t sorted_lds[kAlignSingleMaxR];
  __shared__ uint64_t tbl[16 * kAlignSingleMaxE];
  for (int i = threadIdx.x; i < 16 * E; i += 1024) cnt[i] = 0;
  align_block(ids, R, E, bm, counts, offsets, sorted_ids, inv_perm, tiles, max_tiles, num_tiles, cnt, scratch,
              sorted_lds, tbl);
}

// Routing and permutation of a small batch in one launch (route_align_fused_fits): wave t routes
// token t (writing topk ids and weights, and the ids into LDS), then the workgroup builds the
// permutation from the LDS copy exactly as align_single_kernel does.
template <int NJ>
__global__ __launch_bounds__(1024) void route_align_small_kernel(const float* __restrict__ logits, int T, int E,
                                                                 int k, int bm, int32_t* topk_ids, float* topk_w,
                                                                 int32_t* counts, int32_t* offsets,
                                                                 int32_t* sorted_ids, int32_t* inv_perm,
                                                                 int32_t* tiles, int max_tiles, int32_t* num_tiles) {
  __shared__ uint64_t rscratch[16 * 2 * kFusedMaxK];
  __shared__ int32_t ids_lds[kFusedMaxR];
  __shared__ int32_t cnt[16 * kAlignSingleMaxE];
  __shared__ int scratch[64];
  __shared__ int32_t sorted_lds[kFusedMaxR];
  __shared__ uint64_t tbl[16 * kAlignSingleMaxE];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 16 * E; i += 1024) cnt[i] = 0;
  if (wave < T) {
    uint64_t* kept = rscratch + wave * 2 * k;
    route_token<NJ>(logits + (size_t)wave * E, E, k, kept, kept + k, topk_ids + (size_t)wave * k,
                    topk_w + (size_t)wave * k, ids_lds + wave * k);
  }
  __syncthreads();
  align_block(ids_lds, T * k, E, bm, counts, offsets, sorted_ids, inv_perm, tiles, max_tiles, num_tiles, cnt,
              scratch, sorted_lds, tbl);
}

// Multi-workgroup path, step 1: per-(workgroup, wave) counts, kAlignChunk slots per workgroup.
__global__ __launch_bounds__(256) void align_hist_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                         int32_t* seg_cnt) {
  extern __shared__ int32_t cnt[];  // [4][E]
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < 4 * E; i += 256) cnt[i] = 0;
  __syncthreads();
  const int f0 = min(R, blockIdx.x * kAlignChunk + wave * (kAlignChunk / 4));
  const int f1 = min(R, f0 + kAlignChunk / 4);
  int id[kSegRegs];
  load_segment(ids, f0, f1, id);
  wave_count(id, f0, f1, cnt + wave * E);
  __syncthreads();
  for (int i = tid; i < 4 * E; i += 256) seg_cnt[(size_t)blockIdx.x * 4 * E + i] = cnt[i];
}

// Step 2: one 1024-thread workgroup turns segment counts into per-expert prefixes, writes counts, offsets,
// tiles and the tile count.
__global__ __launch_bounds__(1024) void align_scan_kernel(int32_t* seg_cnt, int nseg, int E, int bm,
                                                          int32_t* counts, int32_t* offsets,
                                                          int32_t* tiles, int max_tiles,
                                                          int32_t* num_tiles) {
  __shared__ int scratch[40];
  __shared__ int32_t s_toff[1025], s_off[1024], s_cnt[1024];  // E <= 1024: one expert per thread
  finish_expert(threadIdx.x, E, nseg, bm, seg_cnt, counts, offsets, tiles, max_tiles, num_tiles, scratch, s_toff,
                s_off, s_cnt);
}

// Step 3: each wave re-walks its segment and scatters from its base rows.
__global__ __launch_bounds__(256) void align_scatter_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                            const int32_t* seg_base, const int32_t* offsets,
                                                            int32_t* sorted_ids, int32_t* inv_perm) {
  extern __shared__ uint64_t dyn[];  // [4][E] peer tables, then [4][E] base rows, then [E] offsets
  uint64_t* tbl = dyn;
  int32_t* base = reinterpret_cast<int32_t*>(dyn + 4 * E);
  int32_t* off = base + 4 * E;
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < 4 * E; i += 256) base[i] = seg_base[(size_t)blockIdx.x * 4 * E + i];
  for (int i = tid; i < E; i += 256) off[i] = offsets[i];
  __syncthreads();
  const int f0 = min(R, blockIdx.x * kAlignChunk + wave * (kAlignChunk / 4));
  const int f1 = min(R, f0 + kAlignChunk / 4);
  int id[kSegRegs];
  load_segment(ids, f0, f1, id);
  wave_scatter(id, f0, f1, base + wave * E, off, tbl + wave * E, sorted_ids, inv_perm);
}

size_t align_workspace_bytes(int R, int E) {
  if (align_single_fits(R, E)) return 0;
  const size_t nblk = (size_t)(R + kAlignChunk - 1) / kAlignChunk;
  return nblk * 4 * (size_t)E * sizeof(int32_t);
}

hipError_t launch_route_align_small(const float* logits, int T, int E, int k, int block_m, int32_t* topk_ids,
                                   float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                                   int32_t* inv_perm, int32_t* tiles, int max_tiles, int32_t* num_tiles,
                                   hipStream_t stream) {
  const int nj = (E + 63) / 64;
#define RA_LAUNCH(NJ_)                                                                                         \
  route_align_small_kernel<NJ_><<<1, 1024, 0, stream>>>(logits, T, E, k, block_m, topk_ids, topk_w, counts, \
                                                         offsets, sorted_ids, inv_perm, tiles, max_tiles, num_tiles)
  if (nj <= 1) RA_LAUNCH(1);
  else if (nj <= 2) RA_LAUNCH(2);
  else if (nj <= 4) RA_LAUNCH(4);
  else RA_LAUNCH(8);
#undef RA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_align(const int32_t* ids, int R, int E, int block_m, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_ids, int32_t* inv_perm, int32_t* tiles,
                        int max_tiles, int32_t* num_tiles, void* workspace, hipStream_t stream) {
  if (align_single_fits(R, E)) {
    align_single_kernel<<<1, 1024, 0, stream>>>(ids, R, E, block_m, counts, offsets, sorted_ids, inv_perm, tiles,
                                                max_tiles, num_tiles);
    return hipGetLastError();
  }
  const int nblk = (R + kAlignChunk - 1) / kAlignChunk;
  int32_t* seg = static_cast<int32_t*>(workspace);
  align_hist_kernel<<<nblk, 256, 4 * (size_t)E * sizeof(int32_t), stream>>>(ids, R, E, seg);
  align_scan_kernel<<<1, 1024, 0, stream>>>(seg, nblk * 4, E, block_m, counts, offsets, tiles, max_tiles,
                                            num_tiles);
  align_scatter_kernel<<<nblk, 256, 4 * (size_t)E * (sizeof(uint64_t) + sizeof(int32_t)) + E * sizeof(int32_t),
                         stream>>>(ids, R, E, seg, offsets, sorted_ids, inv_perm);
  return hipGetLastError();
}

}  // namespace moe
