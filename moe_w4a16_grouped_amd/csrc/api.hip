// C-ABI of libmoe_w4a16: host-side validation, workspace carving and launch sequencing.
// Every entry point validates its arguments before launching anything, reports failures through a
// status code plus a thread-local message, and only enqueues work on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "launch.h"
#include "moe_w4a16.h"

// The static scratch array of moe_ffn_forward_noalloc (see scratch_of_current_device below).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

moe_status_t ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

constexpr int64_t kMaxRows = int64_t(1) << 26;
// The W4A16 grouped GEMMs address a weight row by a 32-bit byte offset within its expert.
constexpr int64_t kMaxExpertCodeBytes = int64_t(0xFFFFF000);

moe_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

moe_status_t check_routing_shape(int32_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1) return fail(MOE_ERR_INVALID_ARG, "need T >= 0, E >= 1, k >= 1 (T=%d E=%d k=%d)", T, E, k);
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "k=%d exceeds E=%d", k, E);
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E=%d exceeds %d", E, MOE_MAX_EXPERTS);
  if ((int64_t)T * k >= kMaxRows) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T*k=%lld must be < 2^26", (long long)T * k);
  return MOE_OK;
}

int64_t max_tiles_of(int64_t R, int64_t E, int64_t bm) { return R / bm + std::min<int64_t>(E, R); }

// Row tile height for the grouped GEMMs given the average rows per expert (measured on MI355X:
// 16 for decode-sized experts, 32 around 25 rows per expert, 64 above; with packed weights, experts
// averaging more than 256 rows go to the 128-row large-tile kernel).
int32_t pick_block_m(int64_t R, int64_t E, bool packed) {
  const int64_t avg = (R + E - 1) / E;
  if (avg <= 16) return 16;
  if (avg <= 32) return 32;
  if (packed && avg > 256) return 128;
  return 64;
}

// Workspace carve-up for moe_ffn_forward (each region 256-byte aligned).
struct FfnLayout {
  size_t ids, w, counts, offsets, sorted, inv, tiles, ntiles, align_ws, h, o, oside, x16, xexp, hflag, hexp, total;
  int32_t block_m, max_tiles;
  bool f16;             // this layout's tile height runs the exact fp16 path (128-row tiles)
  int32_t hexp_stride;  // h's 32-column blocks (exponent flags per tile, exponents per row)
};

// The layer runs the exact fp16 path on 128-row tiles (packed weights, experts averaging more than 256
// rows), where the grouped GEMMs are bound by the matrix cores: measured on MI355X with 4096 tokens
// over 8 experts top-2 (H 4096, I 14336), gate_up 2.0-2.1 ms and down 1.03-1.09 ms against 2.13-2.19
// and 1.22-1.27 ms for the bf16 kernels.  With 64-row tiles (8192 tokens, 512 experts top-10) the
// fp16 and bf16 GEMMs take the same time and the conversion of x would be extra work, so those stay
// on the bf16 path; with 32-row tiles (800 tokens, 256 experts) the fp16 kernels need twice the
// registers and the layer took 184-186 us against 143-144 us.
bool uses_f16(int32_t block_m) { return block_m >= 128; }

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

// The tile list is sized for the canonical-layout tile height, which is never larger than the packed
// one, so one workspace size serves both layouts.
// extra_rows: rows of h and O past the T*k routed rows (the shared expert's, when it runs in the
// routed launches).
FfnLayout ffn_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, bool packed, int64_t extra_rows = 0) {
  FfnLayout L{};
  const int64_t R = T * k;
  L.block_m = pick_block_m(R, E, packed);
  L.max_tiles = (int32_t)max_tiles_of(R, E, L.block_m);
  const int64_t tile_cap = std::max<int64_t>(L.max_tiles, max_tiles_of(R, E, pick_block_m(R, E, false)));
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += up256(bytes); return at; };
  L.ids = take(R * 4);
  L.w = take(R * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted = take(R * 4);
  L.inv = take(R * 4);
  L.tiles = take((size_t)std::max<int64_t>(tile_cap, 1) * 12);
  L.ntiles = take(4);
  L.align_ws = take(moe::align_workspace_bytes((int)R, (int)E));
  L.h = take((size_t)(R + extra_rows) * I * 2);
  L.o = take((size_t)(R + extra_rows) * H * 2);                  // fp16 down output
  L.oside = take((size_t)(R + extra_rows) * ((H + 7) / 8) * 4);  // its side values (scaled segments only)
  // fp16 path: x in fp16 with row exponents, and h's block exponents (the canonical tile height is
  // 64 whenever either layout's is 64 or 128, so the regions exist for both)
  L.f16 = uses_f16(L.block_m);
  L.hexp_stride = (int32_t)((I + 31) / 32);
  const bool any_f16 = uses_f16(pick_block_m(R, E, true));
  L.x16 = take(any_f16 ? (size_t)T * H * 2 : 0);
  L.xexp = take(any_f16 ? (size_t)T * 4 : 0);
  L.hflag = take(any_f16 ? (size_t)(tile_cap + (extra_rows + 15) / 16) * L.hexp_stride : 0);
  L.hexp = take(any_f16 ? (size_t)(R + extra_rows) * L.hexp_stride : 0);
  L.total = off;
  return L;
}

// Shape checks shared by the layer entry points (gate_up [E, 2I, H], down [E, H, I]); they apply
// to an empty batch too.
moe_status_t check_weight_shape(int32_t H, int32_t I, int32_t weight_layout, const char* who) {
  if (H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "%s: H=%d and I=%d must be positive multiples of 32", who, H, I);
  if (weight_layout != MOE_LAYOUT_CANONICAL && weight_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown weight_layout %d", who, weight_layout);
  if (weight_layout == MOE_LAYOUT_PACKED && (H % 128 != 0 || I % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "%s: packed weights need H %% 128 == 0 and I %% 128 == 0 (H=%d I=%d)", who,
                H, I);
  if ((int64_t)H * I > kMaxExpertCodeBytes)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "%s: one expert's gate_up codes (H*I = %lld bytes) must stay below 4 GiB", who,
                (long long)H * I);
  return MOE_OK;
}

moe_status_t check_weight_ptrs(const uint8_t* w13_q, const uint16_t* w13_s, const uint8_t* w2_q, const uint16_t* w2_s,
                               int32_t weight_layout, const char* who) {
  if (!w13_q || !w13_s || !w2_q || !w2_s) return fail(MOE_ERR_INVALID_ARG, "%s: NULL weight pointer", who);
  if (!aligned16(w13_q) || !aligned16(w2_q) || !aligned2(w13_s) || !aligned2(w2_s) ||
      (weight_layout == MOE_LAYOUT_PACKED && ((reinterpret_cast<uintptr_t>(w13_s) | reinterpret_cast<uintptr_t>(w2_s)) & 7u)))
    return fail(MOE_ERR_MISALIGNED, "%s: weight codes need 16-byte alignment (packed scales 8-byte)", who);
  return MOE_OK;
}

// Pointer checks of the routed layer (called for T > 0).
// (workspace_needed = false: the call brings no workspace, as in the entry point without allocation.)
moe_status_t check_ffn_ptrs(const uint16_t* x, const uint8_t* w13_q, const uint16_t* w13_s, const uint8_t* w2_q,
                            const uint16_t* w2_s, int32_t weight_layout, const uint16_t* y,
                            const int32_t* topk_ids_out, const float* topk_w_out, const void* workspace,
                            const char* who, bool workspace_needed = true) {
  if (moe_status_t st = check_weight_ptrs(w13_q, w13_s, w2_q, w2_s, weight_layout, who)) return st;
  if (!x || !y || (workspace_needed && !workspace)) return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(x) || !aligned16(y) || (workspace_needed && !aligned16(workspace)) ||
      (topk_ids_out && !aligned4(topk_ids_out)) || (topk_w_out && !aligned4(topk_w_out)))
    return fail(MOE_ERR_MISALIGNED, "%s: x, y and workspace need 16-byte alignment", who);
  return MOE_OK;
}

// Dense SwiGLU FFN (one expert applied to every row): gate_up with SiLU*mul into h, then down into
// out (fp32).  Both projections run the grouped-GEMM kernels in dense mode (no tile list).
// Row-tile height of one dense projection with `cols` output columns: the largest tile whose grid
// alone has a workgroup per CU (256), else 16 (split-K when there are at most 32 row tiles).  The
// column-block widths are those of the kernels launch_grouped_gemm picks for each height.
int dense_block_m(int64_t T, int64_t cols, bool silu, bool packed) {
  for (int bm : {128, 64, 32}) {
    int64_t bn = bm == 128 ? (packed ? 256 : 128) : bm == 64 ? 256 : 128;
    if (silu) bn /= 2;  // gate and up columns share a tile
    if (((T + bm - 1) / bm) * ((cols + bn - 1) / bn) >= 256) return bm;
  }
  return 16;
}

hipError_t run_dense_ffn(const uint16_t* x, int T, int H, int I, const uint8_t* w13_q, const uint16_t* w13_s,
                         const uint8_t* w2_q, const uint16_t* w2_s, int weight_layout, uint16_t* h, float* out,
                         hipStream_t s) {
  const int packed = weight_layout == MOE_LAYOUT_PACKED;
  const int bm1 = dense_block_m(T, I, true, packed), bm2 = dense_block_m(T, H, false, packed);
  moe::GemmArgs g1{x, nullptr, 1, w13_q, w13_s, 2 * I, H, nullptr, nullptr, (T + bm1 - 1) / bm1, T, h,
                   MOE_EPI_SILU_MUL, 0, packed};
  hipError_t e = moe::launch_grouped_gemm(g1, bm1, s);
  if (e != hipSuccess) return e;
  moe::GemmArgs g2{h, nullptr, 1, w2_q, w2_s, H, I, nullptr, nullptr, (T + bm2 - 1) / bm2, T, out, MOE_EPI_NONE, 1,
                   packed};
  return moe::launch_grouped_gemm(g2, bm2, s);
}

// Weights of a shared expert that runs inside the routed launches (its intermediate size equals
// the routed one), or all NULL.
struct SharedW {
  const uint8_t* w13_q;
  const uint16_t* w13_s;
  const uint8_t* w2_q;
  const uint16_t* w2_s;
};

// The routed layer after validation: routing and permutation, the two grouped GEMMs and the
// combine.  A shared expert is either run in the grouped GEMMs (sw.w13_q set: its tiles follow the
// routed ones, its rows of h and O follow the T*k routed rows) or was run before (shared_out set);
// either way its output is added in the combine.
moe_status_t run_ffn(const uint16_t* x, const float* router_logits, int32_t T, int32_t H, int32_t I, int32_t E,
                     int32_t k, const uint8_t* w13_q, const uint16_t* w13_s, const uint8_t* w2_q, const uint16_t* w2_s,
                     int32_t weight_layout, uint16_t* y, int32_t* topk_ids_out, float* topk_w_out, char* ws,
                     const FfnLayout& L, const SharedW& sw, const float* shared_out, hipStream_t s) {
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(ws + L.ntiles);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  uint16_t* o = reinterpret_cast<uint16_t*>(ws + L.o);
  float* oside = reinterpret_cast<float*>(ws + L.oside);
  const int R = T * k;
  const int packed = weight_layout == MOE_LAYOUT_PACKED;
  const int shared_tiles = sw.w13_q ? (T + L.block_m - 1) / L.block_m : 0;
  hipError_t e;
  moe::GemmArgs g1{x, sorted, k, w13_q, w13_s, 2 * I, H, tiles, ntiles, L.max_tiles + shared_tiles, 0, h,
                   MOE_EPI_SILU_MUL, 0, packed, sw.w13_q, sw.w13_s, T, R, 0};
  uint16_t* x16 = reinterpret_cast<uint16_t*>(ws + L.x16);
  int32_t* xexp = reinterpret_cast<int32_t*>(ws + L.xexp);
  uint8_t* hflag = reinterpret_cast<uint8_t*>(ws + L.hflag);
  uint8_t* hexp = reinterpret_cast<uint8_t*>(ws + L.hexp);
  if (L.f16) {
    // exact fp16 path: gate_up reads x in fp16 (row exponents), writes h in fp16 (block exponents)
    g1.A = x16;
    g1.a_f16 = 1;
    g1.a_row_exp = xexp;
    g1.out_f32 = 3;
    g1.c_blk_flag = hflag;
    g1.c_row_blk_exp = hexp;
    g1.c_blk_stride = L.hexp_stride;
  }
  if (moe::route_prologue_fits(T, E, k) && L.block_m == 16) {
    // small batch: the gate_up launch routes and permutes in its own prologue
    g1.route_logits = router_logits;
    g1.route_T = T;
    g1.route_E = E;
    g1.route_k = k;
    g1.route_ids = ids;
    g1.route_w = w;
    g1.route_tiles = tiles;
    g1.route_num_tiles = ntiles;
    g1.route_sorted = sorted;
    g1.route_inv = inv;
  } else if (moe::route_align_fused_fits(T, E, k)) {
    e = moe::launch_route_align_small(router_logits, T, E, k, L.block_m, ids, w, counts, offsets, sorted, inv,
                                      tiles, L.max_tiles, ntiles, s);
    if (e != hipSuccess) return hip_status(e, "route+align launch");
  } else {
    e = moe::launch_route_topk(router_logits, T, E, k, ids, w, s);
    if (e != hipSuccess) return hip_status(e, "route launch");
    e = moe::launch_align(ids, R, E, L.block_m, counts, offsets, sorted, inv, tiles, L.max_tiles, ntiles,
                          ws + L.align_ws, s);
    if (e != hipSuccess) return hip_status(e, "align launch");
  }
  if (L.f16) {
    e = moe::launch_x_to_f16(x, T, H, x16, xexp, s);
    if (e != hipSuccess) return hip_status(e, "x to fp16 launch");
  }
  e = moe::launch_grouped_gemm(g1, L.block_m, s);
  if (e != hipSuccess) return hip_status(e, "gate_up launch");
  // the down projection writes O as fp16 with in-band per-(row, 8 columns) exponents (kind 2)
  moe::GemmArgs g2{h, nullptr, 1, w2_q, w2_s, H, I, tiles, ntiles, L.max_tiles + shared_tiles, 0, o, MOE_EPI_NONE, 2,
                   packed, sw.w2_q, sw.w2_s, T, R, 0};
  g2.C_side = oside;
  if (L.f16) {
    g2.a_f16 = 1;
    g2.a_blk_flag = hflag;
    g2.a_row_blk_exp = hexp;
    g2.a_blk_stride = L.hexp_stride;
  }
  e = moe::launch_grouped_gemm(g2, L.block_m, s);
  if (e != hipSuccess) return hip_status(e, "down launch");
  e = moe::launch_combine(o, oside, inv, w, shared_out, sw.w13_q ? R : -1, T, k, H, y, s);
  return hip_status(e, "combine launch");
}

// MOE_DUMP=1 in the environment: after a layer call's launches, synchronise its stream and print one
// line of diagnostics to stderr, in the spirit of the Atlas page's per-layer dump of expert ids
// ("告别Python堆栈：Atlas用纯Rust重写LLM推理，在GB10上跑赢vLLM", section "KV Cache量化、MTP推测解码和调试工具链"):
// the shape, the tile height and tile count, the rows per expert (least, most, experts without
// rows), the most tiles of one expert, the ten largest router logits of token 0 (expert:value) and
// the L2 norms of x and y.  It only reads device memory, so results are unchanged; it is skipped on
// a stream under graph capture.  Read on every call (getenv), off unless the value is exactly "1".
bool dump_enabled() {
  const char* v = getenv("MOE_DUMP");
  return v && v[0] == '1' && v[1] == '\0';
}

moe_status_t dump_layer(const uint16_t* x, const float* logits, const int32_t* ids, const int32_t* ntiles,
                        const uint16_t* y, int32_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t block_m,
                        hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return ok();
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "MOE_DUMP synchronize");
  const size_t R = (size_t)T * k, n = (size_t)T * H;
  std::vector<int32_t> hid(R);
  std::vector<float> hl(E);
  std::vector<uint16_t> hx(n), hy(n);
  int32_t nt = 0;
  if ((e = hipMemcpy(hid.data(), ids, R * sizeof(int32_t), hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(hl.data(), logits, E * sizeof(float), hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(&nt, ntiles, sizeof(int32_t), hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(hx.data(), x, n * sizeof(uint16_t), hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(hy.data(), y, n * sizeof(uint16_t), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_status(e, "MOE_DUMP copy");
  std::vector<int64_t> cnt(E, 0);
  for (int32_t id : hid)
    if (id >= 0 && id < E) ++cnt[id];
  int64_t cmin = cnt[0], cmax = cnt[0], tiles_max = 0;
  int empty = 0;
  for (int64_t c : cnt) {
    cmin = std::min(cmin, c);
    cmax = std::max(cmax, c);
    empty += c == 0;
    tiles_max = std::max(tiles_max, (c + block_m - 1) / block_m);
  }
  std::vector<int> order(E);
  for (int i = 0; i < E; ++i) order[i] = i;
  const int top = std::min(E, 10);
  std::partial_sort(order.begin(), order.begin() + top, order.end(),
                    [&](int a, int b) { return hl[a] > hl[b] || (hl[a] == hl[b] && a < b); });
  auto norm = [](const std::vector<uint16_t>& v) {
    double acc = 0.0;
    for (uint16_t b : v) {
      uint32_t u = (uint32_t)b << 16;
      float f;
      memcpy(&f, &u, 4);
      acc += (double)f * f;
    }
    return std::sqrt(acc);
  };
  char buf[512];
  int len = 0;
  for (int i = 0; i < top && len < (int)sizeof(buf) - 32; ++i)
    len += snprintf(buf + len, sizeof(buf) - len, "%s%d:%.6g", i ? " " : "", order[i], hl[order[i]]);
  fprintf(stderr,
          "moe_dump: T=%d H=%d I=%d E=%d k=%d block_m=%d tiles=%d rows_per_expert min=%lld max=%lld empty=%d "
          "max_tiles_per_expert=%lld logits0_top=[%s] x_norm=%.9g y_norm=%.9g\n",
          T, H, I, E, k, block_m, nt, (long long)cmin, (long long)cmax, empty, (long long)tiles_max, buf, norm(hx),
          norm(hy));
  fflush(stderr);
  return ok();
}

// Scratch of the layer entry point that allocates nothing: a static device array of fixed size.
// Each GPU the library runs on holds its own copy (allocated when the code object is loaded on that
// device) until the process ends.  Host code never passes the array's name to a kernel or a copy:
// that name is a host-side stand-in, not a device address.  The device address is looked up once
// per device, with that device current, and kept.  Every call on one GPU shares that GPU's array
// and it keeps the last call's contents; no kernel of the layer needs it cleared (every region is
// written before it is read), and calls that overlap in time on one GPU race.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

size_t scratch_capacity() { return sizeof(scratch); }

moe_status_t scratch_of_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "moe_ffn_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_ffn_forward_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "moe_ffn_forward_noalloc: hipGetSymbolAddress(scratch)");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u))
      return fail(MOE_ERR_HIP, "moe_ffn_forward_noalloc: scratch address %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Workspace of the MXFP4 layer: the routing regions of ffn_layout (canonical tile heights), then
// x quantized (codes [T, H/2], scales [T, H/32]), h quantized (codes [R, I/2], scales [R, I/32])
// and O: fp32 [R, H], or from 256 rows on fp16 with in-band exponents [R, H] with its side values fp32
// [R, ceil(H/8)] (the down projection's output kind 2, as in the W4A16 layer).  Measured on MI355X
// (256 experts, top-8, H 2048): the fp16 O takes 8192 skewed tokens from 531 to 418 us and 800 tokens
// from 135.7 to 133.5 us; at 8 tokens it costs 0.6 us, at 64 tokens it gains 0.6 us.
struct MxLayout {
  FfnLayout L;
  bool o16;  // O as fp16 with in-band exponents
  size_t xq, xs, hq, hs, o, oside, total;
};

// The quantized x and h regions hold either row-major rows (T and R of them) or the tile-blocked
// layout of the tile list (max_tiles * block_m rows), whichever is larger, so one size serves both
// weight layouts.
// Row-tile height of the MXFP4 layer: the canonical W4A16 choice, but experts averaging more than 128
// rows take the 128 x 256 LDS-staged kernel when both K dimensions are multiples of 128 (its tile list
// is never longer than the 64-row one, so the canonical tile capacity of ffn_layout covers it).
int32_t pick_mx_block_m(int64_t R, int64_t E, int64_t H, int64_t I) {
  const int64_t avg = (R + E - 1) / E;
  if (avg > 128 && H % 128 == 0 && I % 128 == 0) return 128;
  return pick_block_m(R, E, false);
}

MxLayout mx_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  MxLayout M{};
  M.L = ffn_layout(T, H, I, E, k, false);
  const int64_t R = T * k;
  M.L.block_m = pick_mx_block_m(R, E, H, I);
  M.L.max_tiles = (int32_t)max_tiles_of(R, E, M.L.block_m);
  const int64_t tiled_rows = (int64_t)M.L.max_tiles * M.L.block_m;
  const int64_t xr = std::max(T, tiled_rows), hr = std::max(R, tiled_rows);
  size_t off = M.L.h;
  auto take = [&](size_t bytes) { size_t at = off; off += up256(bytes); return at; };
  M.xq = take((size_t)xr * H / 2);
  M.xs = take((size_t)xr * H / 32);
  M.hq = take((size_t)hr * I / 2);
  M.hs = take((size_t)hr * I / 32);
  M.o16 = R >= 256;
  M.o = take((size_t)R * H * (M.o16 ? 2 : 4));
  M.oside = M.o16 ? take((size_t)R * ((H + 7) / 8) * 4) : 0;
  M.total = off;
  return M;
}

// Workspace of the FP8 layer: the routing regions of ffn_layout (canonical tile heights), then
// x quantized (codes [T, H], scales [T, H/128]), h in fp32 [R, I], h quantized (codes [R, I],
// scales [R, I/128]) and O: fp32 [R, H], or (o16) fp16 with in-band exponents [R, H] and its side
// values fp32 [R, ceil(H/8)].
struct F8Layout {
  FfnLayout L;
  bool o16;  // O as fp16 with in-band exponents: 128-row tiles and at least 16384 rows
  size_t xq, xs, hf, hq, hs, o, oside, total;
};

// Row-tile height of the FP8 layer: as the canonical W4A16 choice, but experts averaging more than
// 128 rows take the 128 x 256 LDS-staged kernel (its tile list is never longer than the 64-row one,
// so the canonical tile capacity of ffn_layout covers it).
int32_t pick_f8_block_m(int64_t R, int64_t E) {
  const int64_t avg = (R + E - 1) / E;
  if (avg > 128) return 128;
  return pick_block_m(R, E, false);
}

F8Layout f8_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  F8Layout M{};
  M.L = ffn_layout(T, H, I, E, k, false);
  const int64_t R = T * k;
  M.L.block_m = pick_f8_block_m(R, E);
  M.L.max_tiles = (int32_t)max_tiles_of(R, E, M.L.block_m);
  size_t off = M.L.h;
  auto take = [&](size_t bytes) { size_t at = off; off += up256(bytes); return at; };
  M.xq = take((size_t)T * H);
  M.xs = take((size_t)T * (H / 128) * 4);
  M.hf = take((size_t)R * I * 4);
  M.hq = take((size_t)R * I);
  M.hs = take((size_t)R * (I / 128) * 4);
  M.o16 = M.L.block_m == 128 && R >= 16384;
  M.o = take((size_t)R * H * (M.o16 ? 2 : 4));
  M.oside = M.o16 ? take((size_t)R * ((H + 7) / 8) * 4) : 0;
  M.total = off;
  return M;
}

constexpr int32_t kF8MaxK = 32768;  // the GEMM stages a tile's activation scales (64 rows x K/128) in LDS

bool f8_dims_ok(int32_t H, int32_t I) {
  return H >= 128 && I >= 128 && H % 128 == 0 && I % 128 == 0 && H <= kF8MaxK && I <= kF8MaxK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return 2; }

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err; }

moe_status_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                            float* topk_w, void* stream) {
  if (moe_status_t st = check_routing_shape(T, E, k)) return st;
  if (T == 0) return ok();
  if (!logits || !topk_ids || !topk_w) return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: NULL pointer");
  if (!aligned4(logits) || !aligned4(topk_ids) || !aligned4(topk_w))
    return fail(MOE_ERR_MISALIGNED, "moe_route_topk: pointers must be 4-byte aligned");
  return hip_status(moe::launch_route_topk(logits, T, E, k, topk_ids, topk_w, (hipStream_t)stream),
                    "moe_route_topk launch");
}

int32_t moe_max_tiles(int32_t T, int32_t k, int32_t E, int32_t block_m) {
  if (T < 0 || k < 1 || E < 1 || block_m < 1) return -1;
  const int64_t v = max_tiles_of((int64_t)T * k, E, block_m);
  return v > INT32_MAX ? -1 : (int32_t)v;
}

size_t moe_align_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1 || (int64_t)T * k >= kMaxRows) return 0;
  return moe::align_workspace_bytes(T * k, E);
}

moe_status_t moe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_ids,
                       int32_t* inv_perm, int32_t* tiles, int32_t max_tiles, int32_t* num_tiles,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (moe_status_t st = check_routing_shape(T, E, k)) return st;
  if (block_m < 1 || block_m > 4096) return fail(MOE_ERR_INVALID_ARG, "moe_align: block_m=%d outside [1, 4096]", block_m);
  const int64_t R = (int64_t)T * k;
  if (!expert_counts || !expert_offsets || !num_tiles || (R > 0 && (!topk_ids || !sorted_ids || !inv_perm || !tiles)))
    return fail(MOE_ERR_INVALID_ARG, "moe_align: NULL pointer");
  for (const void* p : {(const void*)topk_ids, (const void*)expert_counts, (const void*)expert_offsets,
                        (const void*)sorted_ids, (const void*)inv_perm, (const void*)tiles, (const void*)num_tiles})
    if (p && !aligned4(p)) return fail(MOE_ERR_MISALIGNED, "moe_align: pointers must be 4-byte aligned");
  const int64_t need_tiles = max_tiles_of(R, E, block_m);
  if (max_tiles < need_tiles)
    return fail(MOE_ERR_WORKSPACE, "moe_align: max_tiles=%d < required %lld", max_tiles, (long long)need_tiles);
  const size_t need_ws = moe::align_workspace_bytes((int)R, E);
  if (workspace_bytes < need_ws || (need_ws > 0 && !workspace))
    return fail(MOE_ERR_WORKSPACE, "moe_align: workspace %zu B < required %zu B", workspace_bytes, need_ws);
  if (need_ws > 0 && !aligned16(workspace)) return fail(MOE_ERR_MISALIGNED, "moe_align: workspace must be 16-byte aligned");
  return hip_status(moe::launch_align(topk_ids, (int)R, E, block_m, expert_counts, expert_offsets, sorted_ids,
                                      inv_perm, tiles, max_tiles, num_tiles, workspace, (hipStream_t)stream),
                    "moe_align launch");
}

moe_status_t moe_w4_prepack(const uint8_t* w_q, const uint16_t* w_s, int32_t E, int32_t N, int32_t K,
                            uint8_t* packed_q, uint16_t* packed_s, void* stream) {
  if (E < 1 || N < 16 || K < 128) return fail(MOE_ERR_INVALID_ARG, "moe_w4_prepack: need E >= 1, N >= 16, K >= 128");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E=%d exceeds %d", E, MOE_MAX_EXPERTS);
  if (N % 16 != 0 || K % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_w4_prepack: N=%d must be a multiple of 16 and K=%d of 128", N, K);
  if (!w_q || !w_s || !packed_q || !packed_s) return fail(MOE_ERR_INVALID_ARG, "moe_w4_prepack: NULL pointer");
  if (!aligned16(w_q) || !aligned16(packed_q) || !aligned2(w_s) || !aligned2(packed_s))
    return fail(MOE_ERR_MISALIGNED, "moe_w4_prepack: codes need 16-byte, scales 2-byte alignment");
  return hip_status(moe::launch_prepack(w_q, w_s, E, N, K, packed_q, packed_s, (hipStream_t)stream), "moe_w4_prepack launch");
}

moe_status_t moe_grouped_gemm_w4a16(const uint16_t* A, const int32_t* a_row_of, int32_t a_row_div,
                                    const uint8_t* Wq, const uint16_t* Ws, int32_t weight_layout,
                                    int32_t E, int32_t N,
                                    int32_t K, const int32_t* tiles, int32_t max_tiles,
                                    const int32_t* num_tiles, int32_t block_m, int32_t epilogue,
                                    void* C, int32_t out_dtype, float* C_side, void* stream) {
  if (E < 1 || N < 1 || K < 1 || max_tiles < 0) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_w4a16: need E, N, K >= 1, max_tiles >= 0");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E=%d exceeds %d", E, MOE_MAX_EXPERTS);
  if (K % 32 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "K=%d must be a multiple of 32", K);
  if ((int64_t)N * K / 2 > kMaxExpertCodeBytes)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "one expert's codes (N*K/2 = %lld bytes) must stay below 4 GiB",
                (long long)N * K / 2);
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "block_m=%d must be 16, 32, 64 or 128", block_m);
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SILU_MUL) return fail(MOE_ERR_INVALID_ARG, "unknown epilogue %d", epilogue);
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_F16E)
    return fail(MOE_ERR_INVALID_ARG, "unknown out_dtype %d", out_dtype);
  if (epilogue == MOE_EPI_SILU_MUL && (N % 2 != 0 || out_dtype != MOE_OUT_BF16))
    return fail(MOE_ERR_INVALID_ARG, "SILU_MUL needs an even N and bf16 output");
  if (out_dtype == MOE_OUT_F16E && max_tiles > 0 && !C_side)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_w4a16: MOE_OUT_F16E needs C_side");
  if (a_row_of && a_row_div < 1) return fail(MOE_ERR_INVALID_ARG, "a_row_div must be >= 1");
  if (weight_layout != MOE_LAYOUT_CANONICAL && weight_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "unknown weight_layout %d", weight_layout);
  if (weight_layout == MOE_LAYOUT_PACKED && (N % 16 != 0 || K % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "packed weights need N %% 16 == 0 and K %% 128 == 0 (N=%d K=%d)", N, K);
  if (weight_layout == MOE_LAYOUT_PACKED && epilogue == MOE_EPI_SILU_MUL && N % 32 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "packed gate_up weights need N %% 32 == 0 (up rows start a 16-row block; N=%d)", N);
  if (max_tiles == 0) return ok();
  if (!A || !Wq || !Ws || !tiles || !num_tiles || !C) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_w4a16: NULL pointer");
  if (!aligned16(A) || !aligned16(Wq) || !aligned16(C) || !aligned2(Ws) || !aligned4(tiles) || !aligned4(num_tiles) ||
      (a_row_of && !aligned4(a_row_of)) || (weight_layout == MOE_LAYOUT_PACKED && (reinterpret_cast<uintptr_t>(Ws) & 7u)))
    return fail(MOE_ERR_MISALIGNED, "moe_grouped_gemm_w4a16: A, Wq, C need 16-byte alignment (packed Ws 8-byte)");
  if ((int64_t)max_tiles * block_m >= kMaxRows + (int64_t)MOE_MAX_EXPERTS * block_m)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "max_tiles=%d too large", max_tiles);
  moe::GemmArgs a{A, a_row_of, a_row_div, Wq, Ws, N, K, tiles, num_tiles, max_tiles, 0, C, epilogue,
                  out_dtype == MOE_OUT_F16E ? 2 : (out_dtype == MOE_OUT_F32 ? 1 : 0), weight_layout == MOE_LAYOUT_PACKED};
  a.C_side = C_side;
  return hip_status(moe::launch_grouped_gemm(a, block_m, (hipStream_t)stream), "moe_grouped_gemm_w4a16 launch");
}

moe_status_t moe_x_to_f16(const uint16_t* x, int32_t T, int32_t H, uint16_t* x16, int32_t* x_exp, void* stream) {
  if (T < 0 || H < 8 || H % 8 != 0) return fail(MOE_ERR_INVALID_ARG, "moe_x_to_f16: need T >= 0 and H a positive multiple of 8");
  if ((int64_t)T >= kMaxRows) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_x_to_f16: T=%d must be < 2^26", T);
  if (T == 0) return ok();
  if (!x || !x16 || !x_exp) return fail(MOE_ERR_INVALID_ARG, "moe_x_to_f16: NULL pointer");
  if (!aligned16(x) || !aligned16(x16) || !aligned4(x_exp))
    return fail(MOE_ERR_MISALIGNED, "moe_x_to_f16: x and x16 need 16-byte alignment");
  return hip_status(moe::launch_x_to_f16(x, T, H, x16, x_exp, (hipStream_t)stream), "moe_x_to_f16 launch");
}

moe_status_t moe_grouped_gemm_w4f16(const uint16_t* A, const int32_t* a_row_exp, const uint8_t* a_blk_flag,
                                    const uint8_t* a_row_blk_exp, const int32_t* a_row_of, int32_t a_row_div,
                                    const uint8_t* Wq, const uint16_t* Ws, int32_t weight_layout, int32_t E, int32_t N,
                                    int32_t K, const int32_t* tiles, int32_t max_tiles, const int32_t* num_tiles,
                                    int32_t block_m, int32_t epilogue, void* C, int32_t out_dtype, void* C_aux,
                                    uint8_t* C_aux2, void* stream) {
  if (E < 1 || N < 1 || K < 1 || max_tiles < 0) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_w4f16: need E, N, K >= 1, max_tiles >= 0");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E=%d exceeds %d", E, MOE_MAX_EXPERTS);
  if (K % 32 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "K=%d must be a multiple of 32", K);
  if ((int64_t)N * K / 2 > kMaxExpertCodeBytes)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "one expert's codes (N*K/2 = %lld bytes) must stay below 4 GiB",
                (long long)N * K / 2);
  if (weight_layout != MOE_LAYOUT_CANONICAL && weight_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "unknown weight_layout %d", weight_layout);
  if (block_m != 64 && !(block_m == 128 && weight_layout == MOE_LAYOUT_PACKED))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_grouped_gemm_w4f16: block_m=%d must be 64, or 128 with packed weights", block_m);
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SILU_MUL) return fail(MOE_ERR_INVALID_ARG, "unknown epilogue %d", epilogue);
  if (epilogue == MOE_EPI_SILU_MUL && (N % 2 != 0 || out_dtype != MOE_OUT_H16))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_w4f16: SILU_MUL needs an even N and MOE_OUT_H16");
  if (epilogue == MOE_EPI_NONE && out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_F16E)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_w4f16: NONE writes MOE_OUT_F32 or MOE_OUT_F16E");
  if (a_row_of && a_row_div < 1) return fail(MOE_ERR_INVALID_ARG, "a_row_div must be >= 1");
  if (weight_layout == MOE_LAYOUT_PACKED && (N % 16 != 0 || K % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "packed weights need N %% 16 == 0 and K %% 128 == 0 (N=%d K=%d)", N, K);
  if (weight_layout == MOE_LAYOUT_PACKED && epilogue == MOE_EPI_SILU_MUL && N % 32 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "packed gate_up weights need N %% 32 == 0 (N=%d)", N);
  if (max_tiles == 0) return ok();
  if (!A || !Wq || !Ws || !tiles || !num_tiles || !C || (out_dtype != MOE_OUT_F32 && !C_aux) ||
      (out_dtype == MOE_OUT_H16 && !C_aux2) || (a_blk_flag && !a_row_blk_exp))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_w4f16: NULL pointer");
  if (!aligned16(A) || !aligned16(Wq) || !aligned16(C) || !aligned2(Ws) || !aligned4(tiles) || !aligned4(num_tiles) ||
      (a_row_of && !aligned4(a_row_of)) || (a_row_exp && !aligned4(a_row_exp)) ||
      (out_dtype == MOE_OUT_F16E && !aligned4(C_aux)) ||
      (weight_layout == MOE_LAYOUT_PACKED && (reinterpret_cast<uintptr_t>(Ws) & 7u)))
    return fail(MOE_ERR_MISALIGNED, "moe_grouped_gemm_w4f16: A, Wq, C need 16-byte alignment (packed Ws 8-byte)");
  if ((int64_t)max_tiles * block_m >= kMaxRows + (int64_t)MOE_MAX_EXPERTS * block_m)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "max_tiles=%d too large", max_tiles);
  moe::GemmArgs a{A, a_row_of, a_row_div, Wq, Ws, N, K, tiles, num_tiles, max_tiles, 0, C, epilogue,
                  epilogue == MOE_EPI_SILU_MUL ? 3 : (out_dtype == MOE_OUT_F16E ? 2 : 1),
                  weight_layout == MOE_LAYOUT_PACKED};
  a.a_f16 = 1;
  a.a_row_exp = a_row_exp;
  a.a_blk_flag = a_blk_flag;
  a.a_row_blk_exp = a_row_blk_exp;
  a.a_blk_stride = (K + 31) / 32;
  if (epilogue == MOE_EPI_SILU_MUL) {
    a.c_blk_flag = static_cast<uint8_t*>(C_aux);
    a.c_row_blk_exp = C_aux2;
    a.c_blk_stride = (N / 2 + 31) / 32;
  } else if (out_dtype == MOE_OUT_F16E) {
    a.C_side = static_cast<float*>(C_aux);
  }
  return hip_status(moe::launch_grouped_gemm(a, block_m, (hipStream_t)stream), "moe_grouped_gemm_w4f16 launch");
}

moe_status_t moe_combine(const void* O, int32_t o_dtype, const float* O_side, const int32_t* inv_perm,
                         const float* topk_w, const float* shared, int32_t T, int32_t k, int32_t H, uint16_t* y,
                         void* stream) {
  if (T < 0 || k < 1 || H < 1) return fail(MOE_ERR_INVALID_ARG, "moe_combine: need T >= 0, k >= 1, H >= 1");
  if (o_dtype != MOE_OUT_F32 && o_dtype != MOE_OUT_F16E)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: o_dtype %d must be MOE_OUT_F32 or MOE_OUT_F16E", o_dtype);
  if (H % 8 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_combine: H=%d must be a multiple of 8", H);
  if ((int64_t)T * k >= kMaxRows) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T*k must be < 2^26");
  if (T == 0) return ok();
  if (!O || !inv_perm || !topk_w || !y || (o_dtype == MOE_OUT_F16E && !O_side))
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: NULL pointer");
  if (!aligned16(O) || !aligned16(y) || !aligned4(inv_perm) || !aligned4(topk_w) || (shared && !aligned16(shared)) ||
      (O_side && !aligned4(O_side)))
    return fail(MOE_ERR_MISALIGNED, "moe_combine: O, shared and y need 16-byte alignment");
  return hip_status(moe::launch_combine(O, o_dtype == MOE_OUT_F16E ? O_side : nullptr, inv_perm, topk_w, shared, -1,
                                        T, k, H, y, (hipStream_t)stream),
                    "moe_combine launch");
}

moe_status_t moe_router_logits(const uint16_t* x, const uint16_t* w_router, int32_t T, int32_t H, int32_t E,
                               float* logits, void* stream) {
  if (T < 0 || E < 1 || H < 32 || H % 32 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_router_logits: need T >= 0, E >= 1, H a positive multiple of 32");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E=%d exceeds %d", E, MOE_MAX_EXPERTS);
  if ((int64_t)T >= kMaxRows) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_router_logits: T=%d must be < 2^26", T);
  if (T == 0) return ok();
  if (!x || !w_router || !logits) return fail(MOE_ERR_INVALID_ARG, "moe_router_logits: NULL pointer");
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(logits))
    return fail(MOE_ERR_MISALIGNED, "moe_router_logits: x and w_router need 16-byte alignment");
  return hip_status(moe::launch_router_logits(x, w_router, T, H, E, logits, (hipStream_t)stream),
                    "moe_router_logits launch");
}

int32_t moe_ffn_block_m(int32_t T, int32_t E, int32_t k, int32_t weight_layout) {
  if (T < 0 || E < 1 || k < 1 || k > E || (int64_t)T * k >= kMaxRows) return -1;
  if (weight_layout != MOE_LAYOUT_CANONICAL && weight_layout != MOE_LAYOUT_PACKED) return -1;
  return pick_block_m((int64_t)T * k, E, weight_layout == MOE_LAYOUT_PACKED);
}

size_t moe_ffn_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1 || k > E || E > MOE_MAX_EXPERTS || (int64_t)T * k >= kMaxRows) return 0;
  return ffn_layout(T, H, I, E, k, false).total;
}

moe_status_t moe_ffn_forward(const uint16_t* x, const float* router_logits, int32_t T, int32_t H,
                             int32_t I, int32_t E, int32_t k, const uint8_t* w13_q,
                             const uint16_t* w13_s, const uint8_t* w2_q, const uint16_t* w2_s,
                             int32_t weight_layout, uint16_t* y, int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (moe_status_t st = check_routing_shape(T, E, k)) return st;
  if (moe_status_t st = check_weight_shape(H, I, weight_layout, "moe_ffn_forward")) return st;
  if (T == 0) return ok();
  if (moe_status_t st = check_ffn_ptrs(x, w13_q, w13_s, w2_q, w2_s, weight_layout, y, topk_ids_out, topk_w_out,
                                       workspace, "moe_ffn_forward"))
    return st;
  if (!router_logits) return fail(MOE_ERR_INVALID_ARG, "moe_ffn_forward: NULL router_logits");
  if (!aligned4(router_logits)) return fail(MOE_ERR_MISALIGNED, "moe_ffn_forward: router_logits need 4-byte alignment");
  const FfnLayout L = ffn_layout(T, H, I, E, k, weight_layout == MOE_LAYOUT_PACKED);
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "moe_ffn_forward: workspace %zu B < required %zu B", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  if (moe_status_t st = run_ffn(x, router_logits, T, H, I, E, k, w13_q, w13_s, w2_q, w2_s, weight_layout, y,
                                topk_ids_out, topk_w_out, ws, L, SharedW{}, nullptr, (hipStream_t)stream))
    return st;
  if (!dump_enabled()) return ok();
  return dump_layer(x, router_logits, topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids),
                    reinterpret_cast<int32_t*>(ws + L.ntiles), y, T, H, I, E, k, L.block_m, (hipStream_t)stream);
}

size_t moe_ffn_noalloc_scratch_bytes(void) { return scratch_capacity(); }

moe_status_t moe_ffn_forward_noalloc(const uint16_t* x, const float* router_logits, int32_t T, int32_t H, int32_t I,
                                     int32_t E, int32_t k, const uint8_t* w13_q, const uint16_t* w13_s,
                                     const uint8_t* w2_q, const uint16_t* w2_s, int32_t weight_layout, uint16_t* y,
                                     int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  if (moe_status_t st = check_routing_shape(T, E, k)) return st;
  if (moe_status_t st = check_weight_shape(H, I, weight_layout, "moe_ffn_forward_noalloc")) return st;
  // The size limit is checked before anything touches the device, so an oversized call fails the
  // same way on any host.
  const FfnLayout L = ffn_layout(T, H, I, E, k, weight_layout == MOE_LAYOUT_PACKED);
  if (L.total > scratch_capacity())
    return fail(MOE_ERR_WORKSPACE,
                "moe_ffn_forward_noalloc: these sizes need %zu B of scratch, above the library's static %zu B "
                "(use moe_ffn_forward with a caller workspace)",
                L.total, scratch_capacity());
  if (T == 0) return ok();
  if (moe_status_t st = check_ffn_ptrs(x, w13_q, w13_s, w2_q, w2_s, weight_layout, y, topk_ids_out, topk_w_out,
                                       nullptr, "moe_ffn_forward_noalloc", false))
    return st;
  if (!router_logits) return fail(MOE_ERR_INVALID_ARG, "moe_ffn_forward_noalloc: NULL router_logits");
  if (!aligned4(router_logits))
    return fail(MOE_ERR_MISALIGNED, "moe_ffn_forward_noalloc: router_logits need 4-byte alignment");
  char* ws = nullptr;
  if (moe_status_t st = scratch_of_current_device(&ws)) return st;
  return run_ffn(x, router_logits, T, H, I, E, k, w13_q, w13_s, w2_q, w2_s, weight_layout, y, topk_ids_out,
                 topk_w_out, ws, L, SharedW{}, nullptr, (hipStream_t)stream);
}

size_t moe_dense_ffn_workspace_bytes(int32_t T, int32_t H, int32_t I) {
  if (T < 0 || H < 1 || I < 1) return 0;
  return up256((size_t)T * I * 2);
}

moe_status_t moe_dense_ffn_w4a16(const uint16_t* x, int32_t T, int32_t H, int32_t I, const uint8_t* w13_q,
                                 const uint16_t* w13_s, const uint8_t* w2_q, const uint16_t* w2_s,
                                 int32_t weight_layout, float* out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (T < 0 || (int64_t)T >= kMaxRows) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_dense_ffn_w4a16: T=%d", T);
  if (moe_status_t st = check_weight_shape(H, I, weight_layout, "moe_dense_ffn_w4a16")) return st;
  if (T == 0) return ok();
  if (moe_status_t st = check_weight_ptrs(w13_q, w13_s, w2_q, w2_s, weight_layout, "moe_dense_ffn_w4a16")) return st;
  if (!x || !out || !workspace) return fail(MOE_ERR_INVALID_ARG, "moe_dense_ffn_w4a16: NULL pointer");
  if (!aligned16(x) || !aligned16(out) || !aligned16(workspace))
    return fail(MOE_ERR_MISALIGNED, "moe_dense_ffn_w4a16: x, out and workspace need 16-byte alignment");
  if (workspace_bytes < moe_dense_ffn_workspace_bytes(T, H, I))
    return fail(MOE_ERR_WORKSPACE, "moe_dense_ffn_w4a16: workspace %zu B < required %zu B", workspace_bytes,
                moe_dense_ffn_workspace_bytes(T, H, I));
  return hip_status(run_dense_ffn(x, T, H, I, w13_q, w13_s, w2_q, w2_s, weight_layout,
                                  static_cast<uint16_t*>(workspace), out, (hipStream_t)stream),
                    "moe_dense_ffn_w4a16 launch");
}

size_t moe_ffn_block_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t Is) {
  const size_t base = moe_ffn_workspace_bytes(T, H, I, E, k);
  if (base == 0 || Is < 0) return 0;
  size_t total = base + up256((size_t)T * E * 4);
  if (Is > 0) total += up256((size_t)T * Is * 2) + up256((size_t)T * H * 4);
  return total;
}

moe_status_t moe_ffn_block_forward(const uint16_t* x, const uint16_t* w_router, int32_t T, int32_t H, int32_t I,
                                   int32_t E, int32_t k, const uint8_t* w13_q, const uint16_t* w13_s,
                                   const uint8_t* w2_q, const uint16_t* w2_s, int32_t Is, const uint8_t* w13s_q,
                                   const uint16_t* w13s_s, const uint8_t* w2s_q, const uint16_t* w2s_s,
                                   int32_t weight_layout, uint16_t* y, float* logits_out, int32_t* topk_ids_out,
                                   float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (moe_status_t st = check_routing_shape(T, E, k)) return st;
  if (moe_status_t st = check_weight_shape(H, I, weight_layout, "moe_ffn_block_forward")) return st;
  if (Is < 0) return fail(MOE_ERR_INVALID_ARG, "moe_ffn_block_forward: Is=%d", Is);
  if (Is > 0)
    if (moe_status_t st = check_weight_shape(H, Is, weight_layout, "moe_ffn_block_forward (shared expert)")) return st;
  if (T == 0) return ok();
  if (moe_status_t st = check_ffn_ptrs(x, w13_q, w13_s, w2_q, w2_s, weight_layout, y, topk_ids_out, topk_w_out,
                                       workspace, "moe_ffn_block_forward"))
    return st;
  if (Is > 0)
    if (moe_status_t st = check_weight_ptrs(w13s_q, w13s_s, w2s_q, w2s_s, weight_layout, "moe_ffn_block_forward (shared expert)"))
      return st;
  if (!w_router) return fail(MOE_ERR_INVALID_ARG, "moe_ffn_block_forward: NULL w_router");
  if (!aligned16(w_router) || (logits_out && !aligned4(logits_out)))
    return fail(MOE_ERR_MISALIGNED, "moe_ffn_block_forward: w_router needs 16-byte alignment");
  const size_t need = moe_ffn_block_workspace_bytes(T, H, I, E, k, Is);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_ffn_block_forward: workspace %zu B < required %zu B", workspace_bytes, need);
  // A shared expert of the routed intermediate size runs inside the routed launches; another size
  // runs as a dense FFN first.
  const bool fused = Is == I;
  const bool packed = weight_layout == MOE_LAYOUT_PACKED;
  const FfnLayout L = ffn_layout(T, H, I, E, k, packed, fused ? T : 0);
  char* ws = static_cast<char*>(workspace);
  size_t off = L.total;
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>(ws + off);
  off += up256((size_t)T * E * 4);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = moe::launch_router_logits(x, w_router, T, H, E, logits, s);
  if (e != hipSuccess) return hip_status(e, "router launch");
  SharedW sw{};
  float* shared_out = nullptr;
  if (fused) {
    sw = SharedW{w13s_q, w13s_s, w2s_q, w2s_s};
  } else if (Is > 0) {
    uint16_t* hs = reinterpret_cast<uint16_t*>(ws + off);
    off += up256((size_t)T * Is * 2);
    shared_out = reinterpret_cast<float*>(ws + off);
    e = run_dense_ffn(x, T, H, Is, w13s_q, w13s_s, w2s_q, w2s_s, weight_layout, hs, shared_out, s);
    if (e != hipSuccess) return hip_status(e, "shared expert launch");
  }
  if (moe_status_t st = run_ffn(x, logits, T, H, I, E, k, w13_q, w13_s, w2_q, w2_s, weight_layout, y, topk_ids_out,
                                topk_w_out, ws, L, sw, shared_out, s))
    return st;
  if (!dump_enabled()) return ok();
  return dump_layer(x, logits, topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids),
                    reinterpret_cast<int32_t*>(ws + L.ntiles), y, T, H, I, E, k, L.block_m, s);
}

// ---- MXFP4 (W4A4) variant -------------------------------------------------------------------------

moe_status_t moe_mx_quantize(const uint16_t* x, int32_t rows, int32_t K, uint8_t* q, uint8_t* s, void* stream) {
  if (rows < 0 || K < 32 || K % 32 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_mx_quantize: need rows >= 0 and K a positive multiple of 32");
  if ((int64_t)rows >= kMaxRows) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_mx_quantize: rows=%d must be < 2^26", rows);
  if (rows == 0) return ok();
  if (!x || !q || !s) return fail(MOE_ERR_INVALID_ARG, "moe_mx_quantize: NULL pointer");
  if (!aligned16(x) || !aligned16(q)) return fail(MOE_ERR_MISALIGNED, "moe_mx_quantize: x and q need 16-byte alignment");
  return hip_status(moe::launch_mx_quant(x, rows, K, q, s, (hipStream_t)stream), "moe_mx_quantize launch");
}

moe_status_t moe_mx_prepack(const uint8_t* w_q, const uint8_t* w_e, int32_t E, int32_t N, int32_t K, uint8_t* packed_q,
                            uint8_t* packed_e, void* stream) {
  if (E < 1 || N < 1 || K < 128) return fail(MOE_ERR_INVALID_ARG, "moe_mx_prepack: need E, N >= 1 and K >= 128");
  if (N % 16 != 0 || K % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_mx_prepack: N=%d must be a multiple of 16 and K=%d of 128", N, K);
  if (!w_q || !w_e || !packed_q || !packed_e) return fail(MOE_ERR_INVALID_ARG, "moe_mx_prepack: NULL pointer");
  if (!aligned16(w_q) || !aligned16(packed_q)) return fail(MOE_ERR_MISALIGNED, "moe_mx_prepack: codes need 16-byte alignment");
  return hip_status(moe::launch_mx_prepack(w_q, w_e, E, N, K, packed_q, packed_e, (hipStream_t)stream),
                    "moe_mx_prepack launch");
}

moe_status_t moe_mx_quantize_tiles(const uint16_t* x, int32_t T, int32_t K, const int32_t* a_row_of,
                                  int32_t a_row_div, const int32_t* tiles, int32_t max_tiles, const int32_t* num_tiles,
                                  int32_t block_m, uint8_t* q, uint8_t* s, void* stream) {
  if (T < 0 || K < 128 || K % 128 != 0 || max_tiles < 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_mx_quantize_tiles: need T >= 0, K a positive multiple of 128, max_tiles >= 0");
  if (block_m != 16 && block_m != 32 && block_m != 64)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_mx_quantize_tiles: block_m=%d must be 16, 32 or 64", block_m);
  if (a_row_of && a_row_div < 1) return fail(MOE_ERR_INVALID_ARG, "a_row_div must be >= 1");
  if ((int64_t)max_tiles * block_m >= kMaxRows + (int64_t)MOE_MAX_EXPERTS * block_m)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "max_tiles=%d too large", max_tiles);
  if (T == 0 || max_tiles == 0) return ok();
  if (!x || !tiles || !num_tiles || !q || !s) return fail(MOE_ERR_INVALID_ARG, "moe_mx_quantize_tiles: NULL pointer");
  if (!aligned16(x) || !aligned16(q) || !aligned4(tiles) || !aligned4(num_tiles) || (a_row_of && !aligned4(a_row_of)))
    return fail(MOE_ERR_MISALIGNED, "moe_mx_quantize_tiles: x and q need 16-byte alignment");
  return hip_status(moe::launch_mx_quant_tiles(x, K, a_row_of, a_row_div, tiles, num_tiles, max_tiles, block_m, q, s,
                                               (hipStream_t)stream),
                    "moe_mx_quantize_tiles launch");
}

moe_status_t moe_grouped_gemm_mxfp4(const uint8_t* Aq, const uint8_t* As, const int32_t* a_row_of, int32_t a_row_div,
                                    const uint8_t* Wq, const uint8_t* We, int32_t weight_layout, int32_t act_layout,
                                    int32_t E, int32_t N, int32_t K,
                                    const int32_t* tiles, int32_t max_tiles, const int32_t* num_tiles, int32_t block_m,
                                    int32_t epilogue, void* C, uint8_t* Cs, int32_t out_dtype, void* stream) {
  if (E < 1 || N < 1 || K < 1 || max_tiles < 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_mxfp4: need E, N, K >= 1, max_tiles >= 0");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E=%d exceeds %d", E, MOE_MAX_EXPERTS);
  if (K % 32 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "K=%d must be a multiple of 32", K);
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_grouped_gemm_mxfp4: block_m=%d must be 16, 32, 64 or 128", block_m);
  if (block_m == 128 && (K % 128 != 0 || act_layout != MOE_ACT_ROWS))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "moe_grouped_gemm_mxfp4: block_m 128 needs K %% 128 == 0 and row-major activations (K=%d)", K);
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SILU_MUL) return fail(MOE_ERR_INVALID_ARG, "unknown epilogue %d", epilogue);
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return fail(MOE_ERR_INVALID_ARG, "unknown out_dtype %d", out_dtype);
  if (epilogue == MOE_EPI_SILU_MUL && N % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "SILU_MUL output is MXFP4: N/2 = %d must be a multiple of 32", N / 2);
  if (a_row_of && a_row_div < 1) return fail(MOE_ERR_INVALID_ARG, "a_row_div must be >= 1");
  if (weight_layout != MOE_LAYOUT_CANONICAL && weight_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "unknown weight_layout %d", weight_layout);
  if (weight_layout == MOE_LAYOUT_PACKED && (N % 16 != 0 || K % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "packed MXFP4 weights need N %% 16 == 0 and K %% 128 == 0 (N=%d K=%d)", N, K);
  if (act_layout != MOE_ACT_ROWS && act_layout != MOE_ACT_TILED)
    return fail(MOE_ERR_INVALID_ARG, "unknown act_layout %d", act_layout);
  if (act_layout == MOE_ACT_TILED && weight_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "tile-blocked activations need packed weights");
  if (act_layout == MOE_ACT_TILED && epilogue == MOE_EPI_SILU_MUL && (N / 2) % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "a tile-blocked h needs N/2 %% 128 == 0 (N=%d)", N);
  if (max_tiles == 0) return ok();
  if (!Aq || !As || !Wq || !We || !tiles || !num_tiles || !C || (epilogue == MOE_EPI_SILU_MUL && !Cs))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_mxfp4: NULL pointer");
  if (!aligned16(Aq) || !aligned16(Wq) || !aligned16(C) || !aligned4(tiles) || !aligned4(num_tiles) ||
      (a_row_of && !aligned4(a_row_of)))
    return fail(MOE_ERR_MISALIGNED, "moe_grouped_gemm_mxfp4: Aq, Wq, C need 16-byte alignment");
  if (block_m == 128 && (!aligned4(As) || !aligned4(We)))
    return fail(MOE_ERR_MISALIGNED, "moe_grouped_gemm_mxfp4: block_m 128 needs 4-byte aligned scale arrays");
  if ((int64_t)max_tiles * block_m >= kMaxRows + (int64_t)MOE_MAX_EXPERTS * block_m)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "max_tiles=%d too large", max_tiles);
  moe::MxGemmArgs a{Aq, As, a_row_of, a_row_div, Wq, We, N, K, tiles, num_tiles, max_tiles, C, Cs, epilogue,
                    out_dtype == MOE_OUT_F32,
                    act_layout == MOE_ACT_TILED ? 2 : (weight_layout == MOE_LAYOUT_PACKED ? 1 : 0)};
  return hip_status(moe::launch_grouped_gemm_mx(a, block_m, (hipStream_t)stream), "moe_grouped_gemm_mxfp4 launch");
}

int32_t moe_ffn_mxfp4_block_m(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1 || k > E || (int64_t)T * k >= kMaxRows || H < 32 || I < 32) return -1;
  return pick_mx_block_m((int64_t)T * k, E, H, I);
}

size_t moe_ffn_mxfp4_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
  if (T < 0 || H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0 || E < 1 || k < 1 || k > E || E > MOE_MAX_EXPERTS ||
      (int64_t)T * k >= kMaxRows)
    return 0;
  return mx_layout(T, H, I, E, k).total;
}

moe_status_t moe_ffn_forward_mxfp4(const uint16_t* x, const float* router_logits, int32_t T, int32_t H, int32_t I,
                                   int32_t E, int32_t k, const uint8_t* w13_q, const uint8_t* w13_e,
                                   const uint8_t* w2_q, const uint8_t* w2_e, int32_t weight_layout, uint16_t* y,
                                   int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (moe_status_t st = check_routing_shape(T, E, k)) return st;
  if (H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_ffn_forward_mxfp4: H=%d and I=%d must be positive multiples of 32", H, I);
  if (weight_layout != MOE_LAYOUT_CANONICAL && weight_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "moe_ffn_forward_mxfp4: unknown weight_layout %d", weight_layout);
  if (weight_layout == MOE_LAYOUT_PACKED && (H % 128 != 0 || I % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "packed MXFP4 weights need H %% 128 == 0 and I %% 128 == 0 (H=%d I=%d)", H, I);
  if (T == 0) return ok();
  if (!x || !router_logits || !w13_q || !w13_e || !w2_q || !w2_e || !y || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "moe_ffn_forward_mxfp4: NULL pointer");
  if (!aligned16(x) || !aligned16(w13_q) || !aligned16(w2_q) || !aligned16(y) || !aligned16(workspace) ||
      !aligned4(router_logits) || (topk_ids_out && !aligned4(topk_ids_out)) || (topk_w_out && !aligned4(topk_w_out)))
    return fail(MOE_ERR_MISALIGNED, "moe_ffn_forward_mxfp4: x, weight codes, y and workspace need 16-byte alignment");
  const MxLayout M = mx_layout(T, H, I, E, k);
  if (workspace_bytes < M.total)
    return fail(MOE_ERR_WORKSPACE, "moe_ffn_forward_mxfp4: workspace %zu B < required %zu B", workspace_bytes, M.total);
  const FfnLayout& L = M.L;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = (hipStream_t)stream;
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(ws + L.ntiles);
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + M.xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(ws + M.xs);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + M.hq);
  uint8_t* hs = reinterpret_cast<uint8_t*>(ws + M.hs);
  void* o = ws + M.o;
  float* oside = M.o16 ? reinterpret_cast<float*>(ws + M.oside) : nullptr;
  const int R = T * k;
  hipError_t e;
  if (moe::route_align_fused_fits(T, E, k)) {
    e = moe::launch_route_align_small(router_logits, T, E, k, L.block_m, ids, w, counts, offsets, sorted, inv,
                                      tiles, L.max_tiles, ntiles, s);
    if (e != hipSuccess) return hip_status(e, "route+align launch");
  } else {
    e = moe::launch_route_topk(router_logits, T, E, k, ids, w, s);
    if (e != hipSuccess) return hip_status(e, "route launch");
    e = moe::launch_align(ids, R, E, L.block_m, counts, offsets, sorted, inv, tiles, L.max_tiles, ntiles,
                          ws + L.align_ws, s);
    if (e != hipSuccess) return hip_status(e, "align launch");
  }
  // packed weights: x gathered into the tile-blocked layout, h written in it by the gate_up epilogue
  // (the 128-row kernel reads row-major activations with either weight layout)
  const int packed = weight_layout == MOE_LAYOUT_PACKED;
  const int mode = L.block_m == 128 ? packed : (packed ? 2 : 0);
  if (L.block_m == 128 && (!aligned4(w13_e) || !aligned4(w2_e)))
    return fail(MOE_ERR_MISALIGNED, "moe_ffn_forward_mxfp4: scale arrays need 4-byte alignment");
  if (mode == 2) e = moe::launch_mx_quant_tiles(x, H, sorted, k, tiles, ntiles, L.max_tiles, L.block_m, xq, xs, s);
  else e = moe::launch_mx_quant(x, T, H, xq, xs, s);
  if (e != hipSuccess) return hip_status(e, "x quantization launch");
  moe::MxGemmArgs g1{xq, xs, sorted, k, w13_q, w13_e, 2 * I, H, tiles, ntiles, L.max_tiles, hq, hs,
                     MOE_EPI_SILU_MUL, 0, mode};
  e = moe::launch_grouped_gemm_mx(g1, L.block_m, s);
  if (e != hipSuccess) return hip_status(e, "gate_up launch");
  // O fp32, or fp16 with in-band per-(row, 8 columns) exponents (kind 2)
  moe::MxGemmArgs g2{hq, hs, nullptr, 1, w2_q, w2_e, H, I, tiles, ntiles, L.max_tiles, o, nullptr, MOE_EPI_NONE,
                     M.o16 ? 2 : 1, mode};
  g2.C_side = oside;
  e = moe::launch_grouped_gemm_mx(g2, L.block_m, s);
  if (e != hipSuccess) return hip_status(e, "down launch");
  return hip_status(moe::launch_combine(o, oside, inv, w, nullptr, -1, T, k, H, y, s), "combine launch");
}

// ---- W4A8 variant (MXFP8 activations on MXFP4 weights) ---------------------------------------------

namespace {

// Workspace of the W4A8 layer: the routing regions of ffn_layout (canonical tile heights), then x
// quantized (codes [T, H], scale bytes [T, H/32]), h quantized (codes [R, I], scale bytes [R, I/32])
// and O: fp32 [R, H], or (o16) fp16 with in-band exponents [R, H] and its side values fp32
// [R, ceil(H/8)].
struct W4a8Layout {
  FfnLayout L;
  // O as fp16 with in-band exponents from 16384 rows on.  Measured on MI355X in alternated A/B runs:
  // 8192 skewed tokens over 512 experts top-10 651 -> 590 us; 800 tokens equal; 32 and 64 tokens
  // +0.3 us and 4096 tokens over 8 experts top-2 +0.3-0.7 % with fp16 O, so those keep fp32.
  bool o16;
  size_t xq, xs, hq, hs, o, oside, total;
};

// Tile heights as the MXFP4 layer: experts averaging more than 128 rows (H, I multiples of 128) take the
// 128 x 256 LDS-staged kernel; the canonical tile capacity of ffn_layout covers its shorter list.
W4a8Layout w4a8_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  W4a8Layout M{};
  M.L = ffn_layout(T, H, I, E, k, false);
  const int64_t R = T * k;
  M.L.block_m = pick_mx_block_m(R, E, H, I);
  M.L.max_tiles = (int32_t)max_tiles_of(R, E, M.L.block_m);
  // row-major rows or the tile-blocked rows of the tile list, whichever is larger
  const int64_t tiled_rows = (int64_t)M.L.max_tiles * M.L.block_m;
  const int64_t xr = std::max(T, tiled_rows), hr = std::max(R, tiled_rows);
  size_t off = M.L.h;
  auto take = [&](size_t bytes) { size_t at = off; off += up256(bytes); return at; };
  M.xq = take((size_t)xr * H);
  M.xs = take((size_t)xr * H / 32);
  M.hq = take((size_t)hr * I);
  M.hs = take((size_t)hr * I / 32);
  M.o16 = R >= 16384;
  M.o = take((size_t)R * H * (M.o16 ? 2 : 4));
  M.oside = M.o16 ? take((size_t)R * ((H + 7) / 8) * 4) : 0;
  M.total = off;
  return M;
}

}  // namespace

moe_status_t moe_mx8_quantize(const uint16_t* x, int32_t rows, int32_t K, uint8_t* q, uint8_t* s, void* stream) {
  if (rows < 0 || K < 32 || K % 32 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_mx8_quantize: need rows >= 0 and K a positive multiple of 32");
  if ((int64_t)rows >= kMaxRows) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_mx8_quantize: rows=%d must be < 2^26", rows);
  if (rows == 0) return ok();
  if (!x || !q || !s) return fail(MOE_ERR_INVALID_ARG, "moe_mx8_quantize: NULL pointer");
  if (!aligned16(x) || !aligned16(q)) return fail(MOE_ERR_MISALIGNED, "moe_mx8_quantize: x and q need 16-byte alignment");
  return hip_status(moe::launch_mx8_quant(x, rows, K, q, s, (hipStream_t)stream), "moe_mx8_quantize launch");
}

moe_status_t moe_mx8_quantize_tiles(const uint16_t* x, int32_t T, int32_t K, const int32_t* a_row_of,
                                   int32_t a_row_div, const int32_t* tiles, int32_t max_tiles, const int32_t* num_tiles,
                                   int32_t block_m, uint8_t* q, uint8_t* s, void* stream) {
  if (T < 0 || K < 128 || K % 128 != 0 || max_tiles < 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_mx8_quantize_tiles: need T >= 0, K a positive multiple of 128, max_tiles >= 0");
  if (block_m != 16 && block_m != 32 && block_m != 64)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_mx8_quantize_tiles: block_m=%d must be 16, 32 or 64", block_m);
  if (a_row_of && a_row_div < 1) return fail(MOE_ERR_INVALID_ARG, "a_row_div must be >= 1");
  if ((int64_t)max_tiles * block_m >= kMaxRows + (int64_t)MOE_MAX_EXPERTS * block_m)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "max_tiles=%d too large", max_tiles);
  if (T == 0 || max_tiles == 0) return ok();
  if (!x || !tiles || !num_tiles || !q || !s) return fail(MOE_ERR_INVALID_ARG, "moe_mx8_quantize_tiles: NULL pointer");
  if (!aligned16(x) || !aligned16(q) || !aligned4(tiles) || !aligned4(num_tiles) || (a_row_of && !aligned4(a_row_of)))
    return fail(MOE_ERR_MISALIGNED, "moe_mx8_quantize_tiles: x and q need 16-byte alignment");
  return hip_status(moe::launch_mx8_quant_tiles(x, K, a_row_of, a_row_div, tiles, num_tiles, max_tiles, block_m, q, s,
                                                (hipStream_t)stream),
                    "moe_mx8_quantize_tiles launch");
}

moe_status_t moe_grouped_gemm_w4a8(const uint8_t* Aq, const uint8_t* As, const int32_t* a_row_of, int32_t a_row_div,
                                   const uint8_t* Wq, const uint8_t* We, int32_t weight_layout, int32_t act_layout,
                                   int32_t E, int32_t N, int32_t K, const int32_t* tiles, int32_t max_tiles,
                                   const int32_t* num_tiles, int32_t block_m, int32_t epilogue, void* C, uint8_t* Cs,
                                   int32_t out_dtype, void* stream) {
  if (E < 1 || N < 1 || K < 1 || max_tiles < 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_w4a8: need E, N, K >= 1, max_tiles >= 0");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E=%d exceeds %d", E, MOE_MAX_EXPERTS);
  if (K % 32 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "K=%d must be a multiple of 32", K);
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_grouped_gemm_w4a8: block_m=%d must be 16, 32, 64 or 128", block_m);
  if (block_m == 128 && K % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_grouped_gemm_w4a8: block_m 128 needs K %% 128 == 0 (K=%d)", K);
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SILU_MUL) return fail(MOE_ERR_INVALID_ARG, "unknown epilogue %d", epilogue);
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32) return fail(MOE_ERR_INVALID_ARG, "unknown out_dtype %d", out_dtype);
  if (epilogue == MOE_EPI_SILU_MUL && N % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "SILU_MUL output is MXFP8: N/2 = %d must be a multiple of 32", N / 2);
  if (a_row_of && a_row_div < 1) return fail(MOE_ERR_INVALID_ARG, "a_row_div must be >= 1");
  if (weight_layout != MOE_LAYOUT_CANONICAL && weight_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "unknown weight_layout %d", weight_layout);
  if (weight_layout == MOE_LAYOUT_PACKED && (N % 16 != 0 || K % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "packed MXFP4 weights need N %% 16 == 0 and K %% 128 == 0 (N=%d K=%d)", N, K);
  if (act_layout != MOE_ACT_ROWS && act_layout != MOE_ACT_TILED)
    return fail(MOE_ERR_INVALID_ARG, "unknown act_layout %d", act_layout);
  if (act_layout == MOE_ACT_TILED && (weight_layout != MOE_LAYOUT_PACKED || block_m == 128))
    return fail(MOE_ERR_INVALID_ARG, "tile-blocked activations need packed weights and tiles of at most 64 rows");
  if (act_layout == MOE_ACT_TILED && epilogue == MOE_EPI_SILU_MUL && (N / 2) % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "a tile-blocked h needs N/2 %% 128 == 0 (N=%d)", N);
  if (max_tiles == 0) return ok();
  if (!Aq || !As || !Wq || !We || !tiles || !num_tiles || !C || (epilogue == MOE_EPI_SILU_MUL && !Cs))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_w4a8: NULL pointer");
  if (!aligned16(Aq) || !aligned16(Wq) || !aligned16(C) || !aligned4(tiles) || !aligned4(num_tiles) ||
      (a_row_of && !aligned4(a_row_of)))
    return fail(MOE_ERR_MISALIGNED, "moe_grouped_gemm_w4a8: Aq, Wq, C need 16-byte alignment");
  if (block_m == 128 && (!aligned4(As) || !aligned4(We)))
    return fail(MOE_ERR_MISALIGNED, "moe_grouped_gemm_w4a8: block_m 128 needs 4-byte aligned scale arrays");
  if ((int64_t)max_tiles * block_m >= kMaxRows + (int64_t)MOE_MAX_EXPERTS * block_m)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "max_tiles=%d too large", max_tiles);
  moe::MxGemmArgs a{Aq, As, a_row_of, a_row_div, Wq, We, N, K, tiles, num_tiles, max_tiles, C, Cs, epilogue,
                    out_dtype == MOE_OUT_F32,
                    act_layout == MOE_ACT_TILED ? 2 : (weight_layout == MOE_LAYOUT_PACKED ? 1 : 0), 1};
  return hip_status(moe::launch_grouped_gemm_mx(a, block_m, (hipStream_t)stream), "moe_grouped_gemm_w4a8 launch");
}

int32_t moe_ffn_w4a8_block_m(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1 || k > E || (int64_t)T * k >= kMaxRows || H < 32 || I < 32) return -1;
  return pick_mx_block_m((int64_t)T * k, E, H, I);
}

size_t moe_ffn_w4a8_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
  if (T < 0 || H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0 || E < 1 || k < 1 || k > E || E > MOE_MAX_EXPERTS ||
      (int64_t)T * k >= kMaxRows)
    return 0;
  return w4a8_layout(T, H, I, E, k).total;
}

moe_status_t moe_ffn_forward_w4a8(const uint16_t* x, const float* router_logits, int32_t T, int32_t H, int32_t I,
                                  int32_t E, int32_t k, const uint8_t* w13_q, const uint8_t* w13_e,
                                  const uint8_t* w2_q, const uint8_t* w2_e, int32_t weight_layout, uint16_t* y,
                                  int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (moe_status_t st = check_routing_shape(T, E, k)) return st;
  if (H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_ffn_forward_w4a8: H=%d and I=%d must be positive multiples of 32", H, I);
  if (weight_layout != MOE_LAYOUT_CANONICAL && weight_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "moe_ffn_forward_w4a8: unknown weight_layout %d", weight_layout);
  if (weight_layout == MOE_LAYOUT_PACKED && (H % 128 != 0 || I % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "packed MXFP4 weights need H %% 128 == 0 and I %% 128 == 0 (H=%d I=%d)", H, I);
  if (T == 0) return ok();
  if (!x || !router_logits || !w13_q || !w13_e || !w2_q || !w2_e || !y || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "moe_ffn_forward_w4a8: NULL pointer");
  if (!aligned16(x) || !aligned16(w13_q) || !aligned16(w2_q) || !aligned16(y) || !aligned16(workspace) ||
      !aligned4(router_logits) || (topk_ids_out && !aligned4(topk_ids_out)) || (topk_w_out && !aligned4(topk_w_out)))
    return fail(MOE_ERR_MISALIGNED, "moe_ffn_forward_w4a8: x, weight codes, y and workspace need 16-byte alignment");
  const W4a8Layout M = w4a8_layout(T, H, I, E, k);
  if (workspace_bytes < M.total)
    return fail(MOE_ERR_WORKSPACE, "moe_ffn_forward_w4a8: workspace %zu B < required %zu B", workspace_bytes, M.total);
  const FfnLayout& L = M.L;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = (hipStream_t)stream;
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(ws + L.ntiles);
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + M.xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(ws + M.xs);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + M.hq);
  uint8_t* hs = reinterpret_cast<uint8_t*>(ws + M.hs);
  void* o = ws + M.o;
  float* oside = M.o16 ? reinterpret_cast<float*>(ws + M.oside) : nullptr;
  const int R = T * k;
  hipError_t e;
  if (moe::route_align_fused_fits(T, E, k)) {
    e = moe::launch_route_align_small(router_logits, T, E, k, L.block_m, ids, w, counts, offsets, sorted, inv,
                                      tiles, L.max_tiles, ntiles, s);
    if (e != hipSuccess) return hip_status(e, "route+align launch");
  } else {
    e = moe::launch_route_topk(router_logits, T, E, k, ids, w, s);
    if (e != hipSuccess) return hip_status(e, "route launch");
    e = moe::launch_align(ids, R, E, L.block_m, counts, offsets, sorted, inv, tiles, L.max_tiles, ntiles,
                          ws + L.align_ws, s);
    if (e != hipSuccess) return hip_status(e, "align launch");
  }
  if (L.block_m == 128 && (!aligned4(w13_e) || !aligned4(w2_e)))
    return fail(MOE_ERR_MISALIGNED, "moe_ffn_forward_w4a8: scale arrays need 4-byte alignment");
  // packed weights: x gathered into the tile-blocked layout, h written in it by the gate_up epilogue
  // (the 128-row kernel reads row-major activations with either weight layout)
  const int packed = weight_layout == MOE_LAYOUT_PACKED;
  const int mode = L.block_m == 128 ? packed : (packed ? 2 : 0);
  if (mode == 2) e = moe::launch_mx8_quant_tiles(x, H, sorted, k, tiles, ntiles, L.max_tiles, L.block_m, xq, xs, s);
  else e = moe::launch_mx8_quant(x, T, H, xq, xs, s);
  if (e != hipSuccess) return hip_status(e, "x quantization launch");
  moe::MxGemmArgs g1{xq, xs, sorted, k, w13_q, w13_e, 2 * I, H, tiles, ntiles, L.max_tiles, hq, hs,
                     MOE_EPI_SILU_MUL, 0, mode, 1};
  e = moe::launch_grouped_gemm_mx(g1, L.block_m, s);
  if (e != hipSuccess) return hip_status(e, "gate_up launch");
  // O fp32, or fp16 with in-band per-(row, 8 columns) exponents (kind 2)
  moe::MxGemmArgs g2{hq, hs, nullptr, 1, w2_q, w2_e, H, I, tiles, ntiles, L.max_tiles, o, nullptr, MOE_EPI_NONE,
                     M.o16 ? 2 : 1, mode, 1};
  g2.C_side = oside;
  e = moe::launch_grouped_gemm_mx(g2, L.block_m, s);
  if (e != hipSuccess) return hip_status(e, "down launch");
  return hip_status(moe::launch_combine(o, oside, inv, w, nullptr, -1, T, k, H, y, s), "combine launch");
}

// ---- FP8 (W8A8, per-1x128) variant ------------------------------------------------------------------

moe_status_t moe_f8_quantize(const void* x, int32_t in_dtype, int32_t rows, int32_t K, uint8_t* q, float* s,
                             void* stream) {
  if (rows < 0 || K < 128 || K % 128 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_f8_quantize: need rows >= 0 and K a positive multiple of 128");
  if (in_dtype != MOE_IN_BF16 && in_dtype != MOE_IN_F32)
    return fail(MOE_ERR_INVALID_ARG, "moe_f8_quantize: unknown in_dtype %d", in_dtype);
  if ((int64_t)rows >= kMaxRows) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_f8_quantize: rows=%d must be < 2^26", rows);
  if (rows == 0) return ok();
  if (!x || !q || !s) return fail(MOE_ERR_INVALID_ARG, "moe_f8_quantize: NULL pointer");
  if (!aligned16(x) || !aligned16(q) || !aligned4(s))
    return fail(MOE_ERR_MISALIGNED, "moe_f8_quantize: x and q need 16-byte alignment, s 4-byte");
  return hip_status(moe::launch_f8_quant(x, in_dtype == MOE_IN_F32, rows, K, q, s, (hipStream_t)stream),
                    "moe_f8_quantize launch");
}

moe_status_t moe_grouped_gemm_f8(const uint8_t* Aq, const float* As, const int32_t* a_row_of, int32_t a_row_div,
                                 const uint8_t* Wq, const float* Ws, int32_t E, int32_t N, int32_t K,
                                 const int32_t* tiles, int32_t max_tiles, const int32_t* num_tiles, int32_t block_m,
                                 int32_t epilogue, void* C, float* Cs, int32_t out_dtype, void* stream) {
  if (E < 1 || N < 1 || K < 1 || max_tiles < 0 || a_row_div < 1)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_f8: need E, N, K, a_row_div >= 1, max_tiles >= 0");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_grouped_gemm_f8: E=%d exceeds %d", E, MOE_MAX_EXPERTS);
  if (K % 128 != 0 || K > kF8MaxK)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_grouped_gemm_f8: K=%d must be a multiple of 128 and <= %d", K, kF8MaxK);
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_grouped_gemm_f8: block_m=%d must be 16, 32, 64 or 128", block_m);
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SILU_MUL)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_f8: unknown epilogue %d", epilogue);
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_F8)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_f8: unknown out_dtype %d", out_dtype);
  if (epilogue == MOE_EPI_SILU_MUL && (N % 2 != 0 || out_dtype == MOE_OUT_BF16))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_f8: SILU_MUL needs an even N and out_dtype F32 or F8");
  if (out_dtype == MOE_OUT_F8 && (epilogue != MOE_EPI_SILU_MUL || block_m != 128 || (N / 2) % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "moe_grouped_gemm_f8: out_dtype F8 needs SILU_MUL, block_m 128 and N/2 %% 128 == 0 (N=%d)", N);
  if (max_tiles == 0) return ok();
  if (!Aq || !As || !Wq || !Ws || !tiles || !num_tiles || !C || (out_dtype == MOE_OUT_F8 && !Cs))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_f8: NULL pointer");
  if (!aligned16(Aq) || !aligned16(Wq) || !aligned16(C) || !aligned4(As) || !aligned4(Ws) || !aligned4(tiles) ||
      (Cs && !aligned4(Cs)))
    return fail(MOE_ERR_MISALIGNED, "moe_grouped_gemm_f8: Aq, Wq, C need 16-byte alignment, As, Ws, Cs 4-byte");
  moe::F8GemmArgs a{Aq, As, a_row_of, a_row_div, Wq, Ws, N, K, tiles, num_tiles, max_tiles, C, epilogue,
                    out_dtype == MOE_OUT_F8 ? 2 : (out_dtype == MOE_OUT_F32 ? 1 : 0), Cs};
  return hip_status(moe::launch_grouped_gemm_f8(a, block_m, (hipStream_t)stream), "moe_grouped_gemm_f8 launch");
}

int32_t moe_ffn_f8_block_m(int32_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1 || k > E || (int64_t)T * k >= kMaxRows) return -1;
  return pick_f8_block_m((int64_t)T * k, E);
}

size_t moe_ffn_f8_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
  if (T < 0 || !f8_dims_ok(H, I) || E < 1 || k < 1 || k > E || E > MOE_MAX_EXPERTS || (int64_t)T * k >= kMaxRows)
    return 0;
  return f8_layout(T, H, I, E, k).total;
}

moe_status_t moe_ffn_forward_f8(const uint16_t* x, const float* router_logits, int32_t T, int32_t H, int32_t I,
                                int32_t E, int32_t k, const uint8_t* w13_q, const float* w13_s, const uint8_t* w2_q,
                                const float* w2_s, uint16_t* y, int32_t* topk_ids_out, float* topk_w_out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (moe_status_t st = check_routing_shape(T, E, k)) return st;
  if (!f8_dims_ok(H, I))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_ffn_forward_f8: H=%d and I=%d must be positive multiples of 128, <= %d",
                H, I, kF8MaxK);
  if (T == 0) return ok();
  if (!x || !router_logits || !w13_q || !w13_s || !w2_q || !w2_s || !y || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "moe_ffn_forward_f8: NULL pointer");
  if (!aligned16(x) || !aligned16(w13_q) || !aligned16(w2_q) || !aligned16(y) || !aligned16(workspace) ||
      !aligned4(w13_s) || !aligned4(w2_s) || !aligned4(router_logits) || (topk_ids_out && !aligned4(topk_ids_out)) ||
      (topk_w_out && !aligned4(topk_w_out)))
    return fail(MOE_ERR_MISALIGNED, "moe_ffn_forward_f8: x, weight codes, y and workspace need 16-byte alignment");
  const F8Layout M = f8_layout(T, H, I, E, k);
  if (workspace_bytes < M.total)
    return fail(MOE_ERR_WORKSPACE, "moe_ffn_forward_f8: workspace %zu B < required %zu B", workspace_bytes, M.total);
  const FfnLayout& L = M.L;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = (hipStream_t)stream;
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(ws + L.ntiles);
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + M.xq);
  float* xs = reinterpret_cast<float*>(ws + M.xs);
  float* hf = reinterpret_cast<float*>(ws + M.hf);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + M.hq);
  float* hs = reinterpret_cast<float*>(ws + M.hs);
  void* o = ws + M.o;
  float* oside = M.o16 ? reinterpret_cast<float*>(ws + M.oside) : nullptr;
  const int R = T * k;
  hipError_t e;
  if (moe::route_align_fused_fits(T, E, k)) {
    e = moe::launch_route_align_small(router_logits, T, E, k, L.block_m, ids, w, counts, offsets, sorted, inv,
                                      tiles, L.max_tiles, ntiles, s);
    if (e != hipSuccess) return hip_status(e, "route+align launch");
  } else {
    e = moe::launch_route_topk(router_logits, T, E, k, ids, w, s);
    if (e != hipSuccess) return hip_status(e, "route launch");
    e = moe::launch_align(ids, R, E, L.block_m, counts, offsets, sorted, inv, tiles, L.max_tiles, ntiles,
                          ws + L.align_ws, s);
    if (e != hipSuccess) return hip_status(e, "align launch");
  }
  e = moe::launch_f8_quant(x, false, T, H, xq, xs, s);
  if (e != hipSuccess) return hip_status(e, "x quantization launch");
  // the 128-row kernel quantizes h in its epilogue (one 1x128 block per row and workgroup)
  const bool fused_h = L.block_m == 128 && I % 128 == 0;
  moe::F8GemmArgs g1{xq, xs, sorted, k, w13_q, w13_s, 2 * I, H, tiles, ntiles, L.max_tiles,
                     fused_h ? static_cast<void*>(hq) : static_cast<void*>(hf), MOE_EPI_SILU_MUL, fused_h ? 2 : 1,
                     fused_h ? hs : nullptr};
  e = moe::launch_grouped_gemm_f8(g1, L.block_m, s);
  if (e != hipSuccess) return hip_status(e, "gate_up launch");
  if (!fused_h) {
    e = moe::launch_f8_quant(hf, true, R, I, hq, hs, s);
    if (e != hipSuccess) return hip_status(e, "h quantization launch");
  }
  // O fp32, or fp16 with in-band per-(row, 8 columns) exponents (kind 3 of the FP8 GEMM)
  moe::F8GemmArgs g2{hq, hs, nullptr, 1, w2_q, w2_s, H, I, tiles, ntiles, L.max_tiles, o, MOE_EPI_NONE,
                     M.o16 ? 3 : 1};
  g2.C_side = oside;
  e = moe::launch_grouped_gemm_f8(g2, L.block_m, s);
  if (e != hipSuccess) return hip_status(e, "down launch");
  return hip_status(moe::launch_combine(o, oside, inv, w, nullptr, -1, T, k, H, y, s), "combine launch");
}

}  // extern "C"
