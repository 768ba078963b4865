// C ABI of the MoE layer: host-side validation, workspace carving, kernel launches.
// Validation runs entirely on the host before anything is enqueued and touches no
// HIP API, so the error paths can be exercised without a GPU.
#include <stddef.h>
#include <algorithm>
#include <atomic>
#include <stdint.h>

#include "../../include/moeq.h"
#include "device.h"
#include "launch.h"

namespace {

using moeq::LayerArgs;
using moeq::Work;

constexpr size_t kAlign = 256;
// Workspace header at offset 0 whatever T is: words that must read zero when a call
// starts (each call leaves them zero): the decode router's arrival flags, one word
// per router block (at most (1024 + 1 + 3) / 4 = 257 blocks), then its logit mailbox
// (moeq::kDecMailboxWords 64-bit words at byte 2048).
constexpr size_t kHeaderBytes = 2048 + 8 * moeq::kDecMailboxWords;
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int32_t kMaxDim = 16384;
constexpr int32_t kMaxExperts = 1024;
constexpr int32_t kMaxTopK = 16;
constexpr int32_t kMaxTokens = 1 << 16;
// MOE_PATH_AUTO takes the decode kernels up to this many tokens, where they measured
// faster than the grouped ones on MI355X.  gpt-oss MXFP4 shape (E 128, top-4, H = I = 2880):
// T = 4 decode 56.8 against grouped 68.3 us, T = 8 88.6 against 98.8 us, T = 10 101.3
// against 102.6 us, T = 12 114.2 against 107.2 us.  CB4 verify shape (E 256, top-8,
// H 2048, I 512, Zipf routing): the decode kernels win up to their limit, T = 32 63.2
// against 90.0 us.
constexpr int32_t kAutoDecodeTokensMx = 10;
constexpr int32_t kAutoDecodeTokensCb4 = 32;

int validate_layer(const moe_layer* L) {
  if (!L) return MOE_ERR_INVALID_ARG;
  if (L->hidden <= 0 || L->inter <= 0 || L->n_experts <= 0 || L->top_k <= 0) return MOE_ERR_INVALID_ARG;
  if (L->hidden % 32 || L->inter % 32) return MOE_ERR_INVALID_ARG;
  if (L->hidden > kMaxDim || L->inter > kMaxDim || L->n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (L->top_k > L->n_experts || L->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (L->wfmt != MOE_WFMT_MXFP4 && L->wfmt != MOE_WFMT_CB4 && L->wfmt != MOE_WFMT_MXFP4_PS &&
      L->wfmt != MOE_WFMT_AFF3)
    return MOE_ERR_INVALID_ARG;
  if (L->has_shared != 0 && L->has_shared != 1) return MOE_ERR_INVALID_ARG;
  if (!L->router_w || !L->gate_up || !L->down) return MOE_ERR_INVALID_ARG;
  if (L->wfmt == MOE_WFMT_CB4 && !L->codebook) return MOE_ERR_INVALID_ARG;
  if (L->wfmt != MOE_WFMT_CB4 && L->codebook) return MOE_ERR_INVALID_ARG;
  if (!aligned16(L->router_w) || (L->router_b && !aligned4(L->router_b))) return MOE_ERR_ALIGNMENT;
  if (L->has_shared && L->shared_gate_w && !aligned16(L->shared_gate_w)) return MOE_ERR_ALIGNMENT;
  if (!aligned16(L->gate_up) || !aligned16(L->down)) return MOE_ERR_ALIGNMENT;
  if (!(L->omit_below >= 0.0f && L->omit_below <= 1.0f)) return MOE_ERR_INVALID_ARG;  // NaN fails too
  if (L->wfmt == MOE_WFMT_AFF3 && (L->hidden % 128 || L->inter % 128)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct Layout {
  size_t logits, ids, pair_w, counts, offsets, perm, active, xplanes, hplanes, xr, o, tickets, slots, items, n_items,
      groups, n_groups, total;
};

Layout layout_for(const moe_layer* L, int32_t T) {
  const size_t E = (size_t)L->n_experts, k = (size_t)L->top_k, H = (size_t)L->hidden, I = (size_t)L->inter;
  const size_t P = (size_t)T * k + (L->has_shared ? (size_t)T : 0);
  Layout o{};
  size_t at = kHeaderBytes;  // the fixed header (synchronisation words) comes first
  auto take = [&](size_t bytes) { size_t r = at; at = align_up(at + bytes, kAlign); return r; };
  // K-split partial logits, of the whole call or of one 32-token chunk of it (3-bit affine)
  const int Tc = T < 32 ? T : 32;
  o.logits = take(std::max((size_t)moeq::router_splits(T, (int)H) * T, (size_t)moeq::router_splits(Tc, (int)H) * Tc) *
                  (E + 1) * 8);
  o.ids = take((size_t)T * k * 4);
  o.pair_w = take(P * 4);
  o.counts = take((E + 1) * 4);
  o.offsets = take((E + 2) * 4);
  o.perm = take(P * 4);
  o.active = take((E + 2) * 4);
  // bf16 planes (CB4 prefill, fp32 x) or fp8 planes + scales (MXFP4 prefill) share a region
  const size_t Hp = align_up(H, 128), Ip = align_up(I, 256);
  o.xplanes = take(std::max(3 * (size_t)T * H * 2, 3 * (size_t)T * Hp + (size_t)T));
  o.hplanes = take(std::max(2 * P * I * 2, 3 * P * Ip + P * (Ip / 256)));
  o.xr = take((size_t)T * H * 2);  // bf16 x of a rescaled-input call (not shared with the planes)
  o.o = take(P * H * 4);
  o.tickets = take((H / 16) * 4);
  o.slots = take((E + 2) * sizeof(moeq::Slot));
  // decode gate/up work items: at most one staging pass per pair of a decode call (at most
  // 32 tokens; larger 3-bit batches run in chunks of 32)
  const size_t Td = (size_t)(T < 32 ? T : 32);
  o.items = take((Td * k + (L->has_shared ? Td : 0) + 1) * sizeof(moeq::Slot));
  o.n_items = take(4);
  o.groups = take((size_t)moeq::max_groups((int)P, (int)E) * 16);
  o.n_groups = take(4);
  o.total = at;
  return o;
}

Work carve(void* ws, const Layout& lo) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  Work w;
  w.resid = nullptr;
  w.logits = reinterpret_cast<double*>(b + lo.logits);
  w.ids = reinterpret_cast<int32_t*>(b + lo.ids);
  w.pair_w = reinterpret_cast<float*>(b + lo.pair_w);
  w.counts = reinterpret_cast<int32_t*>(b + lo.counts);
  w.offsets = reinterpret_cast<int32_t*>(b + lo.offsets);
  w.perm = reinterpret_cast<int32_t*>(b + lo.perm);
  w.active = reinterpret_cast<int32_t*>(b + lo.active);
  w.xplanes = reinterpret_cast<uint16_t*>(b + lo.xplanes);
  w.hplanes = reinterpret_cast<uint16_t*>(b + lo.hplanes);
  w.o = reinterpret_cast<float*>(b + lo.o);
  w.xr = reinterpret_cast<uint16_t*>(b + lo.xr);
  w.tickets = reinterpret_cast<uint32_t*>(b + lo.tickets);
  w.slots = reinterpret_cast<moeq::Slot*>(b + lo.slots);
  w.items = reinterpret_cast<moeq::Slot*>(b + lo.items);
  w.n_items = reinterpret_cast<int32_t*>(b + lo.n_items);
  w.hf32 = reinterpret_cast<float*>(b + lo.hplanes);
  w.xq = b + lo.xplanes;
  w.hq = b + lo.hplanes;
  w.groups = reinterpret_cast<int4*>(b + lo.groups);
  w.n_groups = reinterpret_cast<int32_t*>(b + lo.n_groups);
  w.rr_flags = reinterpret_cast<uint32_t*>(b);
  w.rr_mbox = reinterpret_cast<uint64_t*>(b + 2048);
  return w;
}

LayerArgs args_of(const moe_layer* L) {
  LayerArgs a;
  a.H = L->hidden; a.I = L->inter; a.E = L->n_experts; a.k = L->top_k;
  a.wfmt = L->wfmt; a.has_shared = L->has_shared;
  a.omit_below = L->omit_below;
  a.router_w = L->router_w; a.router_b = L->router_b;
  a.gate_up = reinterpret_cast<const uint8_t* const*>(L->gate_up);
  a.down = reinterpret_cast<const uint8_t* const*>(L->down);
  a.codebook = L->codebook;
  a.shared_gate_w = L->has_shared ? L->shared_gate_w : nullptr;
  return a;
}

int check_ws(const moe_layer* L, int32_t T, void* ws, size_t ws_bytes) {
  if (!ws) return MOE_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return MOE_ERR_ALIGNMENT;
  if (ws_bytes < layout_for(L, T).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// x_dtype kRmsInput: x is the previous layer's fp32 y and the layer's input is
// bf16(y / sqrt(mean(y^2) + eps)) per token, as moe_rms_rescale computes it.
constexpr int32_t kRmsInput = 2;

int forward_impl(const moe_layer* L, const void* x, int32_t x_dtype, int32_t T, float* y, void* ws,
                        size_t ws_bytes, void* stream, int32_t path, int32_t* dbg_ids, float* dbg_w,
                        int32_t* dbg_counts, int32_t* dbg_offsets, int32_t* dbg_perm, const moeq::Timing& tm,
                        float eps = 0.0f, bool residual = false) {
  int st = validate_layer(L);
  if (st) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16 && x_dtype != kRmsInput) return MOE_ERR_INVALID_ARG;
  if (path != MOE_PATH_AUTO && path != MOE_PATH_DECODE && path != MOE_PATH_PREFILL) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y)) return MOE_ERR_ALIGNMENT;
  if ((dbg_ids && !aligned4(dbg_ids)) || (dbg_w && !aligned4(dbg_w)) || (dbg_counts && !aligned4(dbg_counts)) ||
      (dbg_offsets && !aligned4(dbg_offsets)) || (dbg_perm && !aligned4(dbg_perm)))
    return MOE_ERR_ALIGNMENT;
  if ((st = check_ws(L, T, ws, ws_bytes))) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Work w = carve(ws, layout_for(L, T));
  w.resid = residual ? static_cast<const float*>(x) : nullptr;  // pre-norm block: y_prev + layer
  const LayerArgs a = args_of(L);
  if (a.wfmt == MOE_WFMT_AFF3) {
    // decode kernels only: a larger batch runs them on chunks of up to 32 tokens (each
    // chunk routed and bucketed on its own, so the whole call's bucketing is not formed)
    const int xd = x_dtype == kRmsInput ? MOE_BF16 : x_dtype;
    if (path == MOE_PATH_PREFILL || !moeq::decode_path_fits(a, T < 32 ? T : 32, xd)) return MOE_ERR_UNSUPPORTED;
    if (T > 32 && (dbg_counts || dbg_offsets || dbg_perm)) return MOE_ERR_UNSUPPORTED;
    const size_t xrow = (size_t)a.H * (x_dtype == MOE_BF16 ? 2 : 4);
    for (int32_t t0 = 0; t0 < T; t0 += 32) {
      const int32_t Tc = T - t0 < 32 ? T - t0 : 32;
      const void* xc = static_cast<const uint8_t*>(x) + (size_t)t0 * xrow;
      w.resid = residual ? static_cast<const float*>(xc) : nullptr;
      const hipError_t e = moeq::launch_decode(a, xc, x_dtype, Tc, w, y + (size_t)t0 * a.H, eps,
                                               dbg_ids ? dbg_ids + (size_t)t0 * a.k : nullptr,
                                               dbg_w ? dbg_w + (size_t)t0 * a.k : nullptr, dbg_counts, dbg_offsets,
                                               dbg_perm, s, tm);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return MOE_OK;
  }
  const bool dec_ok = moeq::decode_path_fits(a, T, x_dtype == kRmsInput ? MOE_BF16 : x_dtype);
  if (path == MOE_PATH_DECODE && !dec_ok) return MOE_ERR_UNSUPPORTED;
  const int32_t auto_max = a.wfmt == MOE_WFMT_CB4 ? kAutoDecodeTokensCb4 : kAutoDecodeTokensMx;
  if (path == MOE_PATH_DECODE || (path == MOE_PATH_AUTO && dec_ok && T <= auto_max))
    return hip_status(moeq::launch_decode(a, x, x_dtype, T, w, y, eps, dbg_ids, dbg_w, dbg_counts, dbg_offsets,
                                          dbg_perm, s, tm));
  hipError_t e = hipSuccess;
  if (x_dtype == kRmsInput) {  // the rescale first, then the grouped path on its bf16 output
    e = moeq::launch_rms_rescale(static_cast<const float*>(x), T, a.H, eps, w.xr, s);
    x = w.xr;
    x_dtype = MOE_BF16;
  }
  if (e == hipSuccess) e = moeq::launch_router_topk(a, x, x_dtype, T, w, dbg_ids, dbg_w, s, tm);
  if (e == hipSuccess)
    e = moeq::launch_bucket(T, a.k, a.E, a.has_shared, w.ids, w, dbg_counts, dbg_offsets, dbg_perm, s, tm);
  if (e == hipSuccess) e = moeq::launch_experts(a, x, x_dtype, T, w, y, s, tm);
  return hip_status(e);
}

// ---- scratch of moe_forward_noalloc -------------------------------------------------
// The workspace of the no-allocation entry point: one array per device the library runs
// on, zero-filled when the code object is loaded and held until the process ends.  Host
// code never uses the array's name as an address (on the host it only names the symbol):
// the device address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept per device below.
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Clears the scratch's synchronisation header (a kernel, not a memset, so that a caller
// may capture the first call in a graph).
__global__ void k_clear_words(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The current device's scratch address (set up on the device's first call: the symbol's
// address and a clear of the header on `s`); nullptr on a HIP error.
void* device_scratch(hipStream_t s, hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || !ptr) return nullptr;
  hipLaunchKernelGGL(k_clear_words, dim3(1), dim3(256), 0, s, static_cast<uint32_t*>(ptr),
                     (int)(kHeaderBytes / 4));
  *err = hipGetLastError();
  if (*err != hipSuccess) return nullptr;
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

extern "C" {

size_t moe_packed_bytes(int32_t wfmt, int32_t rows, int32_t cols) {
  if (rows <= 0 || cols <= 0 || cols % 32 || rows % 16) return 0;
  if (wfmt != MOE_WFMT_MXFP4 && wfmt != MOE_WFMT_CB4 && wfmt != MOE_WFMT_MXFP4_PS && wfmt != MOE_WFMT_AFF3) return 0;
  if (wfmt == MOE_WFMT_AFF3)
    return cols % 128 ? 0 : align_up((size_t)rows * cols * 3 / 8, 256) + (size_t)rows * (cols / 64) * 4;
  const size_t code = (size_t)rows * cols / 2;
  const size_t nblk = (size_t)rows * cols / 32;
  if (wfmt == MOE_WFMT_MXFP4_PS) return align_up(code, 256) + (size_t)rows + nblk / 2;
  return align_up(code, 256) + nblk * (wfmt == MOE_WFMT_MXFP4 ? 1 : 2);
}

size_t moe_workspace_bytes(const moe_layer* L, int32_t T_max) {
  if (validate_layer(L) != MOE_OK || T_max < 0 || T_max > kMaxTokens) return 0;
  return layout_for(L, T_max).total;
}

int moe_router_topk(const moe_layer* L, const void* x, int32_t x_dtype, int32_t T, int32_t* topk_ids,
                    float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  int st = validate_layer(L);
  if (st) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;  // nothing is read or written; empty buffers may be NULL
  if (!x || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned4(topk_ids) || !aligned4(topk_w)) return MOE_ERR_ALIGNMENT;
  if ((st = check_ws(L, T, ws, ws_bytes))) return st;
  const Work w = carve(ws, layout_for(L, T));
  return hip_status(moeq::launch_router_topk(args_of(L), x, x_dtype, T, w, topk_ids, topk_w,
                                             static_cast<hipStream_t>(stream)));
}

int moe_bucket(const moe_layer* L, const int32_t* topk_ids, int32_t T, int32_t* counts, int32_t* offsets,
               int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  int st = validate_layer(L);
  if (st) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !counts || !offsets || !perm) return MOE_ERR_INVALID_ARG;
  if (!aligned4(topk_ids) || !aligned4(counts) || !aligned4(offsets) || !aligned4(perm)) return MOE_ERR_ALIGNMENT;
  if ((st = check_ws(L, T, ws, ws_bytes))) return st;
  const Work w = carve(ws, layout_for(L, T));
  return hip_status(moeq::launch_bucket(T, L->top_k, L->n_experts, L->has_shared, topk_ids, w, counts, offsets,
                                        perm, static_cast<hipStream_t>(stream)));
}

int moe_forward(const moe_layer* L, const void* x, int32_t x_dtype, int32_t T, float* y, void* ws,
                size_t ws_bytes, void* stream, int32_t path, int32_t* dbg_ids, float* dbg_w, int32_t* dbg_counts,
                int32_t* dbg_offsets, int32_t* dbg_perm) {
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  return forward_impl(L, x, x_dtype, T, y, ws, ws_bytes, stream, path, dbg_ids, dbg_w, dbg_counts, dbg_offsets,
                      dbg_perm, moeq::Timing());
}

int moe_forward_noalloc(const moe_layer* L, const void* x, int32_t x_dtype, int32_t T, float* y, void* stream,
                        int32_t path) {
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  int st = validate_layer(L);
  if (st) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (layout_for(L, T).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void* ws = device_scratch(static_cast<hipStream_t>(stream), &e);
  if (!ws) return MOE_ERR_HIP;
  return forward_impl(L, x, x_dtype, T, y, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, path, nullptr, nullptr, nullptr,
                      nullptr, nullptr, moeq::Timing());
}

int moe_forward_timed(const moe_layer* L, const void* x, int32_t x_dtype, int32_t T, float* y, void* ws,
                      size_t ws_bytes, void* stream, int32_t path, void* const* stage_events) {
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  moeq::Timing tm;
  tm.ev = stage_events;
  return forward_impl(L, x, x_dtype, T, y, ws, ws_bytes, stream, path, nullptr, nullptr, nullptr, nullptr,
                      nullptr, tm);
}

int moe_forward_rms(const moe_layer* L, const float* y_prev, float eps, int32_t residual, int32_t T, float* y,
                    void* ws, size_t ws_bytes, void* stream, int32_t path, void* const* stage_events) {
  if (!(eps >= 0.0f) || (residual != 0 && residual != 1)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && y_prev == y) return MOE_ERR_INVALID_ARG;
  moeq::Timing tm;
  tm.ev = stage_events;
  return forward_impl(L, y_prev, kRmsInput, T, y, ws, ws_bytes, stream, path, nullptr, nullptr, nullptr, nullptr,
                      nullptr, tm, eps, residual == 1);
}

int moe_dequant(int32_t wfmt, const void* packed, const int8_t* codebook, int32_t rows, int32_t cols, float* out,
                void* stream) {
  if (wfmt != MOE_WFMT_MXFP4 && wfmt != MOE_WFMT_CB4 && wfmt != MOE_WFMT_MXFP4_PS && wfmt != MOE_WFMT_AFF3)
    return MOE_ERR_INVALID_ARG;
  if (wfmt == MOE_WFMT_AFF3 && cols % 128) return MOE_ERR_INVALID_ARG;
  if (rows <= 0 || cols <= 0 || cols % 32 || rows % 16) return MOE_ERR_INVALID_ARG;
  if ((size_t)rows * (size_t)cols > ((size_t)1 << 34)) return MOE_ERR_UNSUPPORTED;
  if (!packed || !out) return MOE_ERR_INVALID_ARG;
  if (wfmt == MOE_WFMT_CB4 && !codebook) return MOE_ERR_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(out)) return MOE_ERR_ALIGNMENT;
  return hip_status(moeq::launch_dequant(wfmt, static_cast<const uint8_t*>(packed), codebook, rows, cols, out,
                                         static_cast<hipStream_t>(stream)));
}

int moe_dequant_grouped(int32_t wfmt, const void* packed, const int8_t* codebook, int32_t rows, int32_t cols,
                        float* out, void* stream) {
  if (wfmt != MOE_WFMT_CB4) return MOE_ERR_UNSUPPORTED;  // the grouped MXFP4 kernels decode nothing
  if (rows <= 0 || cols <= 0 || cols % 32 || rows % 16) return MOE_ERR_INVALID_ARG;
  if ((size_t)rows * (size_t)cols > ((size_t)1 << 34)) return MOE_ERR_UNSUPPORTED;
  if (!packed || !out || !codebook) return MOE_ERR_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(out)) return MOE_ERR_ALIGNMENT;
  return hip_status(moeq::launch_pf_dequant_cb4(static_cast<const uint8_t*>(packed), codebook, rows, cols, out,
                                                static_cast<hipStream_t>(stream)));
}

int moe_rms_rescale(const float* y, int32_t T, int32_t H, float eps, void* x_next_bf16, void* stream) {
  if (T < 0 || H <= 0 || !(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!y || !x_next_bf16) return MOE_ERR_INVALID_ARG;
  return hip_status(moeq::launch_rms_rescale(y, T, H, eps, static_cast<uint16_t*>(x_next_bf16),
                                             static_cast<hipStream_t>(stream)));
}

int moe_hbm_read_probe(const void* buf, size_t bytes, uint32_t* out, int32_t blocks, void* stream) {
  if (!buf || !out || bytes == 0 || bytes % 16 || blocks <= 0 || blocks > (1 << 20)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(buf) || !aligned4(out)) return MOE_ERR_ALIGNMENT;
  return hip_status(moeq::launch_read_probe(buf, bytes, out, blocks, static_cast<hipStream_t>(stream)));
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_ALIGNMENT: return "misaligned buffer";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
