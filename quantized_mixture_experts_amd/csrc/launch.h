// Host-side launchers of the kernels (one per kernel family).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include "device.h"

namespace moeq {

// Kernel stages of one forward call.  A stage whose work is fused into another
// kernel on the chosen path launches nothing and leaves its events untouched.
enum Stage {
  kStageRouter = 0, kStageTopk, kStageBucket, kStageGateUp, kStageDown, kStageCombine,
  kStageActQuant,  // fp8 activation planes of the block-scaled (MXFP4) prefill path
  kNumStages
};

// Optional start/stop events per stage, stamped by the dispatch packet itself
// (hipExtLaunchKernel), i.e. the kernel's own execution interval.
struct Timing {
  void* const* ev = nullptr;  // [2 * kNumStages] hipEvent_t, each may be null
  hipEvent_t start(int s) const { return ev ? static_cast<hipEvent_t>(ev[2 * s]) : nullptr; }
  hipEvent_t stop(int s) const { return ev ? static_cast<hipEvent_t>(ev[2 * s + 1]) : nullptr; }
};

// Plain launches when no events are requested (stream capture friendly); otherwise the
// dispatch packet carries the stage's start/stop events.
#define MOEQ_LAUNCH(tm, stage, kernel, grid, block, shmem, stream, ...)                                   \
  do {                                                                                                    \
    if ((tm).ev)                                                                                          \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, (tm).start(stage), (tm).stop(stage), 0,   \
                            __VA_ARGS__);                                                                 \
    else                                                                                                  \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                                \
  } while (0)

// K-split of the matrix-core router for small batches (up to 32 tokens fill one token
// tile, so the expert tiles alone would leave most CUs idle): each split writes partial
// logits [T][E+1] at logits + z * T * (E + 1), summed in z order by the top-k.
constexpr int kRouterMaxSplits = 8;  // the top-k loads at most this many partial sums
inline int router_splits(int T, int H) {
  if (T > 32) return 1;
  const int nch = H / 16;  // 16-column chunks
  return nch >= kRouterMaxSplits * 16 ? kRouterMaxSplits : (nch >= 4 * 16 ? 4 : 1);
}

// the matrix-core router alone: K-split partial logits [nsplit][T][E+1] in w.logits
hipError_t launch_router(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, hipStream_t s,
                         const Timing& tm = Timing());
hipError_t launch_router_topk(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w,
                              int32_t* dbg_ids, float* dbg_w, hipStream_t s,
                              const Timing& tm = Timing());
hipError_t launch_bucket(int T, int k, int E, int has_shared, const int32_t* ids, const Work& w,
                         int32_t* dbg_counts, int32_t* dbg_offsets, int32_t* dbg_perm, hipStream_t s,
                         const Timing& tm = Timing());
hipError_t launch_experts(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, float* y,
                          hipStream_t s, const Timing& tm = Timing());
// y[t] = sum_j g[t,j] o[t*k+j] (+ shared), fixed order, from the o rows in the workspace.
hipError_t launch_combine(const LayerArgs& L, int T, const Work& w, float* y, hipStream_t s, const Timing& tm);
// Decode path (T <= 32 and the activation tiles fit in LDS).  x_dtype 2: x is the previous
// layer's fp32 y and the layer's input is its bf16 RMS rescale with eps (written to w.xr).
bool decode_path_fits(const LayerArgs& L, int T, int x_dtype);
hipError_t launch_decode(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, float* y, float eps,
                         int32_t* dbg_ids, float* dbg_w, int32_t* dbg_counts, int32_t* dbg_offsets,
                         int32_t* dbg_perm, hipStream_t s, const Timing& tm);
// the grouped (prefill) CB4 kernels' decode table and lookup over a whole matrix
hipError_t launch_pf_dequant_cb4(const uint8_t* packed, const int8_t* codebook, int rows, int cols, float* out,
                                 hipStream_t s);
hipError_t launch_dequant(int wfmt, const uint8_t* packed, const int8_t* codebook, int rows, int cols,
                          float* out, hipStream_t s);
hipError_t launch_rms_rescale(const float* y, int T, int H, float eps, uint16_t* out, hipStream_t s);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t s);

}  // namespace moeq
