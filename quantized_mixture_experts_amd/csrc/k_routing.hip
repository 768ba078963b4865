// Router logits (fp64 accumulation), top-k with softmax gates, and the stable
// bucketing of (token, expert) pairs by expert.
//
// The router emits, per token, k expert ids and their normalised weights ("Nebula"
// page, "How it works"; "How Neural runs a 120-billion-parameter model on one gaming
// PC", "How one token and one prompt are processed").  Pairs are grouped by expert on
// the GPU, with no host synchronisation (NInfer Qwen3.8-Flash-Next page, MoE
// execution notes; the Neural page's "Prompt processing" counts a host-side routing
// sync among its costs, which this design avoids).
#include "device.h"
#include "launch.h"

namespace moeq {

// ---------------------------------------------------------------------------
// Router logits: l[t][e] = sum_h x[t][h] * W[e][h] + b[e].
// Products of an fp32 weight and an fp32/bf16 activation are exact in fp64 and are
// summed in fp64, so the result differs from any other fp64 summation order only
// in the last bits; ties and near-ties are then ordered the same way as a plain
// fp64 evaluation.  Row E (when a shared-gate vector exists) holds w_sg . x[t].
// A wave owns one expert row for a tile of kTokTile tokens.
// For fp32 activations the first block column also writes the exact 3-plane bf16
// split of x used by the MFMA kernels.
// ---------------------------------------------------------------------------
constexpr int kTokTile = 8;

template <int XDT>
__global__ __launch_bounds__(256) void k_router_logits(LayerArgs L, const void* __restrict__ x, int T,
                                                       int erows, double* __restrict__ logits,
                                                       uint16_t* __restrict__ xplanes) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wave;
  const int t0 = blockIdx.y * kTokTile;
  const int H = L.H;
  const int nt = min(kTokTile, T - t0);

  if (XDT == 0 && blockIdx.x == 0) {
    // exact split x = hi + mid + lo (each bf16) for the tokens of this tile
    const float* xf = (const float*)x;
    for (int idx = threadIdx.x; idx < nt * H; idx += blockDim.x) {
      const int t = t0 + idx / H, h = idx % H;
      const float v = xf[(size_t)t * H + h];
      const uint32_t p0 = f32_to_bf16_rne(v);
      const float r1 = v - bf16_bits_to_f32(p0);
      const uint32_t p1 = f32_to_bf16_rne(r1);
      const float r2 = r1 - bf16_bits_to_f32(p1);
      const uint32_t p2 = f32_to_bf16_rne(r2);
      const size_t o = (size_t)t * H + h;
      xplanes[o] = (uint16_t)p0;
      xplanes[(size_t)T * H + o] = (uint16_t)p1;
      xplanes[(size_t)2 * T * H + o] = (uint16_t)p2;
    }
  }
  if (e >= erows) return;

  const float* w = (e < L.E) ? L.router_w + (size_t)e * H : L.shared_gate_w;
  double acc[kTokTile];
#pragma unroll
  for (int t = 0; t < kTokTile; ++t) acc[t] = 0.0;

  for (int h = lane * 4; h < H; h += 4 * kWave) {
    const float4 wv = *(const float4*)(w + h);
#pragma unroll
    for (int t = 0; t < kTokTile; ++t) {
      if (t < nt) {
        float x0, x1, x2, x3;
        if (XDT == 0) {
          const float4 xv = *(const float4*)((const float*)x + (size_t)(t0 + t) * H + h);
          x0 = xv.x; x1 = xv.y; x2 = xv.z; x3 = xv.w;
        } else {
          const uint2 xb = *(const uint2*)((const uint16_t*)x + (size_t)(t0 + t) * H + h);
          x0 = bf16_bits_to_f32(xb.x & 0xFFFFu); x1 = bf16_bits_to_f32(xb.x >> 16);
          x2 = bf16_bits_to_f32(xb.y & 0xFFFFu); x3 = bf16_bits_to_f32(xb.y >> 16);
        }
        double a = acc[t];
        a = fma((double)wv.x, (double)x0, a);
        a = fma((double)wv.y, (double)x1, a);
        a = fma((double)wv.z, (double)x2, a);
        a = fma((double)wv.w, (double)x3, a);
        acc[t] = a;
      }
    }
  }
  const double bias = (e < L.E && L.router_b) ? (double)L.router_b[e] : 0.0;
#pragma unroll
  for (int t = 0; t < kTokTile; ++t) {
    const double s = wave_sum_f64(acc[t]);
    if (lane == 0 && t < nt) logits[(size_t)(t0 + t) * (L.E + 1) + e] = s + bias;
  }
}

// ---------------------------------------------------------------------------
// Top-k + softmax gates.  One wave per token; lane i holds experts i, i+64, ...
// Round j takes the largest remaining logit, ties to the lower index.
// g_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), in fp64, stored as fp32.
// Also writes the per-pair weights: pair_w[t*k+j] = g[t][j]; with a shared expert
// pair_w[T*k+t] = 1 or sigmoid(shared logit).
// ---------------------------------------------------------------------------
constexpr int kMaxEPerLane = 16;  // E <= 1024

__global__ __launch_bounds__(256) void k_topk(LayerArgs L, int T, const double* __restrict__ logits,
                                              int32_t* __restrict__ ids, float* __restrict__ pair_w,
                                              int32_t* __restrict__ dbg_ids, float* __restrict__ dbg_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int E = L.E, k = L.k;
  const double* lt = logits + (size_t)t * (E + 1);
  double v[kMaxEPerLane];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kMaxEPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? lt[e] : 0.0;
  }
  double lsel[16];
  int isel[16];
  for (int j = 0; j < k; ++j) {
    // local best: largest value, lowest index among equals (i ascending = index ascending)
    double bv = 0.0;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxEPerLane; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u)) {
        if (bi == 0x7FFFFFFF || v[i] > bv) { bv = v[i]; bi = e; }
      }
    }
    // wave argmax with the same order
    wave_argmax(bv, bi);
    lsel[j] = bv;
    isel[j] = bi;
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
  }
  if (lane == 0) {
    double z[16], sum = 0.0;
    for (int j = 0; j < k; ++j) { z[j] = exp(lsel[j] - lsel[0]); sum += z[j]; }
    for (int j = 0; j < k; ++j) {
      const float g = (float)(z[j] / sum);
      ids[t * k + j] = isel[j];
      pair_w[t * k + j] = g;
      if (dbg_ids) dbg_ids[t * k + j] = isel[j];
      if (dbg_w) dbg_w[t * k + j] = g;
    }
    if (L.has_shared) {
      float s = 1.0f;
      if (L.shared_gate_w) s = (float)(1.0 / (1.0 + exp(-lt[E])));
      pair_w[T * k + t] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Bucketing.  One block per bucket e in [0, E]; bucket E is the shared expert.
// Every block builds the full histogram of the routed ids in LDS, so each one knows
//   counts[e] = #{p : id_p = e}, offsets[e] = #{p : id_p < e},
//   its rank among the non-empty buckets (the active list), and
//   its first prefill work group (groups of up to kGroupPairs consecutive bucket
//   positions of one expert, numbered in bucket order),
// with no grid-wide scan.  perm[offsets[e] + r] = the r-th pair (increasing p) with
// id_p = e, by ballot compaction.  The result is deterministic.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bucket(int T, int k, int E, int has_shared,
                                                const int32_t* __restrict__ ids, int32_t* __restrict__ counts,
                                                int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                int32_t* __restrict__ active, int4* __restrict__ groups,
                                                int32_t* __restrict__ n_groups, int32_t* __restrict__ dbg_counts,
                                                int32_t* __restrict__ dbg_offsets, int32_t* __restrict__ dbg_perm) {
  __shared__ int hist[1024];
  __shared__ int red[5][4];
  __shared__ int wave_tot[4];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Pr = T * k;
  for (int i = tid; i < E; i += 256) hist[i] = 0;
  __syncthreads();
  for (int p = tid; p < Pr; p += 256) {
    const int id = ids[p];
    if (id >= 0 && id < E) atomicAdd(&hist[id], 1);
  }
  __syncthreads();
  // pairs, non-empty buckets and groups below e; non-empty buckets and groups overall
  int v[5] = {0, 0, 0, 0, 0};
  for (int i = tid; i < E; i += 256) {
    const int c = hist[i], ng = (c + kGroupPairs - 1) / kGroupPairs;
    if (i < e) { v[0] += c; v[1] += c > 0; v[2] += ng; }
    v[3] += c > 0;
    v[4] += ng;
  }
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const int r = wave_sum_i32(v[q]);
    if (lane == 0) red[q][wave] = r;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 5; ++q) v[q] = red[q][0] + red[q][1] + red[q][2] + red[q][3];
  const int lt = v[0], below = v[1], g_below = v[2], total = v[3], g_total = v[4];
  if (e == E) {
    const int cnt = has_shared ? T : 0;
    const int ngs = (cnt + kGroupPairs - 1) / kGroupPairs;
    if (tid == 0) {
      counts[E] = cnt; offsets[E] = Pr; offsets[E + 1] = Pr + cnt;
      active[0] = total + (cnt > 0);
      if (cnt > 0) active[1 + total] = E;
      *n_groups = g_total + ngs;
      if (dbg_counts) dbg_counts[E] = cnt;
      if (dbg_offsets) { dbg_offsets[E] = Pr; dbg_offsets[E + 1] = Pr + cnt; }
    }
    for (int i = tid; i < ngs; i += 256)
      groups[g_total + i] = make_int4(E, Pr + kGroupPairs * i, min(kGroupPairs, cnt - kGroupPairs * i), 0);
    for (int t = tid; t < cnt; t += 256) {
      perm[Pr + t] = Pr + t;
      if (dbg_perm) dbg_perm[Pr + t] = Pr + t;
    }
    return;
  }
  const int eq = hist[e];
  if (tid == 0) {
    counts[e] = eq; offsets[e] = lt;
    if (eq > 0) active[1 + below] = e;
    if (dbg_counts) dbg_counts[e] = eq;
    if (dbg_offsets) dbg_offsets[e] = lt;
  }
  if (eq == 0) return;
  const int ng = (eq + kGroupPairs - 1) / kGroupPairs;
  for (int i = tid; i < ng; i += 256)
    groups[g_below + i] = make_int4(e, lt + kGroupPairs * i, min(kGroupPairs, eq - kGroupPairs * i), 0);
  int running = 0;
  for (int base = 0; base < Pr; base += 256) {
    const int p = base + tid;
    const bool flag = p < Pr && ids[p] == e;
    const uint64_t m = __ballot(flag);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) wave_tot[wave] = __popcll(m);
    __syncthreads();
    int woff = 0;
    for (int w = 0; w < wave; ++w) woff += wave_tot[w];
    if (flag) {
      const int pos = lt + running + woff + before;
      perm[pos] = p;
      if (dbg_perm) dbg_perm[pos] = p;
    }
    running += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
hipError_t launch_router_topk(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w,
                              int32_t* dbg_ids, float* dbg_w, hipStream_t s, const Timing& tm) {
  const int erows = L.E + ((L.has_shared && L.shared_gate_w) ? 1 : 0);
  dim3 grid((erows + 3) / 4, (T + kTokTile - 1) / kTokTile);
  if (x_dtype == 0)
    MOEQ_LAUNCH(tm, kStageRouter, k_router_logits<0>, grid, dim3(256), 0, s, L, x, T, erows, w.logits, w.xplanes);
  else
    MOEQ_LAUNCH(tm, kStageRouter, k_router_logits<1>, grid, dim3(256), 0, s, L, x, T, erows, w.logits, w.xplanes);
  MOEQ_LAUNCH(tm, kStageTopk, k_topk, dim3((T + 3) / 4), dim3(256), 0, s, L, T, (const double*)w.logits, w.ids,
              w.pair_w, dbg_ids, dbg_w);
  return hipGetLastError();
}

hipError_t launch_bucket(int T, int k, int E, int has_shared, const int32_t* ids, const Work& w,
                         int32_t* dbg_counts, int32_t* dbg_offsets, int32_t* dbg_perm, hipStream_t s,
                         const Timing& tm) {
  MOEQ_LAUNCH(tm, kStageBucket, k_bucket, dim3(E + 1), dim3(256), 0, s, T, k, E, has_shared, ids, w.counts,
              w.offsets, w.perm, w.active, w.groups, w.n_groups, dbg_counts, dbg_offsets, dbg_perm);
  return hipGetLastError();
}

}  // namespace moeq
