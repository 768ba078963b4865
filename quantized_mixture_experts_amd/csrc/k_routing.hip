// Router logits (fp64 accumulation), top-k with softmax gates, and the stable
// bucketing of (token, expert) pairs by expert.
//
// The router emits, per token, k expert ids and their normalised weights ("Nebula"
// page, "How it works"; "How Neural runs a 120-billion-parameter model on one gaming
// PC", "How one token and one prompt are processed").  The device sorts the pairs into
// per-expert groups itself, with no host synchronisation (NInfer Qwen3.8-Flash-Next page, MoE
// execution notes; the Neural page's "Prompt processing" counts a host-side routing
// sync among its costs, which this design avoids).
#include "device.h"
#include "launch.h"

namespace moeq {

// ---------------------------------------------------------------------------
// Router logits for larger batches on the fp64 matrix cores (v_mfma_f64_16x16x4f64:
// lane l supplies A[l%16][l/16] and B[l/16][l%16] and holds D[4r + l/16][l%16]).
// A = activations (tokens x k), B = router rows (k x experts); every product of a
// bf16/fp32 activation and an fp32 weight is exact in fp64 and the matrix core sums in
// fp64, so only the summation order differs from a plain fp64 loop.
// Block: 32 tokens x 16 expert rows; its 8 waves (two per SIMD, so that one wave's
// loads are in flight while the other's MFMAs run) split K in 16-column chunks (wave w
// takes chunks w, w+8, ...) and are summed in wave order.  Each lane loads 4
// consecutive k of its token rows and its expert row; MFMA step q pairs element q of
// both, so a chunk's 4 steps cover its 16 columns.  Row E (with a shared-gate vector)
// is w_sg.  Blocks of the first expert tile also write the exact 3-plane bf16 split of
// fp32 x used by the projections.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) double f64x4_t;

constexpr int kRouterWaves = 8;

template <int XDT>
__global__ __launch_bounds__(64 * kRouterWaves) void k_router_mfma(LayerArgs L, const void* __restrict__ x, int T,
                                                                  int erows, double* __restrict__ logits,
                                                                  uint16_t* __restrict__ xplanes) {
  __shared__ double red[kRouterWaves - 1][2][4][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, kk = lane >> 4;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 16;
  const int H = L.H;
  const int z = blockIdx.z, nsplit = gridDim.z;  // this block's share of the 16-column chunks

  if (XDT == 0 && blockIdx.y == 0 && z == 0) {
    const float* xf = (const float*)x;
    const int nt = min(32, T - t0);
    for (int idx = threadIdx.x; idx < nt * H; idx += 64 * kRouterWaves) {
      const size_t o = (size_t)t0 * H + idx;
      const float v = xf[o];
      const uint32_t p0 = f32_to_bf16_rne(v);
      const float r1 = v - bf16_bits_to_f32(p0);
      const uint32_t p1 = f32_to_bf16_rne(r1);
      const uint32_t p2 = f32_to_bf16_rne(r1 - bf16_bits_to_f32(p1));
      xplanes[o] = (uint16_t)p0;
      xplanes[(size_t)T * H + o] = (uint16_t)p1;
      xplanes[(size_t)2 * T * H + o] = (uint16_t)p2;
    }
  }
  // this lane's rows (clamped into range; clamped results are not stored)
  const int ta = min(t0 + i, T - 1), tb = min(t0 + 16 + i, T - 1);
  const int e = e0 + i;
  const float* wrow = e < L.E ? L.router_w + (size_t)e * H : (e < erows ? L.shared_gate_w : L.router_w);
  f64x4_t acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
  const int nch = H >> 4;
  const int ch_beg = z * nch / nsplit, ch_end = (z + 1) * nch / nsplit;
#pragma unroll 4
  for (int ch = ch_beg + wave; ch < ch_end; ch += kRouterWaves) {
    const int k = 16 * ch + 4 * kk;
    double a0[4], a1[4], b[4];
    const float4 wv = *(const float4*)(wrow + k);
    b[0] = wv.x; b[1] = wv.y; b[2] = wv.z; b[3] = wv.w;
    if (XDT == 0) {
      const float4 xa = *(const float4*)((const float*)x + (size_t)ta * H + k);
      const float4 xb = *(const float4*)((const float*)x + (size_t)tb * H + k);
      a0[0] = xa.x; a0[1] = xa.y; a0[2] = xa.z; a0[3] = xa.w;
      a1[0] = xb.x; a1[1] = xb.y; a1[2] = xb.z; a1[3] = xb.w;
    } else {
      const uint2 xa = *(const uint2*)((const uint16_t*)x + (size_t)ta * H + k);
      const uint2 xb = *(const uint2*)((const uint16_t*)x + (size_t)tb * H + k);
      a0[0] = bf16_bits_to_f32(xa.x & 0xFFFFu); a0[1] = bf16_bits_to_f32(xa.x >> 16);
      a0[2] = bf16_bits_to_f32(xa.y & 0xFFFFu); a0[3] = bf16_bits_to_f32(xa.y >> 16);
      a1[0] = bf16_bits_to_f32(xb.x & 0xFFFFu); a1[1] = bf16_bits_to_f32(xb.x >> 16);
      a1[2] = bf16_bits_to_f32(xb.y & 0xFFFFu); a1[3] = bf16_bits_to_f32(xb.y >> 16);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0[q], b[q], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1[q], b[q], acc1, 0, 0, 0);
    }
  }
  // the fp64 matrix-core results settle before any read (its latency is not measured here:
  // twice the 24-cycle wait)
  mfma_settle(acc0, acc1);
  mfma_settle(acc0, acc1);
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) { red[wave - 1][0][r][lane] = acc0[r]; red[wave - 1][1][r][lane] = acc1[r]; }
  }
  __syncthreads();
  if (wave == 0) {
    const int col = e0 + i;  // expert of this lane's outputs
    const double bias = (z == 0 && col < L.E && L.router_b) ? (double)L.router_b[col] : 0.0;
    double* out = logits + (size_t)z * T * (L.E + 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      double s0 = acc0[r], s1 = acc1[r];
#pragma unroll
      for (int v = 0; v < kRouterWaves - 1; ++v) {
        s0 += red[v][0][r][lane];
        s1 += red[v][1][r][lane];
      }
      const int row = 4 * r + kk;  // token within the 16-token tile
      if (col < erows) {
        if (t0 + row < T) out[(size_t)(t0 + row) * (L.E + 1) + col] = s0 + bias;
        if (t0 + 16 + row < T) out[(size_t)(t0 + 16 + row) * (L.E + 1) + col] = s1 + bias;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k + softmax gates.  One wave per token (the per-lane sorted candidates of
// topk_tokens, ties to the lower index); lane j < k computes exp(l_j - l_0) and a wave
// sum normalises them: g_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), in fp64, stored as
// fp32.  Also the per-pair weights: pair_w[t*k+j] = g[t][j]; with a shared expert
// pair_w[T*k+t] = 1 or sigmoid(shared logit).
// ---------------------------------------------------------------------------
template <int NPER>
__device__ __forceinline__ void topk_one(const double* logits, int E, int k, int t, int* s_exp, double* s_l,
                                         int nsplit, size_t split_stride) {
  const int tok[1] = {t}, slot[1] = {0};
  if (nsplit == 1) topk_tokens<NPER, 1, false, 1>(logits, E, k, tok, slot, s_exp, s_l);
  else topk_tokens<NPER, 1, false, kRouterMaxSplits>(logits, E, k, tok, slot, s_exp, s_l, nsplit, split_stride);
}

__global__ __launch_bounds__(256) void k_topk(LayerArgs L, int T, const double* __restrict__ logits, int nsplit,
                                              int32_t* __restrict__ ids, float* __restrict__ pair_w,
                                              int32_t* __restrict__ dbg_ids, float* __restrict__ dbg_w) {
  __shared__ int s_exp[4][16];
  __shared__ double s_l[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // no block-wide synchronisation below
  const int E = L.E, k = L.k;
  const size_t sstride = (size_t)T * (E + 1);
  const int nper = (E + 63) >> 6;
  if (nper <= 1) topk_one<1>(logits, E, k, t, s_exp[wave], s_l[wave], nsplit, sstride);
  else if (nper <= 2) topk_one<2>(logits, E, k, t, s_exp[wave], s_l[wave], nsplit, sstride);
  else if (nper <= 4) topk_one<4>(logits, E, k, t, s_exp[wave], s_l[wave], nsplit, sstride);
  else if (nper <= 8) topk_one<8>(logits, E, k, t, s_exp[wave], s_l[wave], nsplit, sstride);
  else topk_one<16>(logits, E, k, t, s_exp[wave], s_l[wave], nsplit, sstride);
  float g;
  const bool keep = pair_gate(s_l[wave][min(lane, k - 1)], s_l[wave][0], k, L.omit_below, &g);
  if (lane < k) {
    const int id = keep ? s_exp[wave][lane] : -1;  // an omitted pair is in no bucket
    ids[t * k + lane] = id;
    pair_w[t * k + lane] = g;
    if (dbg_ids) dbg_ids[t * k + lane] = id;
    if (dbg_w) dbg_w[t * k + lane] = g;
  }
  if (L.has_shared && lane == 0) {
    float s = 1.0f;
    if (L.shared_gate_w) {
      double pz[kRouterMaxSplits];  // every split loaded first (clamped index), added in order
#pragma unroll
      for (int z = 0; z < kRouterMaxSplits; ++z) pz[z] = logits[(size_t)min(z, nsplit - 1) * sstride + (size_t)t * (E + 1) + E];
      double ls = pz[0];
#pragma unroll
      for (int z = 1; z < kRouterMaxSplits; ++z) ls = z < nsplit ? ls + pz[z] : ls;
      s = (float)(1.0 / (1.0 + exp(-ls)));
    }
    pair_w[T * k + t] = s;
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
// Each of the 16 waves scans its own contiguous range of pairs, 8 loads in flight per
// lane (the ids are read in two passes, histogram and placement).
constexpr int kBucketWaves = 16;
constexpr int kBucketBatch = 8;

// ids of pairs base + 64 u + lane (u < kBucketBatch), -1 past the wave's range end p1
// (loads clamped to the last pair, so every load is in bounds).
__device__ __forceinline__ void bucket_load(const int32_t* __restrict__ ids, int base, int p1, int Pr,
                                            int (&id)[kBucketBatch]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kBucketBatch; ++u) {
    const int p = base + 64 * u + lane;
    const int v = ids[min(p, Pr - 1)];
    id[u] = p < p1 ? v : -1;
  }
}

__global__ __launch_bounds__(64 * kBucketWaves) void k_bucket(int T, int k, int E, int has_shared,
                                                const int32_t* __restrict__ ids, int32_t* __restrict__ counts,
                                                int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                int32_t* __restrict__ active, int4* __restrict__ groups,
                                                int32_t* __restrict__ n_groups, int32_t* __restrict__ dbg_counts,
                                                int32_t* __restrict__ dbg_offsets, int32_t* __restrict__ dbg_perm) {
  constexpr int NT = 64 * kBucketWaves;
  __shared__ int hist[1024];
  __shared__ int red[6][kBucketWaves];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Pr = T * k;
  // each wave owns the contiguous pair range [wave * chunk, (wave + 1) * chunk)
  const int chunk = ((Pr + kBucketWaves - 1) / kBucketWaves + 63) / 64 * 64;
  const int p0 = wave * chunk, p1 = min(Pr, p0 + chunk);
  for (int i = tid; i < E; i += NT) hist[i] = 0;
  __syncthreads();
  int mine = 0;  // pairs of this wave's range routed to e
  for (int base = p0; base < p1; base += 64 * kBucketBatch) {
    int id[kBucketBatch];
    bucket_load(ids, base, p1, Pr, id);
#pragma unroll
    for (int u = 0; u < kBucketBatch; ++u) {
      if (id[u] >= 0 && id[u] < E) atomicAdd(&hist[id[u]], 1);
      mine += __popcll(__ballot(id[u] == e));
    }
  }
  if (lane == 0) red[5][wave] = mine;
  __syncthreads();
  // pairs, non-empty buckets and groups below e; non-empty buckets and groups overall
  int v[5] = {0, 0, 0, 0, 0};
  for (int i = tid; i < E; i += NT) {
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
  for (int q = 0; q < 5; ++q) {
    int acc = 0;
#pragma unroll
    for (int w2 = 0; w2 < kBucketWaves; ++w2) acc += red[q][w2];
    v[q] = acc;
  }
  const int lt = v[0], below = v[1], g_below = v[2], total = v[3], g_total = v[4];
  if (e == E) {
    const int cnt = has_shared ? T : 0;
    const int ngs = (cnt + kGroupPairs - 1) / kGroupPairs;
    // lt = the routed pairs placed in buckets 0 .. E-1 (all Pr, unless some were omitted)
    if (tid == 0) {
      counts[E] = cnt; offsets[E] = lt; offsets[E + 1] = lt + cnt;
      active[0] = total + (cnt > 0);
      if (cnt > 0) active[1 + total] = E;
      *n_groups = g_total + ngs;
      if (dbg_counts) dbg_counts[E] = cnt;
      if (dbg_offsets) { dbg_offsets[E] = lt; dbg_offsets[E + 1] = lt + cnt; }
    }
    for (int i = tid; i < ngs; i += NT)
      groups[g_total + i] = make_int4(E, lt + kGroupPairs * i, min(kGroupPairs, cnt - kGroupPairs * i), 0);
    for (int t = tid; t < cnt; t += NT) {
      perm[lt + t] = Pr + t;
      if (dbg_perm) dbg_perm[lt + t] = Pr + t;
    }
    for (int i = lt + cnt + tid; i < Pr + cnt; i += NT) {  // past the placed pairs
      perm[i] = -1;
      if (dbg_perm) dbg_perm[i] = -1;
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
  for (int i = tid; i < ng; i += NT)
    groups[g_below + i] = make_int4(e, lt + kGroupPairs * i, min(kGroupPairs, eq - kGroupPairs * i), 0);
  // stable positions: earlier waves' matches, then this wave's in increasing p
  int pos = lt;
  for (int w2 = 0; w2 < wave; ++w2) pos += red[5][w2];
  if (red[5][wave] == 0) return;
  for (int base = p0; base < p1; base += 64 * kBucketBatch) {
    int id[kBucketBatch];
    bucket_load(ids, base, p1, Pr, id);
#pragma unroll
    for (int u = 0; u < kBucketBatch; ++u) {
      const bool flag = id[u] == e;
      const uint64_t m = __ballot(flag);
      if (flag) {
        const int at = pos + __popcll(m & ((1ull << lane) - 1ull));
        const int p = base + 64 * u + lane;
        perm[at] = p;
        if (dbg_perm) dbg_perm[at] = p;
      }
      pos += __popcll(m);
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
hipError_t launch_router(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, hipStream_t s,
                         const Timing& tm) {
  const int erows = L.E + ((L.has_shared && L.shared_gate_w) ? 1 : 0);
  const int nsplit = router_splits(T, L.H);
  dim3 grid((T + 31) / 32, (erows + 15) / 16, nsplit);
  if (x_dtype == 0)
    MOEQ_LAUNCH(tm, kStageRouter, k_router_mfma<0>, grid, dim3(64 * kRouterWaves), 0, s, L, x, T, erows, w.logits, w.xplanes);
  else
    MOEQ_LAUNCH(tm, kStageRouter, k_router_mfma<1>, grid, dim3(64 * kRouterWaves), 0, s, L, x, T, erows, w.logits, w.xplanes);
  return hipGetLastError();
}

hipError_t launch_router_topk(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w,
                              int32_t* dbg_ids, float* dbg_w, hipStream_t s, const Timing& tm) {
  hipError_t e = launch_router(L, x, x_dtype, T, w, s, tm);
  if (e != hipSuccess) return e;
  MOEQ_LAUNCH(tm, kStageTopk, k_topk, dim3((T + 3) / 4), dim3(256), 0, s, L, T, (const double*)w.logits,
              router_splits(T, L.H), w.ids, w.pair_w, dbg_ids, dbg_w);
  return hipGetLastError();
}

hipError_t launch_bucket(int T, int k, int E, int has_shared, const int32_t* ids, const Work& w,
                         int32_t* dbg_counts, int32_t* dbg_offsets, int32_t* dbg_perm, hipStream_t s,
                         const Timing& tm) {
  MOEQ_LAUNCH(tm, kStageBucket, k_bucket, dim3(E + 1), dim3(64 * kBucketWaves), 0, s, T, k, E, has_shared, ids,
              w.counts, w.offsets, w.perm, w.active, w.groups, w.n_groups, dbg_counts, dbg_offsets, dbg_perm);
  return hipGetLastError();
}

}  // namespace moeq
