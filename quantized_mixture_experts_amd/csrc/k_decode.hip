// Decode path (few tokens per call, e.g. a draft/verify window of up to 17 tokens):
//   1. routing, by token count:
//      - one token: k_dec_rr computes the router logits (one expert row per block) and
//        stores them; every gate/up block of step 2 takes the top-k of those logits
//        itself (the same selection in every block) and routes, so no route kernel runs;
//      - 2..7 tokens: k_dec_rr also routes: every block posts its logits and then checks
//        once whether all of them are there; a block that sees them all does the top-k
//        + gates, the stable bucketing of the pairs and the active-expert slot records,
//        and clears the per-tile arrival counters of step 3;
//      - 8 tokens and more: the K-split matrix-core router, then k_dec_topk_route (one
//        wave per token for the top-k; the last block to finish routes).
//   2. k_dec_gateup:   fused dequant + gate/up + SwiGLU per (16-row tile, active expert).
//   3. k_dec_down / k_dec_down_rows: dequant + down per (row tile, active expert); the
//                      last block to finish a tile sums the gate-weighted expert outputs
//                      of that tile in a fixed order (routed j ascending, then shared),
//                      so no float atomics and a run-to-run identical result (NInfer
//                      Qwen3.8-Flash-Next page, MoE execution notes: a token's down
//                      projection runs over all of its experts, and the weighted sum is
//                      formed so that it does not depend on which expert finishes first).
// Each selected expert's weights are streamed from HBM once per call for all of its
// tokens (same page and notes: the pairs are grouped by expert so that an expert's rows
// are read in one pass); an expert whose tokens exceed one LDS staging pass streams them
// once per pass.  Weight loads for a wave's whole K range are
// issued before the first MFMA so that a wave keeps its full share of HBM requests in
// flight.
// No block ever waits for another: a block that needs the results of others checks
// once, after its own results have landed, and leaves the work to a later block when
// something is missing.  The last block to check sees everything, so the work is always
// done, whatever blocks the GPU keeps resident together.
#include "device.h"
#include "launch.h"

namespace moeq {

// From this many tokens the decode path routes with two kernels (the matrix-core router,
// then the per-token top-k with the route) instead of the single router/route kernel,
// whose fp64 reductions and one-CU top-k grow with T.
constexpr int kDecSplitRouteT = 8;
// bf16 elements of the rescaled rows a router block keeps in LDS when it folds the RMS
// rescale in (T * H at most: 48 KB)
constexpr int kRmsFoldElems = 24576;

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory
// operations of this wave are outstanding, leaving the other counters alone.
constexpr int waitcnt_vm_le(int n) {
  return (n > 63 ? 63 : n) & 15 | (7 << 4) | (15 << 8) | (((n > 63 ? 63 : n) >> 4) << 14);
}
// The same, also waiting for all of this wave's LDS stores and scalar loads (lgkmcnt 0):
// the barrier after it does not wait for memory by itself.
constexpr int waitcnt_vm_le_lgkm0(int n) { return waitcnt_vm_le(n) & ~(15 << 8); }
// vector-memory instructions one prefetch_step issues per 16-row tile: MXFP4 one 16-byte
// code load and one scale byte (the packed scale store: one delta byte); CB4 one 16-byte
// code load and one 8-byte load of the row's four fp16 scales (a last step of fewer than
// four blocks: four 2-byte scale loads, so more, never fewer); 3-bit affine one 12-byte
// code load and one 8-byte (scale, bias) load.  The waits after the staging loads count
// on at least these: the code and scale loads of a step read different planes, so the
// compiler cannot merge them into one instruction.
template <int FMT>
constexpr int loads_per_step() { return 2; }
constexpr int kDecMaxTokens = 32;  // two 16-slot MFMA token tiles

__device__ __forceinline__ int dec_token_of_pair(int p, int T, int k) { return p < T * k ? p / k : p - T * k; }

// padded LDS row stride (in bf16 elements) with (stride/2) % 64 == 4 dwords
__host__ __device__ __forceinline__ int lds_row_stride(int K) {
  int dw = K / 2;
  int pad = (4 - (dw % 64) + 64) % 64;
  return 2 * (dw + pad);
}

// ---------------------------------------------------------------------------
// 1+2. Router and route in one kernel.  Each 1024-thread block computes 4 expert rows
// of router logits (4 waves per row split its columns; all tokens; fp64 accumulation
// of exact products, partial sums added in a fixed order) and writes them through to
// the device-coherent level; without the route (one token) a block computes one row
// with its 16 waves.  Each block then checks once whether every logit has
// arrived; a block that sees them all does the top-k, the softmax gates and the
// bucketing:
//    top-k: one wave per token, k rounds of a wave argmax (ties to the lower index);
//    gates: lane j < k computes exp(l_j - l_0), a wave sum normalises them (fp64);
//    buckets: integer counts, one wave-scan over the E+1 buckets of the packed pair
//    (count, non-empty flag), then each pair's stable rank among earlier pairs of
//    the same expert; one slot record per active expert for the projections.
// The mailbox entries and arrival flags live in the workspace's fixed header; the routing
// block clears them, so they read zero at the start of every call once the header was
// zeroed before the first use.
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 1024;
// Expert rows per router block: 4 (4 waves each) when the block also routes, 1 (16 waves
// splitting the row) when it only stores the logits, so that the W_r stream of one token
// spreads over E + 1 CUs instead of a quarter of them (each CU keeps only so many
// requests in flight).
template <bool ROUTE>
constexpr int router_rows() { return ROUTE ? 4 : 1; }
constexpr int kMaxPairsDec = kDecMaxTokens * 16 + kDecMaxTokens;

// Top-k of the tokens a wave takes (t0, and t1 when below T) from the logit mailbox,
// where the blocks of this kernel post each logit l as ~bits(l) (0: not posted yet).
// Every wave of the block loads its tokens' entries once (and lane 0 the shared-gate
// logit, column E, when want_sg); if any is missing the block leaves the routing to a
// later block and false is returned, uniformly over the block.  Otherwise the entries are
// cleared for the next call and the selections written: s_exp/s_l[t * k + j], and the
// shared-gate logit to s_sg[t].  Every wave of the block calls this (one barrier each).
template <int NPER>
__device__ __forceinline__ bool topk_mbox(uint64_t* __restrict__ mbox, int E, int k, int T, int t0, int t1,
                                          bool want_sg, int* s_flag, int* s_exp, double* s_l, double* s_sg) {
  const int lane = threadIdx.x & 63;
  const int nt = t1 < T ? 2 : (t0 < T ? 1 : 0);  // wave-uniform
  const int tok[2] = {t0, t1};
  uint64_t raw[2][NPER], sgr[2] = {1ull, 1ull};
  bool missing = false;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t < nt) {
      const uint64_t* row = mbox + (size_t)tok[t] * (E + 1);
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const int e = lane + 64 * i;
        raw[t][i] = __hip_atomic_load(row + min(e, E - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        missing |= e < E && raw[t][i] == 0ull;
      }
      if (want_sg && lane == 0) {
        sgr[t] = __hip_atomic_load(row + E, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        missing |= sgr[t] == 0ull;
      }
    }
  }
  if (__ballot(missing) != 0ull && lane == 0) *s_flag = 1;
  __syncthreads();
  if (*s_flag) return false;
  double lv[2][NPER];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t < nt) {
      uint64_t* row = mbox + (size_t)tok[t] * (E + 1);
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const int e = lane + 64 * i;
        lv[t][i] = __builtin_bit_cast(double, ~raw[t][i]);
        if (e < E) __hip_atomic_store(row + e, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (want_sg && lane == 0) {
        __hip_atomic_store(row + E, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_sg[tok[t]] = __builtin_bit_cast(double, ~sgr[t]);
      }
    }
  }
  if (nt == 2) {
    topk_select<NPER, 2>(lv, E, k, tok, s_exp, s_l);
  } else if (nt == 1) {
    double lw[1][NPER];
    const int tk[1] = {t0};
#pragma unroll
    for (int i = 0; i < NPER; ++i) lw[0][i] = lv[0][i];
    topk_select<NPER, 1>(lw, E, k, tk, s_exp, s_l);
  }
  return true;
}

// Top-k of the tokens a wave takes from the logits in memory (written by other blocks of
// this kernel and known to be complete).
template <int NPER>
__device__ __forceinline__ void topk_wave(const double* __restrict__ logits, int E, int k, int T, int t0, int t1,
                                          int* s_exp, double* s_l) {
  if (t1 < T) {
    const int tok[2] = {t0, t1};
    topk_tokens<NPER, 2, true>(logits, E, k, tok, tok, s_exp, s_l);
  } else if (t0 < T) {
    const int tok[1] = {t0};
    topk_tokens<NPER, 1, true>(logits, E, k, tok, tok, s_exp, s_l);
  }
}

// Partial logits of one expert row for all T tokens over the columns [h0, h1), by one
// wave: sum_h x[t][h] w[h] in fp64 (every product exact).  Branch-free: each lane loads
// its kPer 4-column chunks of the row once per chunk pass (addresses clamped into the
// row, values past it masked at use) together with the activation chunks of the first
// kTB tokens (token index clamped), so a pass starts with one round trip for all its
// loads.  part[t] receives the wave's sum for token t (summed over passes in order).
template <int XDT>
struct RouterX;
template <>
struct RouterX<0> {  // fp32 activations
  using chunk = f32x4_t;
  __device__ static chunk load(const void* x, size_t off) {
    return *(const __attribute__((address_space(1))) f32x4_t*)((const float*)x + off);
  }
  __device__ static float get(const chunk& c, int q) { return c[q]; }
};
template <>
struct RouterX<1> {  // bf16 activations
  using chunk = uint64_t;
  __device__ static chunk load(const void* x, size_t off) {
    return *(const __attribute__((address_space(1))) uint64_t*)((const uint16_t*)x + off);
  }
  __device__ static float get(const chunk& c, int q) { return bf16_bits_to_f32((uint32_t)(c >> (16 * q)) & 0xFFFFu); }
};

// Activation chunk of token u at column c.  XDT 2: x is the block's LDS copy of the bf16
// RMS rescale of the previous layer's y.
template <int XDT>
__device__ __forceinline__ typename RouterX<XDT == 2 ? 1 : XDT>::chunk router_x(const void* x, int u, int H, int c) {
  if constexpr (XDT == 2) {
    return *(const uint64_t*)((const uint16_t*)x + (size_t)u * H + c);
  } else {
    return RouterX<XDT>::load(x, (size_t)u * H + c);
  }
}

// float4 chunks of W_r per lane and pass: a 2880-column row's quarter (4 waves a row) or
// sixteenth (16 waves a row) in one pass
template <bool ROUTE>
constexpr int router_per() { return ROUTE ? 3 : 1; }

// The first pass's router-weight chunks of this lane (issued early, e.g. before the RMS
// rescale that the activations need).
template <int KPER>
__device__ __forceinline__ void router_w_first(const float* __restrict__ wrow, int h0, int h1,
                                               f32x4_t (&wv)[KPER]) {
  const int lane = threadIdx.x & 63;
  const int c_beg = h0 / 4, c_end = h1 / 4;
#pragma unroll
  for (int i = 0; i < KPER; ++i) {
    const int c = max(c_beg, min(c_beg + lane + 64 * i, c_end - 1));
    wv[i] = c_end > c_beg ? *(const __attribute__((address_space(1))) f32x4_t*)(wrow + 4 * c) : f32x4_t{0, 0, 0, 0};
  }
}

template <int XDT, int KPER>
__device__ __forceinline__ void router_part(const float* __restrict__ wrow, const void* __restrict__ x, int T, int H,
                                            int h0, int h1, double* __restrict__ part, const f32x4_t (&wfirst)[KPER]) {
  using RX = RouterX<XDT == 2 ? 1 : XDT>;
  const int lane = threadIdx.x & 63;
  constexpr int kPer = KPER;
  constexpr int kTB = 4;
  const int c_beg = h0 / 4, c_end = h1 / 4;
  if (c_end <= c_beg) {
    if (lane == 0)
      for (int t = 0; t < T; ++t) part[t] = 0.0;
    return;
  }
  for (int c0 = c_beg; c0 < c_end; c0 += 64 * kPer) {
    f32x4_t wv[kPer];
    int cc[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      cc[i] = min(c0 + lane + 64 * i, c_end - 1);
      wv[i] = c0 == c_beg ? wfirst[i] : *(const __attribute__((address_space(1))) f32x4_t*)(wrow + 4 * cc[i]);
    }
    typename RX::chunk xq[kTB][kPer];
#pragma unroll
    for (int u = 0; u < kTB; ++u)
      if (u < T) {  // uniform; the block's loads share one CU's address unit
#pragma unroll
        for (int i = 0; i < kPer; ++i) xq[u][i] = router_x<XDT>(x, u, H, 4 * cc[i]);
      }
    for (int t0 = 0; t0 < T; t0 += kTB) {
#pragma unroll
      for (int u = 0; u < kTB; ++u) {
        // token slots past T are skipped (uniform): the waves of a SIMD run their fp64
        // sums one after another, so dead slots would lengthen every block
        if (t0 + u >= T) break;
        double a = 0.0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const bool ok = c0 + lane + 64 * i < c_end;
#pragma unroll
          for (int q = 0; q < 4; ++q) a = fma(ok ? (double)wv[i][q] : 0.0, (double)RX::get(xq[u][i], q), a);
        }
        const double sum = wave_sum_f64(a);
        if (lane == 0 && t0 + u < T) part[t0 + u] = c0 == c_beg ? sum : part[t0 + u] + sum;
      }
#pragma unroll
      for (int u = 0; u < kTB; ++u)
        if (t0 + kTB + u < T) {
#pragma unroll
          for (int i = 0; i < kPer; ++i) xq[u][i] = router_x<XDT>(x, t0 + kTB + u, H, 4 * cc[i]);
        }
    }
  }
}

// Expert pointers of the buckets e = tid + u blockDim.x (u < NPP) a thread of the routing
// block writes slot records for, loaded before they are needed (at most 1,025 buckets:
// NPP blockDim.x must cover them).
template <int NPP>
struct BucketPtrs {
  const uint8_t* gu[NPP];
  const uint8_t* dn[NPP];
};
template <int NPP>
__device__ __forceinline__ void load_bucket_ptrs(const LayerArgs& L, BucketPtrs<NPP>& bp) {
  const int last = L.E + (L.has_shared ? 1 : 0) - 1;
#pragma unroll
  for (int u = 0; u < NPP; ++u) {
    const int ie = min((int)threadIdx.x + u * (int)blockDim.x, last);
    bp.gu[u] = L.gate_up[ie];
    bp.dn[u] = L.down[ie];
  }
}

// Routing after top-k (s_exp[p] = the expert of pair p for p < P, s_cnt zeroed): LDS
// histogram, scan and stable ranks -> counts, offsets, perm, the active list and one slot
// record per active expert.  Every thread of the block takes part (any block size with
// NPP blockDim.x > E).
// s_tmask[e] (zeroed with s_cnt): bit t set when token t has a pair in bucket e (T <= 32).
// A token's routed experts are distinct, so the stable rank of pair p (of token t) in its
// bucket, the number of earlier pairs in the same bucket, is the number of earlier tokens
// in it: popcount(s_tmask[e] & (2^t - 1)).
// The gate/up work items: pass j of an active expert (its pairs j xg .. j xg + xg - 1) is
// item record w.items[q] with the expert's passes on consecutive q, in expert order, and
// *w.n_items their number (at most max_items, the host's bound that sizes the gate/up
// grid).  Quotients by xg (at most 32) of numbers below 1,024 are (n m) >> 20 with
// m = 2^20 / xg + 1, exact in that range.
// The bucket scan runs on one packed word per bucket: pairs (bits 0..9), non-empty
// buckets (bits 10..20) and staging passes (bits 21..30); none of the three totals can
// reach its field's limit (at most 544 pairs and passes, 1,025 buckets).
static_assert(kMaxPairsDec < 1024, "packed bucket scan");
__device__ __forceinline__ int incl_pairs(int x) { return x & 0x3FF; }
__device__ __forceinline__ int incl_active(int x) { return (x >> 10) & 0x7FF; }
__device__ __forceinline__ int incl_items(int x) { return (int)((uint32_t)x >> 21); }
template <int NPP>
__device__ __forceinline__ void dec_route_tail(const LayerArgs& L, int T, const Work& w, int max_slots, int xg,
                                               int max_items, const int* s_exp, int* s_cnt, uint32_t* s_tmask,
                                               int* s_incl, const BucketPtrs<NPP>& bp,
                                               int32_t* __restrict__ dbg_counts, int32_t* __restrict__ dbg_offsets,
                                               int32_t* __restrict__ dbg_perm) {
  __shared__ int s_ctot[(1024 + 1 + 63) / 64];  // each 64-bucket chunk's sum
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nthr = (int)blockDim.x;
  const int E = L.E, k = L.k;
  const int nb = E + 1;
  const int Pr = T * k;
  const int P = Pr + (L.has_shared ? T : 0);
  for (int p = tid; p < P; p += nthr) {
    const int e = s_exp[p];
    if (e >= 0) {  // expert -1: an omitted pair
      atomicAdd(&s_cnt[e], 1);
      atomicOr(&s_tmask[e], 1u << dec_token_of_pair(p, T, k));
    }
  }
  __syncthreads();
  // inclusive scan of (count, non-empty flag, passes) over the buckets: every wave scans
  // 64-bucket chunks (DPP row shifts inside 16-lane rows, then the row totals), then each
  // bucket adds the sums of the chunks before its own
  const uint32_t xgm = (1u << 20) / (uint32_t)xg + 1u;
  const int nchunks = (nb + 63) >> 6;
  for (int c = wave; c < nchunks; c += nthr >> 6) {
    const int i = 64 * c + lane;
    const int cv = i < nb ? s_cnt[i] : 0;
    int x = cv | ((cv > 0 ? 1 : 0) << 10) | (int)(((uint32_t)(cv + xg - 1) * xgm >> 20) << 21);
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
    const int r2 = __builtin_amdgcn_readlane(x, 47), r3 = __builtin_amdgcn_readlane(x, 63);
    const int row = lane >> 4;
    x += (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
    if (i < nb) s_incl[i] = x;
    if (lane == 0) s_ctot[c] = r0 + r1 + r2 + r3;
  }
  __syncthreads();
  for (int i = tid; i < nb; i += nthr) {
    int pre = 0;
    for (int c = 0; c < (i >> 6); ++c) pre += s_ctot[c];
    s_incl[i] += pre;
  }
  __syncthreads();
  const int n_active = incl_active(s_incl[nb - 1]);
  const int placed = incl_pairs(s_incl[nb - 1]);  // pairs in the buckets (omitted ones are not)
  const int n_items = incl_items(s_incl[nb - 1]);
#pragma unroll
  for (int u = 0; u < NPP; ++u) {
    const int e = tid + u * nthr;
    if (e >= nb) break;
    const int c = s_cnt[e];
    const int off = incl_pairs(s_incl[e]) - c;
    w.counts[e] = c;
    w.offsets[e] = off;
    if (dbg_counts) dbg_counts[e] = c;
    if (dbg_offsets) dbg_offsets[e] = off;
    if (c > 0) {
      const int a = incl_active(s_incl[e]) - 1;
      w.active[1 + a] = e;
      Slot& sl = w.slots[a];
      sl.e = e; sl.cnt = c; sl.off = off; sl.n_active = n_active;
      sl.gate_up = bp.gu[u];
      sl.down = bp.dn[u];
      const int np = (int)((uint32_t)(c + xg - 1) * xgm >> 20);
      const int q0 = incl_items(s_incl[e]) - np;
      for (int j = 0; j < np && q0 + j < max_items; ++j) {  // (the bound holds for every routing)
        Slot& it = w.items[q0 + j];
        it.e = e; it.cnt = min(xg, c - j * xg); it.off = off + j * xg; it.n_active = n_active;
        it.gate_up = bp.gu[u];
        it.down = bp.dn[u];
      }
    }
  }
  for (int a = n_active + tid; a < max_slots; a += nthr) {
    Slot& sl = w.slots[a];
    sl.e = 0; sl.cnt = 0; sl.off = 0; sl.n_active = n_active;
    sl.gate_up = nullptr;
    sl.down = nullptr;
  }
  if (tid == 0) {
    w.offsets[nb] = placed;
    if (dbg_offsets) dbg_offsets[nb] = placed;
    w.active[0] = n_active;
    *w.n_items = min(n_items, max_items);
  }
  for (int i = placed + tid; i < P; i += nthr) {  // past the placed pairs
    w.perm[i] = -1;
    if (dbg_perm) dbg_perm[i] = -1;
  }
  for (int p = tid; p < P; p += nthr) {
    const int e = s_exp[p];
    if (e < 0) continue;
    const int r = __popc(s_tmask[e] & ((1u << dec_token_of_pair(p, T, k)) - 1u));  // stable rank
    const int c = s_cnt[e];
    const int pos = incl_pairs(s_incl[e]) - c + r;
    w.perm[pos] = p;
    if (dbg_perm) dbg_perm[pos] = p;
    if (r < kSlotRows) w.slots[incl_active(s_incl[e]) - 1].rows[r] = p;
    const int j = (int)((uint32_t)r * xgm >> 20), rj = r - j * xg;
    const int q = incl_items(s_incl[e]) - (int)((uint32_t)(c + xg - 1) * xgm >> 20) + j;
    if (rj < kSlotRows && q < max_items) w.items[q].rows[rj] = p;
  }
}

// ROUTE false (one token, self-routed projections): the logits are stored to w.logits and
// the kernel ends; the gate/up kernel routes.
// MBOX (T (E+1) <= kDecMailboxWords): the logits go through the mailbox in the workspace
// header as ~bits(l), so a posted entry is its own arrival mark; otherwise through
// w.logits, each block raising its arrival flag (header word blockIdx) once they have
// landed.  Either way each block then checks once whether everything has arrived, and a
// block that sees it all routes (more than one may: they write the same values), clearing
// the mailbox entries or flags so that the header reads zero again after the call.
template <int XDT, bool MBOX, bool ROUTE>
__global__ __launch_bounds__(kRouteThreads) void k_dec_rr(LayerArgs L, const void* __restrict__ x, int T, int erows,
                                                          Work w, int max_slots, int xg, int max_items,
                                                          uint32_t* __restrict__ rr_flags,
                                                          int ntickets, int nzero_o, float eps,
                                                          int32_t* __restrict__ dbg_ids,
                                                          float* __restrict__ dbg_w, int32_t* __restrict__ dbg_counts,
                                                          int32_t* __restrict__ dbg_offsets,
                                                          int32_t* __restrict__ dbg_perm) {
  __shared__ __align__(16) int s_exp[kMaxPairsDec];   // expert of each pair
  __shared__ double s_l[kMaxPairsDec];  // its logit (routed pairs)
  __shared__ int s_cnt[1024 + 1];
  __shared__ uint32_t s_tmask[1024 + 1];  // tokens with a pair in each bucket
  __shared__ int s_incl[1024 + 1];      // inclusive scan of the packed (pairs, buckets, passes)
  __shared__ double s_part[kRouteThreads / 64][kDecMaxTokens];
  __shared__ double s_sg[kDecMaxTokens];  // shared-gate logits read from the mailbox
  __shared__ int s_flag;                // something this block needs has not arrived
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int kWaves = kRouteThreads / 64;
  const int E = L.E, k = L.k, H = L.H;
  const int nb = E + 1;

  if (tid == 0) s_flag = 0;
  if (blockIdx.x == 0) {
    for (int i = tid; i < ntickets; i += kRouteThreads) w.tickets[i] = 0u;  // this call's combine tickets
    // the o mailbox of the one-token combine (nzero_o words, 0 = not posted)
    for (int i = tid; i < nzero_o; i += kRouteThreads) reinterpret_cast<uint32_t*>(w.o)[i] = 0u;
    if (XDT == 0) {  // exact 3-plane bf16 split of fp32 x for the projections
      const float* xf = (const float*)x;
      for (int idx = tid; idx < T * H; idx += kRouteThreads) {
        const float v = xf[idx];
        const uint32_t p0 = f32_to_bf16_rne(v);
        const float r1 = v - bf16_bits_to_f32(p0);
        const uint32_t p1 = f32_to_bf16_rne(r1);
        const uint32_t p2 = f32_to_bf16_rne(r1 - bf16_bits_to_f32(p1));
        w.xplanes[idx] = (uint16_t)p0;
        w.xplanes[(size_t)T * H + idx] = (uint16_t)p1;
        w.xplanes[(size_t)2 * T * H + idx] = (uint16_t)p2;
      }
    }
  }
  for (int i = tid; i < nb; i += kRouteThreads) {
    s_cnt[i] = 0;
    s_tmask[i] = 0u;
  }
  // rows blockIdx.x ROWS + wave / SPLIT; wave % SPLIT takes a 1/SPLIT share of the row's
  // columns; the first pass of its weights is requested now, before the activations are ready
  constexpr int ROWS = router_rows<ROUTE>(), SPLIT = kWaves / ROWS, KPER = router_per<ROUTE>();
  const int e_row = blockIdx.x * ROWS + wave / SPLIT, part = wave % SPLIT;
  const int qh = ((H / SPLIT + 3) / 4) * 4;  // columns per share, a multiple of 4
  const int h0 = min(H, part * qh), h1 = min(H, (part + 1) * qh);
  const float* wrow = e_row < E ? L.router_w + (size_t)e_row * H : L.shared_gate_w;
  f32x4_t wfirst[KPER];
  if (e_row < erows) router_w_first<KPER>(wrow, h0, h1, wfirst);
  const void* xr = x;  // the router's activations (XDT 2: the block's LDS copy of the rescale)
  if constexpr (XDT == 2) {
    __shared__ double s_d[kDecSplitRouteT];  // each token's sqrt(mean(y^2) + eps)
    __shared__ double s_rd[kDecSplitRouteT];  // and its fp64 reciprocal
    __shared__ __align__(16) uint16_t s_x[kRmsFoldElems];
    // With the rescale kernel's exact arithmetic (rms_partial over 256 threads, the 4 wave
    // sums in wave order, rms_divisor, rms_apply).  Group g of the block's four 256-thread
    // groups takes tokens g, g + 4.
    __shared__ double s_ms[kDecSplitRouteT][4];
    const int grp = wave >> 2, i = tid & 255;
    static_assert(kDecSplitRouteT <= 2 * (kWaves / 4), "a group holds at most two tokens' values");
    if (H <= kRmsRegCols && T == 1) {
      // one token: group 0 reads the row once (16 values a thread, kept for LDS), and
      // all 16 waves take the quotients (3 values a thread instead of 12 for group 0 alone)
      __shared__ float s_y[kRmsRegCols];
      if (grp == 0) {
        float v[16];
        const double sq = wave_sum_f64(rms_partial_keep((const float*)x, H, i, v));
        if (lane == 0) s_ms[0][wave & 3] = sq;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (i + 256 * u < H) s_y[i + 256 * u] = v[u];
      }
      __syncthreads();
      if (tid == 0) {
        const double d = rms_divisor(s_ms[0][0], s_ms[0][1], s_ms[0][2], s_ms[0][3], H, eps);
        s_d[0] = d;
        s_rd[0] = 1.0 / d;
      }
      __syncthreads();
      const double d = s_d[0], rd = s_rd[0];
      for (int n = tid; n < H; n += kRouteThreads) {
        const uint16_t q = rms_apply(s_y[n], d, rd);
        s_x[n] = q;
        if (blockIdx.x == 0) w.xr[n] = q;
      }
      __syncthreads();
    } else if (H <= kRmsRegCols) {
      // each row read once: the group's (at most two) tokens keep their values in
      // registers from the sum of squares to the quotient
      float v[2][16];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = grp + (kWaves / 4) * j;
        if (t < T) {  // wave-uniform
          const double sq = wave_sum_f64(rms_partial_keep((const float*)x + (size_t)t * H, H, i, v[j]));
          if (lane == 0) s_ms[t][wave & 3] = sq;
        }
      }
      __syncthreads();
      if (tid < T) {
        const double d = rms_divisor(s_ms[tid][0], s_ms[tid][1], s_ms[tid][2], s_ms[tid][3], H, eps);
        s_d[tid] = d;
        s_rd[tid] = 1.0 / d;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = grp + (kWaves / 4) * j;
        if (t < T) {
          const double d = s_d[t], rd = s_rd[t];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int n = i + 256 * u;
            const uint16_t q = rms_apply(v[j][u], d, rd);
            if (n < H) {
              s_x[t * H + n] = q;
              if (blockIdx.x == 0) w.xr[(size_t)t * H + n] = q;
            }
          }
        }
      }
      __syncthreads();
    } else {
      for (int t = grp; t < T; t += kWaves / 4) {
        const double sq = wave_sum_f64(rms_partial((const float*)x + (size_t)t * H, H, i));
        if (lane == 0) s_ms[t][wave & 3] = sq;
      }
      __syncthreads();
      if (tid < T) {
        const double d = rms_divisor(s_ms[tid][0], s_ms[tid][1], s_ms[tid][2], s_ms[tid][3], H, eps);
        s_d[tid] = d;
        s_rd[tid] = 1.0 / d;
      }
      __syncthreads();
      // the rescaled rows once per block into LDS (block 0 also writes them for the projections),
      // token by token, 8 values in flight per thread
      for (int t = 0; t < T; ++t) {
        for (int n0 = tid; n0 < H; n0 += 8 * kRouteThreads) {
          uint16_t v[8];
          rms_apply8((const float*)x + (size_t)t * H, n0, kRouteThreads, H, s_d[t], s_rd[t], v);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int n = n0 + kRouteThreads * u;
            if (n < H) {
              s_x[t * H + n] = v[u];
              if (blockIdx.x == 0) w.xr[(size_t)t * H + n] = v[u];
            }
          }
        }
      }
      __syncthreads();
    }
    xr = s_x;
  }
  {
    // the bias of the logit this thread finishes (if any), loaded before the sums
    double bias = 0.0;
    if (tid < ROWS * T) {
      const int er = blockIdx.x * ROWS + tid / T;
      if (er < E && L.router_b) bias = (double)L.router_b[er];
    }
    if (e_row < erows) router_part<XDT, KPER>(wrow, xr, T, H, h0, h1, s_part[wave], wfirst);
    __syncthreads();
    if (tid < ROWS * T) {
      const int r = tid / T, t = tid % T;
      const int er = blockIdx.x * ROWS + r;
      if (er < erows) {
        double v = s_part[SPLIT * r][t];  // the shares added in column order
#pragma unroll
        for (int q = 1; q < SPLIT; ++q) v += s_part[SPLIT * r + q][t];
        if (er < E && L.router_b) v += bias;
        if (!ROUTE)
          w.logits[(size_t)t * (E + 1) + er] = v;
        else if (MBOX)
          __hip_atomic_store(w.rr_mbox + (size_t)t * (E + 1) + er, ~__builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        else
          __hip_atomic_store(w.logits + (size_t)t * (E + 1) + er, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if constexpr (!ROUTE) return;
  // This block's posts have landed (acknowledged) before any of its checks is issued, so the
  // block whose check comes last sees every post.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (!MBOX) {
    if (wave == 0) {
      if (lane == 0) __hip_atomic_store(rr_flags + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      bool missing = false;
      for (int b = lane; b < (int)gridDim.x; b += 64)
        missing |= __hip_atomic_load(rr_flags + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;
      if (__ballot(missing) != 0ull && lane == 0) s_flag = 1;
    }
    __syncthreads();
    if (s_flag) return;
    for (int b = tid; b < (int)gridDim.x; b += kRouteThreads)
      __hip_atomic_store(rr_flags + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // this thread's buckets' expert pointers for the slot records: issued now, used at the end
  BucketPtrs<2> bp;
  load_bucket_ptrs(L, bp);

  const int Pr = T * k;
  const bool want_sg = L.has_shared && L.shared_gate_w;
  // top-k: wave w takes tokens w and w + 16 (T <= 32), side by side
  {
    const int t0 = wave, t1 = wave + kWaves;
    const int nper = (E + 63) >> 6;
    if (MBOX) {
      bool ok;
      if (nper <= 1) ok = topk_mbox<1>(w.rr_mbox, E, k, T, t0, t1, want_sg, &s_flag, s_exp, s_l, s_sg);
      else if (nper <= 2) ok = topk_mbox<2>(w.rr_mbox, E, k, T, t0, t1, want_sg, &s_flag, s_exp, s_l, s_sg);
      else if (nper <= 4) ok = topk_mbox<4>(w.rr_mbox, E, k, T, t0, t1, want_sg, &s_flag, s_exp, s_l, s_sg);
      else if (nper <= 8) ok = topk_mbox<8>(w.rr_mbox, E, k, T, t0, t1, want_sg, &s_flag, s_exp, s_l, s_sg);
      else ok = topk_mbox<16>(w.rr_mbox, E, k, T, t0, t1, want_sg, &s_flag, s_exp, s_l, s_sg);
      if (!ok) return;  // block-uniform: a later block routes
    } else {
      if (nper <= 1) topk_wave<1>(w.logits, E, k, T, t0, t1, s_exp, s_l);
      else if (nper <= 2) topk_wave<2>(w.logits, E, k, T, t0, t1, s_exp, s_l);
      else if (nper <= 4) topk_wave<4>(w.logits, E, k, T, t0, t1, s_exp, s_l);
      else if (nper <= 8) topk_wave<8>(w.logits, E, k, T, t0, t1, s_exp, s_l);
      else topk_wave<16>(w.logits, E, k, T, t0, t1, s_exp, s_l);
    }
    for (int t = t0; t < T && t <= t1; t += kWaves) {
      float gte;
      const bool keep = pair_gate(s_l[t * k + min(lane, k - 1)], s_l[t * k], k, L.omit_below, &gte);
      if (lane < k) {
        const int p = t * k + lane;
        const int id = keep ? s_exp[p] : -1;  // an omitted pair is in no bucket
        s_exp[p] = id;
        w.ids[p] = id;
        w.pair_w[p] = gte;
        if (dbg_ids) dbg_ids[p] = id;
        if (dbg_w) dbg_w[p] = gte;
      }
      if (L.has_shared && lane == 0) {
        double sg = 1.0;
        if (want_sg) {
          const double ls = MBOX ? s_sg[t]
                                 : __hip_atomic_load(w.logits + (size_t)t * (E + 1) + E, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
          sg = 1.0 / (1.0 + exp(-ls));
        }
        w.pair_w[Pr + t] = (float)sg;
        s_exp[Pr + t] = E;
      }
    }
  }
  __syncthreads();
  dec_route_tail(L, T, w, max_slots, xg, max_items, s_exp, s_cnt, s_tmask, s_incl, bp, dbg_counts, dbg_offsets,
                 dbg_perm);
}


// Decode routing of 8..32 tokens after the matrix-core router (K-split partial logits
// [nsplit][T][E+1] in w.logits, added in split order): one wave per token takes the top-k
// (ties to the lower index), the softmax gates with the omission rule and the
// shared-expert weight, 4 tokens per block.  Each block then checks once, after its
// results have landed, whether it is the last one to finish (an arrival counter in the
// workspace header); that block routes: the combine tickets, histogram, scan, slot records.
// No block waits for another.
template <int NPER>
__device__ __forceinline__ void dec_topk_token(const double* logits, int E, int k, int t, int* s_exp, double* s_l,
                                               int nsplit, size_t sstride) {
  const int tok[1] = {t}, slot[1] = {0};
  if (nsplit == 1) topk_tokens<NPER, 1, false, 1>(logits, E, k, tok, slot, s_exp, s_l);
  else topk_tokens<NPER, 1, false, kRouterMaxSplits>(logits, E, k, tok, slot, s_exp, s_l, nsplit, sstride);
}
// the header word counting the top-k blocks that have finished (the router kernel's
// arrival flags use the words below E / 4 + 1)
constexpr int kTopkDoneWord = 511;
constexpr int kTopkRouteThreads = 256;  // 4 tokens per block
// the bucket pointers of the routing kernels cover every bucket of up to 1,024 experts
// plus the shared one
static_assert(2 * kRouteThreads > 1024 && 5 * kTopkRouteThreads > 1024, "bucket pointer prefetch");

__global__ __launch_bounds__(kTopkRouteThreads) void k_dec_topk_route(LayerArgs L, int T, Work w, int nsplit,
                                                                      int max_slots, int xg, int max_items,
                                                                      int ntickets,
                                                                      int32_t* __restrict__ dbg_ids,
                                                                      float* __restrict__ dbg_w,
                                                                      int32_t* __restrict__ dbg_counts,
                                                                      int32_t* __restrict__ dbg_offsets,
                                                                      int32_t* __restrict__ dbg_perm) {
  __shared__ int s_sel[4][16];
  __shared__ double s_l[4][16];
  __shared__ __align__(16) int s_exp[kMaxPairsDec];
  __shared__ int s_cnt[1024 + 1];
  __shared__ uint32_t s_tmask[1024 + 1];
  __shared__ int s_incl[1024 + 1];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = L.E, k = L.k, nb = E + 1;
  const int Pr = T * k;
  const int P = Pr + (L.has_shared ? T : 0);
  const int t = blockIdx.x * 4 + wave;
  // the expert pointers of this thread's buckets, for the slot records if this block routes
  // (loaded by every block, before its top-k, so that the routing block never waits on them)
  BucketPtrs<5> bp;
  load_bucket_ptrs(L, bp);
  if (t < T) {  // wave-uniform
    const size_t sstride = (size_t)T * (E + 1);
    const int nper = (E + 63) >> 6;
    if (nper <= 1) dec_topk_token<1>(w.logits, E, k, t, s_sel[wave], s_l[wave], nsplit, sstride);
    else if (nper <= 2) dec_topk_token<2>(w.logits, E, k, t, s_sel[wave], s_l[wave], nsplit, sstride);
    else if (nper <= 4) dec_topk_token<4>(w.logits, E, k, t, s_sel[wave], s_l[wave], nsplit, sstride);
    else if (nper <= 8) dec_topk_token<8>(w.logits, E, k, t, s_sel[wave], s_l[wave], nsplit, sstride);
    else dec_topk_token<16>(w.logits, E, k, t, s_sel[wave], s_l[wave], nsplit, sstride);
    float g;
    const bool keep = pair_gate(s_l[wave][min(lane, k - 1)], s_l[wave][0], k, L.omit_below, &g);
    if (lane < k) {
      const int id = keep ? s_sel[wave][lane] : -1;  // an omitted pair is in no bucket
      __hip_atomic_store(&w.ids[t * k + lane], id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      w.pair_w[t * k + lane] = g;
      if (dbg_ids) dbg_ids[t * k + lane] = id;
      if (dbg_w) dbg_w[t * k + lane] = g;
    }
    if (L.has_shared && lane == 0) {
      float sg = 1.0f;
      if (L.shared_gate_w) {
        double pz[kRouterMaxSplits];  // every split loaded first (clamped index), added in order
#pragma unroll
        for (int z = 0; z < kRouterMaxSplits; ++z)
          pz[z] = w.logits[(size_t)min(z, nsplit - 1) * sstride + (size_t)t * (E + 1) + E];
        double ls = pz[0];
#pragma unroll
        for (int z = 1; z < kRouterMaxSplits; ++z) ls = z < nsplit ? ls + pz[z] : ls;
        sg = (float)(1.0 / (1.0 + exp(-ls)));
      }
      w.pair_w[Pr + t] = sg;
    }
  }
  // this block's ids have landed (device-scope stores); one arrival, checked once
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&w.rr_flags[kTopkDoneWord], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  if (tid == 0) __hip_atomic_store(&w.rr_flags[kTopkDoneWord], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = tid; i < ntickets; i += kTopkRouteThreads) w.tickets[i] = 0u;  // this call's combine tickets
  for (int i = tid; i < nb; i += kTopkRouteThreads) {
    s_cnt[i] = 0;
    s_tmask[i] = 0u;
  }
  for (int p = tid; p < P; p += kTopkRouteThreads)
    s_exp[p] = p < Pr ? __hip_atomic_load(&w.ids[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : E;
  __syncthreads();
  dec_route_tail(L, T, w, max_slots, xg, max_items, s_exp, s_cnt, s_tmask, s_incl, bp, dbg_counts, dbg_offsets,
                 dbg_perm);
}

// ---------------------------------------------------------------------------
// Shared pieces of the two projection kernels.
// MFMA mapping (v_mfma_f32_16x16x32_bf16): A = activations (16 token slots x 32 k),
// B = decoded weights (32 k x 16 rows); lane l supplies A[l%16][8(l/16)..] and
// B[8(l/16)..][l%16] and holds D[4(l/16)+i][l%16].
// MXFP4: lane group g owns block 4ks+g of its row (16 code bytes); MFMA j uses
//        values 8j..8j+7 of it, so A supplies x[32(4ks+g) + 8j ..].  The E8M0
//        scale is folded into the bf16 values (exact).
// CB4:   MFMA j covers block 4ks+j; lane group g owns bytes 4g..4g+3 of it, A
//        supplies x[32(4ks+j) + 8g ..]; the fp16 scale multiplies the block's
//        fp32 MFMA result (scale * codebook value is not exact in bf16).
// ---------------------------------------------------------------------------
template <int FMT, int KSW>
struct WeightRegs;

template <int KSW>
struct WeightRegs<1, KSW> {
  u32x4_t c[KSW];
  uint32_t s[KSW];
};
template <int KSW>
struct WeightRegs<3, KSW> {  // the packed scale store: s holds the byte with the delta nibble
  u32x4_t c[KSW];
  uint32_t s[KSW];
};
template <int KSW>
struct WeightRegs<4, KSW> {  // 3-bit affine: 12 code bytes and the (scale, bias) fp16 pairs of 2 groups
  u32x3_t c[KSW];
  uint64_t s[KSW];
};
template <int KSW>
struct WeightRegs<2, KSW> {
  u32x4_t c[KSW];      // block 4ks + g of row m (16 bytes), as stored
  uint32_t s[KSW][2];  // fp16 scale bits of blocks 4ks..4ks+3 of row m, two per dword
};

// Loads of one wave's k-steps ks0, ks0+stride, ... of one 16-row weight tile (stride 4:
// the 4 waves split K; stride 1: the wave takes every k-step).  Straight-line
// code with clamped addresses and no use of the loaded values here, so each k-step's
// MFMAs wait only for their own loads.  Out-of-range data is never used: k-steps past
// the row are skipped and k blocks past the row meet a zero activation operand.
template <int FMT, int KSW>
__device__ __forceinline__ void prefetch_step(WeightRegs<FMT, KSW>& r, int i, const PackedTile& pt, int nkb, int ks0,
                                              int nks, int m, int g, int stride = 4) {
  // every form below issues one code load and (for a full step) one scale load; a partial
  // CB4 step's four 2-byte scale loads only lengthen the counted waits
  constexpr int kCodeLoads = 1, kScaleLoadsFullStep = 1;
  static_assert(kCodeLoads + kScaleLoadsFullStep == loads_per_step<FMT>(), "per-step load count");
  {
    const int ks = ks0 + stride * i;
    if constexpr (fmt_is_mx(FMT)) {
      // block 4 ksc + g of row m (a block past the row: the step's first block), as the
      // wave-uniform step base plus a 32-bit lane offset
      const int ksc = ks < nks ? ks : 0;
      const int gc = 4 * ksc + g < nkb ? g : 0;
      r.c[i] = __builtin_nontemporal_load(
          (const __attribute__((address_space(1))) u32x4_t*)(pt.codes + (size_t)ksc * 1024 + (uint32_t)(gc * 256 + 16 * m)));
      const uint32_t si = (uint32_t)(gc * 16 + m);
      r.s[i] = FMT == 3 ? (pt.scales + (size_t)ksc * 32)[si >> 1] : (pt.scales + (size_t)ksc * 64)[si];
    } else if constexpr (FMT == 4) {
      const int ksc = ks < nks ? ks : 0;
      r.c[i] = __builtin_nontemporal_load(
          (const __attribute__((address_space(1))) u32x3_t*)(pt.codes + 768 * ksc + 12 * (16 * g + m)));
      r.s[i] = *(const __attribute__((address_space(1))) uint64_t*)(pt.scales + 128 * ksc + 8 * m);
    } else {
      // block 4 ksc + g of row m, as MXFP4 (a block past the row: the step's first block,
      // whose values then meet zero activations); the lane rows are transposed at use
      const int ksc = ks < nks ? ks : 0;
      // the step's scale unit holds rb = min(4, blocks left) entries per row, row-major
      const int rb = min(4, nkb - 4 * ksc);
      const int gc = g < rb ? g : 0;
      r.c[i] = __builtin_nontemporal_load(
          (const __attribute__((address_space(1))) u32x4_t*)(pt.codes + (size_t)ksc * 1024 + (uint32_t)(gc * 256 + 16 * m)));
      if (rb == 4) {  // uniform: the row's four scales are 8 contiguous bytes
        typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
        const u32x2_t sv = *(const __attribute__((address_space(1))) u32x2_t*)(pt.scales + (size_t)ksc * 128 + 8 * m);
        r.s[i][0] = sv[0];
        r.s[i][1] = sv[1];
      } else {  // a block past the row takes the row's last scale
        const uint32_t so = 2u * __umul24((uint32_t)m, (uint32_t)rb);
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          h[j] = *(const __attribute__((address_space(1))) uint16_t*)(pt.scales + ((size_t)ksc * 128 + 2 * min(j, rb - 1)) + so);
        r.s[i][0] = h[0] | (h[1] << 16);
        r.s[i][1] = h[2] | (h[3] << 16);
      }
    }
  }
}

template <int FMT, int KSW>
__device__ __forceinline__ void prefetch_weights(WeightRegs<FMT, KSW>& r, const PackedTile& pt, int nkb, int ks0,
                                                 int nks, int m, int g, int stride = 4) {
#pragma unroll
  for (int i = 0; i < KSW; ++i) prefetch_step<FMT, KSW>(r, i, pt, nkb, ks0, nks, m, g, stride);
}

// Two tiles (gate and up rows) k-step by k-step, so a k-step's MFMAs of both tiles
// depend only on that step's loads.
template <int FMT, int KSW>
__device__ __forceinline__ void prefetch_weights2(WeightRegs<FMT, KSW>& ra, const PackedTile& pa,
                                                  WeightRegs<FMT, KSW>& rb, const PackedTile& pb, int nkb, int ks0,
                                                  int nks, int m, int g) {
#pragma unroll
  for (int i = 0; i < KSW; ++i) {
    prefetch_step<FMT, KSW>(ra, i, pa, nkb, ks0, nks, m, g);
    prefetch_step<FMT, KSW>(rb, i, pb, nkb, ks0, nks, m, g);
  }
}

// An empty use of k-step i's weight registers.
template <int FMT, int KSW>
__device__ __forceinline__ void consume_weights(const WeightRegs<FMT, KSW>& r, int i) {
  if constexpr (fmt_is_mx(FMT)) {
    asm volatile("" ::"v"(r.c[i]), "v"(r.s[i]));
  } else if constexpr (FMT == 4) {
    asm volatile("" ::"v"(r.c[i]), "v"(r.s[i]));
  } else {
    asm volatile("" ::"v"(r.c[i]), "v"(r.s[i][0]), "v"(r.s[i][1]));
  }
}

// acc[tt] += A(token tile tt, planes) x B(weights of k-step i) for one weight matrix.
// sbase: the packed scale store's base byte of this lane's weight row (format 3 only).
// arow[tt]: this lane's activation row for token tile tt in LDS (slot 16 tt + m, or the
// tile's zero row for a slot past the staged rows).  Staged rows are zero from column K
// to the end of the last k-step, so 32-blocks past the row add exact zeros (the weights
// they meet are clamped real blocks); k-steps past the row (ks is wave-uniform) are
// skipped.  No per-lane masking: every MFMA reads its operands unconditionally.
template <int FMT, int NP, int NTT, int KSW>
__device__ __forceinline__ void mma_kstep(const WeightRegs<FMT, KSW>& r, int i, int ks, int nks,
                                          const uint16_t* const (&arow)[NTT], size_t plane_stride, int live,
                                          const uint32_t* lut, uint32_t sbase, f32x4_t (&acc)[NTT],
                                          const float* xsum = nullptr, int ngrp = 0) {
  if (ks >= nks) {
    // the step's loads were issued (clamped addresses) but are not used: read their
    // registers here, so that no load is left outstanding past this point (the compiler
    // would otherwise wait for all loads before those registers' next use)
    consume_weights<FMT, KSW>(r, i);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  if constexpr (fmt_is_mx(FMT)) {
    const float sc = e8m0_to_f32(FMT == 3 ? ps_e8m0(sbase, r.s[i], m) : r.s[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t b = fp4x8_to_bf16(r.c[i][j], sc);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        if (tt < live) {
          const uint16_t* ap = arow[tt] + 128 * ks + 32 * g + 8 * j;
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const u32x4_t av = *(const u32x4_t*)(ap + p * plane_stride);
            acc[tt] = mfma_bf16(__builtin_bit_cast(bf16x8_t, av), b, acc[tt]);
          }
        }
      }
    }
  } else if constexpr (FMT == 4) {
    // 3-bit affine: per 64-column group G (MFMAs 2G, 2G+1) the matrix cores sum
    // (128 + q) x exactly per product; s (that) + (b - 128 s) X, X the group's activation
    // sum per token slot (xsum[slot * ngrp + group], zero past the staged rows), is the
    // group's sum of (s q + b) x.
    uint32_t o[16];
    aff3_pairs(r.c[i], o);
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      const float sc = half_bits_to_f32((uint16_t)(r.s[i] >> (32 * G)));
      const float bc = fmaf(-128.0f, sc, half_bits_to_f32((uint16_t)(r.s[i] >> (32 * G + 16))));
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        if (tt < live) {
          f32x4_t tmp[1] = {{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * G + jj;
            const u32x4_t bw = {o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
            const uint16_t* ap = arow[tt] + 128 * ks + 32 * j + 8 * g;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const u32x4_t av = *(const u32x4_t*)(ap + p * plane_stride);
              tmp[0] = mfma_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bw), tmp[0]);
            }
          }
          mfma_settle(tmp[0]);
          const float* xg = xsum + (size_t)(16 * tt + 4 * g) * ngrp + 2 * ks + G;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[tt][q] = fmaf(bc, xg[(size_t)q * ngrp], fmaf(sc, tmp[0][q], acc[tt][q]));
        }
      }
    }
  } else {
    // lane row g then holds bytes 4g..4g+3 of block 4ks + j in dword j: MFMA j covers
    // block 4ks + j alone, so its fp32 result takes the block's scale.  The 4 blocks'
    // MFMAs first, then their scaled sums (block order j per output).
    u32x4_t cw = r.c[i];
    xpose_rows4(cw);
    bf16x8_t b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = cb4x8_to_bf16(cw[j], lut);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      if (tt < live) {
        f32x4_t tmp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t* ap = arow[tt] + 128 * ks + 32 * j + 8 * g;
          tmp[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const u32x4_t av = *(const u32x4_t*)(ap + p * plane_stride);
            tmp[j] = mfma_bf16(__builtin_bit_cast(bf16x8_t, av), b[j], tmp[j]);
          }
        }
        mfma_settle4(tmp);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float sc = half_bits_to_f32((uint16_t)(r.s[i][j >> 1] >> (16 * (j & 1))));
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[tt][q] = fmaf(sc, tmp[j][q], acc[tt][q]);
        }
      }
    }
  }
}

// This lane's activation rows (one per token tile) in a staged LDS tile: slot 16 tt + m
// when it holds a staged row (slot < xrows), else the zero row (index zrow).
template <int NTT>
__device__ __forceinline__ void dec_arows(const uint16_t* xs, int xstride, int xrows, int zrow,
                                          const uint16_t* (&arow)[NTT]) {
  const int m = threadIdx.x & 15;
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int sl = 16 * tt + m;
    arow[tt] = xs + (size_t)(sl < xrows ? sl : zrow) * xstride;
  }
}

// Zero the parts of a staged LDS tile that the MFMAs read but no staging load writes:
// the zero row (index zrow of every plane, all kc columns) and columns K .. kc-1 of the
// rows 0 .. nrows-1 (kc = K rounded up to whole 128-column k-steps).  LDS stores by the
// whole block; the caller's barrier orders them before the MFMAs (after an lgkmcnt wait).
template <int NP>
__device__ __forceinline__ void zero_tile_pad(uint16_t* xs, int xstride, size_t lds_plane, int K, int kc, int zrow,
                                              int nrows) {
  typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
  const u32x4_t zv = {0u, 0u, 0u, 0u};
  // LDS stores through LDS pointers made from the 32-bit LDS address (the low half of
  // the generic pointer)
  auto lds = [](const uint16_t* q) { return (lds_u32x4*)(uint32_t)(uintptr_t)q; };
  const int zc = kc >> 3;  // 16-byte chunks
  for (int idx = threadIdx.x; idx < NP * zc; idx += blockDim.x) {
    const int q = idx / zc, c = idx - q * zc;
    *lds(xs + q * lds_plane + (size_t)zrow * xstride + 8 * c) = zv;
  }
  const int pc = (kc - K) >> 3;  // K is a multiple of 32 columns
  for (int idx = threadIdx.x; idx < NP * nrows * pc; idx += blockDim.x) {
    const int q = idx / (nrows * pc), rc = idx - q * nrows * pc;
    const int row = rc / pc, c = rc - row * pc;
    *lds(xs + q * lds_plane + (size_t)row * xstride + K + 8 * c) = zv;
  }
}

// Stage the activation rows of slots tb .. tb+nrows-1 of this expert into LDS (bf16
// planes).  The slot loop is uniform, so the pair ids arrive through scalar loads and
// only the 16-byte row chunks use vector loads (issued behind the weight prefetch).
template <int NP, bool BY_TOKEN>
__device__ __forceinline__ void stage_rows(uint16_t* xs, int xstride, size_t lds_plane, const uint16_t* src,
                                           size_t src_plane, int K, const int32_t* __restrict__ perm_slots,
                                           int nrows, int T, int k) {
  const int chunks = K / 8;  // 16-byte chunks per row
  for (int s = 0; s < nrows; ++s) {
    const int p = perm_slots[s];
    const int r = BY_TOKEN ? dec_token_of_pair(p, T, k) : p;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const u32x4_t v = *(const u32x4_t*)(src + q * src_plane + (size_t)r * K + 8 * c);
        *(u32x4_t*)(xs + q * lds_plane + (size_t)s * xstride + 8 * c) = v;
      }
    }
  }
}

// The 4 waves copy the activation rows of slots tb .. tb+nrows-1 of this expert into
// LDS with direct global->LDS loads (64 lanes x 16 bytes per instruction, no
// registers).  Issued before the weight loads, they complete first in each wave's
// in-order load counter, so waiting for them leaves the weights in flight.  Pair ids
// come from the slot record (scalar) or, past its first rows, from perm.
// Direct global->LDS copy of 16 bytes per lane to LDS address lds + 16 * lane (the
// LDS base is wave-uniform).  Issued as inline assembly so that the compiler does not
// track it: the caller waits for it explicitly (s_waitcnt vmcnt) before a barrier,
// while later loads stay in flight.
__device__ __forceinline__ void load_lds_16(const void* gptr, void* lds) {
  // the low 32 bits of a generic pointer into LDS are its LDS address (no address-space
  // cast, whose null test the code generator can emit in an illegal form)
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr),
               "v"((const __attribute__((address_space(1))) void*)gptr)
               : "memory", "m0");
}

template <int NP, bool BY_TOKEN>
__device__ __forceinline__ void stage_rows_lds(uint16_t* xs, int xstride, size_t lds_plane, const uint16_t* src,
                                               size_t src_plane, int K, const Slot* __restrict__ slot_rec,
                                               const int32_t* __restrict__ perm_e, int tb, int nrows, int T, int k) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_bytes = K * 2;
  const int nchunk = (row_bytes + 1023) >> 10;  // 1 KB per instruction
  // lane s holds the source row of slot tb + s (one load for all rows of the pass)
  int myrow = 0;
  {
    const int slot = tb + lane;
    const int pair = lane < nrows ? (slot < kSlotRows ? slot_rec->rows[slot] : perm_e[slot]) : 0;
    myrow = BY_TOKEN ? dec_token_of_pair(pair, T, k) : pair;
  }
  // settle the row ids here: the compiler then places no wait inside the loop, where a
  // wait for them would also wait for each earlier direct load (it does not track those)
  // and issue the rows one round trip at a time
  asm volatile("" ::"v"(myrow));
  const int jobs = nrows * nchunk * NP;
  for (int job = wave; job < jobs; job += 4) {  // wave-uniform
    const int q = job % NP;
    const int rc = job / NP;
    const int srow = rc / nchunk, ch = rc % nchunk;
    const int r = __builtin_amdgcn_readlane(myrow, srow);
    const uint8_t* g = (const uint8_t*)(src + q * src_plane + (size_t)r * K) + 1024 * ch + 16 * lane;
    uint8_t* d = (uint8_t*)(xs + q * lds_plane + (size_t)srow * xstride) + 1024 * ch;
    if (1024 * ch + 16 * lane < row_bytes) load_lds_16(g, d);
  }
}

// 3-bit affine: xsum[slot * (K/64) + G] = the sum of the staged activation planes of
// slot over the 64 columns of group G, in a fixed order (0 for slots past xrows), for the
// affine bias term.  Then a barrier on LDS only (the weight loads stay in flight).
template <int NP>
__device__ __forceinline__ void dec_group_sums(float* xsum, const uint16_t* xs, int xstride, size_t lds_plane, int K,
                                               int nslots, int xrows) {
  const int ng = K >> 6;
  for (int idx = threadIdx.x; idx < nslots * ng; idx += blockDim.x) {
    const int sl = idx / ng, G = idx % ng;
    float sum = 0.f;
    if (sl < xrows) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const u32x4_t v = *(const u32x4_t*)(xs + p * lds_plane + (size_t)sl * xstride + 64 * G + 8 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) sum += bf16_bits_to_f32(v[e] & 0xFFFFu) + bf16_bits_to_f32(v[e] >> 16);
        }
    }
    xsum[idx] = sum;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// LDS columns of a staged activation row: K rounded up to whole 128-column k-steps (zero
// past K), and the row stride.
__host__ __device__ inline int dec_kcols(int K) { return (K + 127) & ~127; }
__host__ __device__ inline int dec_xstride(int K) { return lds_row_stride(dec_kcols(K)); }
// Dynamic LDS of a projection block: the activation tile (NP planes of xrows staged rows
// and one zero row), which the split-K reduction buffer later reuses, then (3-bit affine)
// the group sums of 16 NTT token slots.  The codebook table is a static LDS array of the
// kernel, so its address is a constant that the table reads carry as an immediate offset.
__host__ __device__ inline size_t dec_tile_bytes(int K, int NP, int NTT, int xrows) {
  const size_t x = (size_t)NP * (xrows + 1) * dec_xstride(K) * 2;
  const size_t red = (size_t)3 * 8 * NTT * 64 * 4;
  return x > red ? x : red;
}
__host__ __device__ inline size_t dec_lds_bytes(int fmt, int K, int NP, int NTT, int xrows) {
  return dec_tile_bytes(K, NP, NTT, xrows) + (fmt == 4 ? (size_t)16 * NTT * (K / 64) * 4 : 0);
}

// One token: its activation row (NP planes) into LDS row 0, the 4 waves splitting the
// 1 KB direct loads (issued before the block knows its expert).
template <int NP>
__device__ __forceinline__ void stage_token0_lds(uint16_t* xs, size_t lds_plane, const uint16_t* src,
                                                 size_t src_plane, int K) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_bytes = K * 2;
  const int nchunk = (row_bytes + 1023) >> 10;
  for (int job = wave; job < nchunk * NP; job += 4) {
    const int q = job % NP, ch = job / NP;
    if (1024 * ch + 16 * lane < row_bytes)
      load_lds_16((const uint8_t*)(src + q * src_plane) + 1024 * ch + 16 * lane, (uint8_t*)(xs + q * lds_plane) + 1024 * ch);
  }
}

// Sum the 4 waves' partial tiles (split-K) in wave order into wave 0.
template <int NV>
__device__ __forceinline__ void reduce4(float (&v)[NV], float* red) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __syncthreads();
  if (wave > 0 && wave < 4) {
#pragma unroll
    for (int i = 0; i < NV; ++i) red[((wave - 1) * NV + i) * 64 + lane] = v[i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int src = 0; src < 3; ++src)
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] += red[(src * NV + i) * 64 + lane];
  }
}

// ---------------------------------------------------------------------------
// One token, self-routed projections: the router kernel only stores the token's logits
// (w.logits[0 .. E], column E the shared-gate logit); every gate/up block then takes the
// top-k itself (wave 0: one wave, 0.5 us), keeps the pairs that pass the omission rule,
// and takes the routed expert of rank blockIdx.y among the kept ones in ascending expert
// order (the shared expert right after them).  Block (0, 0) writes the call's routing
// outputs (ids, pair weights, counts, offsets, perm, active list, debug copies) and block
// (0, y) the slot record y that the down kernel reads; the blocks read none of them, so
// the kernel has no cross-block dependency.  E <= kSelfRouteMaxE.
// ---------------------------------------------------------------------------
constexpr int kSelfRouteMaxE = 256;
template <int NPER>
__device__ __forceinline__ void dec_self_route(const LayerArgs& L, const Work& w, Slot* s_rec,
                                               int32_t* __restrict__ dbg_ids, float* __restrict__ dbg_w,
                                               int32_t* __restrict__ dbg_counts, int32_t* __restrict__ dbg_offsets,
                                               int32_t* __restrict__ dbg_perm) {
  __shared__ int s_exp[16];
  __shared__ double s_l[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = L.E, k = L.k, sh = L.has_shared;
  const int y = blockIdx.y;
  if (wave == 0) {
    double lv[1][NPER];
    uint64_t gp[NPER + 1];
#pragma unroll
    for (int i = 0; i < NPER; ++i) lv[0][i] = w.logits[min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i <= NPER; ++i) gp[i] = (uint64_t)L.gate_up[min(lane + 64 * i, E + sh - 1)];
    const double lsg = (sh && L.shared_gate_w) ? w.logits[E] : 0.0;
    const int tok[1] = {0};
    topk_select<NPER, 1>(lv, E, k, tok, s_exp, s_l);
    // the gates decide only with omission; otherwise only block (0, 0) needs them
    float g = 0.0f;
    bool keep = lane < k;
    if (L.omit_below > 0.0f || (blockIdx.x == 0 && y == 0))
      keep = pair_gate(s_l[min(lane, k - 1)], s_l[0], k, L.omit_below, &g);
    const bool kept = lane < k && keep;
    const int id = lane < k ? s_exp[lane] : 0;
    const uint64_t km = __ballot(kept);
    const int n_kept = __popcll(km);
    int r = 0;  // rank of this lane's expert among the kept ones (ids are distinct)
    for (int j = 0; j < k; ++j) r += ((km >> j) & 1ull) && __builtin_amdgcn_readlane(id, j) < id;
    // this block's slot
    int e_mine = -1, p_mine = -1;
    const uint64_t mine = __ballot(kept && r == y);
    if (mine) {
      const int j = __ffsll((long long)mine) - 1;
      e_mine = __builtin_amdgcn_readlane(id, j);
      p_mine = j;  // pair t*k + j of token 0
    } else if (sh && y == n_kept) {
      e_mine = E;
      p_mine = k;  // the shared pair T*k + t
    }
    uint64_t ptr = 0;
    if (e_mine >= 0) {
#pragma unroll
      for (int i = 0; i <= NPER; ++i) {
        const uint64_t v = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(gp[i] >> 32), e_mine & 63) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)gp[i], e_mine & 63);
        if ((e_mine >> 6) == i) ptr = v;
      }
    }
    const int n_active = n_kept + sh;
    if (lane == 0) {
      s_rec->e = e_mine < 0 ? 0 : e_mine;
      s_rec->cnt = e_mine < 0 ? 0 : 1;
      s_rec->off = y;
      s_rec->n_active = n_active;
      s_rec->gate_up = (const uint8_t*)ptr;
      s_rec->rows[0] = p_mine;
    }
    if (blockIdx.x == 0) {
      if (lane == 0) {  // the slot record of row y for the down kernel
        Slot& sl = w.slots[y];
        sl.e = e_mine < 0 ? 0 : e_mine;
        sl.cnt = e_mine < 0 ? 0 : 1;
        sl.off = y;
        sl.n_active = n_active;
        sl.gate_up = (const uint8_t*)ptr;
        sl.down = e_mine < 0 ? nullptr : L.down[e_mine];
        sl.rows[0] = p_mine;
      }
      if (y == 0) {  // the call's routing outputs
        if (lane < k) {
          const int idv = kept ? id : -1;
          w.ids[lane] = idv;
          w.pair_w[lane] = g;
          if (dbg_ids) dbg_ids[lane] = idv;
          if (dbg_w) dbg_w[lane] = g;
          if (kept) {
            w.perm[r] = lane;
            w.active[1 + r] = id;
            if (dbg_perm) dbg_perm[r] = lane;
          }
        }
        for (int i = n_active + lane; i < k + sh; i += 64) {  // past the placed pairs
          w.perm[i] = -1;
          if (dbg_perm) dbg_perm[i] = -1;
        }
        if (lane == 0) {
          if (sh) {
            w.pair_w[k] = L.shared_gate_w ? (float)(1.0 / (1.0 + exp(-lsg))) : 1.0f;
            w.perm[n_kept] = k;
            w.active[1 + n_kept] = E;
            if (dbg_perm) dbg_perm[n_kept] = k;
          }
          w.active[0] = n_active;
          w.offsets[E + 1] = n_active;
          if (dbg_offsets) dbg_offsets[E + 1] = n_active;
        }
        // counts and exclusive offsets of every bucket: the kept experts have one pair each
        for (int e = lane; e <= E; e += 64) {
          int below = 0, c = 0;
          for (int j = 0; j < k; ++j) {
            const int idj = __builtin_amdgcn_readlane(id, j);
            const bool kj = (km >> j) & 1ull;
            below += kj && idj < e;
            c += kj && idj == e;
          }
          if (e == E) { below = n_kept; c = sh; }
          w.counts[e] = c;
          w.offsets[e] = below;
          if (dbg_counts) dbg_counts[e] = c;
          if (dbg_offsets) dbg_offsets[e] = below;
        }
      }
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// 3. Fused gate/up + SwiGLU per (16-row tile, active expert), 4 waves split K.
//    Each wave first issues direct-to-LDS loads of its share of the expert's
//    activation rows, then all its weight loads; it waits only for the former before
//    the staging barrier, and each k-step's MFMAs then wait only for that step's
//    weights while the rest are still in flight.
// ---------------------------------------------------------------------------
// One block's share of the gate/up projection: the 16-row gate and up tiles x of one
// active expert (slot record sr), passes of xrows_max pairs starting at pair tb0, every
// tb_step pairs.  SR: the caller has staged and padded row 0.
template <int FMT, int NP, int NTT, int KSW, bool SR>
__device__ __forceinline__ void dec_gateup_item(const LayerArgs& L, int T, const Work& w, const uint16_t* act,
                                                size_t act_plane, int xrows_max, const Slot* sr, int x, int tb0,
                                                int tb_step, uint8_t* smem, const uint32_t* lut) {
  const int cnt = sr->cnt, off = sr->off;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int H = L.H, I = L.I, k = L.k;
  const int K = H, nkb = K >> 5, nks = (nkb + 3) >> 2;
  const int xstride = dec_xstride(K);
  const size_t lds_plane = (size_t)(xrows_max + 1) * xstride;  // staged rows, then the zero row
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + dec_tile_bytes(K, NP, NTT, xrows_max));  // 3-bit affine
  const PackedTile pg = packed_tile<FMT>(sr->gate_up, 2 * I, K, x);
  const PackedTile pu = packed_tile<FMT>(sr->gate_up, 2 * I, K, I / 16 + x);
  // the packed scale store's row bases, loaded before the staging loads (not counted below)
  const uint32_t bg = FMT == 3 ? (uint32_t)pg.bases[n] : 0u, bu = FMT == 3 ? (uint32_t)pu.bases[n] : 0u;
  const int nchunks = (nks + 4 * KSW - 1) / (4 * KSW);

  for (int tb = tb0; tb < cnt; tb += tb_step) {
    const int live = min(NTT, (cnt - tb + 15) / 16);
    const int xrows = min(cnt - tb, xrows_max);
    const uint16_t* arow[NTT];
    dec_arows<NTT>(xs, xstride, xrows, xrows_max, arow);
    f32x4_t accg[NTT], accu[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) { accg[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; accu[tt] = accg[tt]; }
    for (int ch = 0; ch < nchunks; ++ch) {
      const int ks0 = ch * 4 * KSW + wave;
      if (ch == 0) {
        if (tb > tb0) __syncthreads();  // the previous pass finished with the LDS tile
        if (!SR) {  // (self-routed: the row was staged before the routing)
          stage_rows_lds<NP, true>(xs, xstride, lds_plane, act, act_plane, K, sr, w.perm + off, tb, xrows, T, k);
          zero_tile_pad<NP>(xs, xstride, lds_plane, K, dec_kcols(K), xrows_max, xrows);
        }
      }
      WeightRegs<FMT, KSW> wg, wu;
      prefetch_weights2<FMT, KSW>(wg, pg, wu, pu, nkb, ks0, nks, n, g);
      if (ch == 0) {
        // this wave's staging loads are complete once at most the weight loads issued
        // after them are outstanding; then every wave's rows are in LDS after the barrier
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_le_lgkm0(2 * KSW * loads_per_step<FMT>()));
        __builtin_amdgcn_s_barrier();
        if constexpr (FMT == 4) dec_group_sums<NP>(xsum, xs, xstride, lds_plane, K, 16 * NTT, xrows);
      }
#pragma unroll
      for (int i = 0; i < KSW; ++i) {
        const int ks = ks0 + 4 * i;
        mma_kstep<FMT, NP, NTT, KSW>(wg, i, ks, nks, arow, lds_plane, live, lut, bg, accg, xsum, nkb >> 1);
        mma_kstep<FMT, NP, NTT, KSW>(wu, i, ks, nks, arow, lds_plane, live, lut, bu, accu, xsum, nkb >> 1);
      }
    }
    // split-K reduction (fixed wave order), SwiGLU, two bf16 planes of h
    mfma_settle_all(accg);
    mfma_settle_all(accu);
    float v[8 * NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) { v[8 * tt + q] = accg[tt][q]; v[8 * tt + 4 + q] = accu[tt][q]; }
    reduce4<8 * NTT>(v, (float*)smem);
    if (wave == 0) {
      const int P = T * k + (L.has_shared ? T : 0);
      const int col = 16 * x + n;
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int slot = tb + 16 * tt + 4 * g + q;
          if (slot < tb + xrows) {  // this pass's pairs only
            const int p = slot < kSlotRows ? sr->rows[slot] : w.perm[off + slot];
            const float h = silu_f32(v[8 * tt + q]) * v[8 * tt + 4 + q];
            const uint32_t hi = f32_to_bf16_rne(h);
            const uint32_t lo = f32_to_bf16_rne(h - bf16_bits_to_f32(hi));
            w.hplanes[(size_t)p * I + col] = (uint16_t)hi;
            w.hplanes[(size_t)P * I + (size_t)p * I + col] = (uint16_t)lo;
          }
        }
      }
    }
  }
}

// Gate/up projection, grid (I/16, work items).  Block row y takes work item y of the
// routing (one staging pass of one active expert; an expert with more pairs than one pass
// stages has its passes on adjacent rows); rows past the last item exit at once.  The
// grid's item count is the host's bound over every routing, so few rows exit (the verify
// window: 139 rows instead of 137 slots x 3 passes).  SR (one token, one pass; grid (I/16,
// slots)): the block routes itself (dec_self_route), staging the token's row meanwhile,
// and keeps its slot record in LDS.
template <int FMT, int NP, int NTT, int KSW, bool SR>
__global__ __launch_bounds__(256, 3) void k_dec_gateup(LayerArgs L, int T, Work w, const uint16_t* __restrict__ act,
                                                       size_t act_plane, int xrows_max, int nslots,
                                                       int32_t* __restrict__ dbg_ids, float* __restrict__ dbg_w,
                                                       int32_t* __restrict__ dbg_counts,
                                                       int32_t* __restrict__ dbg_offsets,
                                                       int32_t* __restrict__ dbg_perm) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ uint32_t s_lut[FMT == 2 ? 256 : 1];  // codebook table (CB4)
  if constexpr (SR) {
    __shared__ Slot s_rec;
    const int xst = dec_xstride(L.H);
    const size_t lpl = (size_t)(xrows_max + 1) * xst;
    stage_token0_lds<NP>((uint16_t*)smem, lpl, act, act_plane, L.H);
    zero_tile_pad<NP>((uint16_t*)smem, xst, lpl, L.H, dec_kcols(L.H), xrows_max, 1);
    const int nper = (L.E + 63) >> 6;
    if (nper <= 1) dec_self_route<1>(L, w, &s_rec, dbg_ids, dbg_w, dbg_counts, dbg_offsets, dbg_perm);
    else if (nper <= 2) dec_self_route<2>(L, w, &s_rec, dbg_ids, dbg_w, dbg_counts, dbg_offsets, dbg_perm);
    else dec_self_route<4>(L, w, &s_rec, dbg_ids, dbg_w, dbg_counts, dbg_offsets, dbg_perm);
    if (s_rec.cnt == 0) {
      __builtin_amdgcn_s_waitcnt(0);  // the staging loads land before the LDS is released
      return;
    }
    if (FMT == 2) build_cb4_lut(s_lut, L.codebook);  // ordered before use by the staging barrier
    dec_gateup_item<FMT, NP, NTT, KSW, SR>(L, T, w, act, act_plane, xrows_max, &s_rec, blockIdx.x, 0, xrows_max,
                                           smem, s_lut);
  } else {
    const Slot* sr = w.items + blockIdx.y;
    // the count and the record are loaded together; rows past the count exit
    const int cnt = sr->cnt, ni = *w.n_items;
    if ((int)blockIdx.y >= ni || cnt == 0) return;
    if (FMT == 2) build_cb4_lut(s_lut, L.codebook);  // ordered before use by the staging barrier
    dec_gateup_item<FMT, NP, NTT, KSW, SR>(L, T, w, act, act_plane, xrows_max, sr, blockIdx.x, 0, xrows_max, smem,
                                           s_lut);
  }
}

// y[t][col0 .. col0+ncols) = sum_j g[t,j] o[t*k+j] (+ shared), j ascending then the shared
// expert: the fixed-order combine of the block that arrives last at a column tile.
// The o rows are read at device scope (written through by the other blocks), the k
// routed ones 8 at a time (clamped loads, in bounds).
__device__ __forceinline__ void dec_combine_cols(const LayerArgs& L, int T, const Work& w, float* __restrict__ y,
                                                 int col0, int ncols) {
  const int H = L.H, k = L.k;
  for (int idx = threadIdx.x; idx < T * ncols; idx += blockDim.x) {
    const int t = idx / ncols;
    const int col = col0 + idx % ncols;
    if (col >= H) continue;
    float s = 0.f;
    for (int j0 = 0; j0 < k; j0 += 8) {
      float ov[8], wv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = min(j0 + u, k - 1);
        ov[u] = __hip_atomic_load(&w.o[(size_t)(t * k + j) * H + col], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wv[u] = w.pair_w[t * k + j];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < k && wv[u] != 0.0f) s = fmaf(wv[u], ov[u], s);  // weight 0: omitted, o not written
    }
    if (L.has_shared) {
      const float o = __hip_atomic_load(&w.o[(size_t)(T * k + t) * H + col], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s = fmaf(w.pair_w[T * k + t], o, s);
    }
    y[(size_t)t * H + col] = w.resid ? w.resid[(size_t)t * H + col] + s : s;
  }
}

// ---------------------------------------------------------------------------
// 4. Down projection + combine for rows of more than 8 k-steps, 4 waves splitting K = I.
//    One token (k_dec_down): grid (H/16, slots); each slot's block posts its 16 o values
//    to a mailbox and the block that finds every pair posted writes y.
//    From 2 tokens (k_dec_down2): grid (H/32, slots); o rows are written through and a
//    relaxed device-scope ticket per 32 columns elects the block that sums y.
//    Either way y is the fixed-order sum (routed j ascending, then shared), the o values
//    travel as write-through stores and no full L2 write-back is needed.
// ---------------------------------------------------------------------------
// Pairs of one token: top-k routed ones plus the shared one.
constexpr int kMaxPairsT1 = 17;

// o posted to the one-token mailbox as ~bits(o): never 0 (the all-ones NaN is replaced
// by another NaN), so 0 marks an entry not yet written.
__device__ __forceinline__ uint32_t omb_encode(float v) {
  const uint32_t b = __float_as_uint(v);
  return ~(b == 0xFFFFFFFFu ? 0xFFC00000u : b);
}

// One token (one pair per slot, one pass): every slot's block posts its 16 o values to the
// mailbox (zeroed by the router kernel) and, once they have landed, reads the other pairs'
// entries once; a block that finds them all sums the column tile over the pairs in the
// fixed order and writes y (more than one may: the same values).  The block whose read
// comes last finds them all, so no block waits and no residency is assumed.
template <int FMT, int KSW>
__device__ __forceinline__ void dec_down_t1_item(const LayerArgs& L, const Work& w, float* __restrict__ y,
                                                 const Slot* slot_rec, int x, uint8_t* smem, const uint32_t* lut) {
  const int off = slot_rec->off;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int H = L.H, I = L.I, k = L.k;
  const int P = k + (L.has_shared ? 1 : 0);
  const int K = I, nkb = K >> 5, nks = (nkb + 3) >> 2;
  const int xstride = dec_xstride(K);
  const size_t lds_plane = 2 * (size_t)xstride;  // the staged row, then the zero row
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + dec_tile_bytes(K, 2, 1, 1));  // 3-bit affine
  const PackedTile pd = packed_tile<FMT>(slot_rec->down, H, K, x);
  const uint32_t bd = FMT == 3 ? (uint32_t)pd.bases[n] : 0u;  // before the staging loads
  const int nchunks = (nks + 4 * KSW - 1) / (4 * KSW);
  const uint16_t* arow[1];
  dec_arows<1>(xs, xstride, 1, 1, arow);
  f32x4_t acc[1] = {{0.f, 0.f, 0.f, 0.f}};
  for (int ch = 0; ch < nchunks; ++ch) {
    const int ks0 = ch * 4 * KSW + wave;
    if (ch == 0) {
      stage_rows_lds<2, false>(xs, xstride, lds_plane, w.hplanes, (size_t)P * I, K, slot_rec, w.perm + off, 0, 1, 1,
                               k);
      zero_tile_pad<2>(xs, xstride, lds_plane, K, dec_kcols(K), 1, 1);
    }
    WeightRegs<FMT, KSW> wd;
    prefetch_weights<FMT, KSW>(wd, pd, nkb, ks0, nks, n, g);
    if (ch == 0) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_le_lgkm0(KSW * loads_per_step<FMT>()));
      __builtin_amdgcn_s_barrier();
      if constexpr (FMT == 4) dec_group_sums<2>(xsum, xs, xstride, lds_plane, K, 16, 1);
    }
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      const int ks = ks0 + 4 * i;
      mma_kstep<FMT, 2, 1, KSW>(wd, i, ks, nks, arow, lds_plane, 1, lut, bd, acc, xsum, nkb >> 1);
    }
  }
  mfma_settle_all(acc);
  float v[4] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
  reduce4<4>(v, (float*)smem);
  if (wave == 0 && g == 0) {
    const int col = 16 * x + n;
    const int p_own = w.perm[off];
    uint32_t* omb = reinterpret_cast<uint32_t*>(w.o);
    const uint32_t mine = omb_encode(v[0]);
    const float rv = w.resid ? w.resid[col] : 0.f;
    __hip_atomic_store(&omb[(size_t)p_own * H + col], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    uint32_t e[kMaxPairsT1];
    float pw[kMaxPairsT1];
    bool miss = false;
#pragma unroll
    for (int u = 0; u < kMaxPairsT1; ++u) {
      const int p = min(u, P - 1);  // routed pairs 0 .. k-1, then the shared one
      pw[u] = w.pair_w[p];
      e[u] = p == p_own ? mine : __hip_atomic_load(&omb[(size_t)p * H + col], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      miss |= e[u] == 0u && pw[u] != 0.0f;  // an omitted pair (weight 0) posts nothing
    }
    if (!miss) {
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < kMaxPairsT1; ++u)
        if (u < P && pw[u] != 0.0f) sum = fmaf(pw[u], __uint_as_float(~e[u]), sum);
      y[col] = w.resid ? rv + sum : sum;
    }
  }
}

// Down projection over two 16-row tiles per block, output columns 32 x .. 32 x + 31 (H is a
// multiple of 32): the steps of dec_down_item with both tiles' weights in flight together
// and one ticket per 32 columns.  A block then streams twice the weight bytes per staged activation row and
// the grid half the blocks; from 2 tokens, where the grid takes several rounds of blocks.
template <int FMT, int NTT, int KSW>
__device__ __forceinline__ void dec_down2_item(const LayerArgs& L, int T, const Work& w, float* __restrict__ y,
                                               uint32_t* __restrict__ tickets, int xrows_max, const Slot* slot_rec,
                                               int x, uint8_t* smem, const uint32_t* lut, int* is_last) {
  const int cnt = slot_rec->cnt, off = slot_rec->off, n_active = slot_rec->n_active;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int H = L.H, I = L.I, k = L.k;
  const int P = T * k + (L.has_shared ? T : 0);
  const int K = I, nkb = K >> 5, nks = (nkb + 3) >> 2;
  const int xstride = dec_xstride(K);
  const size_t lds_plane = (size_t)(xrows_max + 1) * xstride;  // staged rows, then the zero row
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + dec_tile_bytes(K, 2, NTT, xrows_max));  // 3-bit affine
  const PackedTile pa = packed_tile<FMT>(slot_rec->down, H, K, 2 * x);
  const PackedTile pb = packed_tile<FMT>(slot_rec->down, H, K, 2 * x + 1);
  // the packed scale store's row bases, before the staging loads (not counted below)
  const uint32_t ba = FMT == 3 ? (uint32_t)pa.bases[n] : 0u, bb = FMT == 3 ? (uint32_t)pb.bases[n] : 0u;
  const int nchunks = (nks + 4 * KSW - 1) / (4 * KSW);

  for (int tb = 0; tb < cnt; tb += xrows_max) {
    const int live = min(NTT, (cnt - tb + 15) / 16);
    const int xrows = min(cnt - tb, xrows_max);
    const uint16_t* arow[NTT];
    dec_arows<NTT>(xs, xstride, xrows, xrows_max, arow);
    f32x4_t acca[NTT], accb[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) { acca[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; accb[tt] = acca[tt]; }
    for (int ch = 0; ch < nchunks; ++ch) {
      const int ks0 = ch * 4 * KSW + wave;
      if (ch == 0) {
        if (tb > 0) __syncthreads();  // the previous pass finished with the LDS tile
        stage_rows_lds<2, false>(xs, xstride, lds_plane, w.hplanes, (size_t)P * I, K, slot_rec, w.perm + off, tb,
                                 xrows, T, k);
        zero_tile_pad<2>(xs, xstride, lds_plane, K, dec_kcols(K), xrows_max, xrows);
      }
      WeightRegs<FMT, KSW> wa, wb;
      prefetch_weights2<FMT, KSW>(wa, pa, wb, pb, nkb, ks0, nks, n, g);
      if (ch == 0) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_le_lgkm0(2 * KSW * loads_per_step<FMT>()));
        __builtin_amdgcn_s_barrier();
        if constexpr (FMT == 4) dec_group_sums<2>(xsum, xs, xstride, lds_plane, K, 16 * NTT, xrows);
      }
#pragma unroll
      for (int i = 0; i < KSW; ++i) {
        const int ks = ks0 + 4 * i;
        mma_kstep<FMT, 2, NTT, KSW>(wa, i, ks, nks, arow, lds_plane, live, lut, ba, acca, xsum, nkb >> 1);
        mma_kstep<FMT, 2, NTT, KSW>(wb, i, ks, nks, arow, lds_plane, live, lut, bb, accb, xsum, nkb >> 1);
      }
    }
    mfma_settle_all(acca);
    mfma_settle_all(accb);
    float v[8 * NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) { v[8 * tt + q] = acca[tt][q]; v[8 * tt + 4 + q] = accb[tt][q]; }
    reduce4<8 * NTT>(v, (float*)smem);
    if (wave == 0) {
      const int col = 32 * x + n;
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int slot = tb + 16 * tt + 4 * g + q;
          if (slot < tb + xrows) {  // this pass's pairs only
            float* orow = w.o + (size_t)w.perm[off + slot] * H;
            __hip_atomic_store(&orow[col], v[8 * tt + q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&orow[col + 16], v[8 * tt + 4 + q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
    }
  }

  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&tickets[x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *is_last = (prev == (uint32_t)(n_active - 1));
  }
  __syncthreads();
  if (!*is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  dec_combine_cols(L, T, w, y, 32 * x, 32);
  if (threadIdx.x == 0) __hip_atomic_store(&tickets[x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// grid (H/32, slots): one block per (32-column tile, active expert)
template <int FMT, int NTT, int KSW>
__global__ __launch_bounds__(256, 3) void k_dec_down2(LayerArgs L, int T, Work w, float* __restrict__ y,
                                                      uint32_t* __restrict__ tickets, int xrows_max) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int is_last;
  __shared__ uint32_t s_lut[FMT == 2 ? 256 : 1];  // codebook table (CB4)
  const Slot* sr = w.slots + blockIdx.y;
  if (sr->cnt == 0) return;
  if (FMT == 2) build_cb4_lut(s_lut, L.codebook);  // ordered before use by the staging barrier
  dec_down2_item<FMT, NTT, KSW>(L, T, w, y, tickets, xrows_max, sr, blockIdx.x, smem, s_lut, &is_last);
}

// one token: grid (H/16, slots), one block per (16-column tile, active expert)
template <int FMT, int KSW>
__global__ __launch_bounds__(256, 3) void k_dec_down(LayerArgs L, Work w, float* __restrict__ y) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ uint32_t s_lut[FMT == 2 ? 256 : 1];  // codebook table (CB4)
  const Slot* sr = w.slots + blockIdx.y;
  if (sr->cnt == 0) return;
  if (FMT == 2) build_cb4_lut(s_lut, L.codebook);  // ordered before use by the staging barrier
  dec_down_t1_item<FMT, KSW>(L, w, y, sr, blockIdx.x, smem, s_lut);
}

// ---------------------------------------------------------------------------
// 4'. Down projection for short rows (K = I of at most 8 k-steps of 128 columns):
// instead of splitting K over the 4 waves, each wave owns one 16-row tile over the
// whole K, so a block covers 64 output columns with no split-K reduction.
// grid = (ceil(H/64), max active slots).  TICKETS: per 64 columns a ticket elects the
// last block, which sums y in the fixed order (few active experts); otherwise o is
// written plainly and a separate combine kernel follows (many active experts, where
// one ticket would take an atomic per expert on a single address).
// ---------------------------------------------------------------------------
template <int FMT, int NTT, int KSW, bool TICKETS>
__device__ __forceinline__ void dec_down_rows_item(const LayerArgs& L, int T, const Work& w, float* __restrict__ y,
                                                   uint32_t* __restrict__ tickets, int xrows_max,
                                                   const Slot* slot_rec, int x, int tb0, int tb_step,
                                                   uint8_t* smem, const uint32_t* lut, int* is_last) {
  const int cnt = slot_rec->cnt, off = slot_rec->off, n_active = slot_rec->n_active;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int H = L.H, I = L.I, k = L.k;
  const int P = T * k + (L.has_shared ? T : 0);
  const int K = I, nkb = K >> 5, nks = (nkb + 3) >> 2;
  const int xstride = dec_xstride(K);
  const size_t lds_plane = (size_t)(xrows_max + 1) * xstride;  // staged rows, then the zero row
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + dec_tile_bytes(K, 2, NTT, xrows_max));  // 3-bit affine
  const int tile = 4 * x + wave;  // this wave's 16 output columns
  const bool tile_ok = 16 * tile < H;
  const PackedTile pd = packed_tile<FMT>(slot_rec->down, H, K, tile_ok ? tile : 0);
  const uint32_t bd = FMT == 3 ? (uint32_t)pd.bases[n] : 0u;  // before the staging loads

  for (int tb = tb0; tb < cnt; tb += tb_step) {
    const int live = min(NTT, (cnt - tb + 15) / 16);
    const int xrows = min(cnt - tb, xrows_max);
    const uint16_t* arow[NTT];
    dec_arows<NTT>(xs, xstride, xrows, xrows_max, arow);
    f32x4_t acc[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (tb > tb0) __syncthreads();  // the previous pass finished with the LDS tile
    stage_rows_lds<2, false>(xs, xstride, lds_plane, w.hplanes, (size_t)P * I, K, slot_rec, w.perm + off, tb, xrows,
                             T, k);
    zero_tile_pad<2>(xs, xstride, lds_plane, K, dec_kcols(K), xrows_max, xrows);
    WeightRegs<FMT, KSW> wd;
    prefetch_weights<FMT, KSW>(wd, pd, nkb, 0, nks, n, g, 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_le_lgkm0(KSW * loads_per_step<FMT>()));
    __builtin_amdgcn_s_barrier();
    if constexpr (FMT == 4) dec_group_sums<2>(xsum, xs, xstride, lds_plane, K, 16 * NTT, xrows);
#pragma unroll
    for (int i = 0; i < KSW; ++i)
      mma_kstep<FMT, 2, NTT, KSW>(wd, i, i, nks, arow, lds_plane, live, lut, bd, acc, xsum, nkb >> 1);
    mfma_settle_all(acc);
    if (tile_ok) {
      const int col = 16 * tile + n;
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int slot = tb + 16 * tt + 4 * g + q;
          if (slot < tb + xrows) {  // this pass's pairs only
            float* dst = &w.o[(size_t)w.perm[off + slot] * H + col];
            if constexpr (TICKETS) __hip_atomic_store(dst, acc[tt][q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *dst = acc[tt][q];
          }
        }
    }
  }
  if constexpr (!TICKETS) return;

  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&tickets[x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *is_last = (prev == (uint32_t)(n_active - 1));
  }
  __syncthreads();
  if (!*is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  dec_combine_cols(L, T, w, y, 64 * x, 64);
  if (threadIdx.x == 0) __hip_atomic_store(&tickets[x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Short-row down projection kernel, grid (ceil(H/64), slots [x passes]).  TICKETS: one
// block row per slot (the ticket counts one arrival per active expert), all passes in the
// block; otherwise block row y takes pass y % npass of slot y / npass, rows past a slot's
// pairs exiting at once.
template <int FMT, int NTT, int KSW, bool TICKETS>
__global__ __launch_bounds__(256, 3) void k_dec_down_rows(LayerArgs L, int T, Work w, float* __restrict__ y,
                                                          uint32_t* __restrict__ tickets, int xrows_max, int nslots) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int is_last;
  __shared__ uint32_t s_lut[FMT == 2 ? 256 : 1];  // codebook table (CB4)
  const int npass = (int)gridDim.y / nslots;
  const Slot* sr = w.slots + blockIdx.y / npass;
  const int tb0 = (int)(blockIdx.y % npass) * xrows_max;
  if (tb0 >= sr->cnt) return;
  if (FMT == 2) build_cb4_lut(s_lut, L.codebook);  // ordered before use by the staging barrier
  dec_down_rows_item<FMT, NTT, KSW, TICKETS>(L, T, w, y, tickets, xrows_max, sr, blockIdx.x, tb0, npass * xrows_max,
                                             smem, s_lut, &is_last);
}

// k-steps per wave: the smallest supported count that covers a quarter of the row's
// 128-column steps (longer rows loop over chunks of 8).
static int pick_ksw(int K) {
  const int nks = (K / 32 + 3) / 4;
  const int per = (nks + 3) / 4;
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 6 ? 6 : 8;
}

// The routing debug outputs of a call (each may be null).
struct DbgOut {
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
};

template <int FMT, int NTT, int KSW, bool SR>
static void launch_gateup_sr(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, int xrows,
                             int max_items, const DbgOut& d, hipStream_t s, const Timing& tm) {
  const int nslots = min(T * L.k, L.E) + (L.has_shared ? 1 : 0);
  const dim3 g1(L.I / 16, SR ? nslots : max_items);
  if (x_dtype == 1)
    MOEQ_LAUNCH(tm, kStageGateUp, (k_dec_gateup<FMT, 1, NTT, KSW, SR>), g1, dim3(256),
                dec_lds_bytes(FMT, L.H, 1, NTT, xrows), s, L, T, w, (const uint16_t*)x, (size_t)0, xrows, nslots, d.ids,
                d.w, d.counts, d.offsets, d.perm);
  else
    MOEQ_LAUNCH(tm, kStageGateUp, (k_dec_gateup<FMT, 3, NTT, KSW, SR>), g1, dim3(256),
                dec_lds_bytes(FMT, L.H, 3, NTT, xrows), s, L, T, w, (const uint16_t*)w.xplanes, (size_t)T * L.H, xrows,
                nslots, d.ids, d.w, d.counts, d.offsets, d.perm);
}
template <int FMT, int NTT, int KSW>
static void launch_gateup_k(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, int xrows,
                            int max_items, bool sr, const DbgOut& d, hipStream_t s, const Timing& tm) {
  if (sr) launch_gateup_sr<FMT, NTT, KSW, true>(L, x, x_dtype, T, w, xrows, max_items, d, s, tm);
  else launch_gateup_sr<FMT, NTT, KSW, false>(L, x, x_dtype, T, w, xrows, max_items, d, s, tm);
}

// Down rows of at most this many 128-column k-steps take the short-row kernel (each wave
// one 16-row tile over the whole row: 64 rows, so more weight bytes, per block).
constexpr int kDownRowsMaxSteps = 8;

// Active slots above which the combine runs as its own kernel instead of ticketed.
constexpr int kTicketSlotsMax = 24;

template <int FMT, int NTT, int KSW>
static void launch_down_rows_k(const LayerArgs& L, int T, const Work& w, float* y, uint32_t* tickets, int xrows,
                               hipStream_t s, const Timing& tm) {
  const int slots = min(T * L.k, L.E) + (L.has_shared ? 1 : 0);
  const size_t lds = dec_lds_bytes(FMT, L.I, 2, NTT, xrows);
  if (slots <= kTicketSlotsMax) {
    MOEQ_LAUNCH(tm, kStageDown, (k_dec_down_rows<FMT, NTT, KSW, true>), dim3((L.H + 63) / 64, slots), dim3(256), lds,
                s, L, T, w, y, tickets, xrows, slots);
  } else {
    const int npass = (T + xrows - 1) / xrows;  // a slot holds at most T pairs
    MOEQ_LAUNCH(tm, kStageDown, (k_dec_down_rows<FMT, NTT, KSW, false>), dim3((L.H + 63) / 64, slots * npass),
                dim3(256), lds, s, L, T, w, y, tickets, xrows, slots);
    (void)launch_combine(L, T, w, y, s, tm);
  }
}

template <int FMT, int NTT, int KSW>
static void launch_down_k(const LayerArgs& L, int T, const Work& w, float* y, uint32_t* tickets, int xrows,
                          bool omb, hipStream_t s, const Timing& tm) {
  const int slots = min(T * L.k, L.E) + (L.has_shared ? 1 : 0);
  if (omb) {  // one token: the mailbox combine, one 16-row tile per block
    MOEQ_LAUNCH(tm, kStageDown, (k_dec_down<FMT, KSW>), dim3(L.H / 16, slots), dim3(256),
                dec_lds_bytes(FMT, L.I, 2, 1, 1), s, L, w, y);
    return;
  }
  // two row tiles per block from 2 tokens (at one token every block of the grid is resident
  // at once, and half as many blocks measured slower)
  MOEQ_LAUNCH(tm, kStageDown, (k_dec_down2<FMT, NTT, KSW>), dim3(L.H / 32, slots), dim3(256),
              dec_lds_bytes(FMT, L.I, 2, NTT, xrows), s, L, T, w, y, tickets, xrows);
}

// The one-token mailbox combine of the split-K down kernel: one token and long down rows
// (no block waits for another, so any grid size works).
static bool use_down_mailbox(const LayerArgs& L, int T) { return T == 1 && (L.I / 32 + 3) / 4 > kDownRowsMaxSteps; }

// Rows of activations a projection block stages per pass: as many of the expert's
// pairs as fit in the staging budget of LDS (at least 1, at most T), so that several
// blocks share a CU whatever T is; an expert with more pairs takes several passes.
// 48 KB lets 3 blocks share a CU.  The codebook gate/up kernel needs few enough registers
// for 4 blocks a CU (at most 128 per lane), so it stages within 36 KB: more of the verify
// window's 1,056 gate/up blocks run at once, for one staging pass more on its hottest
// expert (gate/up 20.4 -> 19.7 us; the 3-bit kernel measured slower so).
constexpr size_t kDecStageBytes = 48 * 1024;
constexpr size_t kDecStageBytesGateUpCb4 = 36 * 1024;
static size_t dec_gateup_stage_bytes(int wfmt) { return wfmt == 2 ? kDecStageBytesGateUpCb4 : kDecStageBytes; }
// The split-K down kernels (rows of more than 8 k-steps) stage their two h planes within
// 36 KB, so 4 blocks share a CU (their registers allow it): the stacked T = 4 down grid of
// 1,350 two-tile blocks then takes 1.3 rounds of the chip instead of 1.8; an expert with
// more pairs than a pass holds loops over passes inside its block.
constexpr size_t kDecStageBytesDownLong = 36 * 1024;
static size_t dec_down_stage_bytes(int I) {
  return (I / 32 + 3) / 4 > kDownRowsMaxSteps ? kDecStageBytesDownLong : kDecStageBytes;
}
static int dec_rows_per_pass(int K, int NP, int T, size_t budget = kDecStageBytes) {
  const size_t row = (size_t)dec_xstride(K) * 2 * NP;
  const int cap = (int)(budget / row) - 1;  // and the zero row
  return max(1, min(T, min(cap, kDecMaxTokens)));
}
// Bound on the gate/up work items (staging passes of xg pairs) over every routing of T
// tokens: A <= min(T k, E) routed experts holding at most T k pairs in all take at most
// sum ceil(c / xg) <= (T k + A (xg - 1)) / xg passes; the shared expert takes ceil(T / xg).
// At most T k + T: the workspace holds that many item records.
static int dec_max_items(const LayerArgs& L, int T, int xg) {
  const int pr = T * L.k, a = min(pr, L.E);
  return (pr + a * (xg - 1)) / xg + (L.has_shared ? (T + xg - 1) / xg : 0);
}

template <int FMT, int NTT>
static void launch_dec_gateup(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, int xrows,
                              int max_items, bool sr, const DbgOut& d, hipStream_t s, const Timing& tm) {
  switch (pick_ksw(L.H)) {
    case 1: launch_gateup_k<FMT, NTT, 1>(L, x, x_dtype, T, w, xrows, max_items, sr, d, s, tm); break;
    case 2: launch_gateup_k<FMT, NTT, 2>(L, x, x_dtype, T, w, xrows, max_items, sr, d, s, tm); break;
    case 4: launch_gateup_k<FMT, NTT, 4>(L, x, x_dtype, T, w, xrows, max_items, sr, d, s, tm); break;
    case 6: launch_gateup_k<FMT, NTT, 6>(L, x, x_dtype, T, w, xrows, max_items, sr, d, s, tm); break;
    default: launch_gateup_k<FMT, NTT, 8>(L, x, x_dtype, T, w, xrows, max_items, sr, d, s, tm); break;
  }
}

template <int FMT, int NTT>
static void launch_dec_down(const LayerArgs& L, int T, const Work& w, float* y, uint32_t* tickets, int xrows,
                            bool omb, hipStream_t s, const Timing& tm) {
  const int nks_dn = (L.I / 32 + 3) / 4;
  if (nks_dn <= kDownRowsMaxSteps) {  // short rows: one 16-row tile per wave over the whole K
    if (nks_dn <= 1) launch_down_rows_k<FMT, NTT, 1>(L, T, w, y, tickets, xrows, s, tm);
    else if (nks_dn <= 2) launch_down_rows_k<FMT, NTT, 2>(L, T, w, y, tickets, xrows, s, tm);
    else if (nks_dn <= 4) launch_down_rows_k<FMT, NTT, 4>(L, T, w, y, tickets, xrows, s, tm);
    else if (nks_dn <= 6) launch_down_rows_k<FMT, NTT, 6>(L, T, w, y, tickets, xrows, s, tm);
    else launch_down_rows_k<FMT, NTT, 8>(L, T, w, y, tickets, xrows, s, tm);
    return;
  }
  switch (pick_ksw(L.I)) {
    case 1: launch_down_k<FMT, NTT, 1>(L, T, w, y, tickets, xrows, omb, s, tm); break;
    case 2: launch_down_k<FMT, NTT, 2>(L, T, w, y, tickets, xrows, omb, s, tm); break;
    case 4: launch_down_k<FMT, NTT, 4>(L, T, w, y, tickets, xrows, omb, s, tm); break;
    case 6: launch_down_k<FMT, NTT, 6>(L, T, w, y, tickets, xrows, omb, s, tm); break;
    default: launch_down_k<FMT, NTT, 8>(L, T, w, y, tickets, xrows, omb, s, tm); break;
  }
}

// Token tiles per pass follow the rows staged per pass (16 or 32).
template <int FMT>
static hipError_t launch_dec_experts(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, float* y,
                                     uint32_t* tickets, bool omb, bool sr, int xg, int max_items, const DbgOut& d,
                                     hipStream_t s, const Timing& tm) {
  const int xd = dec_rows_per_pass(L.I, 2, T, dec_down_stage_bytes(L.I));
  if (xg <= 16) launch_dec_gateup<FMT, 1>(L, x, x_dtype, T, w, xg, max_items, sr, d, s, tm);
  else launch_dec_gateup<FMT, 2>(L, x, x_dtype, T, w, xg, max_items, false, d, s, tm);
  if (xd <= 16) launch_dec_down<FMT, 1>(L, T, w, y, tickets, xd, omb, s, tm);
  else launch_dec_down<FMT, 2>(L, T, w, y, tickets, xd, false, s, tm);
  return hipGetLastError();
}

bool decode_path_fits(const LayerArgs& L, int T, int x_dtype) {
  if (T > kDecMaxTokens) return false;
  const int np = x_dtype == 1 ? 1 : 3;
  const int xg = dec_rows_per_pass(L.H, np, T, dec_gateup_stage_bytes(L.wfmt));
  const int xd = dec_rows_per_pass(L.I, 2, T, dec_down_stage_bytes(L.I));
  const size_t g = dec_lds_bytes(L.wfmt, L.H, np, xg <= 16 ? 1 : 2, xg);
  const size_t d = dec_lds_bytes(L.wfmt, L.I, 2, xd <= 16 ? 1 : 2, xd);
  return g <= 160 * 1024 && d <= 160 * 1024;
}

template <int XDT>
static void launch_rr(const LayerArgs& L, const void* x, int T, int erows, const Work& w, int max_slots, int xg,
                      int max_items, int ntickets, int nzero_o, float eps, bool sr, int32_t* dbg_ids, float* dbg_w,
                      int32_t* dbg_counts, int32_t* dbg_offsets, int32_t* dbg_perm, hipStream_t s,
                      const Timing& tm) {
  const int rows = sr ? router_rows<false>() : router_rows<true>();
  const dim3 grid((erows + rows - 1) / rows);
  if (sr)  // logits only: the gate/up kernel routes
    MOEQ_LAUNCH(tm, kStageRouter, (k_dec_rr<XDT, false, false>), grid, dim3(kRouteThreads), 0, s, L, x, T, erows, w,
                max_slots, xg, max_items, w.rr_flags, ntickets, nzero_o, eps, nullptr, nullptr, nullptr, nullptr,
                nullptr);
  else if (T * (L.E + 1) <= kDecMailboxWords)
    MOEQ_LAUNCH(tm, kStageRouter, (k_dec_rr<XDT, true, true>), grid, dim3(kRouteThreads), 0, s, L, x, T, erows, w,
                max_slots, xg, max_items, w.rr_flags, ntickets, nzero_o, eps, dbg_ids, dbg_w, dbg_counts,
                dbg_offsets, dbg_perm);
  else
    MOEQ_LAUNCH(tm, kStageRouter, (k_dec_rr<XDT, false, true>), grid, dim3(kRouteThreads), 0, s, L, x, T, erows, w,
                max_slots, xg, max_items, w.rr_flags, ntickets, nzero_o, eps, dbg_ids, dbg_w, dbg_counts,
                dbg_offsets, dbg_perm);
}

hipError_t launch_decode(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, float* y, float eps,
                         int32_t* dbg_ids, float* dbg_w, int32_t* dbg_counts, int32_t* dbg_offsets,
                         int32_t* dbg_perm, hipStream_t s, const Timing& tm) {
  const int erows = L.E + ((L.has_shared && L.shared_gate_w) ? 1 : 0);
  const int ntickets = L.H / 16;
  const int max_slots = min(T * L.k, L.E) + (L.has_shared ? 1 : 0);
  const bool omb = use_down_mailbox(L, T);
  const int nzero_o = omb ? (L.k + (L.has_shared ? 1 : 0)) * L.H : 0;  // T == 1
  // x_dtype 2: x is the previous layer's fp32 y, and the layer takes its bf16 RMS rescale
  // in w.xr.  Below the split, when the rows fit the router block's LDS copy, the router
  // kernel rescales them (one launch fewer); otherwise the rescale kernel runs first.
  if (x_dtype == 2 && (T >= kDecSplitRouteT || T * L.H > kRmsFoldElems)) {
    hipError_t e = launch_rms_rescale((const float*)x, T, L.H, eps, w.xr, s);
    if (e != hipSuccess) return e;
    x = w.xr;
    x_dtype = 1;
  }
  const void* xp = x_dtype == 2 ? (const void*)w.xr : x;
  const int xdp = x_dtype == 2 ? 1 : x_dtype;
  // one token: the router kernel stores the logits and the gate/up blocks route themselves
  const bool sr = T == 1 && L.E <= kSelfRouteMaxE;
  const DbgOut d{dbg_ids, dbg_w, dbg_counts, dbg_offsets, dbg_perm};
  // the gate/up staging pass and the bound on its work items, for the route
  const int xg = dec_rows_per_pass(L.H, xdp == 1 ? 1 : 3, T, dec_gateup_stage_bytes(L.wfmt));
  const int max_items = dec_max_items(L, T, xg);
  if (T >= kDecSplitRouteT) {
    // the fp64 matrix-core router, then one wave per token for the top-k, the last block
    // to finish routing
    hipError_t e = launch_router(L, xp, xdp, T, w, s, tm);
    if (e != hipSuccess) return e;
    MOEQ_LAUNCH(tm, kStageTopk, k_dec_topk_route, dim3((T + 3) / 4), dim3(kTopkRouteThreads), 0, s, L, T, w,
                router_splits(T, L.H), max_slots, xg, max_items, ntickets, dbg_ids, dbg_w, dbg_counts, dbg_offsets,
                dbg_perm);
  } else if (x_dtype == 0) {
    launch_rr<0>(L, x, T, erows, w, max_slots, xg, max_items, ntickets, nzero_o, eps, sr, dbg_ids, dbg_w, dbg_counts,
                 dbg_offsets, dbg_perm, s, tm);
  } else if (x_dtype == 1) {
    launch_rr<1>(L, x, T, erows, w, max_slots, xg, max_items, ntickets, nzero_o, eps, sr, dbg_ids, dbg_w, dbg_counts,
                 dbg_offsets, dbg_perm, s, tm);
  } else {
    launch_rr<2>(L, x, T, erows, w, max_slots, xg, max_items, ntickets, nzero_o, eps, sr, dbg_ids, dbg_w, dbg_counts,
                 dbg_offsets, dbg_perm, s, tm);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (L.wfmt) {
    case 1: return launch_dec_experts<1>(L, xp, xdp, T, w, y, w.tickets, omb, sr, xg, max_items, d, s, tm);
    case 3: return launch_dec_experts<3>(L, xp, xdp, T, w, y, w.tickets, omb, sr, xg, max_items, d, s, tm);
    case 4: return launch_dec_experts<4>(L, xp, xdp, T, w, y, w.tickets, omb, sr, xg, max_items, d, s, tm);
    default: return launch_dec_experts<2>(L, xp, xdp, T, w, y, w.tickets, omb, sr, xg, max_items, d, s, tm);
  }
}

}  // namespace moeq
