// Decode path (few tokens per call, e.g. a draft/verify window of up to 17 tokens):
//   1. k_dec_router:   router logits, one expert row per block, loads issued up front;
//                      block 0 also clears the per-tile arrival counters of step 4.
//   2. k_dec_route:    one block: top-k + gates for every token, then the stable
//                      bucketing of the pairs and the active-expert list.
//   3. k_dec_gateup:   fused dequant + gate/up + SwiGLU per (16-row tile, active expert).
//   4. k_dec_down:     dequant + down per (16-row tile, active expert); the last block
//                      to finish a tile sums the gate-weighted expert outputs of that
//                      tile in a fixed order (routed j ascending, then shared), so no
//                      float atomics and a run-to-run identical result (NInfer
//                      Qwen3.8-Flash-Next page, MoE execution notes: one token's down
//                      runs over all its experts and the weighted sum must not depend
//                      on the order experts finish in).
// Each selected expert's weights are streamed from HBM exactly once per call, for all
// of its tokens (same page: one pass over each selected expert's rows for all of its
// tokens).  Weight loads for a wave's whole K range are issued before the first MFMA
// so that a wave keeps its full share of HBM requests in flight.
#include "device.h"
#include "launch.h"

namespace moeq {

constexpr int kDecKSW = 6;         // k-steps (of 128 columns) per wave per k-chunk
constexpr int kDecMaxTokens = 32;  // two 16-slot MFMA token tiles

__device__ __forceinline__ int dec_token_of_pair(int p, int T, int k) { return p < T * k ? p / k : p - T * k; }

// padded LDS row stride (in bf16 elements) with (stride/2) % 64 == 4 dwords
__host__ __device__ __forceinline__ int lds_row_stride(int K) {
  int dw = K / 2;
  int pad = (4 - (dw % 64) + 64) % 64;
  return 2 * (dw + pad);
}

// ---------------------------------------------------------------------------
// 1. Router logits (fp64 accumulation of exact products), one expert row per block,
//    4 waves splitting H.  x is read from global memory (tiny for decode batches).
// ---------------------------------------------------------------------------
template <int XDT>
__global__ __launch_bounds__(256) void k_dec_router(LayerArgs L, const void* __restrict__ x, int T, int erows,
                                                    double* __restrict__ logits, uint16_t* __restrict__ xplanes,
                                                    uint32_t* __restrict__ tickets, int ntickets) {
  __shared__ double part[4][kDecMaxTokens];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x;
  const int H = L.H;
  if (e == 0) {
    for (int i = threadIdx.x; i < ntickets; i += 256) tickets[i] = 0u;
  }
  if (XDT == 0 && e == 0) {
    const float* xf = (const float*)x;
    for (int idx = threadIdx.x; idx < T * H; idx += 256) {
      const float v = xf[idx];
      const uint32_t p0 = f32_to_bf16_rne(v);
      const float r1 = v - bf16_bits_to_f32(p0);
      const uint32_t p1 = f32_to_bf16_rne(r1);
      const uint32_t p2 = f32_to_bf16_rne(r1 - bf16_bits_to_f32(p1));
      xplanes[idx] = (uint16_t)p0;
      xplanes[(size_t)T * H + idx] = (uint16_t)p1;
      xplanes[(size_t)2 * T * H + idx] = (uint16_t)p2;
    }
  }
  const float* w = (e < L.E) ? L.router_w + (size_t)e * H : L.shared_gate_w;
  // wave `wave` owns float4 columns c = wave*64 + lane + 256*i
  constexpr int kMaxPer = 16;  // H <= 16384
  const int nf4 = H / 4;
  float4 wv[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = wave * 64 + lane + 256 * i;
    wv[i] = (c < nf4) ? *(const float4*)(w + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int t = 0; t < T; ++t) {
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int c = wave * 64 + lane + 256 * i;
      if (c < nf4) {
        float x0, x1, x2, x3;
        if (XDT == 0) {
          const float4 xv = *(const float4*)((const float*)x + (size_t)t * H + 4 * c);
          x0 = xv.x; x1 = xv.y; x2 = xv.z; x3 = xv.w;
        } else {
          const uint2 xb = *(const uint2*)((const uint16_t*)x + (size_t)t * H + 4 * c);
          x0 = bf16_bits_to_f32(xb.x & 0xFFFFu); x1 = bf16_bits_to_f32(xb.x >> 16);
          x2 = bf16_bits_to_f32(xb.y & 0xFFFFu); x3 = bf16_bits_to_f32(xb.y >> 16);
        }
        acc = fma((double)wv[i].x, (double)x0, acc);
        acc = fma((double)wv[i].y, (double)x1, acc);
        acc = fma((double)wv[i].z, (double)x2, acc);
        acc = fma((double)wv[i].w, (double)x3, acc);
      }
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) part[wave][t] = acc;
  }
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    double s = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
    if (e < L.E && L.router_b) s += (double)L.router_b[e];
    logits[(size_t)t * (L.E + 1) + e] = s;
  }
}

// ---------------------------------------------------------------------------
// 2. Top-k + gates + bucketing in one block (T <= kDecMaxTokens).
//    top-k: one wave per token, k rounds of a wave argmax (ties to the lower index);
//    gates: lane j < k computes exp(l_j - l_0), a wave sum normalises them (fp64);
//    buckets: integer counts, one wave-scan over the E+1 buckets of the packed pair
//    (count, non-empty flag), then each pair's stable rank among earlier pairs of
//    the same expert.
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 256;
constexpr int kMaxPairsDec = kDecMaxTokens * 16 + kDecMaxTokens;

__global__ __launch_bounds__(kRouteThreads) void k_dec_route(LayerArgs L, int T, const double* __restrict__ logits,
                                                             Work w, int32_t* __restrict__ dbg_ids,
                                                             float* __restrict__ dbg_w, int32_t* __restrict__ dbg_counts,
                                                             int32_t* __restrict__ dbg_offsets,
                                                             int32_t* __restrict__ dbg_perm) {
  __shared__ int s_exp[kMaxPairsDec];   // expert of each pair
  __shared__ double s_l[kMaxPairsDec];  // its logit (routed pairs)
  __shared__ int s_cnt[1024 + 1];
  __shared__ int s_incl[1024 + 1];      // inclusive scan: count (low 16 bits), non-empty flags (high)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = L.E, k = L.k;
  const int Pr = T * k;
  const int P = Pr + (L.has_shared ? T : 0);
  for (int i = tid; i <= E; i += kRouteThreads) s_cnt[i] = 0;

  for (int t = wave; t < T; t += kRouteThreads / 64) {
    const double* lt = logits + (size_t)t * (E + 1);
    double v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      v[i] = (e < E) ? lt[e] : 0.0;
    }
    uint32_t taken = 0;
    for (int j = 0; j < k; ++j) {
      double bv = 0.0;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !((taken >> i) & 1u) && (bi == 0x7FFFFFFF || v[i] > bv)) { bv = v[i]; bi = e; }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const double ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == 0) { s_exp[t * k + j] = bi; s_l[t * k + j] = bv; }
    }
    // gates: lane j < k
    const double l0 = s_l[t * k];
    const double z = lane < k ? exp(s_l[t * k + lane] - l0) : 0.0;
    const double zs = wave_sum_f64(z);
    if (lane < k) {
      const int p = t * k + lane;
      const float gte = (float)(z / zs);
      const int id = s_exp[p];
      w.ids[p] = id;
      w.pair_w[p] = gte;
      if (dbg_ids) dbg_ids[p] = id;
      if (dbg_w) dbg_w[p] = gte;
    }
    if (L.has_shared && lane == 0) {
      w.pair_w[Pr + t] = L.shared_gate_w ? (float)(1.0 / (1.0 + exp(-lt[E]))) : 1.0f;
      s_exp[Pr + t] = E;
    }
  }
  __syncthreads();
  for (int p = tid; p < P; p += kRouteThreads) atomicAdd(&s_cnt[s_exp[p]], 1);
  __syncthreads();
  const int nb = E + 1;
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < nb; base += 64) {
      const int i = base + lane;
      const int c = i < nb ? s_cnt[i] : 0;
      int x = c | ((c > 0 ? 1 : 0) << 16);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
      }
      x += carry;
      if (i < nb) s_incl[i] = x;
      carry = __shfl(x, 63, kWave);
    }
  }
  __syncthreads();
  for (int e = tid; e < nb; e += kRouteThreads) {
    const int c = s_cnt[e];
    const int off = (s_incl[e] & 0xFFFF) - c;
    w.counts[e] = c;
    w.offsets[e] = off;
    if (dbg_counts) dbg_counts[e] = c;
    if (dbg_offsets) dbg_offsets[e] = off;
    if (c > 0) w.active[1 + (s_incl[e] >> 16) - 1] = e;
  }
  if (tid == 0) {
    w.offsets[nb] = P;
    if (dbg_offsets) dbg_offsets[nb] = P;
    w.active[0] = s_incl[nb - 1] >> 16;
  }
  for (int p = tid; p < P; p += kRouteThreads) {
    const int e = s_exp[p];
    int r = 0;
    for (int q = 0; q < p; ++q) r += (s_exp[q] == e);
    const int pos = (s_incl[e] & 0xFFFF) - s_cnt[e] + r;
    w.perm[pos] = p;
    if (dbg_perm) dbg_perm[pos] = p;
  }
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
template <int FMT>
struct WeightRegs;

template <>
struct WeightRegs<1> {
  u32x4_t c[kDecKSW];
  uint32_t s[kDecKSW];
};
template <>
struct WeightRegs<2> {
  uint32_t c[kDecKSW][4];
  uint32_t s[kDecKSW][2];  // 4 fp16 scales of blocks 4ks..4ks+3
};

template <int FMT>
__device__ __forceinline__ void prefetch_weights(WeightRegs<FMT>& r, const uint8_t* codes_row,
                                                 const uint8_t* scales_row, int nkb, int ks0, int nks, int g) {
#pragma unroll
  for (int i = 0; i < kDecKSW; ++i) {
    const int ks = ks0 + 4 * i;
    if constexpr (FMT == 1) {
      const int kb = 4 * ks + g;
      const bool v = ks < nks && kb < nkb;
      r.c[i] = v ? __builtin_nontemporal_load((const u32x4_t*)(codes_row + (size_t)kb * 16)) : u32x4_t{0, 0, 0, 0};
      r.s[i] = v ? scales_row[kb] : 127u;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = 4 * ks + j;
        const bool v = ks < nks && kb < nkb;
        r.c[i][j] = v ? __builtin_nontemporal_load((const uint32_t*)(codes_row + (size_t)kb * 16 + 4 * g)) : 0u;
      }
      const uint16_t* sp = (const uint16_t*)scales_row;
      uint32_t s01 = 0, s23 = 0;
      if (ks < nks) {
        const int kb = 4 * ks;
        const uint32_t a = sp[kb];
        const uint32_t b = (kb + 1 < nkb) ? sp[kb + 1] : 0u;
        const uint32_t c = (kb + 2 < nkb) ? sp[kb + 2] : 0u;
        const uint32_t d = (kb + 3 < nkb) ? sp[kb + 3] : 0u;
        s01 = a | (b << 16);
        s23 = c | (d << 16);
      }
      r.s[i][0] = s01;
      r.s[i][1] = s23;
    }
  }
}

// acc[tt] += A(token tile tt, planes) x B(weights of k-step i) for one weight matrix.
// xrows = activation rows staged in LDS; A is zero for slots >= xrows and for k >= K.
template <int FMT, int NP, int NTT>
__device__ __forceinline__ void mma_kstep(const WeightRegs<FMT>& r, int i, int ks, int nkb, const uint16_t* xs,
                                          int xstride, size_t plane_stride, int live, int xrows,
                                          const uint32_t* lut, f32x4_t (&acc)[NTT]) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  if constexpr (FMT == 1) {
    const float sc = e8m0_to_f32(r.s[i]);
    const bool kval = 4 * ks + g < nkb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t b = fp4x8_to_bf16(r.c[i][j], sc);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        if (tt < live) {
          const bool ok = kval && (16 * tt + m < xrows);
          const uint16_t* ap = xs + (size_t)(ok ? 16 * tt + m : 0) * xstride + (ok ? 128 * ks + 32 * g + 8 * j : 0);
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            u32x4_t av = *(const u32x4_t*)(ap + p * plane_stride);
            if (!ok) av = u32x4_t{0, 0, 0, 0};
            acc[tt] = mfma_bf16(__builtin_bit_cast(bf16x8_t, av), b, acc[tt]);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (4 * ks + j < nkb) {
        const bf16x8_t b = cb4x8_to_bf16(r.c[i][j], lut);
        const uint32_t sbits = (r.s[i][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        const float sc = half_bits_to_f32((uint16_t)sbits);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          if (tt < live) {
            const bool ok = 16 * tt + m < xrows;
            const uint16_t* ap = xs + (size_t)(ok ? 16 * tt + m : 0) * xstride + 128 * ks + 32 * j + 8 * g;
            f32x4_t tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              u32x4_t av = *(const u32x4_t*)(ap + p * plane_stride);
              if (!ok) av = u32x4_t{0, 0, 0, 0};
              tmp = mfma_bf16(__builtin_bit_cast(bf16x8_t, av), b, tmp);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[tt][q] = fmaf(sc, tmp[q], acc[tt][q]);
          }
        }
      }
    }
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

// Sum the 4 waves' partial tiles (split-K) in wave order into wave 0.
template <int NV>
__device__ __forceinline__ void reduce4(float (&v)[NV], float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (wave > 0) {
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
// 3. Fused gate/up + SwiGLU.  grid = (I/16, max active slots), 4 waves split K.
// dynamic LDS: [NP][slots][xstride] bf16 activations, then the CB4 table.
// ---------------------------------------------------------------------------
template <int FMT, int NP, int NTT>
__global__ __launch_bounds__(256, 3) void k_dec_gateup(LayerArgs L, int T, Work w, const uint16_t* __restrict__ act,
                                                    size_t act_plane, int xrows_max) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int a = blockIdx.y;
  if (a >= w.active[0]) return;
  const int e = w.active[1 + a];
  const int cnt = w.counts[e], off = w.offsets[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int H = L.H, I = L.I, k = L.k;
  const int K = H, nkb = K >> 5, nks = (nkb + 3) >> 2;
  const int xstride = lds_row_stride(K);
  const int nslots = 16 * NTT;
  const size_t lds_plane = (size_t)xrows_max * xstride;
  uint32_t* lut = (uint32_t*)smem;
  uint16_t* xs = (uint16_t*)(smem + 1024);

  const uint8_t* base = L.gate_up[e];
  const size_t scale_off = ((size_t)2 * I * K / 2 + 255) / 256 * 256;
  const int rg = 16 * blockIdx.x + n, ru = I + rg;
  const int sb = FMT == 1 ? 1 : 2;

  // k-chunks of 4 waves x kDecKSW k-steps; weights of a chunk are prefetched first
  const int nchunks = (nks + 4 * kDecKSW - 1) / (4 * kDecKSW);
  f32x4_t accg[NTT], accu[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) { accg[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; accu[tt] = accg[tt]; }

  for (int tb = 0; tb < cnt; tb += nslots) {
    const int live = min(NTT, (cnt - tb + 15) / 16);
    const int xrows = min(cnt - tb, xrows_max);
    for (int ch = 0; ch < nchunks; ++ch) {
      WeightRegs<FMT> wg, wu;
      const int ks0 = ch * 4 * kDecKSW + wave;
      prefetch_weights<FMT>(wg, base + (size_t)rg * (K / 2), base + scale_off + (size_t)rg * nkb * sb, nkb, ks0,
                            nks, g);
      prefetch_weights<FMT>(wu, base + (size_t)ru * (K / 2), base + scale_off + (size_t)ru * nkb * sb, nkb, ks0,
                            nks, g);
      if (ch == 0) {
        __syncthreads();  // the previous pass finished with the LDS tile
        if (FMT == 2 && tb == 0) build_cb4_lut(lut, L.codebook);
        stage_rows<NP, true>(xs, xstride, lds_plane, act, act_plane, K, w.perm + off + tb, xrows, T, k);
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < kDecKSW; ++i) {
        const int ks = ks0 + 4 * i;
        if (ks < nks) {
          mma_kstep<FMT, NP, NTT>(wg, i, ks, nkb, xs, xstride, lds_plane, live, xrows, lut, accg);
          mma_kstep<FMT, NP, NTT>(wu, i, ks, nkb, xs, xstride, lds_plane, live, xrows, lut, accu);
        }
      }
    }
    // split-K reduction (fixed wave order), SwiGLU, two bf16 planes of h
    float v[8 * NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) { v[8 * tt + q] = accg[tt][q]; v[8 * tt + 4 + q] = accu[tt][q]; }
    reduce4<8 * NTT>(v, (float*)(smem + 1024));
    if (wave == 0) {
      const int P = T * k + (L.has_shared ? T : 0);
      const int col = 16 * blockIdx.x + n;
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int slot = tb + 16 * tt + 4 * g + q;
          if (slot < cnt) {
            const int p = w.perm[off + slot];
            const float h = silu_f32(v[8 * tt + q]) * v[8 * tt + 4 + q];
            const uint32_t hi = f32_to_bf16_rne(h);
            const uint32_t lo = f32_to_bf16_rne(h - bf16_bits_to_f32(hi));
            w.hplanes[(size_t)p * I + col] = (uint16_t)hi;
            w.hplanes[(size_t)P * I + (size_t)p * I + col] = (uint16_t)lo;
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) { accg[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; accu[tt] = accg[tt]; }
  }
}

// ---------------------------------------------------------------------------
// 4. Down projection + combine.  grid = (H/16, max active slots), 4 waves split K=I.
// Each block writes o_p[16 cols] for its expert's pairs; the last block to arrive
// at a column tile computes y[t][tile] for every token in a fixed order.
// ---------------------------------------------------------------------------
template <int FMT, int NTT>
__global__ __launch_bounds__(256, 3) void k_dec_down(LayerArgs L, int T, Work w, float* __restrict__ y,
                                                  uint32_t* __restrict__ tickets, int xrows_max) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int is_last;
  const int a = blockIdx.y;
  const int n_active = w.active[0];
  if (a >= n_active) return;
  const int e = w.active[1 + a];
  const int cnt = w.counts[e], off = w.offsets[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int H = L.H, I = L.I, k = L.k;
  const int P = T * k + (L.has_shared ? T : 0);
  const int K = I, nkb = K >> 5, nks = (nkb + 3) >> 2;
  const int xstride = lds_row_stride(K);
  const int nslots = 16 * NTT;
  const size_t lds_plane = (size_t)xrows_max * xstride;
  uint32_t* lut = (uint32_t*)smem;
  uint16_t* xs = (uint16_t*)(smem + 1024);

  const uint8_t* base = L.down[e];
  const size_t scale_off = ((size_t)H * K / 2 + 255) / 256 * 256;
  const int r = 16 * blockIdx.x + n;
  const int sb = FMT == 1 ? 1 : 2;
  const int nchunks = (nks + 4 * kDecKSW - 1) / (4 * kDecKSW);
  f32x4_t acc[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int tb = 0; tb < cnt; tb += nslots) {
    const int live = min(NTT, (cnt - tb + 15) / 16);
    const int xrows = min(cnt - tb, xrows_max);
    for (int ch = 0; ch < nchunks; ++ch) {
      WeightRegs<FMT> wd;
      const int ks0 = ch * 4 * kDecKSW + wave;
      prefetch_weights<FMT>(wd, base + (size_t)r * (K / 2), base + scale_off + (size_t)r * nkb * sb, nkb, ks0, nks,
                            g);
      if (ch == 0) {
        __syncthreads();
        if (FMT == 2 && tb == 0) build_cb4_lut(lut, L.codebook);
        stage_rows<2, false>(xs, xstride, lds_plane, w.hplanes, (size_t)P * I, K, w.perm + off + tb, xrows, T, k);
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < kDecKSW; ++i) {
        const int ks = ks0 + 4 * i;
        if (ks < nks) mma_kstep<FMT, 2, NTT>(wd, i, ks, nkb, xs, xstride, lds_plane, live, xrows, lut, acc);
      }
    }
    float v[4 * NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) v[4 * tt + q] = acc[tt][q];
    reduce4<4 * NTT>(v, (float*)(smem + 1024));
    if (wave == 0) {
      const int col = 16 * blockIdx.x + n;
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int slot = tb + 16 * tt + 4 * g + q;
          // write-through store (device coherence point), read back by the tile's last block
          if (slot < cnt)
            __hip_atomic_store(&w.o[(size_t)w.perm[off + slot] * H + col], v[4 * tt + q], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Arrival at this column tile; the last of the n_active blocks combines it.  The o
  // values were stored write-through (scope agent); waiting for their completion
  // before the ticket makes them visible to the last block's coherent loads, without
  // a full L2 write-back.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&tickets[blockIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == (uint32_t)(n_active - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  for (int idx = threadIdx.x; idx < T * 16; idx += 256) {
    const int t = idx >> 4;
    const int col = 16 * blockIdx.x + (idx & 15);
    float s = 0.f;
    for (int j = 0; j < k; ++j) {
      const float o = __hip_atomic_load(&w.o[(size_t)(t * k + j) * H + col], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s = fmaf(w.pair_w[t * k + j], o, s);
    }
    if (L.has_shared) {
      const float o = __hip_atomic_load(&w.o[(size_t)(T * k + t) * H + col], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s = fmaf(w.pair_w[T * k + t], o, s);
    }
    y[(size_t)t * H + col] = s;
  }
  if (threadIdx.x == 0) __hip_atomic_store(&tickets[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// LDS of a projection block: 1 KB codebook table, then the activation tile of
// xrows rows (NP planes), which the split-K reduction buffer later reuses.
static size_t dec_lds_bytes(int K, int NP, int NTT, int xrows) {
  const size_t x = (size_t)NP * xrows * lds_row_stride(K) * 2;
  const size_t red = (size_t)3 * 8 * NTT * 64 * 4;
  return 1024 + (x > red ? x : red);
}

template <int FMT, int NTT>
static hipError_t launch_dec_experts(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, float* y,
                                     uint32_t* tickets, hipStream_t s, const Timing& tm) {
  const int max_slots = min(T * L.k, L.E) + (L.has_shared ? 1 : 0);
  const dim3 g1(L.I / 16, max_slots), g2(L.H / 16, max_slots);
  const int xrows = min(T, 16 * NTT);  // an expert holds at most T pairs
  if (x_dtype == 1) {
    const size_t lds = dec_lds_bytes(L.H, 1, NTT, xrows);
    MOEQ_LAUNCH(tm, kStageGateUp, (k_dec_gateup<FMT, 1, NTT>), g1, dim3(256), lds, s, L, T, w,
                (const uint16_t*)x, (size_t)0, xrows);
  } else {
    const size_t lds = dec_lds_bytes(L.H, 3, NTT, xrows);
    MOEQ_LAUNCH(tm, kStageGateUp, (k_dec_gateup<FMT, 3, NTT>), g1, dim3(256), lds, s, L, T, w,
                (const uint16_t*)w.xplanes, (size_t)T * L.H, xrows);
  }
  const size_t lds2 = dec_lds_bytes(L.I, 2, NTT, xrows);
  MOEQ_LAUNCH(tm, kStageDown, (k_dec_down<FMT, NTT>), g2, dim3(256), lds2, s, L, T, w, y, tickets, xrows);
  return hipGetLastError();
}

bool decode_path_fits(const LayerArgs& L, int T, int x_dtype) {
  if (T > kDecMaxTokens) return false;
  const int NTT = T <= 16 ? 1 : 2;
  const size_t g = dec_lds_bytes(L.H, x_dtype == 1 ? 1 : 3, NTT, T);
  const size_t d = dec_lds_bytes(L.I, 2, NTT, T);
  return g <= 160 * 1024 && d <= 160 * 1024;
}

hipError_t launch_decode(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, float* y,
                         int32_t* dbg_ids, float* dbg_w, int32_t* dbg_counts, int32_t* dbg_offsets,
                         int32_t* dbg_perm, hipStream_t s, const Timing& tm) {
  const int erows = L.E + ((L.has_shared && L.shared_gate_w) ? 1 : 0);
  const int ntickets = L.H / 16;
  if (x_dtype == 0)
    MOEQ_LAUNCH(tm, kStageRouter, k_dec_router<0>, dim3(erows), dim3(256), 0, s, L, x, T, erows, w.logits,
                w.xplanes, w.tickets, ntickets);
  else
    MOEQ_LAUNCH(tm, kStageRouter, k_dec_router<1>, dim3(erows), dim3(256), 0, s, L, x, T, erows, w.logits,
                w.xplanes, w.tickets, ntickets);
  MOEQ_LAUNCH(tm, kStageTopk, k_dec_route, dim3(1), dim3(kRouteThreads), 0, s, L, T, (const double*)w.logits, w,
              dbg_ids, dbg_w, dbg_counts, dbg_offsets, dbg_perm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (T <= 16)
    return L.wfmt == 1 ? launch_dec_experts<1, 1>(L, x, x_dtype, T, w, y, w.tickets, s, tm)
                       : launch_dec_experts<2, 1>(L, x, x_dtype, T, w, y, w.tickets, s, tm);
  return L.wfmt == 1 ? launch_dec_experts<1, 2>(L, x, x_dtype, T, w, y, w.tickets, s, tm)
                     : launch_dec_experts<2, 2>(L, x, x_dtype, T, w, y, w.tickets, s, tm);
}

}  // namespace moeq
