// Expert projections on bucketed pairs: fused dequant + gate/up + SwiGLU, the down
// projection, and the fixed-order gate-weighted combine.
//
// Each selected expert's rows are read once for all of its tokens (NInfer
// Qwen3.8-Flash-Next page, MoE execution notes: one pass over each selected
// expert's rows for all of its tokens, a fused gate/up kernel per block of rows of
// one expert, and a down pass that sums one token's experts in a fixed order).
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, D[16][16] += A[16][32] * B[32][16]):
//   A = activations: 16 token slots of one expert x 32 k values, bf16 planes;
//   B = weights:     32 k values x 16 weight rows, decoded in registers;
//   lane l supplies A[l%16][8(l/16) .. +7] and B[8(l/16) .. +7][l%16] and holds
//   D[4(l/16) + i][l%16], i = 0..3.
// Decoded weights are exact in bf16:
//   MXFP4: e2m1 * 2^(u-127) (two significant bits), the block scale folded in;
//   CB4:   the int8 codebook value; the fp16 block scale multiplies the fp32 MFMA
//          result of that 32-wide block (the product scale*value needs up to 18
//          bits and is not exact in bf16).
// Activations are exact bf16 sums of planes: bf16 x is one plane, fp32 x three
// planes (hi + mid + lo, exact), and the SwiGLU output h two planes (hi + lo,
// relative error <= 2^-17).  So every product is exact and only the fp32
// accumulation rounds.
// A block = 4 waves that split the K loop (k-step ks = wave, wave+4, ...) and
// reduce their partial tiles through LDS in a fixed order, so results are
// deterministic run to run.
#include "device.h"
#include "launch.h"

namespace moeq {

constexpr int kMaxTokTiles = 4;  // token slots per pass = 16 * NTT

__device__ __forceinline__ int token_of_pair(int p, int T, int k) { return p < T * k ? p / k : p - T * k; }

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)p);
}

__device__ __forceinline__ bf16x8_t zero_bf16x8() { return __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0}); }

// One 16-row weight tile (rows wrow0 .. wrow0+15 of the packed matrix `base`, K cols)
// against up to NTT*16 activation rows; NW weight tiles share the activations (gate
// and up for the fused kernel).  acc[w][tt] is the D tile of weight tile w, token
// tile tt.  act_rows[tt] is this lane's activation row index (-1 = empty slot).
template <int FMT, int NP, int NTT, int NW>
__device__ __forceinline__ void tile_mma(const uint8_t* const* bases, const int* wrow0, int nrows_total, int K,
                                         const uint16_t* act, size_t plane_stride, const int* act_rows,
                                         int ntiles_live, const uint32_t* lut, f32x4_t (&acc)[NW][NTT]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int nkb = K >> 5;
  const int nks = (nkb + 3) >> 2;
  const size_t scale_off = ((size_t)nrows_total * K / 2 + 255) / 256 * 256;
  const uint8_t* codes[NW];
  const uint8_t* scales[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const size_t row = (size_t)(wrow0[w] + n);
    codes[w] = bases[w] + row * (K / 2);
    scales[w] = bases[w] + scale_off + row * nkb * (FMT == 1 ? 1 : 2);
  }
  for (int ks = wave; ks < nks; ks += 4) {
    if (FMT == 1) {
      // MXFP4: lane group g owns the whole block kb = 4ks+g of its row; MFMA j takes
      // values 8j..8j+7 of it, so A must supply x[32kb + 8j .. +7] for the same g.
      const int kb = 4 * ks + g;
      const bool kv = kb < nkb;
      u32x4_t cw[NW];
      float sw[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        cw[w] = kv ? *(const u32x4_t*)(codes[w] + (size_t)kb * 16) : u32x4_t{0, 0, 0, 0};
        sw[w] = kv ? e8m0_to_f32(scales[w][kb]) : 1.0f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t b[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) b[w] = fp4x8_to_bf16(cw[w][j], sw[w]);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          if (tt < ntiles_live) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const int r = act_rows[tt];
              const bf16x8_t a = (kv && r >= 0)
                  ? load_bf16x8(act + p * plane_stride + (size_t)r * K + 32 * kb + 8 * j)
                  : zero_bf16x8();
#pragma unroll
              for (int w = 0; w < NW; ++w) acc[w][tt] = mfma_bf16(a, b[w], acc[w][tt]);
            }
          }
        }
      }
    } else {
      // CB4: MFMA j covers block kb = 4ks+j entirely (K = 32 = one block); lane group g
      // supplies quarter g (bytes 4g..4g+3) of that block, A supplies x[32kb + 8g ..].
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = 4 * ks + j;
        if (kb >= nkb) break;
        bf16x8_t b[NW];
        float sw[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const uint32_t cq = *(const uint32_t*)(codes[w] + (size_t)kb * 16 + 4 * g);
          b[w] = cb4x8_to_bf16(cq, lut);
          const uint16_t sb = *(const uint16_t*)(scales[w] + 2 * (size_t)kb);
          sw[w] = half_bits_to_f32(sb);
        }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          if (tt < ntiles_live) {
            f32x4_t tmp[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) tmp[w] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < NP; ++p) {
              const int r = act_rows[tt];
              const bf16x8_t a = (r >= 0) ? load_bf16x8(act + p * plane_stride + (size_t)r * K + 32 * kb + 8 * g)
                                          : zero_bf16x8();
#pragma unroll
              for (int w = 0; w < NW; ++w) tmp[w] = mfma_bf16(a, b[w], tmp[w]);
            }
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[w][tt][i] = fmaf(sw[w], tmp[w][i], acc[w][tt][i]);
          }
        }
      }
    }
  }
}

// Sum the 4 waves' partial tiles in wave order into wave 0's registers.
template <int NW, int NTT>
__device__ __forceinline__ void reduce_waves(f32x4_t (&acc)[NW][NTT], float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NV = NW * NTT * 4;
  if (wave > 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((wave - 1) * NV + (w * NTT + tt) * 4 + i) * 64 + lane] = acc[w][tt][i];
  }
  __syncthreads();
  if (wave == 0) {
    for (int src = 0; src < 3; ++src) {
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[w][tt][i] += red[(src * NV + (w * NTT + tt) * 4 + i) * 64 + lane];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Fused gate/up + SwiGLU.  grid = (I/16 row tiles, active-expert slots).
// h_p[i] = silu(gate_i . x_t) * (up_i . x_t), stored as two bf16 planes.
// ---------------------------------------------------------------------------
template <int FMT, int NP, int NTT>
__global__ __launch_bounds__(256) void k_gateup(LayerArgs L, int T, Work w, const uint16_t* __restrict__ act,
                                                size_t act_plane_stride) {
  __shared__ float red[3 * 2 * NTT * 4 * 64];
  __shared__ uint32_t lut[256];
  const int a = blockIdx.y;
  const int n_active = w.active[0];
  if (a >= n_active) return;
  if (FMT == 2) {
    build_cb4_lut(lut, L.codebook);
    __syncthreads();
  }
  const int e = w.active[1 + a];
  const int cnt = w.counts[e], off = w.offsets[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int I = L.I, H = L.H, k = L.k;
  const int P = T * k + (L.has_shared ? T : 0);
  const uint8_t* base = L.gate_up[e];
  const uint8_t* bases[2] = {base, base};
  const int wrow0[2] = {16 * (int)blockIdx.x, I + 16 * (int)blockIdx.x};

  for (int tb = 0; tb < cnt; tb += 16 * NTT) {
    int rows[NTT];
    const int live = min(NTT, (cnt - tb + 15) / 16);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const int slot = tb + 16 * tt + (lane & 15);
      rows[tt] = slot < cnt ? token_of_pair(w.perm[off + slot], T, k) : -1;
    }
    f32x4_t acc[2][NTT];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) acc[q][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    tile_mma<FMT, NP, NTT, 2>(bases, wrow0, 2 * I, H, act, act_plane_stride, rows, live, lut, acc);
    reduce_waves<2, NTT>(acc, red);
    if (wave == 0) {
      const int col = 16 * blockIdx.x + (lane & 15);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = tb + 16 * tt + 4 * (lane >> 4) + i;
          if (slot < cnt) {
            const int p = w.perm[off + slot];
            const float h = silu_f32(acc[0][tt][i]) * acc[1][tt][i];
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

// ---------------------------------------------------------------------------
// Down projection.  grid = (H/16 row tiles, active-expert slots).
// o_p[n] = Wd[n,:] . h_p  (fp32, before the gate).
// ---------------------------------------------------------------------------
template <int FMT, int NTT>
__global__ __launch_bounds__(256) void k_down(LayerArgs L, int T, Work w) {
  __shared__ float red[3 * 1 * NTT * 4 * 64];
  __shared__ uint32_t lut[256];
  const int a = blockIdx.y;
  const int n_active = w.active[0];
  if (a >= n_active) return;
  if (FMT == 2) {
    build_cb4_lut(lut, L.codebook);
    __syncthreads();
  }
  const int e = w.active[1 + a];
  const int cnt = w.counts[e], off = w.offsets[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int I = L.I, H = L.H, k = L.k;
  const int P = T * k + (L.has_shared ? T : 0);
  const uint8_t* bases[1] = {L.down[e]};
  const int wrow0[1] = {16 * (int)blockIdx.x};

  for (int tb = 0; tb < cnt; tb += 16 * NTT) {
    int rows[NTT];
    const int live = min(NTT, (cnt - tb + 15) / 16);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const int slot = tb + 16 * tt + (lane & 15);
      rows[tt] = slot < cnt ? w.perm[off + slot] : -1;  // h rows are indexed by pair
    }
    f32x4_t acc[1][NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[0][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    tile_mma<FMT, 2, NTT, 1>(bases, wrow0, H, I, w.hplanes, (size_t)P * I, rows, live, lut, acc);
    reduce_waves<1, NTT>(acc, red);
    if (wave == 0) {
      const int col = 16 * blockIdx.x + (lane & 15);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = tb + 16 * tt + 4 * (lane >> 4) + i;
          if (slot < cnt) w.o[(size_t)w.perm[off + slot] * H + col] = acc[0][tt][i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: y[t][n] = sum_j pair_w[t*k+j] * o[t*k+j][n] (+ pair_w[T*k+t] * o[T*k+t][n]),
// j ascending and the shared expert last, a fixed order for every run.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(int T, int H, int k, int has_shared, const float* __restrict__ o,
                                                 const float* __restrict__ pair_w, float* __restrict__ y) {
  const int t = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= H) return;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s = fmaf(pair_w[t * k + j], o[(size_t)(t * k + j) * H + n], s);
  if (has_shared) s = fmaf(pair_w[T * k + t], o[(size_t)(T * k + t) * H + n], s);
  y[(size_t)t * H + n] = s;
}

// ---------------------------------------------------------------------------
template <int FMT, int NTT>
static void launch_experts_fmt(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w,
                               int max_slots, hipStream_t s, const Timing& tm) {
  dim3 g1(L.I / 16, max_slots), g2(L.H / 16, max_slots);
  if (x_dtype == 1)
    MOEQ_LAUNCH(tm, kStageGateUp, (k_gateup<FMT, 1, NTT>), g1, dim3(256), 0, s, L, T, w, (const uint16_t*)x,
                (size_t)0);
  else
    MOEQ_LAUNCH(tm, kStageGateUp, (k_gateup<FMT, 3, NTT>), g1, dim3(256), 0, s, L, T, w,
                (const uint16_t*)w.xplanes, (size_t)T * L.H);
  MOEQ_LAUNCH(tm, kStageDown, (k_down<FMT, NTT>), g2, dim3(256), 0, s, L, T, w);
}

hipError_t launch_experts(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, float* y,
                          hipStream_t s, const Timing& tm) {
  const int max_slots = min(T * L.k, L.E) + (L.has_shared ? 1 : 0);
  const int ntt = T <= 16 ? 1 : (T <= 32 ? 2 : 4);
  if (L.wfmt == 1) {
    if (ntt == 1) launch_experts_fmt<1, 1>(L, x, x_dtype, T, w, max_slots, s, tm);
    else if (ntt == 2) launch_experts_fmt<1, 2>(L, x, x_dtype, T, w, max_slots, s, tm);
    else launch_experts_fmt<1, 4>(L, x, x_dtype, T, w, max_slots, s, tm);
  } else {
    if (ntt == 1) launch_experts_fmt<2, 1>(L, x, x_dtype, T, w, max_slots, s, tm);
    else if (ntt == 2) launch_experts_fmt<2, 2>(L, x, x_dtype, T, w, max_slots, s, tm);
    else launch_experts_fmt<2, 4>(L, x, x_dtype, T, w, max_slots, s, tm);
  }
  MOEQ_LAUNCH(tm, kStageCombine, k_combine, dim3((L.H + 255) / 256, T), dim3(256), 0, s, T, L.H, L.k,
              L.has_shared, (const float*)w.o, (const float*)w.pair_w, y);
  return hipGetLastError();
}

}  // namespace moeq
