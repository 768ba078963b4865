// Device-side helpers shared by the kernels of the MoE layer (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(3))) uint32_t u32x3_t;

// Global-memory views of pointers that come from memory (expert tables, slot records):
// loads through them compile to global_load (vector memory only) instead of flat_load,
// whose completion also counts against the LDS counter and forces full waits.
typedef const __attribute__((address_space(1))) uint8_t gbyte_t;
__device__ __forceinline__ gbyte_t* as_global(const void* p) { return (gbyte_t*)p; }

// ---- packed storage of one matrix [N][K] (N % 16 == 0, K % 32 == 0), tile-major ----
// Rows form tiles of 16 and a row's nkb = K/32 blocks form steps of 4 (the last step may
// hold r = nkb - 4s < 4 blocks).  Code unit (tile t, step s) starts at byte t*8K + 1024s
// and holds block g of the step for row m at (16g + m)*16, so the 64 lanes of a load with
// lane = 16g + m read one contiguous kilobyte.  The scale plane starts at
// round_up(N*K/2, 256); scale unit (t, s) starts at index t*16*nkb + 64s and holds MXFP4
// (g, m) at 16g + m, CB4 (m, g) at m*r + g (fp16, so 8 contiguous bytes per row and step).
// Keeping a 16-row step contiguous lets DRAM serve it from one open page.
// Packed scale store (format 3, MXFP4 codes): the scale plane is replaced, at the same
// offset S, by N base bytes in row order and then one 4-bit delta per block at the nibble
// whose index is the block's MXFP4 scale index (low nibble first); a block's E8M0 byte is
// base(row) + delta.  A tile's deltas start at byte S + N + t*8*nkb.
struct PackedTile {
  gbyte_t* codes;   // code unit (t, 0)
  gbyte_t* scales;  // scale unit (t, 0), bytes (format 3: the tile's first delta byte)
  gbyte_t* bases;   // format 3: the base bytes of the tile's 16 rows
};
// Formats: 1 MXFP4, 2 CB4, 3 MXFP4 with the packed scale store, 4 3-bit affine.
__host__ __device__ constexpr bool fmt_is_mx(int fmt) { return fmt == 1 || fmt == 3; }
// 3-bit affine (format 4, K % 128 == 0): tile t's code units (one per 128-column step s,
// 768 bytes, lane 16g + m's 12 bytes at 12 (16g + m)) start at t*6K; the scale plane at
// round_up(N*K*3/8, 256) holds per (t, s) 128 bytes, row m's (scale, bias) fp16 pairs of
// the step's two 64-column groups at 8m.
template <int FMT>
__device__ __forceinline__ PackedTile packed_tile(const void* base, int N, int K, int t) {
  gbyte_t* b = as_global(base);
  if constexpr (FMT == 4) {
    const size_t soff4 = ((size_t)N * K * 3 / 8 + 255) / 256 * 256;
    return {b + (size_t)t * 6 * K, b + soff4 + (size_t)t * K, nullptr};
  }
  const size_t soff = ((size_t)N * K / 2 + 255) / 256 * 256;
  if constexpr (FMT == 3)
    return {b + (size_t)t * 8 * K, b + soff + N + (size_t)t * 8 * (K / 32), b + soff + 16 * (size_t)t};
  return {b + (size_t)t * 8 * K, b + soff + (size_t)t * 16 * (K / 32) * (FMT == 1 ? 1 : 2), nullptr};
}
// block kb (< nkb) of row m of a tile: byte offset of its 16 code bytes in the tile
__device__ __forceinline__ uint32_t pk_code(int kb, int m) {
  return (uint32_t)(kb >> 2) * 1024u + (uint32_t)(((kb & 3) * 16 + m) * 16);
}
// its scale's index within the tile's scales (MXFP4 bytes / CB4 fp16 entries; in the
// packed scale store, the index of its delta nibble)
__device__ __forceinline__ uint32_t pk_scale_mx(int kb, int m) { return (uint32_t)(kb >> 2) * 64u + (kb & 3) * 16 + m; }
// E8M0 byte of a block in the packed scale store: the row's base plus the delta nibble
// (dbyte = the byte holding it, m = the row within its tile: even rows in the low nibble)
__device__ __forceinline__ uint32_t ps_e8m0(uint32_t base, uint32_t dbyte, int m) {
  return base + ((dbyte >> ((m & 1) * 4)) & 15u);
}
__device__ __forceinline__ uint32_t pk_scale_cb(int kb, int m, int nkb) {
  const int s = kb >> 2, r = min(4, nkb - 4 * s);
  return (uint32_t)s * 64u + (uint32_t)(m * r + (kb & 3));
}

// Layer descriptor as the kernels see it (copied by value into kernel arguments).
struct LayerArgs {
  int H, I, E, k, wfmt, has_shared;
  float omit_below;  // marginal-expert omission threshold (0: every routed pair kept)
  const float* router_w;
  const float* router_b;
  const uint8_t* const* gate_up;
  const uint8_t* const* down;
  const int8_t* codebook;
  const float* shared_gate_w;
};

struct Slot;

// Per-call scratch carved out of the caller's workspace.
struct Work {
  double* logits;      // [T][E + 1] (column E: shared-gate logit)
  int32_t* ids;        // [T][k]
  float* pair_w;       // [P]   gate of pair p (routed) or shared weight (p >= T*k)
  int32_t* counts;     // [E + 1]
  int32_t* offsets;    // [E + 2]
  int32_t* perm;       // [P]
  int32_t* active;     // [E + 2]  active[0] = number of active experts, then their ids ascending
  uint16_t* xplanes;   // [3][T][H] bf16 planes of fp32 activations (x = p0 + p1 + p2)
  uint16_t* hplanes;   // [2][P][I] bf16 planes of the SwiGLU output (h ~= p0 + p1)
  uint16_t* xr;        // [T][H] bf16 RMS rescale of the previous layer's y (rescaled-input calls)
  const float* resid;  // [T][H] fp32 added to y after the combine, or null
  float* o;            // [P][H]  expert outputs (down projection, before the gate)
  uint32_t* tickets;   // [H/16] arrival counters of the decode combine
  float* hf32;         // [P][I] SwiGLU output of the decode path (aliases hplanes)
  uint8_t* xq;         // MXFP4 prefill: fp8 planes [NPX][T][Hp] + [T] E8M0 row scales (aliases xplanes)
  uint8_t* hq;         // MXFP4 prefill: fp8 planes [3][P][Ip] + [P][Ip/256] E8M0 chunk scales (aliases hplanes)
  struct Slot* slots;  // [min(T*k, E) + 1] decode work records, one per active-expert slot
  struct Slot* items;  // [P] decode gate/up work items: one record per staging pass of an
                       // active expert (its pairs off .. off + cnt)
  int32_t* n_items;    // [1] number of valid entries of items
  int4* groups;        // prefill work groups: (expert, first bucket position, pairs <= 64, 0)
  int32_t* n_groups;   // [1] number of valid entries of groups
  uint32_t* rr_flags;  // decode router arrival flags, one per block: in the workspace's fixed
                       // header, zero between calls
  uint64_t* rr_mbox;   // decode router logit mailbox [T][E+1] (T (E+1) <= kDecMailboxWords): in
                       // the fixed header, zero between calls; a logit l is posted as ~bits(l)
};
// Words of the decode router's logit mailbox.  ~bits(l) is never 0: that needs the
// all-ones NaN, which fp64 arithmetic on fp32/bf16 data does not produce.
constexpr int kDecMailboxWords = 2048;

// Pairs per prefill work group (four 16-row MFMA token tiles).
constexpr int kGroupPairs = 64;
// Upper bound of the number of prefill groups: every non-empty bucket adds at most one
// partial group to the P / kGroupPairs full ones.
__host__ __device__ inline int max_groups(int P, int E) { return P / kGroupPairs + E + 2; }

// One active expert of a decode call: everything a projection block needs, in one
// 128-byte record (scalar loads).  cnt == 0 marks an unused slot.  rows[] holds the
// first kSlotRows pair ids of the expert's bucket (the rest are read from perm).
constexpr int kSlotRows = 24;
struct __align__(128) Slot {
  int32_t e, cnt, off, n_active;
  const uint8_t* gate_up;
  const uint8_t* down;
  int32_t rows[kSlotRows];
};
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// IEEE fp16 bits -> fp32 (exact, subnormals included).
__device__ __forceinline__ float half_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Round-to-nearest-even fp64 -> bf16 bits, for finite v that is 0 or of magnitude in the
// bf16 normal range: the fraction is rounded at bf16's last kept bit (bit 45 of the fp64
// fraction) on the integer bits, and the result, having 8 significant bits, converts to
// fp32 exactly.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
  constexpr uint64_t kDrop = (1ull << 45) - 1;  // fraction bits below bf16's seventh
  uint64_t b = __builtin_bit_cast(uint64_t, v);
  b = (b + (kDrop >> 1) + ((b >> 45) & 1ull)) & ~kDrop;
  return __float_as_uint((float)__builtin_bit_cast(double, b)) >> 16;
}

// ---- RMS rescale between stacked layers: x = bf16_rne(y / sqrt(mean(y^2) + eps)) ----
// One thread's share of a row's sum of squares, n = i, i + 256, ... (fp64: every square
// of an fp32 value is exact; the sum rounds in this order).  A row is summed by 256
// threads (4 waves), the wave sums added in wave order; the rescale kernel and the
// router kernel that folds the rescale in both use exactly these steps.
__device__ __forceinline__ double rms_partial(const float* __restrict__ yt, int H, int i) {
  double s = 0.0;
  // 8 loads in flight per batch; a slot past the row adds fma(0, 0, s) = s exactly, so the
  // sum is the in-order sum over n = i, i + 256, ...
  for (int n0 = i; n0 < H; n0 += 8 * 256) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = n0 + 256 * u < H ? yt[n0 + 256 * u] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) s = fma((double)v[u], (double)v[u], s);
  }
  return s;
}
// Rows of at most this many columns keep a thread's values in registers from the sum of
// squares to the quotient (16 per thread of 256), so the row is read once.
constexpr int kRmsRegCols = 16 * 256;
// rms_partial of a row of at most kRmsRegCols columns, its values kept in v: all 16 loads
// are issued at once (slots past the row read as 0), then summed in the same order as
// rms_partial, so the result is bit-identical.
__device__ __forceinline__ double rms_partial_keep(const float* __restrict__ yt, int H, int i, float (&v)[16]) {
#pragma unroll
  for (int u = 0; u < 16; ++u) v[u] = i + 256 * u < H ? yt[i + 256 * u] : 0.0f;
  double s = 0.0;
#pragma unroll
  for (int u = 0; u < 16; ++u) s = fma((double)v[u], (double)v[u], s);
  return s;
}
__device__ __forceinline__ double rms_divisor(double s0, double s1, double s2, double s3, int H, float eps) {
  return sqrt((((s0 + s1) + s2) + s3) / (double)H + (double)eps);
}
// The fp64 quotient y / d (correctly rounded), then rounded to bf16.  rd = 1 / d in fp64:
// y * rd lies within 2 ulp of the quotient, so both round to the same bf16 unless the
// product's 45 dropped bits are within 8 ulp of the midpoint between two bf16 values;
// only then is the quotient itself computed.  The result is the bf16 of y / d, bit for bit.
__device__ __forceinline__ uint16_t rms_apply(float y, double d, double rd) {
  double q = (double)y * rd;
  const int64_t dropped = (int64_t)(__builtin_bit_cast(uint64_t, q) & ((1ull << 45) - 1));
  const bool near = dropped - (1ll << 44) <= 8 && (1ll << 44) - dropped <= 8;
  if (__ballot(near)) {  // a wave-uniform branch: the division runs only where it can matter
    if (near) q = (double)y / d;
  }
  return (uint16_t)f64_to_bf16_rne(q);
}
// rms_apply of 8 values of a row: n = i + stride u (u < 8, those below H), loads first.
__device__ __forceinline__ void rms_apply8(const float* __restrict__ y, int i, int stride, int n_end, double d,
                                           double rd, uint16_t (&out)[8]) {
  float v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = i + stride * u < n_end ? y[i + stride * u] : 0.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u) out[u] = rms_apply(v[u], d, rd);
}

// ---- cross-lane helpers on DPP row rotations (a few cycles each) plus readlane ----
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __builtin_bit_cast(long long, v);
  const int lo = dpp_i32<CTRL>((int)(b & 0xFFFFFFFFll));
  const int hi = dpp_i32<CTRL>((int)(b >> 32));
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long b = __builtin_bit_cast(long long, v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}
constexpr int kDppRowRor1 = 0x121, kDppRowRor2 = 0x122, kDppRowRor4 = 0x124, kDppRowRor8 = 0x128;

// Sum over the 64 lanes, returned to every lane; fixed association order.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<kDppRowRor1>(v);
  v += dpp_f64<kDppRowRor2>(v);
  v += dpp_f64<kDppRowRor4>(v);
  v += dpp_f64<kDppRowRor8>(v);  // every lane of a 16-lane row holds the row sum
  return ((readlane_f64(v, 0) + readlane_f64(v, 16)) + readlane_f64(v, 32)) + readlane_f64(v, 48);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __builtin_bit_cast(float, dpp_i32<kDppRowRor1>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, dpp_i32<kDppRowRor2>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, dpp_i32<kDppRowRor4>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, dpp_i32<kDppRowRor8>(__builtin_bit_cast(int, v)));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return ((r0 + r1) + r2) + r3;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  v += dpp_i32<kDppRowRor1>(v);
  v += dpp_i32<kDppRowRor2>(v);
  v += dpp_i32<kDppRowRor4>(v);
  v += dpp_i32<kDppRowRor8>(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}

// Softmax gate of routed pair j = lane (< k) of one token: lj its logit, l0 the token's
// largest: g_j = exp(lj - l0) / sum_j' exp(l_j' - l0) in fp64.  With omit_below > 0
// (uniform) a pair j > 0 whose g_j is below omit_below (decided in fp64) is omitted: it
// gets gate 0 and false is returned; the kept gates are renormalised over the kept pairs,
// exp(lj - l0) / sum over kept.  Every lane of the wave calls this.
__device__ __forceinline__ bool pair_gate(double lj, double l0, int k, float omit_below, float* g) {
  const int lane = threadIdx.x & 63;
  const double z = lane < k ? exp(lj - l0) : 0.0;
  const double zs = wave_sum_f64(z);
  bool keep = lane < k;
  double zk = zs;
  if (omit_below > 0.0f) {
    keep = keep && (lane == 0 || z / zs >= (double)omit_below);
    zk = wave_sum_f64(keep ? z : 0.0);
  }
  *g = keep ? (float)(z / zk) : 0.0f;
  return keep;
}

// ---- top-k of NT tokens per wave (NT = 1 or 2, processed side by side) -------------------
// Lane l holds the candidates e = l + 64 i, i < NPER, of each token as selection keys,
// sorted once; every round takes the wave maximum of the lanes' heads and the lane holding
// it moves up its next candidate.
// ---- top-k on 64-bit selection keys ----
// key(v, e): the fp64 bits of v mapped to an unsigned integer of the same order (sign
// bit flipped for v >= 0, all bits inverted for v < 0), with the low 10 bits replaced
// by 1023 - e.  A larger key is a larger logit, and on equal upper bits the lower
// expert index; so one unsigned maximum picks the winner, exact ties going to the lower
// index.  Two logits that differ only in the 10 dropped bits (less than 2^-42 of their
// magnitude) also order by index.  Key 0 marks an empty candidate (E <= 1024).
__device__ __forceinline__ uint64_t topk_key(double v, int e) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t o = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return (o & ~1023ull) | (uint64_t)(1023 - e);
}
__device__ __forceinline__ int topk_key_index(uint64_t key) { return 1023 - (int)(key & 1023ull); }
// The logit a key stands for (its dropped low bits zero in the key's order).
__device__ __forceinline__ double topk_key_value(uint64_t key) {
  const uint64_t o = key & ~1023ull;
  const uint64_t b = (o >> 63) ? (o & 0x7FFFFFFFFFFFFFFFull) : ~o;
  return __builtin_bit_cast(double, b);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
// Maximum over the wave of 32-bit unsigned values: every lane's row maximum by DPP row
// rotations, then the maximum of the four rows'.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
  m = max(m, (uint32_t)dpp_i32<kDppRowRor1>((int)m));
  m = max(m, (uint32_t)dpp_i32<kDppRowRor2>((int)m));
  m = max(m, (uint32_t)dpp_i32<kDppRowRor4>((int)m));
  m = max(m, (uint32_t)dpp_i32<kDppRowRor8>((int)m));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)m, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)m, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)m, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)m, 48);
  return max(max(a, b), max(c, d));
}
// Maximum over the wave of distinct 64-bit keys: the high words' maximum H, then the low
// word of the one lane holding H or, when several lanes hold it, the maximum of their low
// words.  32-bit steps are half the instructions of 64-bit compares and selects.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
  const uint32_t H = wave_max_u32(hi);
  const uint64_t tied = __ballot(hi == H);
  uint32_t L;
  if (__popcll(tied) == 1)  // uniform
    L = (uint32_t)__builtin_amdgcn_readlane((int)lo, __ffsll((long long)tied) - 1);
  else
    L = wave_max_u32(hi == H ? lo : 0u);
  return ((uint64_t)H << 32) | L;
}
// Descending order of a lane's candidates (odd-even transposition, static indices).
template <int NPER>
__device__ __forceinline__ void sort_lane(uint64_t (&v)[NPER]) {
#pragma unroll
  for (int pass = 0; pass < NPER; ++pass) {
#pragma unroll
    for (int i = pass & 1; i + 1 < NPER; i += 2) {
      const uint64_t hi = max_u64(v[i], v[i + 1]), lo = v[i] > v[i + 1] ? v[i + 1] : v[i];
      v[i] = hi;
      v[i + 1] = lo;
    }
  }
}
// Selection of the top k of NT tokens from each lane's candidate logits lv[t][i] (expert
// e = lane + 64 i; entries with e >= E are ignored).  Token t's selections go to
// s_exp/s_l[slot[t] * k + j] (written by lane 0), j = 0 .. k-1 in selection order.
template <int NPER, int NT>
__device__ __forceinline__ void topk_select(const double (&lv)[NT][NPER], int E, int k, const int (&slot)[NT],
                                            int* s_exp, double* s_l) {
  const int lane = threadIdx.x & 63;
  uint64_t v[NT][NPER];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = lane + 64 * i;
      v[t][i] = e < E ? topk_key(lv[t][i], e) : 0ull;
    }
#pragma unroll
  for (int t = 0; t < NT; ++t) sort_lane<NPER>(v[t]);
  // lane j keeps the j-th selection; the selections are written once, after the rounds
  uint64_t sel[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) sel[t] = 0ull;
  for (int j = 0; j < k; ++j) {
    uint64_t m[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) m[t] = wave_max_key(v[t][0]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sel[t] = lane == j ? m[t] : sel[t];
      if (v[t][0] == m[t]) {  // keys are unique: exactly one lane moves up its next candidate
#pragma unroll
        for (int i = 0; i + 1 < NPER; ++i) v[t][i] = v[t][i + 1];
        v[t][NPER - 1] = 0ull;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (lane < k) {
      s_exp[slot[t] * k + lane] = topk_key_index(sel[t]);
      s_l[slot[t] * k + lane] = topk_key_value(sel[t]);
    }
  }
}

// Top-k of NT tokens whose logits are in memory ([T][E + 1] rows).  COHERENT: they were
// written by other blocks of the running kernel (device-scope loads).
// The logits may come as nsplit <= MAXS partial sums (a K-split router), split z at
// logits + z * split_stride; every split is loaded before any is added (clamped split
// index: no branch around the loads), and they are added in z order.
template <int NPER, int NT, bool COHERENT, int MAXS = 1>
__device__ __forceinline__ void topk_tokens(const double* __restrict__ logits, int E, int k, const int (&tok)[NT],
                                            const int (&slot)[NT], int* s_exp, double* s_l, int nsplit = 1,
                                            size_t split_stride = 0) {
  const int lane = threadIdx.x & 63;
  double part[NT][NPER][MAXS];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      // every lane loads (index clamped into the row): no branch around the loads
      const int e = lane + 64 * i;
      const double* src = logits + (size_t)tok[t] * (E + 1) + min(e, E - 1);
#pragma unroll
      for (int z = 0; z < MAXS; ++z) {
        const double* sz = src + (size_t)min(z, nsplit - 1) * split_stride;
        part[t][i][z] = COHERENT ? __hip_atomic_load(sz, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *sz;
      }
    }
  double lv[NT][NPER];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      lv[t][i] = part[t][i][0];
#pragma unroll
      for (int z = 1; z < MAXS; ++z) lv[t][i] = z < nsplit ? lv[t][i] + part[t][i][z] : lv[t][i];
    }
  topk_select<NPER, NT>(lv, E, k, slot, s_exp, s_l);
}

// 3-bit affine: the 16 bf16 pairs (128 + q) of one lane's 12 code bytes of a step, pair
// P = 4j + d holding values i = 2d, 2d+1 of MFMA j (columns 32j + 8g + i).  Pairs 0..14
// sit at bits 3 (P % 5) and 16 + 3 (P % 5) of word P / 5; pair 15's bit k is bit 15 (and
// 31) of word k.  0x4300 | q is the bf16 of 128 + q (q < 8 sits in the mantissa), so one
// shift and one and-or make a pair.
__device__ __forceinline__ void aff3_pairs(const u32x3_t w, uint32_t (&o)[16]) {
#pragma unroll
  for (int P = 0; P < 15; ++P) o[P] = ((w[P / 5] >> (3 * (P % 5))) & 0x00070007u) | 0x43004300u;
  o[15] = ((w[0] >> 15) & 0x00010001u) | ((w[1] >> 14) & 0x00020002u) | ((w[2] >> 13) & 0x00040004u) | 0x43004300u;
}

// E8M0 byte -> fp32 2^(u-127) (u = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t u) {
  return __uint_as_float(u == 0 ? 0x00400000u : (u << 23));
}

// Four E2M1 code bytes (8 values, element 2j in the low nibble of byte j) times a
// power-of-two scale, as 8 bf16 values.  Exact: E2M1 values carry two significant
// bits and the scale only shifts the exponent.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t codes, float scale) {
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  bf16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Four codebook-index bytes -> 8 bf16 codebook values through a 256-entry LDS table
// whose entry b packs (codebook[b & 15], codebook[b >> 4]).  int8 values are exact
// in bf16.
// Byte I of c times 4 (the byte offset of table entry c.byte[I]) in one instruction: a
// shift whose source operand selects the byte (SDWA).  Pure register arithmetic.
template <int I>
__device__ __forceinline__ uint32_t byte_x4(uint32_t c) {
  uint32_t r;
  if constexpr (I == 0)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(c));
  else if constexpr (I == 1)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(c));
  else if constexpr (I == 2)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(c));
  else
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(c));
  return r;
}
__device__ __forceinline__ bf16x8_t cb4x8_to_bf16(uint32_t codes, const uint32_t* lut) {
  const uint8_t* t = (const uint8_t*)lut;
  u32x4_t v;
  v[0] = *(const uint32_t*)(t + byte_x4<0>(codes));
  v[1] = *(const uint32_t*)(t + byte_x4<1>(codes));
  v[2] = *(const uint32_t*)(t + byte_x4<2>(codes));
  v[3] = *(const uint32_t*)(t + byte_x4<3>(codes));
  return __builtin_bit_cast(bf16x8_t, v);
}

// 4 x 4 transpose of dwords across the four 16-lane rows of a wave: on return, register
// j of row g holds what register g of row j held.  v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second, v_permlane16_swap the odd
// rows of the first with the even rows of the second.
__device__ __forceinline__ void xpose_rows4(u32x4_t& d) {
  const auto a = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto e = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  d = u32x4_t{c[0], c[1], e[0], e[1]};
}

// bf16 bits of an int8 value (exact).
__device__ __forceinline__ uint32_t int8_to_bf16_bits(int v) {
  return __float_as_uint((float)v) >> 16;
}

__device__ __forceinline__ void build_cb4_lut(uint32_t* lut, const int8_t* codebook) {
  for (int b = threadIdx.x; b < 256; b += blockDim.x) {
    uint32_t lo = int8_to_bf16_bits(codebook[b & 15]);
    uint32_t hi = int8_to_bf16_bits(codebook[b >> 4]);
    lut[b] = lo | (hi << 16);
  }
}

// Matrix-core results about to be read by vector, LDS or memory instructions.  Such reads
// need idle cycles after the MFMA that the hardware does not enforce: measured on gfx950,
// at least 7 for 16x16x32 bf16 and 11 for the scaled 16x16x128 fp8/fp4; with the
// compiler's minimum spacing (mostly scalar instructions in between) reads have returned
// stale registers.  The asm takes the results as read-write operands, so no read can move
// above it, and idles 16 (SETTLE_SHORT) or 24 cycles.
#define MOEQ_SETTLE_ASM "s_nop 7\n\ts_nop 7\n\ts_nop 7"
#define MOEQ_SETTLE_SHORT_ASM "s_nop 7\n\ts_nop 7"
template <typename A>
__device__ __forceinline__ void mfma_settle(A& a) {
  asm volatile(MOEQ_SETTLE_ASM : "+v"(a));
}
template <typename A, typename B>
__device__ __forceinline__ void mfma_settle(A& a, B& b) {
  asm volatile(MOEQ_SETTLE_ASM : "+v"(a), "+v"(b));
}
template <typename A>
__device__ __forceinline__ void mfma_settle4(A (&t)[4], bool short_wait = false) {
  if (short_wait) asm volatile(MOEQ_SETTLE_SHORT_ASM : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]));
  else asm volatile(MOEQ_SETTLE_ASM : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]));
}
// every element of an accumulator array, all operands of one asm (so that it follows every
// MFMA that produces them)
template <typename A, int N>
__device__ __forceinline__ void mfma_settle_all(A (&t)[N]) {
  static_assert(N == 1 || N == 2 || N == 4, "1, 2 or 4 accumulators");
  if constexpr (N == 1) mfma_settle(t[0]);
  else if constexpr (N == 2) mfma_settle(t[0], t[1]);
  else mfma_settle4(t);
}
// a [4][NTT] accumulator block (NTT <= 4)
template <typename A, int NTT>
__device__ __forceinline__ void mfma_settle_block(A (&t)[4][NTT]) {
  static_assert(NTT >= 1 && NTT <= 4, "up to 4 token tiles");
  if constexpr (NTT == 1)
    asm volatile(MOEQ_SETTLE_ASM : "+v"(t[0][0]), "+v"(t[1][0]), "+v"(t[2][0]), "+v"(t[3][0]));
  else if constexpr (NTT == 2)
    asm volatile(MOEQ_SETTLE_ASM : "+v"(t[0][0]), "+v"(t[1][0]), "+v"(t[2][0]), "+v"(t[3][0]), "+v"(t[0][1]),
                 "+v"(t[1][1]), "+v"(t[2][1]), "+v"(t[3][1]));
  else if constexpr (NTT == 3)
    asm volatile(MOEQ_SETTLE_ASM : "+v"(t[0][0]), "+v"(t[1][0]), "+v"(t[2][0]), "+v"(t[3][0]), "+v"(t[0][1]),
                 "+v"(t[1][1]), "+v"(t[2][1]), "+v"(t[3][1]), "+v"(t[0][2]), "+v"(t[1][2]), "+v"(t[2][2]),
                 "+v"(t[3][2]));
  else
    asm volatile(MOEQ_SETTLE_ASM : "+v"(t[0][0]), "+v"(t[1][0]), "+v"(t[2][0]), "+v"(t[3][0]), "+v"(t[0][1]),
                 "+v"(t[1][1]), "+v"(t[2][1]), "+v"(t[3][1]), "+v"(t[0][2]), "+v"(t[1][2]), "+v"(t[2][2]),
                 "+v"(t[3][2]), "+v"(t[0][3]), "+v"(t[1][3]), "+v"(t[2][3]), "+v"(t[3][3]));
}

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + expf(-a)); }

}  // namespace moeq
