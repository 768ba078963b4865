// Prefill path: grouped GEMMs over the bucketed (token, expert) pairs.
//
// Work unit: a group = up to 64 consecutive bucket positions of one expert (the
// bucketing kernel lists them in bucket order).  A block of 8 waves covers 512 weight
// rows of that expert for the group's pairs; every wave owns a 64-row x 64-pair tile
// (4 x 4 tiles of v_mfma_f32_16x16x32_bf16) over the whole K range, so there is no
// split-K reduction.  In the fused gate/up kernel a wave holds 32 gate rows and the 32
// matching up rows, so SwiGLU is applied in registers.  Each selected expert's rows
// are read from HBM once per group (once in total when it has at most 64 pairs), the
// grouping the NInfer Qwen3.8-Flash-Next page describes for its MoE execution (pairs
// grouped by expert, one pass over each selected expert's rows for all its tokens).
//
// Pipeline (k-step = 128 columns):
//   - activations: the group's 64 rows are copied into LDS one k-step chunk at a time
//     (direct global->LDS loads; the 16-byte pieces of a row are XOR-swizzled by row so
//     that the MFMA operand reads hit 16 distinct bank groups), D-1 chunks ahead, in D
//     rotating buffers;
//   - weights: each wave streams its own rows' codes into a register ring D k-steps
//     ahead; MXFP4 block scales (one 64-byte unit per row tile and k-step) are copied
//     into LDS for the block's 32 row tiles, D k-steps at a time, by one direct
//     global->LDS load per wave, into two alternating buffers (a byte load per lane and
//     row tile per k-step would cost as many memory instructions as the codes);
//   - only the activation rows of the group's live 16-row token tiles are staged;
//   - the k loop is unrolled by D, so ring slots and buffers are compile-time indices
//     and the wait before each step is a constant vmcnt (every wave issues the same
//     number of loads per step; loads past the row end re-read a real block that is
//     then masked, so nothing outside the matrices is touched).
// Operands as in the decode kernels: A = activation rows (bf16 planes, exact), B =
// decoded weights (MXFP4 with its E8M0 scale folded in, exact; CB4 codebook values,
// with the fp16 block scale applied to each 32-column block's fp32 MFMA result).
#include "device.h"
#include "launch.h"

namespace moeq {

constexpr int kPfWaves = 8;  // waves per block (eight 64-row wave tiles: 512 weight rows)

constexpr int kPfRowBytes = 256;                         // one staged row chunk: 128 bf16
constexpr int kPfPlaneBytes = kGroupPairs * kPfRowBytes;  // 16 KB per plane per buffer

// CB4 decode table at LDS offset 0, in one of two forms:
//  - replicated, one copy per lane: the entry for code byte b (two bf16 values) of lane
//    l sits at byte 256 b + 4 l, so the 64 lanes of a lookup always hit 64 distinct
//    dword slots of one 256-byte row, whatever their code bytes (no bank conflicts),
//    and a lookup address is one byte permute of the code word; 64 KB;
//  - a single 1 KB copy (lookups conflict by chance) where the 64 KB do not fit beside
//    the activation buffers.
constexpr int kPfLutReplBytes = 256 * 64 * 4;
constexpr int kPfLdsMax = 160 * 1024;

__host__ __device__ constexpr bool pf_lut_repl(int fmt, int np, int d) {
  return fmt == 2 && kPfLutReplBytes + d * np * kPfPlaneBytes + 4 * kGroupPairs <= kPfLdsMax;
}
__host__ __device__ constexpr int pf_lut_bytes(int fmt, int np, int d) {
  return fmt != 2 ? 0 : pf_lut_repl(fmt, np, d) ? kPfLutReplBytes : 1024;
}
// MXFP4 scale buffers: two groups of D k-steps; group buffer = 8 waves x 1 KB, step u
// of the group at 2 KB u, row tile (wave w, tile rt) at 64 (4 w + rt) inside it.
constexpr int kPfScaleGroupBytes = 8 * 1024;
__host__ __device__ constexpr int pf_scale_lds_bytes(int fmt) { return fmt == 1 ? 2 * kPfScaleGroupBytes : 0; }
// LUT, then the D x NP activation buffers, then the MXFP4 scale buffers, then the
// group's 64 pair ids.
__host__ __device__ constexpr int pf_lds_bytes(int fmt, int np, int d) {
  return pf_lut_bytes(fmt, np, d) + d * np * kPfPlaneBytes + pf_scale_lds_bytes(fmt);
}
__host__ __device__ constexpr int pf_lds_total(int fmt, int np, int d) {
  return pf_lds_bytes(fmt, np, d) + 4 * kGroupPairs;
}

__device__ __forceinline__ void pf_build_lut(uint32_t* lut, const int8_t* codebook) {
  for (int i = threadIdx.x; i < 256 * 64; i += blockDim.x) {
    const int b = i >> 6;
    lut[i] = int8_to_bf16_bits(codebook[b & 15]) | (int8_to_bf16_bits(codebook[b >> 4]) << 16);
  }
}

// Eight CB4 values (one code word) -> bf16: byte i of the code word indexes row i of the
// table; the address is (code byte << 8) | (4 lane), assembled by v_perm_b32 from the
// code word (high source) and the lane offset (low source).
__device__ __forceinline__ bf16x8_t pf_cb4x8(uint32_t codes, uint32_t lane_off) {
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t addr = __builtin_amdgcn_perm(codes, lane_off, 0x0C0C0000u | ((4u + i) << 8));
    v[i] = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)addr;
  }
  return __builtin_bit_cast(bf16x8_t, v);
}

// s_waitcnt immediate: at most n vector-memory operations of this wave outstanding.
__host__ __device__ constexpr int pf_vm_le(int n) {
  return ((n > 63 ? 63 : n) & 15) | (7 << 4) | (15 << 8) | (((n > 63 ? 63 : n) >> 4) << 14);
}

// Weight registers of one k-step for the wave's 4 row tiles.
// SCL (CB4 only): 1 = the 4 block scales of a row arrive in one 8-byte load (K % 128 == 0),
//                 0 = four 2-byte loads.
template <int FMT, int SCL>
struct PfStep;
template <int SCL>
struct PfStep<1, SCL> {
  u32x4_t c[4];  // the scales are staged in LDS
};
template <>
struct PfStep<2, 0> {
  uint32_t c[4][4];
  uint32_t s[4][4];
};
template <>
struct PfStep<2, 1> {
  uint32_t c[4][4];
  uint64_t s[4];  // fp16 scale bits of blocks 4ks..4ks+3, block j in bits 16j..16j+15
};
template <int FMT, int SCL>
__host__ __device__ constexpr int pf_loads_per_step() {
  return FMT == 1 ? 4 : (SCL ? 20 : 32);
}

__device__ __forceinline__ void pf_load_lds_16(gbyte_t* gptr, void* lds) {
  const uint32_t lds_addr =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(gptr) : "memory");
}

// Loads of k-step ks (clamped to the last step: such registers are never used).  A block
// past the row end re-reads the row's last block (masked at use).  For a full step the
// 64 lanes of one code load read one contiguous kilobyte of the tile-major storage.
template <int FMT, int SCL>
__device__ __forceinline__ void pf_load_step(PfStep<FMT, SCL>& r, const PackedTile (&pt)[4], int ks, int nks,
                                             int nkb, int m, int g) {
  const int kc = ks < nks ? ks : nks - 1;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    if constexpr (FMT == 1) {
      const int kb = min(4 * kc + g, nkb - 1);
      r.c[rt] = __builtin_nontemporal_load(
          (const __attribute__((address_space(1))) u32x4_t*)(pt[rt].codes + pk_code(kb, m)));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = min(4 * kc + j, nkb - 1);
        r.c[rt][j] = __builtin_nontemporal_load(
            (const __attribute__((address_space(1))) uint32_t*)(pt[rt].codes + pk_code(kb, m) + 4 * g));
      }
      if constexpr (SCL == 1) {  // every step holds 4 blocks: row m's 4 scales are 8 contiguous bytes
        r.s[rt] = *(const __attribute__((address_space(1))) uint64_t*)(pt[rt].scales + (size_t)128 * kc + 8 * m);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kb = min(4 * kc + j, nkb - 1);
          r.s[rt][j] = *(const __attribute__((address_space(1))) uint16_t*)(pt[rt].scales + 2 * pk_scale_cb(kb, m, nkb));
        }
      }
    }
  }
}

// Branch-free: all 4 row tiles are computed (a row tile past the matrix holds clamped
// real rows whose results are not stored) and NTT token tiles are live.
// sb (MXFP4): this lane's scale byte of row tile 0 for step ks in LDS (tile rt at +64 rt).
template <int FMT, int NP, int SCL, int NTT, bool REPL>
__device__ __forceinline__ void pf_mma_step(const PfStep<FMT, SCL>& r, const uint8_t* xb, int ks, int nkb,
                                            uint32_t lane_off, const uint32_t* lut, const uint8_t* sb,
                                            f32x4_t (&acc)[4][NTT]) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  if constexpr (FMT == 1) {
    const bool kval = 4 * ks + g < nkb;
    float sc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) sc[rt] = e8m0_to_f32(sb[64 * rt]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8_t b[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) b[rt] = fp4x8_to_bf16(kval ? r.c[rt][j] : 0u, sc[rt]);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const bf16x8_t a = *(const bf16x8_t*)(xb + p * kPfPlaneBytes + (16 * tt + m) * kPfRowBytes +
                                                16 * ((4 * g + j) ^ m));
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) acc[rt][tt] = mfma_bf16(a, b[rt], acc[rt][tt]);
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // a block past the row adds 0 x (finite products); with 8-byte scale loads K is a
      // multiple of 128 and every block of a step is real
      const bool kval = SCL == 1 || 4 * ks + j < nkb;
      {
        bf16x8_t b[4];
        float sc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          if constexpr (REPL) b[rt] = pf_cb4x8(r.c[rt][j], lane_off);
          else b[rt] = cb4x8_to_bf16(r.c[rt][j], lut);
          uint32_t sb;
          if constexpr (SCL == 1) sb = (uint32_t)(r.s[rt] >> (16 * j));
          else sb = r.s[rt][j];
          sc[rt] = kval ? half_bits_to_f32((uint16_t)(sb & 0xFFFFu)) : 0.0f;
        }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          f32x4_t tmp[4];
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) tmp[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const bf16x8_t a = *(const bf16x8_t*)(xb + p * kPfPlaneBytes + (16 * tt + m) * kPfRowBytes +
                                                  16 * ((4 * j + g) ^ m));
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) tmp[rt] = mfma_bf16(a, b[rt], tmp[rt]);
          }
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[rt][tt][q] = fmaf(sc[rt], tmp[rt][q], acc[rt][tt][q]);
        }
      }
    }
  }
}

__device__ __forceinline__ int pf_token_of_pair(int p, int T, int k) { return p < T * k ? p / k : p - T * k; }

// Per-block state of one projection, shared by the token-tile specialisations.
struct PfCtx {
  PackedTile tile[4];      // the wave's 4 row tiles (uniform)
  gbyte_t* src[4];         // activation source rows of this lane's staging loads (16/W of them)
  int piece[4];            // byte offset of this lane's 16-byte piece in a staged row chunk
  uint8_t* xs;             // LDS activation buffers [D][NP][64 rows][256 B]
  uint32_t lane_off;       // 4 x lane: this lane's column of the replicated CB4 table
  const uint32_t* lut;     // the CB4 table (LDS offset 0)
  int start;               // the group's first bucket position
  const int* s_pair;       // the group's pair ids in LDS (when they fit there)
  gbyte_t* ssrc;           // MXFP4: scale unit (this lane's staging tile, step 0) + 16 x chunk
  uint8_t* sbuf;           // MXFP4: LDS scale buffers
  int sstep;               // MXFP4: the step of a D-step group whose scales this wave stages
  int schunk;              // MXFP4: this lane's 16-byte chunk (block g) of a scale unit
  int soff;                // MXFP4: this lane's scale byte of its row tile 0 in a staged step
  size_t act_plane_bytes;
  int nks, nkb, row_bytes, wave, g, m;
  uint32_t rt_mask;
};

// Copy staged chunk s (clamped to the last one) of the group's rows into buffer buf: the
// one-kilobyte loads per plane (4 rows each) are spread over the W waves, this wave
// taking u = wave + W q, q < NQ (16 / W loads cover all 64 rows; fewer cover the rows of
// the live token tiles).
template <int NP, int W, int NQ>
__device__ __forceinline__ void pf_stage(const PfCtx& c, int s, int buf) {
  const int sc = s < c.nks ? s : c.nks - 1;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    int off = kPfRowBytes * sc + c.piece[q];
    off = off + 16 <= c.row_bytes ? off : 0;  // past the row end: real data, never used
#pragma unroll
    for (int p = 0; p < NP; ++p)
      pf_load_lds_16(c.src[q] + p * c.act_plane_bytes + off,
                     c.xs + (buf * NP + p) * kPfPlaneBytes + (c.wave + W * q) * 1024);
  }
}

// Stage the MXFP4 scales of steps s..s+D-1 (clamped to the last step) of the block's 32
// row tiles into group buffer par: one 1 KB load per wave, wave w taking step w/2 of the
// group (a wave past the group's steps re-reads its last step into its own slice) and
// the 16 tiles 16 (w & 1).. of it, 4 lanes per 64-byte unit.  Chunks past a partial
// last unit re-read chunk 0 of it (those blocks are masked at use).
template <int D>
__device__ __forceinline__ void pf_stage_scales(const PfCtx& c, int s, int par) {
  const int st = min(s + c.sstep, c.nks - 1);
  const int nb = min(4, c.nkb - 4 * st);
  const int ch = c.schunk < nb ? c.schunk : 0;
  pf_load_lds_16(c.ssrc + 64 * st + 16 * (ch - c.schunk), c.sbuf + par * kPfScaleGroupBytes + c.wave * 1024);
}

// The vmcnt wait at the start of the k-step in ring slot U that covers chunk s: chunk s
// was staged D-1 steps earlier and was followed by that step's weights and by D-2 whole
// steps (chunk + weights, plus the scale load of a slot-0 step, which precedes its chunk).
template <int FMT, int SCL, int D, int NQNP>
__host__ __device__ constexpr int pf_wait_count(int U) {
  int n = pf_loads_per_step<FMT, SCL>();
  for (int v = 2; v < D; ++v) n += NQNP + pf_loads_per_step<FMT, SCL>() + ((FMT == 1 && (U + v) % D == 0) ? 1 : 0);
  return n;
}

// Marks a ring slot's registers as produced here: the compiler may not move their uses
// (or its own waits for them) above this point, which keeps the uses of slot U inside
// step U instead of hoisting them to the loop head where the later slots are in flight.
template <int SCL>
__device__ __forceinline__ void pf_pin(PfStep<1, SCL>& r) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) asm volatile("" : "+v"(r.c[rt]));
}
__device__ __forceinline__ void pf_pin(PfStep<2, 0>& r) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(r.c[rt][j]), "+v"(r.s[rt][j]));
}
__device__ __forceinline__ void pf_pin(PfStep<2, 1>& r) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(r.c[rt][j]));
    asm volatile("" : "+v"(r.s[rt]));
  }
}

// Activation staging loads per wave per plane and k-step for NTT live token tiles.
template <int W, int NTT>
__host__ __device__ constexpr int pf_nq() {
  return (4 * NTT + W - 1) / W < 16 / W ? (4 * NTT + W - 1) / W : 16 / W;
}

// One k-step (s = a multiple of D plus U): wait for chunk s, stage (in a slot-0 step) the
// MXFP4 scales of the next D-step group and chunk s+D-1 into buffers every wave has
// finished with, MFMAs, then the weights of step s+D into the ring slot just consumed.
// The wait covers chunk s and every load issued before it (this wave's weights of step s
// and the scales of step s's group); the barrier then makes every wave's staged data
// visible and frees the buffers of step s-1.  Straight-line code: every wave issues the
// same loads at every step, so the wait is a constant.
template <int FMT, int NP, int D, int SCL, int NTT, int U, int W>
__device__ __forceinline__ void pf_kstep(const PfCtx& c, PfStep<FMT, SCL> (&ring)[D], int s, f32x4_t (&acc)[4][NTT]) {
  constexpr int NQ = pf_nq<W, NTT>();
  constexpr int kWait = pf_wait_count<FMT, SCL, D, NQ * NP>(U);
  static_assert(kWait <= 63, "too many loads in flight for the vmcnt counter");
  __builtin_amdgcn_s_waitcnt(pf_vm_le(kWait));
  __builtin_amdgcn_s_barrier();
  const int grp = s / D;
  if constexpr (FMT == 1 && U == 0) pf_stage_scales<D>(c, s + D, (grp + 1) & 1);
  pf_stage<NP, W, NQ>(c, s + D - 1, (U + D - 1) % D);
  pf_pin(ring[U]);
  const uint8_t* sb = c.sbuf + (grp & 1) * kPfScaleGroupBytes + U * 2048 + c.soff;
  pf_mma_step<FMT, NP, SCL, NTT, pf_lut_repl(FMT, NP, D)>(ring[U], c.xs + U * NP * kPfPlaneBytes, s, c.nkb,
                                                         c.lane_off, c.lut, sb, acc);
  pf_load_step<FMT, SCL>(ring[U], c.tile, s + D, c.nks, c.nkb, c.m, c.g);
}

// The last R (< D) k-steps, straight-line.
template <int FMT, int NP, int D, int SCL, int NTT, int R, int W>
__device__ __forceinline__ void pf_tail(const PfCtx& c, PfStep<FMT, SCL> (&ring)[D], int s0, f32x4_t (&acc)[4][NTT]) {
  if constexpr (R >= 1) pf_kstep<FMT, NP, D, SCL, NTT, 0, W>(c, ring, s0, acc);
  if constexpr (R >= 2) pf_kstep<FMT, NP, D, SCL, NTT, 1, W>(c, ring, s0 + 1, acc);
  if constexpr (R >= 3) pf_kstep<FMT, NP, D, SCL, NTT, 2, W>(c, ring, s0 + 2, acc);
  static_assert(R < 4, "tail longer than supported");
}

// Main loop and epilogue for a group with NTT live token tiles.
template <int FMT, int NP, int D, bool GATEUP, int SCL, int NTT, int W>
__device__ __forceinline__ void pf_run(const PfCtx& c, const LayerArgs& L, int T, const Work& w, int wt, int nt) {
  f32x4_t acc[4][NTT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[rt][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  PfStep<FMT, SCL> ring[D];
  if constexpr (FMT == 1) pf_stage_scales<D>(c, 0, 0);
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if (j < D - 1) pf_stage<NP, W, pf_nq<W, NTT>()>(c, j, j);
    pf_load_step<FMT, SCL>(ring[j], c.tile, j, c.nks, c.nkb, c.m, c.g);
  }
  const int nfull = c.nks / D * D;
  for (int s0 = 0; s0 < nfull; s0 += D) {
    pf_kstep<FMT, NP, D, SCL, NTT, 0, W>(c, ring, s0, acc);
    if constexpr (D > 1) pf_kstep<FMT, NP, D, SCL, NTT, (D > 1 ? 1 : 0), W>(c, ring, s0 + 1, acc);
    if constexpr (D > 2) pf_kstep<FMT, NP, D, SCL, NTT, (D > 2 ? 2 : 0), W>(c, ring, s0 + 2, acc);
    if constexpr (D > 3) pf_kstep<FMT, NP, D, SCL, NTT, (D > 3 ? 3 : 0), W>(c, ring, s0 + 3, acc);
    static_assert(D <= 4, "deeper rings need more unrolled steps");
  }
  switch (c.nks - nfull) {
    case 1: pf_tail<FMT, NP, D, SCL, NTT, 1, W>(c, ring, nfull, acc); break;
    case 2: pf_tail<FMT, NP, D, SCL, NTT, (D > 2 ? 2 : 1), W>(c, ring, nfull, acc); break;
    case 3: pf_tail<FMT, NP, D, SCL, NTT, (D > 3 ? 3 : 1), W>(c, ring, nfull, acc); break;
    default: break;
  }
  // the trailing (never used) loads must land before the block's LDS is released
  __builtin_amdgcn_s_waitcnt(pf_vm_le(0));

  const int g = c.g, m = c.m;
  // pair ids of this lane's output slots, fetched together before the stores
  int pid[NTT][4];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int slot = min(16 * tt + 4 * g + q, nt - 1);
      pid[tt][q] = c.s_pair[slot];
    }
  if (GATEUP) {
    if (c.rt_mask) {
      const int I = L.I;
      const int P = T * L.k + (L.has_shared ? T : 0);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int col = 32 * wt + 16 * rt + m;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int slot = 16 * tt + 4 * g + q;
            if (slot < nt) {
              const int p = pid[tt][q];
              const float h = silu_f32(acc[rt][tt][q]) * acc[rt + 2][tt][q];
              const uint32_t hi = f32_to_bf16_rne(h);
              const uint32_t lo = f32_to_bf16_rne(h - bf16_bits_to_f32(hi));
              w.hplanes[(size_t)p * I + col] = (uint16_t)hi;
              w.hplanes[(size_t)P * I + (size_t)p * I + col] = (uint16_t)lo;
            }
          }
        }
      }
    }
  } else {
    const int H = L.H;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if ((c.rt_mask >> rt) & 1u) {
        const int col = 64 * wt + 16 * rt + m;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int slot = 16 * tt + 4 * g + q;
            if (slot < nt) w.o[(size_t)pid[tt][q] * H + col] = acc[rt][tt][q];
          }
        }
      }
    }
  }
}

// One projection of the prefill path.
//   GATEUP: rows of gate_up [2I][H] (K = H); wave tile wt = gate rows 32wt..32wt+31 and
//           up rows I+32wt..; A = x rows of the group's tokens (NP bf16 planes);
//           writes h (two bf16 planes) for the group's pairs.
//   down:   rows of down [H][I] (K = I); wave tile wt = rows 64wt..64wt+63; A = h rows
//           of the group's pairs (two planes); writes o (fp32) for the group's pairs.
// grid = RB row blocks x max groups; blocks past RB * n_groups exit.  Block ids are
// remapped so that the row blocks of one group run on one XCD (consecutive hardware
// ids go to different XCDs), where they share the group's activation rows in L2.
template <int FMT, int NP, int D, bool GATEUP, int SCL, int W>
__global__ __launch_bounds__(64 * W) void k_pf_proj(LayerArgs L, int T, Work w, const uint16_t* __restrict__ act,
                                                   size_t act_plane, int RB) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int ng = *w.n_groups;
  const int M = RB * ng;
  const int bid = blockIdx.x;
  if (bid >= M) return;
  const int M8 = M & ~7;
  const int logical = bid < M8 ? (bid & 7) * (M8 >> 3) + (bid >> 3) : bid;
  const int rb = logical % RB, gi = logical / RB;
  const int4 grp = w.groups[gi];
  const int e = grp.x, start = grp.y, nt = grp.z;

  PfCtx c;
  const int lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.m = lane & 15;
  c.g = lane >> 4;
  const int H = L.H, I = L.I, k = L.k;
  const int K = GATEUP ? H : I;
  c.nkb = K >> 5;
  c.nks = (c.nkb + 3) >> 2;
  c.row_bytes = 2 * K;
  c.act_plane_bytes = act_plane * 2;
  const int wt = rb * W + c.wave;

  c.xs = smem + pf_lut_bytes(FMT, NP, D);
  c.start = start;
  c.lane_off = 4u * (uint32_t)lane;
  c.lut = (const uint32_t*)smem;
  if (FMT == 2) {
    if constexpr (pf_lut_repl(FMT, NP, D)) pf_build_lut((uint32_t*)smem, L.codebook);
    else build_cb4_lut((uint32_t*)smem, L.codebook);
  }
  int* s_pair = (int*)(smem + pf_lds_bytes(FMT, NP, D));
  c.s_pair = s_pair;
  if (threadIdx.x < kGroupPairs)
    s_pair[threadIdx.x] = w.perm[start + ((int)threadIdx.x < nt ? (int)threadIdx.x : 0)];
  __syncthreads();

#pragma unroll
  for (int q = 0; q < 16 / W; ++q) {
    const int row = 4 * (c.wave + W * q) + (lane >> 4);
    const int p = w.perm[start + (row < nt ? row : 0)];
    const int r = GATEUP ? pf_token_of_pair(p, T, k) : p;
    c.src[q] = as_global(act) + (size_t)r * K * 2;
    c.piece[q] = 16 * ((lane & 15) ^ (row & 15));
  }

  const void* base = GATEUP ? L.gate_up[e] : L.down[e];
  const int rows_total = GATEUP ? 2 * I : H;
  // row tile rt of wave tile wt: GATEUP gate rows 32wt.. (rt 0, 1) and up rows I+32wt..
  // (rt 2, 3); down rows 64wt + 16rt..  A tile past the matrix reads tile 0 (its results
  // are not stored).
  auto tile_of = [&](int wtile, int rt, bool& ok) {
    int row0;
    if (GATEUP) {
      ok = 32 * wtile < I;
      row0 = (rt < 2 ? 0 : I) + 32 * wtile + 16 * (rt & 1);
    } else {
      row0 = 64 * wtile + 16 * rt;
      ok = row0 < H;
    }
    return packed_tile(base, rows_total, K, ok ? row0 / 16 : 0, FMT == 1 ? 1 : 2);
  };
  c.rt_mask = 0;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    bool ok;
    c.tile[rt] = tile_of(wt, rt, ok);
    if (ok) c.rt_mask |= 1u << rt;
  }
  if constexpr (FMT == 1) {
    static_assert(W == 8, "the scale staging assumes 8 waves (32 row tiles) per block");
    bool ok;
    const int wv = 4 * (c.wave & 1) + (lane >> 4);  // the wave owning this lane's staged tile
    c.schunk = lane & 3;
    c.ssrc = tile_of(rb * W + wv, (lane >> 2) & 3, ok).scales + 16 * c.schunk;
    c.sstep = min(c.wave >> 1, D - 1);
    c.sbuf = smem + pf_lut_bytes(FMT, NP, D) + D * NP * kPfPlaneBytes;
    c.soff = 256 * c.wave + 16 * c.g + c.m;
  } else {
    c.ssrc = nullptr;
    c.sbuf = nullptr;
    c.sstep = c.schunk = c.soff = 0;
  }

  switch ((nt + 15) >> 4) {
    case 1: pf_run<FMT, NP, D, GATEUP, SCL, 1, W>(c, L, T, w, wt, nt); break;
    case 2: pf_run<FMT, NP, D, GATEUP, SCL, 2, W>(c, L, T, w, wt, nt); break;
    case 3: pf_run<FMT, NP, D, GATEUP, SCL, 3, W>(c, L, T, w, wt, nt); break;
    default: pf_run<FMT, NP, D, GATEUP, SCL, 4, W>(c, L, T, w, wt, nt); break;
  }
}

// ---------------------------------------------------------------------------
// Combine: y[t][n] = sum_j pair_w[t*k+j] * o[t*k+j][n] (+ pair_w[T*k+t] * o[T*k+t][n]),
// j ascending and the shared expert last, a fixed order for every run.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pf_combine(int T, int H, int k, int has_shared, const float* __restrict__ o,
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
template <int FMT, int NP, int D, bool GATEUP, int SCL, int W>
static void pf_launch(const LayerArgs& L, int T, const Work& w, const uint16_t* act, size_t act_plane, int RB,
                      int max_groups_, int stage, hipStream_t s, const Timing& tm) {
  constexpr int lds = pf_lds_total(FMT, NP, D);
  static_assert(lds <= kPfLdsMax, "LDS budget of one workgroup");
  auto kern = k_pf_proj<FMT, NP, D, GATEUP, SCL, W>;
  // more than 64 KB of dynamic LDS: raise the kernel's limit once per instantiation
  static const bool lds_ok =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
  (void)lds_ok;
  MOEQ_LAUNCH(tm, stage, kern, dim3(RB * max_groups_), dim3(64 * W), lds, s, L, T, w, act, act_plane, RB);
}

// Waves per block: WG for the gate/up kernel, WD for the down kernel.
template <int FMT, int SCL, int D, int WG, int WD, int DD>
static void pf_launch_fmt(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, int mg,
                          hipStream_t s, const Timing& tm) {
  const int rb_gu = ((L.I / 32) + WG - 1) / WG;
  const int rb_dn = (((L.H + 63) / 64) + WD - 1) / WD;
  const int P = T * L.k + (L.has_shared ? T : 0);
  if (x_dtype == 1)
    pf_launch<FMT, 1, D, true, SCL, WG>(L, T, w, (const uint16_t*)x, 0, rb_gu, mg, kStageGateUp, s, tm);
  else  // three exact bf16 planes of fp32 x: 2 buffers fit in LDS beside the MXFP4 scales / CB4 table
    pf_launch<FMT, 3, 2, true, SCL, kPfWaves>(L, T, w, w.xplanes, (size_t)T * L.H,
                                                               (L.I / 32 + kPfWaves - 1) / kPfWaves,
                                                        mg, kStageGateUp, s, tm);
  pf_launch<FMT, 2, DD, false, SCL, WD>(L, T, w, w.hplanes, (size_t)P * L.I, rb_dn, mg, kStageDown, s, tm);
}

hipError_t launch_experts(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, float* y,
                          hipStream_t s, const Timing& tm) {
  const int P = T * L.k + (L.has_shared ? T : 0);
  const int mg = max_groups(P, L.E);
  if (L.wfmt == 1) {
    pf_launch_fmt<1, 0, 4, kPfWaves, kPfWaves, 4>(L, x, x_dtype, T, w, mg, s, tm);
  } else {
    // both K ranges must be multiples of 128 for the 8-byte scale loads
    if (L.H % 128 == 0 && L.I % 128 == 0)
      pf_launch_fmt<2, 1, 3, kPfWaves, kPfWaves, 3>(L, x, x_dtype, T, w, mg, s, tm);
    else
      pf_launch_fmt<2, 0, 2, kPfWaves, kPfWaves, 2>(L, x, x_dtype, T, w, mg, s, tm);
  }
  return launch_combine(L, T, w, y, s, tm);
}

hipError_t launch_combine(const LayerArgs& L, int T, const Work& w, float* y, hipStream_t s, const Timing& tm) {
  MOEQ_LAUNCH(tm, kStageCombine, k_pf_combine, dim3((L.H + 255) / 256, T), dim3(256), 0, s, T, L.H, L.k,
              L.has_shared, (const float*)w.o, (const float*)w.pair_w, y);
  return hipGetLastError();
}

}  // namespace moeq
