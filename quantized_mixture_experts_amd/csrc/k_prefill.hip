// Prefill path: grouped GEMMs over the bucketed (token, expert) pairs.
//
// Work unit: a group = up to 64 consecutive bucket positions of one expert (the
// bucketing kernel lists them in bucket order).  A block of 8 waves covers 512 weight
// rows of that expert for the group's pairs; every wave owns a 64-row x 64-pair tile
// (4 x 4 MFMA tiles of 16 x 16) over the whole K range, so there is no split-K
// reduction.  In the fused gate/up kernel a wave holds 32 gate rows and the 32
// matching up rows, so SwiGLU is applied in registers.  Each selected expert's rows
// are read from HBM once per group (once in total when it has at most 64 pairs), the
// grouping the NInfer Qwen3.8-Flash-Next page describes for its MoE execution: the
// routed pairs are sorted into per-expert groups and an expert's weights are streamed
// once for every token routed to it.
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
//   - only the activation rows of the group's live 16-row token tiles are staged (CB4);
//   - the k loop is unrolled by D, so ring slots and buffers are compile-time indices
//     and the wait before each step is a constant vmcnt (every wave issues the same
//     number of loads per step; loads past the row end re-read a real block that is
//     then masked, so nothing outside the matrices is touched).
// Operands:
//   - CB4 (v_mfma_f32_16x16x32_bf16): A = activation rows as bf16 planes (exact), B =
//     codebook values from the LDS table (exact in bf16), the fp16 block scale applied
//     to each 32-column block's fp32 MFMA result;
//   - MXFP4 (v_mfma_scale_f32_16x16x128_f8f6f4): A = the activations as fp8 e4m3 planes
//     with E8M0 scales, B = the stored E2M1 codes and their E8M0 scales as they are.
#include "device.h"
#include "launch.h"

namespace moeq {

constexpr int kPfWaves = 8;  // waves per block (eight 64-row wave tiles: 512 weight rows)

constexpr int kPfRowBytes = 256;                         // CB4 path: one staged row chunk, 128 bf16
constexpr int kPfPlaneBytes = kGroupPairs * kPfRowBytes;  // 16 KB per plane per buffer
constexpr int kMxRowBytes = 128;                          // MXFP4 path: one staged row chunk, 128 fp8
constexpr int kMxPlaneBytes = kGroupPairs * kMxRowBytes;  // 8 KB per plane per buffer
constexpr int kMxChunkCols = 256;  // h columns per activation scale (one gate/up block's columns)
constexpr int kMxAScaleStride = 64;  // LDS activation scales: 64 rows x up to 64 chunks (I <= 16384)
__host__ __device__ constexpr int pf_row_bytes(int fmt) { return fmt_is_mx(fmt) ? kMxRowBytes : kPfRowBytes; }
__host__ __device__ constexpr int pf_plane_bytes(int fmt) { return fmt_is_mx(fmt) ? kMxPlaneBytes : kPfPlaneBytes; }

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
__host__ __device__ constexpr int pf_scale_lds_bytes(int fmt) { return fmt_is_mx(fmt) ? 2 * kPfScaleGroupBytes : 0; }
// MXFP4: the rows' activation scales, then the gate/up epilogue's per-wave row maxima
// [64 rows][8 waves] (a region of its own, so that waves still in their last k-step are
// not disturbed)
__host__ __device__ constexpr int pf_ascale_lds_bytes(int fmt) {
  return fmt_is_mx(fmt) ? kGroupPairs * kMxAScaleStride + kGroupPairs * 8 * 4 : 0;
}
// LUT, then the D x NP activation buffers, then (MXFP4) the weight scale buffers and the
// rows' activation scales, then the group's 64 pair ids.
__host__ __device__ constexpr int pf_lds_bytes(int fmt, int np, int d) {
  return pf_lut_bytes(fmt, np, d) + d * np * pf_plane_bytes(fmt) + pf_scale_lds_bytes(fmt) + pf_ascale_lds_bytes(fmt);
}
__host__ __device__ constexpr int pf_lds_total(int fmt, int np, int d) {
  return pf_lds_bytes(fmt, np, d) + 4 * kGroupPairs;
}

// Wave w writes rows b = w + 8k (k < 32) of the replicated table: the low value is
// codebook[b & 15] = codebook[w + 8 (k & 1)], the high one codebook[b >> 4] =
// codebook[k >> 1].  The 16 codebook values are read once (one byte per lane) and
// broadcast with readlane, so the table costs one global load per lane.
template <int W>
__device__ __forceinline__ void pf_build_lut(uint32_t* lut, const int8_t* codebook) {
  static_assert(W == 8, "rows b = wave + 8k assume 8 waves");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t bits = int8_to_bf16_bits(codebook[lane & 15]);
  const uint32_t lo0 = __builtin_amdgcn_readlane(bits, wave), lo1 = __builtin_amdgcn_readlane(bits, wave + 8);
#pragma unroll
  for (int k = 0; k < 32; ++k)
    lut[(wave + 8 * k) * 64 + lane] = ((k & 1) ? lo1 : lo0) | (__builtin_amdgcn_readlane(bits, k >> 1) << 16);
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
struct PfStep<3, SCL> {  // the packed scale store: the scales are staged in LDS as for MXFP4
  u32x4_t c[4];
};
template <int SCL>
struct PfStep<1, SCL> {
  u32x4_t c[4];  // the scales are staged in LDS
};
// CB4 codes: c[rt] is block 4 ks + g of row m as stored (one 16-byte load); the step's
// MFMAs transpose it across the four lane rows first (xpose_rows4), so that dword j holds
// bytes 4g..4g+3 of block 4 ks + j.
template <>
struct PfStep<2, 0> {
  u32x4_t c[4];
  uint32_t s[4][4];
};
template <>
struct PfStep<2, 1> {
  u32x4_t c[4];
  uint64_t s[4];  // fp16 scale bits of blocks 4ks..4ks+3, block j in bits 16j..16j+15
};
// vector-memory instructions of one k-step's weights: MXFP4 one 16-byte code load per row
// tile (the scales come through LDS); CB4 one 16-byte code load and one 8-byte scale load
// (or four 2-byte ones) per row tile
template <int FMT, int SCL>
__host__ __device__ constexpr int pf_loads_per_step() {
  return fmt_is_mx(FMT) ? 4 : (SCL ? 8 : 20);
}

__device__ __forceinline__ void pf_load_lds_16(gbyte_t* gptr, void* lds) {
  const uint32_t lds_addr =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(gptr) : "memory", "m0");
}

// Loads of k-step ks (clamped to the last step: such registers are never used).  A block
// past the row end re-reads the row's last block (masked at use).  For a full step the
// 64 lanes of one code load read one contiguous kilobyte of the tile-major storage.
template <int FMT, int SCL>
__device__ __forceinline__ void pf_load_step(PfStep<FMT, SCL>& r, const PackedTile (&pt)[4], int ks, int nks,
                                             int nkb, int m, int g) {
  // the memory instructions of one row tile below (the counted waits rely on their sum)
  constexpr int kCodeLoads = 1, kScaleLoads = fmt_is_mx(FMT) ? 0 : (SCL ? 1 : 4);
  static_assert(4 * (kCodeLoads + kScaleLoads) == pf_loads_per_step<FMT, SCL>(), "per-step load count");
  const int kc = ks < nks ? ks : nks - 1;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    if constexpr (fmt_is_mx(FMT)) {
      const int kb = min(4 * kc + g, nkb - 1);
      r.c[rt] = __builtin_nontemporal_load(
          (const __attribute__((address_space(1))) u32x4_t*)(pt[rt].codes + pk_code(kb, m)));
    } else {
      const int kb = min(4 * kc + g, nkb - 1);
      r.c[rt] = __builtin_nontemporal_load(
          (const __attribute__((address_space(1))) u32x4_t*)(pt[rt].codes + pk_code(kb, m)));
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
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

// MXFP4 A operand of v_mfma_scale_f32_16x16x128_f8f6f4 for token row `row` of a staged
// fp8 chunk: lane 16g + m supplies columns 16g..16g+15 (bytes 0..15) and 64+16g..
// 64+16g+15 (bytes 16..31) of its row.  The 16-byte pieces of row r sit at piece ^
// ((r >> 1) & 7) in LDS, which spreads the 16 rows of a read over 16 bank groups.
__device__ __forceinline__ i32x8_t pf_mx_a(const uint8_t* plane, int row, int g) {
  const int sw = (row >> 1) & 7;
  const uint8_t* rb = plane + row * kMxRowBytes;
  const u32x4_t lo = *(const u32x4_t*)(rb + 16 * (g ^ sw));
  const u32x4_t hi = *(const u32x4_t*)(rb + 16 * ((4 + g) ^ sw));
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// sb (MXFP4): this lane's weight scale byte of row tile 0 for step ks in LDS (tile rt at
// +64 rt); ab (MXFP4): this lane's activation scale byte of token row m of the step
// (token tile tt at +16 x kMxAScaleStride x tt).
template <int FMT, int NP, int SCL, int NTT, bool REPL>
__device__ __forceinline__ void pf_mma_step(const PfStep<FMT, SCL>& r, const uint8_t* xb, int ks, int nkb,
                                            uint32_t lane_off, const uint32_t* lut, const uint8_t* sb,
                                            const uint8_t* ab, f32x4_t (&acc)[4][NTT]) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  if constexpr (fmt_is_mx(FMT)) {
    // Block-scaled matrix cores: A = NP fp8 e4m3 planes of the activations with one E8M0
    // scale per row (chunk), B = the E2M1 codes exactly as stored (lane 16g + m holds
    // block g of weight row m, which is the B operand layout) with their E8M0 scales.
    // Columns past K meet zero activations (the planes are zero-padded), so a clamped
    // block of a partial last step adds nothing.
    i32x8_t bw[4];
    int sbv[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      bw[rt] = i32x8_t{(int)r.c[rt][0], (int)r.c[rt][1], (int)r.c[rt][2], (int)r.c[rt][3], 0, 0, 0, 0};
      sbv[rt] = sb[64 * rt];
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const int sa = ab[16 * kMxAScaleStride * tt];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const i32x8_t a = pf_mx_a(xb + p * kMxPlaneBytes, 16 * tt + m, g);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          acc[rt][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bw[rt], acc[rt][tt], 0, 4, 0, sa, 0,
                                                                        sbv[rt]);
      }
    }
  } else {
    // lane row g held block 4 ks + g; after the transpose dword j holds bytes 4g..4g+3 of
    // block 4 ks + j (a clamped block of a partial last step: the row's last block)
    u32x4_t cw[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      cw[rt] = r.c[rt];
      xpose_rows4(cw[rt]);
    }
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
          if constexpr (REPL) b[rt] = pf_cb4x8(cw[rt][j], lane_off);
          else b[rt] = cb4x8_to_bf16(cw[rt][j], lut);
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
          mfma_settle4(tmp, true);
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
  gbyte_t* dsrc;           // packed scale store: this lane's 8 delta bytes (chunk) of its staging tile, step 0
  u32x4_t sbase;           // packed scale store: the base bytes of the 16 rows of this lane's staging tile
  const uint8_t* ascale;   // MXFP4: LDS activation scales [64 rows][kMxAScaleStride], row m
  float* cmax;             // MXFP4 gate/up epilogue: LDS row maxima [64 rows][8 waves]
  size_t act_plane_bytes;
  int nks, nkb, row_bytes, wave, g, m;
  uint32_t rt_mask;
};

// Copy staged chunk s (clamped to the last one) of the group's rows into buffer buf: the
// one-kilobyte loads per plane (4 rows each) are spread over the W waves, this wave
// taking u = wave + W q, q < NQ (16 / W loads cover all 64 rows; fewer cover the rows of
// the live token tiles).
// MXFP4: fp8 rows of 128 bytes, 8 rows per 1 KB load, so every wave issues one load per
// plane for all 64 rows.
template <int FMT, int NP, int W, int NQ>
__device__ __forceinline__ void pf_stage(const PfCtx& c, int s, int buf) {
  const int sc = s < c.nks ? s : c.nks - 1;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    int off = pf_row_bytes(FMT) * sc + c.piece[q];
    off = off + 16 <= c.row_bytes ? off : 0;  // past the row end: real data, never used
#pragma unroll
    for (int p = 0; p < NP; ++p)
      pf_load_lds_16(c.src[q] + p * c.act_plane_bytes + off,
                     c.xs + (buf * NP + p) * pf_plane_bytes(FMT) + (c.wave + W * q) * 1024);
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

// Packed scale store: the lane's 16 deltas (rows 0..15 of block `schunk` of its staging
// tile) for the steps pf_stage_scales would stage, one 8-byte register load in place of
// the direct load (so the per-step load counts are the same) ...
__device__ __forceinline__ uint64_t pf_load_deltas(const PfCtx& c, int s) {
  const int st = min(s + c.sstep, c.nks - 1);
  const int nb = min(4, c.nkb - 4 * st);
  const int ch = c.schunk < nb ? c.schunk : 0;
  return *(const __attribute__((address_space(1))) uint64_t*)(c.dsrc + 32 * st + 8 * (ch - c.schunk));
}
// ... and, once they are needed, the 16 E8M0 bytes (row base + delta nibble j for row j)
// written where the direct load would have put them; the LDS write is complete before
// the next step's barrier.
__device__ __forceinline__ void pf_put_scales(const PfCtx& c, uint64_t d, int par) {
  const int lane = threadIdx.x & 63;
  u32x4_t v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t n = (uint32_t)(d >> (16 * q)) & 0xFFFFu;
    const uint32_t x = (n & 0xFu) | ((n & 0xF0u) << 4) | ((n & 0xF00u) << 8) | ((n & 0xF000u) << 12);
    v[q] = c.sbase[q] + x;  // base + delta <= 255 in every byte: no carries between bytes
  }
  *(u32x4_t*)(c.sbuf + par * kPfScaleGroupBytes + c.wave * 1024 + 16 * lane) = v;
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), the other counters untouched
}

// The vmcnt wait at the start of the k-step in ring slot U that covers chunk s: chunk s
// was staged D-1 steps earlier and was followed by that step's weights and by D-2 whole
// steps (chunk + weights, plus the scale load of a slot-0 step, which precedes its chunk).
template <int FMT, int SCL, int D, int NQNP>
__host__ __device__ constexpr int pf_wait_count(int U) {
  int n = pf_loads_per_step<FMT, SCL>();
  for (int v = 2; v < D; ++v) n += NQNP + pf_loads_per_step<FMT, SCL>() + ((fmt_is_mx(FMT) && (U + v) % D == 0) ? 1 : 0);
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
template <int SCL>
__device__ __forceinline__ void pf_pin(PfStep<3, SCL>& r) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) asm volatile("" : "+v"(r.c[rt]));
}
__device__ __forceinline__ void pf_pin(PfStep<2, 0>& r) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    asm volatile("" : "+v"(r.c[rt]));
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(r.s[rt][j]));
  }
}
__device__ __forceinline__ void pf_pin(PfStep<2, 1>& r) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) asm volatile("" : "+v"(r.c[rt]), "+v"(r.s[rt]));
}

// Activation staging loads per wave per plane and k-step for NTT live token tiles (CB4:
// 4 rows per load; MXFP4: one load covers 8 rows, all 64 are staged).
template <int FMT, int W, int NTT>
__host__ __device__ constexpr int pf_nq() {
  return fmt_is_mx(FMT) ? 64 / 8 / W : ((4 * NTT + W - 1) / W < 16 / W ? (4 * NTT + W - 1) / W : 16 / W);
}

// One k-step (s = a multiple of D plus U): wait for chunk s, stage (in a slot-0 step) the
// MXFP4 scales of the next D-step group and chunk s+D-1 into buffers every wave has
// finished with, MFMAs, then the weights of step s+D into the ring slot just consumed.
// The wait covers chunk s and every load issued before it (this wave's weights of step s
// and the scales of step s's group); the barrier then makes every wave's staged data
// visible and frees the buffers of step s-1.  Straight-line code: every wave issues the
// same loads at every step, so the wait is a constant.
template <int FMT, int NP, int D, bool GATEUP, int SCL, int NTT, int U, int W>
__device__ __forceinline__ void pf_kstep(const PfCtx& c, PfStep<FMT, SCL> (&ring)[D], int s, f32x4_t (&acc)[4][NTT],
                                         uint64_t& pend) {
  constexpr int NQ = pf_nq<FMT, W, NTT>();
  constexpr int kWait = pf_wait_count<FMT, SCL, D, NQ * NP>(U);
  static_assert(kWait <= 63, "too many loads in flight for the vmcnt counter");
  __builtin_amdgcn_s_waitcnt(pf_vm_le(kWait));
  __builtin_amdgcn_s_barrier();
  const int grp = s / D;
  if constexpr (FMT == 1 && U == 0) pf_stage_scales<D>(c, s + D, (grp + 1) & 1);
  if constexpr (FMT == 3 && U == 0) pend = pf_load_deltas(c, s + D);
  pf_stage<FMT, NP, W, NQ>(c, s + D - 1, (U + D - 1) % D);
  pf_pin(ring[U]);
  const uint8_t* sb = c.sbuf + (grp & 1) * kPfScaleGroupBytes + U * 2048 + c.soff;
  // activation scale chunk of step s: one per row for x, one per 256 columns for h
  const uint8_t* ab = c.ascale + (GATEUP ? 0 : (s * 128) / kMxChunkCols);
  pf_mma_step<FMT, NP, SCL, NTT, pf_lut_repl(FMT, NP, D)>(ring[U], c.xs + U * NP * pf_plane_bytes(FMT), s, c.nkb,
                                                         c.lane_off, c.lut, sb, ab, acc);
  pf_load_step<FMT, SCL>(ring[U], c.tile, s + D, c.nks, c.nkb, c.m, c.g);
  // the next group's scales, in the buffer every wave finished with at this group's start
  if constexpr (FMT == 3 && U == D - 1) pf_put_scales(c, pend, (grp + 1) & 1);
}

// The last R (< D) k-steps, straight-line.
template <int FMT, int NP, int D, bool GATEUP, int SCL, int NTT, int R, int W>
__device__ __forceinline__ void pf_tail(const PfCtx& c, PfStep<FMT, SCL> (&ring)[D], int s0, f32x4_t (&acc)[4][NTT],
                                        uint64_t& pend) {
  if constexpr (R >= 1) pf_kstep<FMT, NP, D, GATEUP, SCL, NTT, 0, W>(c, ring, s0, acc, pend);
  if constexpr (R >= 2) pf_kstep<FMT, NP, D, GATEUP, SCL, NTT, 1, W>(c, ring, s0 + 1, acc, pend);
  if constexpr (R >= 3) pf_kstep<FMT, NP, D, GATEUP, SCL, NTT, 2, W>(c, ring, s0 + 2, acc, pend);
  static_assert(R < 4, "tail longer than supported");
}

// Largest value of v over the 16 lanes of this lane's DPP row.
__device__ __forceinline__ float pf_row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  return v;
}

// fp8 e4m3 (round to nearest even) of one value, and its value.
__device__ __forceinline__ uint32_t pf_to_fp8(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}
__device__ __forceinline__ float pf_from_fp8(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// E8M0 exponent e of a block whose largest magnitude is amax: amax / 2^e in [128, 256),
// so that the fp8 planes of v / 2^e stay below the e4m3 maximum (448); e = 0 for a zero
// block.
__device__ __forceinline__ int pf_mx_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;  // floor(log2) for normal amax
  const int e = (amax < 1.17549435e-38f ? -126 : ex) - 7;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// MXFP4 gate/up epilogue: h = silu(gate) * up in registers, then h as three fp8 planes
// with one E8M0 scale per (pair, 256-column chunk), the chunk this block computes:
// h ~= 2^e (p0 + p1 + p2), p_i = fp8(the remainder after p0..p_{i-1}), so about 12
// significant bits below the chunk maximum.  The bytes are assembled in LDS (the
// staging buffers are free) and written as 16-byte rows; columns past I are zeros.
template <int NTT, int W>
__device__ __forceinline__ void pf_mx_h_epilogue(const PfCtx& c, const LayerArgs& L, int T, const Work& w, int wt,
                                                 int nt, const f32x4_t (&acc)[4][NTT]) {
  static_assert(W == 8, "row maxima are kept for 8 waves");
  const int g = c.g, m = c.m;
  const int I = L.I;
  const int Ip = (I + kMxChunkCols - 1) / kMxChunkCols * kMxChunkCols;
  const int nch = Ip / kMxChunkCols;
  const size_t P = (size_t)T * L.k + (L.has_shared ? T : 0);
  const int rb = wt / W;
  uint8_t* hb = c.xs;  // [3][64 rows][256 columns], once every wave is past the k loop
  // h of this lane: rows 16 tt + 4 g + q, columns 32 wt + 16 rt + m (rt = 0, 1);
  // silu(a) = a / (1 + e^-a) with the hardware exp2 and reciprocal (a few ulp)
  float hv[NTT][4][2];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float a = acc[rt][tt][q];
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * a));
        hv[tt][q][rt] = c.rt_mask ? a * sg * acc[rt + 2][tt][q] : 0.0f;
      }
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float r = pf_row16_max(fmaxf(fabsf(hv[tt][q][0]), fabsf(hv[tt][q][1])));
      if (m == 0) c.cmax[(16 * tt + 4 * g + q) * 8 + c.wave] = r;
    }
  __syncthreads();  // row maxima complete; every wave is past its last read of the staged chunks
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 16 * tt + 4 * g + q;
      const f32x4_t m0 = *(const f32x4_t*)(c.cmax + 8 * row);
      const f32x4_t m1 = *(const f32x4_t*)(c.cmax + 8 * row + 4);
      const float cm = fmaxf(fmaxf(fmaxf(m0[0], m0[1]), fmaxf(m0[2], m0[3])),
                             fmaxf(fmaxf(m1[0], m1[1]), fmaxf(m1[2], m1[3])));
      const int e = pf_mx_exp(cm);
      float v0 = ldexpf(hv[tt][q][0], -e), v1 = ldexpf(hv[tt][q][1], -e);
      uint8_t* dst = hb + row * kMxChunkCols + 32 * c.wave + m;
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        const uint32_t b = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
        const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, false);
        v0 -= f[0];
        v1 -= f[1];
        dst[pl * kGroupPairs * kMxChunkCols] = (uint8_t)(b & 0xFFu);
        dst[pl * kGroupPairs * kMxChunkCols + 16] = (uint8_t)((b >> 8) & 0xFFu);
      }
      if (c.wave == 0 && m == 0 && row < nt)
        w.hq[3 * P * Ip + (size_t)c.s_pair[row] * nch + rb] = (uint8_t)(e + 127);
    }
  __syncthreads();
  // 3 planes x nt rows x 256 bytes, 16 bytes per thread and pass
  for (int idx = threadIdx.x; idx < 3 * kGroupPairs * 16; idx += 64 * W) {
    const int pl = idx / (kGroupPairs * 16), row = (idx / 16) % kGroupPairs, ch = idx % 16;
    if (row < nt) {
      const size_t p = (size_t)c.s_pair[row];
      *(u32x4_t*)(w.hq + pl * P * Ip + p * Ip + (size_t)kMxChunkCols * rb + 16 * ch) =
          *(const u32x4_t*)(hb + (pl * kGroupPairs + row) * kMxChunkCols + 16 * ch);
    }
  }
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
  uint64_t pend = 0;  // packed scale store: the next group's deltas, between its load and its use
  if constexpr (FMT == 1) pf_stage_scales<D>(c, 0, 0);
  if constexpr (FMT == 3) pf_put_scales(c, pf_load_deltas(c, 0), 0);
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if (j < D - 1) pf_stage<FMT, NP, W, pf_nq<FMT, W, NTT>()>(c, j, j);
    pf_load_step<FMT, SCL>(ring[j], c.tile, j, c.nks, c.nkb, c.m, c.g);
  }
  const int nfull = c.nks / D * D;
  for (int s0 = 0; s0 < nfull; s0 += D) {
    pf_kstep<FMT, NP, D, GATEUP, SCL, NTT, 0, W>(c, ring, s0, acc, pend);
    if constexpr (D > 1) pf_kstep<FMT, NP, D, GATEUP, SCL, NTT, (D > 1 ? 1 : 0), W>(c, ring, s0 + 1, acc, pend);
    if constexpr (D > 2) pf_kstep<FMT, NP, D, GATEUP, SCL, NTT, (D > 2 ? 2 : 0), W>(c, ring, s0 + 2, acc, pend);
    if constexpr (D > 3) pf_kstep<FMT, NP, D, GATEUP, SCL, NTT, (D > 3 ? 3 : 0), W>(c, ring, s0 + 3, acc, pend);
    static_assert(D <= 4, "deeper rings need more unrolled steps");
  }
  switch (c.nks - nfull) {
    case 1: pf_tail<FMT, NP, D, GATEUP, SCL, NTT, 1, W>(c, ring, nfull, acc, pend); break;
    case 2: pf_tail<FMT, NP, D, GATEUP, SCL, NTT, (D > 2 ? 2 : 1), W>(c, ring, nfull, acc, pend); break;
    case 3: pf_tail<FMT, NP, D, GATEUP, SCL, NTT, (D > 3 ? 3 : 1), W>(c, ring, nfull, acc, pend); break;
    default: break;
  }
  // the trailing (never used) loads must land before the block's LDS is released
  __builtin_amdgcn_s_waitcnt(pf_vm_le(0));
  // the accumulators settle before the epilogue reads them (one wait for all)
  mfma_settle_block(acc);

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
  if constexpr (GATEUP && fmt_is_mx(FMT)) {
    pf_mx_h_epilogue<NTT, W>(c, L, T, w, wt, nt, acc);
  } else if constexpr (GATEUP) {
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
__global__ __launch_bounds__(64 * W) void k_pf_proj(LayerArgs L, int T, Work w, const uint8_t* __restrict__ act,
                                                   size_t act_plane_bytes, int RB) {
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
  // activation row stride: bf16 rows of K (CB4); fp8 rows padded to whole k-steps (x) or
  // whole 256-column chunks (h) (MXFP4)
  c.row_bytes = fmt_is_mx(FMT) ? (GATEUP ? (H + 127) / 128 * 128 : (I + kMxChunkCols - 1) / kMxChunkCols * kMxChunkCols)
                         : 2 * K;
  c.act_plane_bytes = act_plane_bytes;
  const int wt = rb * W + c.wave;

  c.xs = smem + pf_lut_bytes(FMT, NP, D);
  c.start = start;
  c.lane_off = 4u * (uint32_t)lane;
  c.lut = (const uint32_t*)smem;
  if (FMT == 2) {
    if constexpr (pf_lut_repl(FMT, NP, D)) pf_build_lut<W>((uint32_t*)smem, L.codebook);
    else build_cb4_lut((uint32_t*)smem, L.codebook);
  }
  int* s_pair = (int*)(smem + pf_lds_bytes(FMT, NP, D));
  c.s_pair = s_pair;
  if (threadIdx.x < kGroupPairs)
    s_pair[threadIdx.x] = w.perm[start + ((int)threadIdx.x < nt ? (int)threadIdx.x : 0)];
  if constexpr (fmt_is_mx(FMT)) {
    // the rows' activation scales (they follow the NP planes): one per x row, one per
    // 256-column chunk of an h row; rows past nt repeat row 0
    uint8_t* as = smem + pf_lds_bytes(FMT, NP, D) - pf_ascale_lds_bytes(FMT);
    c.cmax = (float*)(as + kGroupPairs * kMxAScaleStride);
    const int nch = GATEUP ? 1 : c.row_bytes / kMxChunkCols;
    const uint8_t* src_scales = act + NP * act_plane_bytes;
    for (int t = threadIdx.x; t < kGroupPairs * nch; t += 64 * W) {
      const int row = t / nch, ch = t % nch;
      const int p = w.perm[start + (row < nt ? row : 0)];
      as[row * kMxAScaleStride + ch] =
          GATEUP ? src_scales[pf_token_of_pair(p, T, k)] : src_scales[(size_t)p * nch + ch];
    }
    c.ascale = as + c.m * kMxAScaleStride;
  } else {
    c.ascale = nullptr;
    c.cmax = nullptr;
  }
  __syncthreads();

  if constexpr (fmt_is_mx(FMT)) {
    // one 1 KB staging load per plane covers rows 8 wave .. 8 wave + 7: lane l loads
    // row 8 wave + l / 8, the 16-byte piece that belongs at LDS piece l % 8
    const int row = 8 * c.wave + (lane >> 3);
    const int p = w.perm[start + (row < nt ? row : 0)];
    const int r = GATEUP ? pf_token_of_pair(p, T, k) : p;
    c.src[0] = as_global(act) + (size_t)r * c.row_bytes;
    c.piece[0] = 16 * ((lane & 7) ^ ((row >> 1) & 7));
  } else {
#pragma unroll
    for (int q = 0; q < 16 / W; ++q) {
      const int row = 4 * (c.wave + W * q) + (lane >> 4);
      const int p = w.perm[start + (row < nt ? row : 0)];
      const int r = GATEUP ? pf_token_of_pair(p, T, k) : p;
      c.src[q] = as_global(act) + (size_t)r * K * 2;
      c.piece[q] = 16 * ((lane & 15) ^ (row & 15));
    }
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
    return packed_tile<FMT>(base, rows_total, K, ok ? row0 / 16 : 0);
  };
  c.rt_mask = 0;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    bool ok;
    c.tile[rt] = tile_of(wt, rt, ok);
    if (ok) c.rt_mask |= 1u << rt;
  }
  if constexpr (fmt_is_mx(FMT)) {
    static_assert(W == 8, "the scale staging assumes 8 waves (32 row tiles) per block");
    bool ok;
    const int wv = 4 * (c.wave & 1) + (lane >> 4);  // the wave owning this lane's staged tile
    c.schunk = lane & 3;
    const PackedTile st = tile_of(rb * W + wv, (lane >> 2) & 3, ok);
    c.ssrc = st.scales + 16 * c.schunk;
    c.sstep = min(c.wave >> 1, D - 1);
    c.sbuf = smem + pf_lut_bytes(FMT, NP, D) + D * NP * pf_plane_bytes(FMT);
    c.soff = 256 * c.wave + 16 * c.g + c.m;
    if constexpr (FMT == 3) {
      c.dsrc = st.scales + 8 * c.schunk;
      c.sbase = *(const __attribute__((address_space(1))) u32x4_t*)st.bases;
    }
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
// j ascending and the shared expert last, a fixed order for every run; resid[t][n] is
// added to the finished sum when given.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pf_combine(int T, int H, int k, int has_shared, const float* __restrict__ o,
                                                    const float* __restrict__ pair_w, const float* __restrict__ resid,
                                                    float* __restrict__ y) {
  const int t = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= H) return;
  // the k (<= 16) routed rows, 8 loads in flight (clamped, in bounds), summed in order
  float s = 0.f;
  for (int j0 = 0; j0 < k; j0 += 8) {
    float ov[8], wv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + u, k - 1);
      ov[u] = o[(size_t)(t * k + j) * H + n];
      wv[u] = pair_w[t * k + j];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < k && wv[u] != 0.0f) s = fmaf(wv[u], ov[u], s);  // weight 0: omitted, o not written
  }
  if (has_shared) s = fmaf(pair_w[T * k + t], o[(size_t)(T * k + t) * H + n], s);
  y[(size_t)t * H + n] = resid ? resid[(size_t)t * H + n] + s : s;
}

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// MXFP4 path: fp8 planes of the activations x with one E8M0 scale per row.
//   x [T][H] bf16 (XDT 1, NPX = 2: exact for entries down to about 2^-9 of the row
//   maximum; smaller ones lose low bits to the e4m3 subnormal floor) or fp32 (XDT 0,
//   NPX = 3); xq = NPX planes
//   [T][Hp] (Hp = H rounded up to 128, zero columns past H), then T scale bytes.
// One block per row: the row maximum, then x / 2^e split into fp8 planes as in the h
// epilogue (2^e maps the row maximum into [128, 256)).
// ---------------------------------------------------------------------------
template <int XDT, int NPX>
__global__ __launch_bounds__(256) void k_mx_xquant(const void* __restrict__ x, int T, int H, int Hp,
                                                   uint8_t* __restrict__ xq) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  auto load4 = [&](int c, float (&v)[4]) {
    if (XDT == 1) {
      const uint2 q = *(const uint2*)((const uint16_t*)x + (size_t)t * H + c);
      v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xFFFF0000u);
      v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xFFFF0000u);
    } else {
      const f32x4_t q = *(const f32x4_t*)((const float*)x + (size_t)t * H + c);
      v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
    }
  };
  float amax = 0.0f;
  for (int c = 4 * threadIdx.x; c < H; c += 1024) {
    float v[4];
    load4(c, v);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = pf_mx_exp(amax);
  if (threadIdx.x == 0) xq[(size_t)NPX * T * Hp + t] = (uint8_t)(e + 127);
  for (int c = 4 * threadIdx.x; c < Hp; c += 1024) {  // H % 32 == 0: a group is all in or all past
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (c < H) {
      load4(c, v);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = ldexpf(v[j], -e);
    }
#pragma unroll
    for (int p = 0; p < NPX; ++p) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t b = pf_to_fp8(v[j]);
        v[j] -= pf_from_fp8(b);
        word |= b << (8 * j);
      }
      *(uint32_t*)(xq + ((size_t)p * T + t) * Hp + c) = word;
    }
  }
}

// The grouped CB4 kernels' decode, exported for a bit-exact test: the replicated table
// built as the projections build it (8 waves) at LDS offset 0, and every 32-value block of
// a matrix decoded by one lane with pf_cb4x8, times the block's fp16 scale in fp32 (the
// product of an int8 value and an fp16 scale needs at most 19 significant bits, so it is
// exact, as the projections' fp32 scaling of an exact block sum is for one term).
__global__ __launch_bounds__(64 * kPfWaves) void k_pf_dequant_cb4(const uint8_t* __restrict__ packed,
                                                                  const int8_t* __restrict__ codebook, int rows,
                                                                  int cols, float* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t smem[];
  pf_build_lut<kPfWaves>((uint32_t*)smem, codebook);
  __syncthreads();
  const int nkb = cols >> 5;
  const size_t blk = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= (size_t)rows * nkb) return;
  const int row = (int)(blk / nkb), kb = (int)(blk % nkb);
  const int m = row & 15;
  const PackedTile pt = packed_tile<2>(packed, rows, cols, row >> 4);
  const u32x4_t c = *(const __attribute__((address_space(1))) u32x4_t*)(pt.codes + pk_code(kb, m));
  const float sc =
      half_bits_to_f32(*(const __attribute__((address_space(1))) uint16_t*)(pt.scales + 2 * pk_scale_cb(kb, m, nkb)));
  const uint32_t lane_off = 4u * (threadIdx.x & 63);
  float* dst = out + blk * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x8_t v = pf_cb4x8(c[q], lane_off);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[8 * q + i] = sc * (float)v[i];
  }
}

hipError_t launch_pf_dequant_cb4(const uint8_t* packed, const int8_t* codebook, int rows, int cols, float* out,
                                 hipStream_t s) {
  static const bool lds_ok = hipFuncSetAttribute((const void*)k_pf_dequant_cb4,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 kPfLutReplBytes) == hipSuccess;
  (void)lds_ok;
  const size_t nblk = (size_t)rows * (cols / 32);
  hipLaunchKernelGGL(k_pf_dequant_cb4, dim3((unsigned)((nblk + 64 * kPfWaves - 1) / (64 * kPfWaves))),
                     dim3(64 * kPfWaves), kPfLutReplBytes, s, packed, codebook, rows, cols, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
template <int FMT, int NP, int D, bool GATEUP, int SCL, int W>
static void pf_launch(const LayerArgs& L, int T, const Work& w, const void* act, size_t act_plane_bytes, int RB,
                      int max_groups_, int stage, hipStream_t s, const Timing& tm) {
  constexpr int lds = pf_lds_total(FMT, NP, D);
  static_assert(lds <= kPfLdsMax, "LDS budget of one workgroup");
  auto kern = k_pf_proj<FMT, NP, D, GATEUP, SCL, W>;
  // more than 64 KB of dynamic LDS: raise the kernel's limit once per instantiation
  static const bool lds_ok =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
  (void)lds_ok;
  MOEQ_LAUNCH(tm, stage, kern, dim3(RB * max_groups_), dim3(64 * W), lds, s, L, T, w, (const uint8_t*)act,
              act_plane_bytes, RB);
}

// CB4: bf16 activation planes (x itself, or three exact planes of fp32 x; h in two
// planes).  Waves per block: WG for the gate/up kernel, WD for the down kernel.
template <int SCL, int D, int WG, int WD, int DD>
static void pf_launch_cb4(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, int mg,
                          hipStream_t s, const Timing& tm) {
  const int rb_gu = ((L.I / 32) + WG - 1) / WG;
  const int rb_dn = (((L.H + 63) / 64) + WD - 1) / WD;
  const size_t P = (size_t)T * L.k + (L.has_shared ? T : 0);
  if (x_dtype == 1)
    pf_launch<2, 1, D, true, SCL, WG>(L, T, w, x, 0, rb_gu, mg, kStageGateUp, s, tm);
  else  // three exact bf16 planes of fp32 x: 2 buffers fit in LDS beside the table
    pf_launch<2, 3, 2, true, SCL, kPfWaves>(L, T, w, w.xplanes, (size_t)T * L.H * 2,
                                            (L.I / 32 + kPfWaves - 1) / kPfWaves, mg, kStageGateUp, s, tm);
  pf_launch<2, 2, DD, false, SCL, WD>(L, T, w, w.hplanes, P * L.I * 2, rb_dn, mg, kStageDown, s, tm);
}

// MXFP4 (FMT 1) and its packed scale store (FMT 3): fp8 activation planes on the
// block-scaled matrix cores (x: 2 planes for bf16, 3 for fp32; h: 3 planes).
template <int FMT>
static void pf_launch_mx(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, int mg,
                         hipStream_t s, const Timing& tm) {
  const int Hp = (L.H + 127) / 128 * 128;
  const size_t Ip = (size_t)(L.I + kMxChunkCols - 1) / kMxChunkCols * kMxChunkCols;
  const size_t P = (size_t)T * L.k + (L.has_shared ? T : 0);
  const int rb_gu = ((L.I / 32) + kPfWaves - 1) / kPfWaves;
  const int rb_dn = (((L.H + 63) / 64) + kPfWaves - 1) / kPfWaves;
  if (x_dtype == 1) {
    MOEQ_LAUNCH(tm, kStageActQuant, (k_mx_xquant<1, 2>), dim3(T), dim3(256), 0, s, x, T, L.H, Hp, w.xq);
    pf_launch<FMT, 2, 4, true, 0, kPfWaves>(L, T, w, w.xq, (size_t)T * Hp, rb_gu, mg, kStageGateUp, s, tm);
  } else {
    MOEQ_LAUNCH(tm, kStageActQuant, (k_mx_xquant<0, 3>), dim3(T), dim3(256), 0, s, x, T, L.H, Hp, w.xq);
    pf_launch<FMT, 3, 3, true, 0, kPfWaves>(L, T, w, w.xq, (size_t)T * Hp, rb_gu, mg, kStageGateUp, s, tm);
  }
  pf_launch<FMT, 3, 3, false, 0, kPfWaves>(L, T, w, w.hq, P * Ip, rb_dn, mg, kStageDown, s, tm);
}

hipError_t launch_experts(const LayerArgs& L, const void* x, int x_dtype, int T, const Work& w, float* y,
                          hipStream_t s, const Timing& tm) {
  const int P = T * L.k + (L.has_shared ? T : 0);
  const int mg = max_groups(P, L.E);
  if (L.wfmt == 1) {
    pf_launch_mx<1>(L, x, x_dtype, T, w, mg, s, tm);
  } else if (L.wfmt == 3) {
    pf_launch_mx<3>(L, x, x_dtype, T, w, mg, s, tm);
  } else {
    // both K ranges must be multiples of 128 for the 8-byte scale loads
    if (L.H % 128 == 0 && L.I % 128 == 0)
      pf_launch_cb4<1, 2, kPfWaves, kPfWaves, 2>(L, x, x_dtype, T, w, mg, s, tm);
    else
      pf_launch_cb4<0, 2, kPfWaves, kPfWaves, 2>(L, x, x_dtype, T, w, mg, s, tm);
  }
  return launch_combine(L, T, w, y, s, tm);
}

hipError_t launch_combine(const LayerArgs& L, int T, const Work& w, float* y, hipStream_t s, const Timing& tm) {
  MOEQ_LAUNCH(tm, kStageCombine, k_pf_combine, dim3((L.H + 255) / 256, T), dim3(256), 0, s, T, L.H, L.k,
              L.has_shared, (const float*)w.o, (const float*)w.pair_w, w.resid, y);
  return hipGetLastError();
}

}  // namespace moeq
