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

// Layer descriptor as the kernels see it (copied by value into kernel arguments).
struct LayerArgs {
  int H, I, E, k, wfmt, has_shared;
  const float* router_w;
  const float* router_b;
  const uint8_t* const* gate_up;
  const uint8_t* const* down;
  const int8_t* codebook;
  const float* shared_gate_w;
};

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
  float* o;            // [P][H]  expert outputs (down projection, before the gate)
  uint32_t* tickets;   // [H/16] arrival counters of the decode down/combine kernel
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// IEEE fp16 bits -> fp32 (exact, subnormals included).
__device__ __forceinline__ float half_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
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
__device__ __forceinline__ bf16x8_t cb4x8_to_bf16(uint32_t codes, const uint32_t* lut) {
  u32x4_t v;
  v[0] = lut[codes & 0xFFu];
  v[1] = lut[(codes >> 8) & 0xFFu];
  v[2] = lut[(codes >> 16) & 0xFFu];
  v[3] = lut[codes >> 24];
  return __builtin_bit_cast(bf16x8_t, v);
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

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + expf(-a)); }

}  // namespace moeq
