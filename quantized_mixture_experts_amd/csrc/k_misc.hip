// Dequantisation export (bit-exact, through the same decode helpers the projection
// kernels use) and the RMS rescale applied between stacked layers.
#include "device.h"
#include "launch.h"

namespace moeq {

// One thread per 32-value block (row, kb): out[row][32kb .. 32kb+31].
template <int FMT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ packed, const int8_t* __restrict__ codebook,
                                                 int rows, int cols, float* __restrict__ out) {
  __shared__ uint32_t lut[256];
  if (FMT == 2) {
    build_cb4_lut(lut, codebook);
    __syncthreads();
  }
  const int nkb = cols >> 5;
  const size_t blk = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= (size_t)rows * nkb) return;
  const int row = (int)(blk / nkb), kb = (int)(blk % nkb);
  const int m = row & 15;
  const PackedTile pt = packed_tile<FMT>(packed, rows, cols, row >> 4);
  const u32x4_t c = *(const __attribute__((address_space(1))) u32x4_t*)(pt.codes + pk_code(kb, m));
  float* dst = out + blk * 32;
  if (fmt_is_mx(FMT)) {
    const float s = e8m0_to_f32(FMT == 3 ? ps_e8m0(pt.bases[m], pt.scales[pk_scale_mx(kb, m) >> 1], m)
                                         : pt.scales[pk_scale_mx(kb, m)]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8_t v = fp4x8_to_bf16(c[q], s);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[8 * q + i] = (float)v[i];
    }
  } else {
    const uint16_t sb =
        *(const __attribute__((address_space(1))) uint16_t*)(pt.scales + 2 * pk_scale_cb(kb, m, nkb));
    const float s = half_bits_to_f32(sb);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8_t v = cb4x8_to_bf16(c[q], lut);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[8 * q + i] = s * (float)v[i];
    }
  }
}

// 3-bit affine: one thread per 8 values (row, columns 8c .. 8c+7), fp32 out = fmaf(s, q, b),
// the fp32 rounding of the exact s * q + b.
__global__ __launch_bounds__(256) void k_dequant_aff3(const uint8_t* __restrict__ packed, int rows, int cols,
                                                      float* __restrict__ out) {
  const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (size_t)rows * (cols / 8)) return;
  const int row = (int)(id / (cols / 8)), c8 = (int)(id % (cols / 8));
  const int m = row & 15, st = c8 / 16, cc = 8 * (c8 % 16);
  const int j = cc / 32, g = (cc % 32) / 8;
  const PackedTile pt = packed_tile<4>(packed, rows, cols, row >> 4);
  const gbyte_t* wp = pt.codes + 768 * st + 12 * (16 * g + m);
  const u32x3_t w = {*(const __attribute__((address_space(1))) uint32_t*)wp,
                     *(const __attribute__((address_space(1))) uint32_t*)(wp + 4),
                     *(const __attribute__((address_space(1))) uint32_t*)(wp + 8)};
  uint32_t o[16];
  aff3_pairs(w, o);
  const uint32_t sb = *(const __attribute__((address_space(1))) uint32_t*)(pt.scales + 128 * st + 8 * m + 4 * (j / 2));
  const float sc = half_bits_to_f32((uint16_t)(sb & 0xFFFFu)), bi = half_bits_to_f32((uint16_t)(sb >> 16));
  float* dst = out + (size_t)row * cols + 8 * c8;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    dst[2 * d] = fmaf(sc, (float)((o[4 * j + d] & 0xFFFFu) - 0x4300u), bi);
    dst[2 * d + 1] = fmaf(sc, (float)((o[4 * j + d] >> 16) - 0x4300u), bi);
  }
}

// x_next[t][n] = bf16_rne(y[t][n] / sqrt(mean_n y^2 + eps)); one block of 256 threads per
// token.  The sum of squares, the mean, the square root and the quotient are fp64 (the
// quotient correctly rounded: rms_apply), then rounded once to bf16.
__global__ __launch_bounds__(256) void k_rms_rescale(const float* __restrict__ y, int H, float eps,
                                                     uint16_t* __restrict__ out) {
  __shared__ double part[4];
  const int t = blockIdx.x;
  const float* yt = y + (size_t)t * H;
  if (H <= kRmsRegCols) {  // the row read once: its values stay in registers
    float v[16];
    const double s = wave_sum_f64(rms_partial_keep(yt, H, threadIdx.x, v));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    const double d = rms_divisor(part[0], part[1], part[2], part[3], H, eps);
    const double rd = 1.0 / d;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int n = threadIdx.x + 256 * u;
      const uint16_t q = rms_apply(v[u], d, rd);
      if (n < H) out[(size_t)t * H + n] = q;
    }
    return;
  }
  const double s = wave_sum_f64(rms_partial(yt, H, threadIdx.x));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  const double d = rms_divisor(part[0], part[1], part[2], part[3], H, eps);
  const double rd = 1.0 / d;
  for (int n0 = threadIdx.x; n0 < H; n0 += 8 * 256) {
    uint16_t v[8];
    rms_apply8(yt, n0, 256, H, d, rd, v);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (n0 + 256 * u < H) out[(size_t)t * H + n0 + 256 * u] = v[u];
  }
}

// Streaming-read probe: every lane reads 16-byte chunks, grid-stride, with nontemporal
// loads, and each block writes the xor of what it read (so the loads are not dropped).
// It measures the HBM read bandwidth a plain stream achieves, the reference point the
// layer's kernels are compared with besides the specification's peak.
__global__ __launch_bounds__(256) void k_read_probe(const u32x4_t* __restrict__ src, size_t n16,
                                                    uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4_t*)(src + i));
    const u32x4_t b = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4_t*)(src + i + stride));
    const u32x4_t c =
        __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4_t*)(src + i + 2 * stride));
    const u32x4_t d =
        __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4_t*)(src + i + 3 * stride));
    acc ^= (a[0] ^ a[1] ^ a[2] ^ a[3]) ^ (b[0] ^ b[1] ^ b[2] ^ b[3]) ^ (c[0] ^ c[1] ^ c[2] ^ c[3]) ^
           (d[0] ^ d[1] ^ d[2] ^ d[3]);
  }
  for (; i < n16; i += stride) {
    const u32x4_t a = src[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  __shared__ uint32_t part[4];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(k_read_probe, dim3(blocks), dim3(256), 0, s, (const u32x4_t*)buf, bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_dequant(int wfmt, const uint8_t* packed, const int8_t* codebook, int rows, int cols,
                          float* out, hipStream_t s) {
  const size_t nblk = (size_t)rows * (cols / 32);
  const dim3 grid((unsigned)((nblk + 255) / 256));
  if (wfmt == 1)
    hipLaunchKernelGGL(k_dequant<1>, grid, dim3(256), 0, s, packed, codebook, rows, cols, out);
  else if (wfmt == 3)
    hipLaunchKernelGGL(k_dequant<3>, grid, dim3(256), 0, s, packed, codebook, rows, cols, out);
  else if (wfmt == 4)
    hipLaunchKernelGGL(k_dequant_aff3, dim3((unsigned)(((size_t)rows * (cols / 8) + 255) / 256)), dim3(256), 0, s,
                       packed, rows, cols, out);
  else
    hipLaunchKernelGGL(k_dequant<2>, grid, dim3(256), 0, s, packed, codebook, rows, cols, out);
  return hipGetLastError();
}

hipError_t launch_rms_rescale(const float* y, int T, int H, float eps, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_rms_rescale, dim3(T), dim3(256), 0, s, y, H, eps, out);
  return hipGetLastError();
}

}  // namespace moeq
