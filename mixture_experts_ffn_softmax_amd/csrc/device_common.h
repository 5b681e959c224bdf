// Device-side helpers shared by the kernels: number formats and wave/block
// reductions.  Formats follow the OCP 8-bit floating point (E4M3FN) and
// bfloat16 definitions; see the public header for where the layer uses them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Largest finite e4m3 magnitude; per-row scales are amax / kE4M3Max.
constexpr float kE4M3Max = 448.0f;

// Finite binary32 -> e4m3 code: round to nearest, ties to even mantissa,
// saturate at +-448, keep the sign of zero.
//  * |v| < 2^-6 lies on the subnormal grid k * 2^-9 (k = 0..8; k = 8 is the
//    smallest normal, code 0x08): scale by 2^9 exactly and round to integer.
//  * otherwise round the binary32 mantissa to 3 bits (a carry moves into the
//    exponent) and rebias the exponent from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), kE4M3Max);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    const uint32_t b = __float_as_uint(a);
    const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return sign | code;
}

// binary32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Block-wide max / sum of one value per thread (blockDim.x a multiple of 64
// or a single partial wave); `red` needs blockDim.x / 64 floats.
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int nw = (blockDim.x + 63) >> 6;
  if (nw == 1) return v;
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int nw = (blockDim.x + 63) >> 6;
  if (nw == 1) return v;
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r += red[i];
  __syncthreads();
  return r;
}

// Exclusive prefix sum over n <= 1024 ints held in LDS `a` (in place) by a
// block of exactly 1024 threads; returns the total.  `tmp` holds 16 ints.
__device__ __forceinline__ int block_exclusive_scan_1024(int* a, int* tmp, int n) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int x = (t < n) ? a[t] : 0;
  int v = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {   // inclusive scan inside the wave
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) tmp[t >> 6] = v;
  __syncthreads();
  if (t < 64) {                               // inclusive scan of the 16 wave totals
    int w = (t < 16) ? tmp[t] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(w, off);
      if (t >= off) w += o;
    }
    if (t < 16) tmp[t] = w;
  }
  __syncthreads();
  const int wave_base = (t >= 64) ? tmp[(t >> 6) - 1] : 0;
  const int total = tmp[15];
  if (t < n) a[t] = wave_base + v - x;
  __syncthreads();
  return total;
}

}  // namespace moe
