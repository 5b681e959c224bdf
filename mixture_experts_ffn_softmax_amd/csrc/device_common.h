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
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal, for data a workgroup reads once and no
// other workgroup of the launch is expected to re-read (streamed weights):
// the caches then do not keep it at the expense of operands that are re-read.
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A weight load of the small GEMMs: non-temporal when NT (each weight tile
// is read by about one row tile of the launch, so caching it gains nothing),
// an ordinary load when several row tiles re-read it.
template <bool NT>
__device__ __forceinline__ uint4 load_w16(const uint8_t* p) {
  if constexpr (NT) return load_stream16(p);
  else return *reinterpret_cast<const uint4*>(p);
}

// Largest finite e4m3 magnitude; per-row scales are amax / kE4M3Max.
constexpr float kE4M3Max = 448.0f;

// Finite binary32 -> e4m3 codes: round to nearest, ties to even mantissa,
// saturate at +-448, keep the sign of zero.  The value is clamped to +-448
// and converted by v_cvt_pk_fp8_f32 (OCP e4m3 on this GPU, round to nearest
// even, subnormals on the 2^-9 grid).  Two values per instruction: a goes to
// byte 2*HI, b to byte 2*HI + 1 of the result; the other half-word is `old`'s.
// Checked against a software encoder (mantissa rounded to 3 bits with the
// carry into the exponent, or k * 2^-9 below 2^-6) for every binary32 of
// magnitude <= 448, both signs: identical codes.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t old) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// binary32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// 1 / s for quot_e4m3, or 0 when it is not finite (s below 2^-126), which
// sends every element to the division.
__device__ __forceinline__ float e4m3_recip(float s) {
  const float r = 1.0f / s;
  return (r < INFINITY) ? r : 0.0f;
}

// Quotients x / s for e4m3 encoding.  The product y = x * r (r = rounded
// 1/s) is within 2.5 binary32 ulps of the exact quotient, so y and the
// rounded quotient q lie within 2 ulps of each other and have the same e4m3
// code unless an e4m3 rounding midpoint (low 20 mantissa bits 0x80000 in the
// normal range) lies between them.  y is kept unless it is within 4 ulps of
// a midpoint, below 2^-6 (the subnormal grid, whose midpoints sit elsewhere)
// or r = 0; if any lane of the wave has such an element, the wave takes the
// IEEE divisions for all eight (a wave-uniform branch, so that the common
// case runs no division).  Checked on the CPU for every bf16 x against 20000
// scales (half of them amax / 448 of a bf16 amax): identical codes; with
// the window cut to the midpoint alone, 2910 of 2.3e8 differ.
__device__ __forceinline__ bool e4m3_near_boundary(float y) {
  const uint32_t yb = __float_as_uint(y) & 0x7FFFFFFFu;
  return yb < 0x3C800000u || ((yb & 0xFFFFFu) - 0x7FFFCu) < 9u;
}

// Four words of two bf16 each (elements 2i in the low half) divided by s ->
// 8 e4m3 codes in element order (r = e4m3_recip(s)).
__device__ __forceinline__ uint2 e4m3_encode8(const uint32_t (&w)[4], float s, float r) {
  float x[8], q[8];
  bool slow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    q[i] = x[i] * r;
    slow |= e4m3_near_boundary(q[i]);
  }
  if (__builtin_expect(__ballot(slow) != 0, 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = x[i] / s;
  }
  uint32_t p0 = e4m3_pack2<false>(q[0], q[1], 0u);
  p0 = e4m3_pack2<true>(q[2], q[3], p0);
  uint32_t p1 = e4m3_pack2<false>(q[4], q[5], 0u);
  p1 = e4m3_pack2<true>(q[6], q[7], p1);
  return make_uint2(p0, p1);
}

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
// or a single partial wave); `red` needs blockDim.x / 64 floats.  A block of
// one wave returns straight after the wave reduction, with no barrier: LDS
// written before the call is not yet published to the other lanes.
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
