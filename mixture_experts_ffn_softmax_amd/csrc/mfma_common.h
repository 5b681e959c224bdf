// Helpers shared by the grouped expert GEMMs and the dense GEMMs: vector
// types of the MFMA operands, exact e2m1 -> bf16 widening, direct-to-LDS
// loads with explicit waits, LDS swizzles, the XCD-aware workgroup order and
// the gate activations.
#pragma once

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace moe {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// 32 e2m1 codes (4 words, element 2i in the low nibble of byte i) times 2^e
// -> 4 x 8 bf16, exact for normal results.
__device__ __forceinline__ void fp4x32_to_bf16(const uint32_t (&w)[4], float scale, v8bf (&out)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 0);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 1);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 2);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 3);
    out[i] = v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);  // 2^(s-127)
}

__device__ __forceinline__ v8i as_v8i(const uint4& a, const uint4& b) {
  return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}
__device__ __forceinline__ v8bf as_v8bf(const uint4& a) { return __builtin_bit_cast(v8bf, a); }

// Calls fn(std::integral_constant<int, i>) for i = I .. N-1: loop bodies whose
// index must be a constant expression.
template <int N, int I = 0, class Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(std::integral_constant<int, I>{});
    static_for<N, I + 1>(fn);
  }
}

// ---- direct-to-LDS loads, waits, barriers ---------------------------------
// Explicit so that the compiler neither drains every outstanding load before
// an LDS read nor moves LDS reads across a barrier.

// 64 lanes x 16 B from `g` (per lane) to LDS [lds, lds + 1024) in lane order.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory");
}
// Wait until at most N of this wave's vector loads are outstanding and its LDS
// reads are done, then barrier.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// LDS swizzles: the 16-byte slot that holds logical chunk c of tile row r.
// A fragment read has 32 lanes on 32 consecutive rows reading the same chunk;
// these make every 8 and every 16 consecutive lanes hit distinct bank groups
// (conflict-free whether the LDS serves 8 or 16 lanes of a 16-byte read per
// cycle).
__device__ __forceinline__ int swz64(int r, int c) { return c ^ (((r >> 1) ^ (r >> 2)) & 3); }   // 64-byte rows
__device__ __forceinline__ int swz128(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }    // 128-byte rows

// Workgroup b < total -> logical tile; each XCD gets a contiguous range.
__device__ __forceinline__ long xcd_remap(long b, long total) {
  const long q = total >> 3, r = total & 7;
  const long x = b & 7, slot = b >> 3;
  return x * q + (x < r ? x : r) + slot;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// SiTU (the Kimi K3 page, §2.6): beta * tanh(g / beta) * sigmoid(g).  Its
// linear factor saturates at +-beta, where SiLU's grows without bound.
__device__ __forceinline__ float situ(float g, float beta) { return beta * tanhf(g / beta) / (1.0f + expf(-g)); }

// fast SiLU for the epilogue (h is rounded to bf16 afterwards): g * 1/(1 + 2^(-g log2 e))
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

}  // namespace moe
