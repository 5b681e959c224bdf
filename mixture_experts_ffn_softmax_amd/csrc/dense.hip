// Dense GEMMs of the LatentMoE block.
//
// The Kimi K3 page, §2.4 (LatentMoE: a down-projection from the hidden size
// to the latent before the routed experts, an up-projection back after their
// RMSNorm, shared experts on the hidden stream) and §2.5 (the projections
// are MXFP4 weight-only, the shared experts bf16).
//
// C[M][N] = epilogue( A[M][K] x B[N][K]^T ) with A bf16 row-major (the
// activations) and B either bf16 [N][K] or MXFP4 (e2m1 codes [N][K/2], e8m0
// [N][K/32]), widened exactly to bf16 while it is staged into LDS.  The
// contraction runs on the bf16 MFMA with fp32 accumulation.
//
// Tile: 128 rows x 128 output channels (64 gate + 64 up channels in the
// gate-up mode), 256 threads = 4 waves of 64 x 64 (2 x 2 fragments of the
// 32x32x16 MFMA).  K steps of 64: both operands go through registers into a
// double-buffered LDS tile (128-byte rows, swizzled), the next step's global
// loads in flight while the current step's MFMAs run.  Output fragments have
// the channel on the lane, so every store instruction writes 32 consecutive
// channels of a row.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "internal.h"
#include "mfma_common.h"

namespace moe {

constexpr int kDnM = 128;   // rows per tile
constexpr int kDnK = 64;    // contraction elements per step: 128-byte bf16 rows

// 16-byte chunk c of LDS row r (8 chunks per row) sits in slot c ^ ((r>>1)&7):
// the 16 rows a 16-lane group reads with one chunk index hit 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int dn_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

template <bool FP4, int MODE>
__global__ __launch_bounds__(256, 2) void dense_kernel(DenseParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][kDnM * kDnK];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][128 * kDnK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;

  // the row tiles of one channel tile are consecutive, so that they read its
  // weights while they are in the XCD's L2
  const long tiles_m = (p.M + kDnM - 1) / kDnM;
  const long t = xcd_remap(blockIdx.x, tiles_m * p.tiles_n);
  const int m0 = (int)(t % tiles_m) * kDnM;
  const int tn = (int)(t / tiles_m);
  constexpr bool gate_up = MODE == kDnGateUp;
  const int n0 = tn * (gate_up ? 64 : 128);
  const int K = p.K, nk = K / kDnK;

  // staging: A (and bf16 B) chunk q = tid + 256 i is row q >> 3, chunk q & 7
  auto b_row = [&](int r) -> long { return gate_up ? (long)(n0 + (r & 63)) : (long)(n0 + r); };
  auto b_mat = [&](int r) -> const uint8_t* {
    return reinterpret_cast<const uint8_t*>(gate_up && r >= 64 ? p.b3 : p.b);
  };
  const uint16_t* asrc[4];
  const uint16_t* bsrc[4] = {nullptr, nullptr, nullptr, nullptr};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i, r = q >> 3, c = q & 7;
    const int gr = min(m0 + r, p.M - 1);
    asrc[i] = p.a + (long)gr * p.lda + c * 8;
    if constexpr (!FP4) bsrc[i] = reinterpret_cast<const uint16_t*>(b_mat(r)) + b_row(r) * K + c * 8;
  }
  // MXFP4 B: thread t stages half (t & 1) of row t >> 1: 16 bytes of codes
  // (32 elements) and their one scale byte per step
  const int fr = tid >> 1, fh = tid & 1;
  const uint8_t* fcode = nullptr;
  const uint8_t* fscale = nullptr;
  if constexpr (FP4) {
    fcode = b_mat(fr) + b_row(fr) * (K / 2) + fh * 16;
    fscale = (gate_up && fr >= 64 ? p.bs3 : p.bs) + b_row(fr) * (K / 32) + fh;
  }

  v4i ra[4], rb[4], rc;   // native vectors: HIP's uint4 struct keeps these arrays out of registers
  uint32_t rs = 0;
  auto load = [&](int ks) {
    static_for<4>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      ra[i] = *reinterpret_cast<const v4i*>(asrc[i] + (long)ks * kDnK);
      if constexpr (!FP4) rb[i] = *reinterpret_cast<const v4i*>(bsrc[i] + (long)ks * kDnK);
    });
    if constexpr (FP4) {
      rc = *reinterpret_cast<const v4i*>(fcode + (long)ks * (kDnK / 2));
      rs = fscale[ks * 2];
    }
  };
  auto store = [&](int buf) {
    static_for<4>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int q = tid + 256 * i, r = q >> 3, c = q & 7;
      *reinterpret_cast<v4i*>(&sa[buf][r * kDnK + dn_slot(r, c) * 8]) = ra[i];
      if constexpr (!FP4) *reinterpret_cast<v4i*>(&sb[buf][r * kDnK + dn_slot(r, c) * 8]) = rb[i];
    });
    if constexpr (FP4) {
      const uint32_t words[4] = {(uint32_t)rc[0], (uint32_t)rc[1], (uint32_t)rc[2], (uint32_t)rc[3]};
      v8bf w[4];
      fp4x32_to_bf16(words, e8m0_to_f32(rs), w);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<v8bf*>(&sb[buf][fr * kDnK + dn_slot(fr, 4 * fh + j) * 8]) = w[j];
    }
  };

  // fragment rows: A rows wm*64 + 32f + l32; B rows wn*64 + 32j + l32, or in
  // the gate-up mode the gate rows wn*32 + l32 (j = 0) and the up rows
  // 64 + wn*32 + l32 (j = 1) of the same channels
  int ar[2], br[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    ar[f] = wm * 64 + 32 * f + l32;
    br[f] = gate_up ? 64 * f + wn * 32 + l32 : wn * 64 + 32 * f + l32;
  }
  v16f acc[2][2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[f][j][v] = 0.0f;

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kDnK / 16; ++kk) {
      const int c = 2 * kk + hi;
      v8bf a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        a[f] = *reinterpret_cast<const v8bf*>(&sa[buf][ar[f] * kDnK + dn_slot(ar[f], c) * 8]);
        b[f] = *reinterpret_cast<const v8bf*>(&sb[buf][br[f] * kDnK + dn_slot(br[f], c) * 8]);
      }
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[f][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[f], b[j], acc[f][j], 0, 0, 0);
    }
  };

  load(0);
  store(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 1 < nk) load(ks + 1);
    compute(ks & 1);
    if (ks + 1 < nk) store((ks + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds channel l32 of each fragment and, in entry
  // v = 4q + s, row 8q + 4hi + s of it
  const bool situ_act = p.act == kActSitu;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * 64 + 32 * f + 8 * (v >> 2) + 4 * hi + (v & 3);
      if (m >= p.M) continue;
      if constexpr (gate_up) {
        const float g = acc[f][0][v], u = acc[f][1][v];
        const float a = situ_act ? situ(g, p.beta) : silu(g);
        const long n = n0 + wn * 32 + l32;
        reinterpret_cast<uint16_t*>(p.c)[(long)m * p.ldc + n] = (uint16_t)bf16_rne(a * u);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const long n = n0 + wn * 64 + 32 * j + l32;
          const long o = (long)m * p.ldc + n;
          const float y = acc[f][j][v];
          if constexpr (MODE == kDnStoreF32) reinterpret_cast<float*>(p.c)[o] = y;
          else if constexpr (MODE == kDnAddBf16) reinterpret_cast<uint16_t*>(p.c)[o] = (uint16_t)bf16_rne(y + p.addend[o]);
          else reinterpret_cast<uint16_t*>(p.c)[o] = (uint16_t)bf16_rne(y);
        }
      }
    }
  }
}

hipError_t launch_dense(const DenseParams& p_in, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (p_in.M == 0) return hipSuccess;
  DenseParams p = p_in;
  p.tiles_n = p.N / (p.mode == kDnGateUp ? 64 : 128);
  const long grid = (long)((p.M + kDnM - 1) / kDnM) * p.tiles_n;
  const bool fp4 = p.bfmt == kMxfp4;
#define MOE_DN(F, M)                                                                                 \
  hipExtLaunchKernelGGL(dense_kernel<F, M>, dim3((unsigned)grid), dim3(256), 0, s, ev_start, ev_stop, 0, p)
  switch (p.mode) {
    case kDnStoreF32: if (fp4) MOE_DN(true, kDnStoreF32); else MOE_DN(false, kDnStoreF32); break;
    case kDnAddBf16: if (fp4) MOE_DN(true, kDnAddBf16); else MOE_DN(false, kDnAddBf16); break;
    case kDnGateUp: if (fp4) MOE_DN(true, kDnGateUp); else MOE_DN(false, kDnGateUp); break;
    default: if (fp4) MOE_DN(true, kDnStoreBf16); else MOE_DN(false, kDnStoreBf16); break;
  }
#undef MOE_DN
  return hipGetLastError();
}

}  // namespace moe
