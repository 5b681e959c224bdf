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
// Tile: BM rows (128, or 64 when 128-row tiles would leave most of the chip
// idle, as in the 512-token down-projection) x 128 output channels (64 gate + 64 up
// channels in the gate-up mode), 256 threads = 4 waves in 2 x 2, each
// (BM / 2) x 64 (BM / 64 x 2 fragments of the 32x32x16 MFMA).  K steps of 64.
// The operands are loaded into registers D steps ahead of the step being
// computed (one step ahead left each workgroup waiting out most of a load's
// latency every step).  A, and bf16 B, are then staged into a
// double-buffered LDS tile (128-byte rows, swizzled) one step ahead; MXFP4 B
// bypasses the LDS: each lane loads the 32 codes and the one scale of its
// own fragment rows and widens them in registers (LDS traffic is what bounds
// these small tiles: a wave's fragment reads cost as many LDS cycles as its
// MFMAs take).  Output fragments have the channel on the lane, so every store
// instruction writes 32 consecutive channels of a row.
//
// K order inside a step: instruction kk of the four 32x32x16 MFMAs of a step
// takes, in lane half hi, the 8 elements of chunk 4 hi + kk, on both
// operands (any assignment of a step's elements to instructions gives the
// same sum, as long as A and B agree); a lane's four chunks are then 32
// contiguous elements, one 16-byte load of MXFP4 codes under one scale.
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

template <bool FP4, int MODE, int BM, int D>
__global__ __launch_bounds__(256, 2) void dense_kernel(DenseParams p) {
  constexpr int FM = BM / 64;   // 32-row fragments per wave
  constexpr int AQ = BM / 32;   // 16-byte A chunks per thread and step (BM rows x 8 chunks)
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][BM * kDnK];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][128 * kDnK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;

  // the row tiles of one channel tile are consecutive, so that they read its
  // weights while they are in the XCD's L2; with a K split, workgroup z of
  // a tile contracts K range [z K / ns, (z + 1) K / ns) into partial z
  const int ns = p.ksplit > 1 ? p.ksplit : 1;
  const long tiles_m = (p.M + BM - 1) / BM;
  const long tiles = tiles_m * p.tiles_n;
  const long tz = xcd_remap(blockIdx.x, tiles * ns);
  const int kz = (int)(tz / tiles);
  const long t = tz - (long)kz * tiles;
  const int m0 = (int)(t % tiles_m) * BM;
  const int tn = (int)(t / tiles_m);
  constexpr bool gate_up = MODE == kDnGateUp;
  const int n0 = tn * (gate_up ? 64 : 128);
  const int K = p.K, kw = K / ns, kb = kz * kw, nk = kw / kDnK;

  // staging: A (and bf16 B) chunk q = tid + 256 i is row q >> 3, chunk q & 7
  auto b_row = [&](int r) -> long { return gate_up ? (long)(n0 + (r & 63)) : (long)(n0 + r); };
  auto b_mat = [&](int r) -> const uint8_t* {
    return reinterpret_cast<const uint8_t*>(gate_up && r >= 64 ? p.b3 : p.b);
  };
  const uint16_t* asrc[AQ];
  const uint16_t* bsrc[4] = {nullptr, nullptr, nullptr, nullptr};
#pragma unroll
  for (int i = 0; i < AQ; ++i) {
    const int q = tid + 256 * i, r = q >> 3, c = q & 7;
    const int gr = min(m0 + r, p.M - 1);
    asrc[i] = p.a + (long)gr * p.lda + kb + c * 8;
  }
  if constexpr (!FP4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, r = q >> 3, c = q & 7;
      bsrc[i] = reinterpret_cast<const uint16_t*>(b_mat(r)) + b_row(r) * K + kb + c * 8;
    }
  // fragment rows: A rows wm * BM / 2 + 32f + l32; B rows wn*64 + 32j + l32,
  // or in the gate-up mode the gate rows wn*32 + l32 (j = 0) and the up rows
  // 64 + wn*32 + l32 (j = 1) of the same channels
  int ar[FM], br[2];
#pragma unroll
  for (int f = 0; f < FM; ++f) ar[f] = wm * (BM / 2) + 32 * f + l32;
#pragma unroll
  for (int j = 0; j < 2; ++j) br[j] = gate_up ? 64 * j + wn * 32 + l32 : wn * 64 + 32 * j + l32;
  // MXFP4 B: lane (l32, hi) of fragment j reads, per step, the 16 bytes of
  // codes of elements [32 hi, +32) of its row and their one scale byte
  const uint8_t* fcode[2] = {nullptr, nullptr};
  const uint8_t* fscale[2] = {nullptr, nullptr};
  if constexpr (FP4)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      fcode[j] = b_mat(br[j]) + b_row(br[j]) * (K / 2) + kb / 2 + hi * 16;
      fscale[j] = (gate_up && br[j] >= 64 ? p.bs3 : p.bs) + b_row(br[j]) * (K / 32) + kb / 32 + hi;
    }

  // one step's operands in registers (native vectors: HIP's uint4 struct
  // keeps arrays of them out of registers)
  struct St {
    v4i a[AQ];
    v4i b[FP4 ? 1 : 4];
    v4i c[2];       // MXFP4: the codes of fragments 0 and 1
    uint32_t s[2];  // and their scales
  };
  auto load = [&](int ks, St& st) {
    static_for<AQ>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      st.a[i] = *reinterpret_cast<const v4i*>(asrc[i] + (long)ks * kDnK);
    });
    if constexpr (FP4) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        st.c[j] = *reinterpret_cast<const v4i*>(fcode[j] + (long)ks * (kDnK / 2));
        st.s[j] = fscale[j][ks * 2];
      }
    } else {
      static_for<4>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        st.b[i] = *reinterpret_cast<const v4i*>(bsrc[i] + (long)ks * kDnK);
      });
    }
  };
  auto store = [&](const St& st, int buf) {
    static_for<AQ>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int q = tid + 256 * i, r = q >> 3, c = q & 7;
      *reinterpret_cast<v4i*>(&sa[buf][r * kDnK + dn_slot(r, c) * 8]) = st.a[i];
    });
    if constexpr (!FP4) {
      static_for<4>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int q = tid + 256 * i, r = q >> 3, c = q & 7;
        *reinterpret_cast<v4i*>(&sb[buf][r * kDnK + dn_slot(r, c) * 8]) = st.b[i];
      });
    }
  };

  v16f acc[FM][2];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[f][j][v] = 0.0f;

  // MXFP4 B of the step being computed, widened: wb[j][kk] is fragment j's
  // operand of instruction kk
  auto compute = [&](int buf, const St& cur) {
    v8bf wb[2][4];
    if constexpr (FP4)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t words[4] = {(uint32_t)cur.c[j][0], (uint32_t)cur.c[j][1], (uint32_t)cur.c[j][2],
                                   (uint32_t)cur.c[j][3]};
        fp4x32_to_bf16(words, e8m0_to_f32(cur.s[j]), wb[j]);
      }
#pragma unroll
    for (int kk = 0; kk < kDnK / 16; ++kk) {
      const int c = 4 * hi + kk;
      v8bf a[FM], b[2];
#pragma unroll
      for (int f = 0; f < FM; ++f) a[f] = *reinterpret_cast<const v8bf*>(&sa[buf][ar[f] * kDnK + dn_slot(ar[f], c) * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = FP4 ? wb[j][kk] : *reinterpret_cast<const v8bf*>(&sb[buf][br[j] * kDnK + dn_slot(br[j], c) * 8]);
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[f][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[f], b[j], acc[f][j], 0, 0, 0);
    }
  };

  // step s's registers are st[s % D] (D >= 2), loaded D steps ahead.  Its A
  // (and bf16 B) goes to LDS buffer s & 1 while step s - 1 is computed; its
  // MXFP4 B is widened when step s is computed, which frees the slot for
  // step s + D.  The loop runs over the steps padded to a multiple of D with
  // every load and LDS store unconditional (a load past the last step
  // re-reads the last step, a store past it fills the buffer nothing reads
  // again): loads issued on every path keep the compiler's count of the
  // loads in flight exact, so each wait is for the one step it needs.
  static_assert(D >= 2, "a step's slot is refilled only after it is computed");
  St st[D];
  static_for<D>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    load(min(j, nk - 1), st[j]);
  });
  store(st[0], 0);
  __syncthreads();
  const int nkp = (nk + D - 1) / D * D;
  for (int k0 = 0; k0 < nkp; k0 += D) {
    static_for<D>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int ks = k0 + j;
      if (ks < nk) compute(ks & 1, st[j]);
      store(st[(j + 1) % D], (ks + 1) & 1);
      load(min(ks + D, nk - 1), st[j]);
      __syncthreads();
    });
  }

  // ---- epilogue: lane holds channel l32 of each fragment and, in entry
  // v = 4q + s, row 8q + 4hi + s of it
  const bool situ_act = p.act == kActSitu;
  // the addend of every entry first (rows past M read row M - 1), so that
  // its loads are in flight together rather than one round trip per entry
  float add[FM][2][16];
  if constexpr (MODE == kDnAddBf16)
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = min(m0 + wm * (BM / 2) + 32 * f + 8 * (v >> 2) + 4 * hi + (v & 3), p.M - 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) add[f][j][v] = p.addend[(long)m * p.ldc + n0 + wn * 64 + 32 * j + l32];
      }
#pragma unroll
  for (int f = 0; f < FM; ++f) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * (BM / 2) + 32 * f + 8 * (v >> 2) + 4 * hi + (v & 3);
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
          if constexpr (MODE == kDnStoreF32) reinterpret_cast<float*>(p.c)[(long)kz * p.M * p.ldc + o] = y;
          else if constexpr (MODE == kDnAddBf16) reinterpret_cast<uint16_t*>(p.c)[o] = (uint16_t)bf16_rne(y + add[f][j][v]);
          else reinterpret_cast<uint16_t*>(p.c)[o] = (uint16_t)bf16_rne(y);
        }
      }
    }
  }
}

// Row-tile height: 128, unless 128-row tiles would occupy fewer than half
// the CUs (the 512-token down-projection: 112 tiles); 64-row tiles double
// the workgroups but read each weight tile twice as often, which costs more
// than it gains once 128-row tiles reach about one workgroup per CU.
static int dense_tile_rows(int M, long tiles_n) { return (long)((M + 127) / 128) * tiles_n >= kNumCUs / 2 ? 128 : 64; }

hipError_t launch_dense(const DenseParams& p_in, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (p_in.M == 0) return hipSuccess;
  DenseParams p = p_in;
  p.tiles_n = p.N / (p.mode == kDnGateUp ? 64 : 128);
  const int bm = dense_tile_rows(p.M, p.tiles_n);
  const long grid = (long)((p.M + bm - 1) / bm) * p.tiles_n;
  const bool fp4 = p.bfmt == kMxfp4;
  // steps in flight: as many as the registers hold at two workgroups per CU
#define MOE_DN_LAUNCH(F, M, B, D)                                                                       \
  hipExtLaunchKernelGGL(dense_kernel<F, M, B, D>, dim3((unsigned)grid), dim3(256), 0, s, ev_start, ev_stop, 0, p)
#define MOE_DN(F, M)                                                 \
  if (bm == 128) {                                                   \
    if (F) MOE_DN_LAUNCH(true, M, 128, 4); else MOE_DN_LAUNCH(false, M, 128, 3); \
  } else {                                                           \
    if (F) MOE_DN_LAUNCH(true, M, 64, 8); else MOE_DN_LAUNCH(false, M, 64, 5);   \
  }
  switch (p.mode) {
    case kDnStoreF32: MOE_DN(fp4, kDnStoreF32); break;
    case kDnAddBf16: MOE_DN(fp4, kDnAddBf16); break;
    case kDnGateUp: MOE_DN(fp4, kDnGateUp); break;
    default: MOE_DN(fp4, kDnStoreBf16); break;
  }
#undef MOE_DN
#undef MOE_DN_LAUNCH
  return hipGetLastError();
}

// out[m][n] = bf16(part[0][m][n] + part[1][m][n] + ...), four channels per
// thread (N is a multiple of 128).
__global__ __launch_bounds__(256) void dense_split_sum_kernel(const float* __restrict__ part, int ns, int M, int N,
                                                              uint16_t* __restrict__ out, long ldc) {
  const long mn = (long)M * N;
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  float4 v = *reinterpret_cast<const float4*>(part + i);
  for (int z = 1; z < ns; ++z) {
    const float4 w = *reinterpret_cast<const float4*>(part + (long)z * mn + i);
    v.x += w.x;
    v.y += w.y;
    v.z += w.z;
    v.w += w.w;
  }
  const long m = i / N, n = i - m * N;
  *reinterpret_cast<uint2*>(out + m * ldc + n) =
      make_uint2(bf16_rne(v.x) | (bf16_rne(v.y) << 16), bf16_rne(v.z) | (bf16_rne(v.w) << 16));
}

hipError_t launch_dense_splitk(const DenseParams& p_in, int ksplit, float* part, hipStream_t s,
                               hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (p_in.M == 0) return hipSuccess;
  if (ksplit < 1 || p_in.mode != kDnStoreBf16 || p_in.K % (kDnK * ksplit) != 0 || p_in.N % 128 != 0)
    return hipErrorInvalidValue;
  DenseParams p = p_in;
  p.mode = kDnStoreF32;
  p.c = part;
  p.ldc = p.N;
  p.ksplit = ksplit;
  p.tiles_n = p.N / 128;
  // 128-row tiles once the split gives them half the CUs (each weight tile
  // is then read by half as many workgroups as with 64-row tiles)
  const long tiles128 = (long)((p.M + 127) / 128) * p.tiles_n;
  const int bm = tiles128 * ksplit >= kNumCUs / 2 ? 128 : 64;
  const long grid = (long)((p.M + bm - 1) / bm) * p.tiles_n * ksplit;
  const bool fp4 = p.bfmt == kMxfp4;
  if (bm == 128) {
    if (fp4) hipExtLaunchKernelGGL(dense_kernel<true, kDnStoreF32, 128, 4>, dim3((unsigned)grid), dim3(256), 0, s, ev_start, nullptr, 0, p);
    else hipExtLaunchKernelGGL(dense_kernel<false, kDnStoreF32, 128, 3>, dim3((unsigned)grid), dim3(256), 0, s, ev_start, nullptr, 0, p);
  } else {
    if (fp4) hipExtLaunchKernelGGL(dense_kernel<true, kDnStoreF32, 64, 8>, dim3((unsigned)grid), dim3(256), 0, s, ev_start, nullptr, 0, p);
    else hipExtLaunchKernelGGL(dense_kernel<false, kDnStoreF32, 64, 5>, dim3((unsigned)grid), dim3(256), 0, s, ev_start, nullptr, 0, p);
  }
  const long groups = (long)p.M * p.N / 4;
  hipExtLaunchKernelGGL(dense_split_sum_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, nullptr, ev_stop,
                        0, part, ksplit, p.M, p.N, reinterpret_cast<uint16_t*>(p_in.c), p_in.ldc);
  return hipGetLastError();
}

}  // namespace moe
