// Grouped expert GEMMs on gfx950 fp8 MFMA (v_mfma_*_16x16x128_f8f6f4).
//
// The Ling-2.6-1T page, §2 (table: the matrix unit runs the W1/W3 gate-up
// and W2 down projections, the vector unit the SiLU, gate multiply and scale
// multiplies) and §5 (per-channel direct_scaled_dot: fp8 tokens and fp8
// weights go straight into the matrix unit over the full K with fp32
// partials; per-token and per-channel scales are applied after the
// reduction).  MXFP4 weights (sglang-jax gap list §4; Kimi K3 page §2.5) use
// the block-scaled form of the same instruction: e2m1 codes with one e8m0
// scale per 32 contraction elements enter each partial product.
//
// Operand roles: the MFMA "A" operand is always a 16-row weight fragment
// (16 output channels x 128 K) and "B" a 16-row token fragment, so that each
// lane ends up holding 4 consecutive channels of one token row: lane l holds
// D[4*(l/16) + v][l%16], v = 0..3.  Lane l supplies row l%16 of its fragment
// and the 32 contraction elements [32*(l/16), 32*(l/16) + 32) of the current
// 128-wide K step; weights and tokens use the same assignment, so any K order
// the hardware applies inside one instruction is the same on both sides.
//
// Work decomposition: a tile is (group, channel tile, row tile).  Row tiles
// never straddle two groups; tile_prefix[g] counts the row tiles before group
// g, so a launch covers ragged, skewed groups with uniform tiles and needs no
// host-side knowledge of the per-expert counts.  Tiles are ordered group,
// channel tile, row tile (the row tiles that share a weight tile are
// consecutive) and then dealt out to the 8 XCDs in contiguous ranges
// (workgroup b runs on XCD b % 8), so that tiles sharing weights run together
// on one XCD and share its L2.
//
// Two variants:
//   large: 128 rows x 256 channel rows per workgroup, 4 waves in a 2 x 2
//          layout (64 rows x 128 channel rows each), A and B tiles staged
//          through a double-buffered, XOR-swizzled LDS ring.  fp8 only.
//   small: 32 rows x 64 channel rows, the 4 waves split the K steps and read
//          their fragments straight from memory into registers (no LDS
//          staging), then reduce through LDS.  For decode-sized groups,
//          where the weight stream is the bound; fp8 and MXFP4.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace moe {

struct GemmParams {
  int fmt;        // WeightFormat of the routed group (shared group: fp8)
  int n_groups;
  int n_routed;
  int K;          // contraction length (elements)
  int N;          // output channels per weight matrix
  int ntiles;     // channel tiles per group
  const int* offsets;
  const int* tile_prefix;
  // Row operand: rows < shared_row0 come from a[0] (row index r), the shared
  // group's rows from a[1] (row index r - shared_row0).
  const uint8_t* a[2];       // [rows][K] e4m3
  const float* a_scale[2];   // [rows]
  long shared_row0;
  const uint8_t* wa[2];  // GEMM1: W1 (gate), GEMM2: W2 -- [0] routed, [1] shared
  const uint8_t* wb[2];  // GEMM1: W3 (up)
  const void* sa[2];
  const void* sb[2];
  float* h;              // GEMM1 output [rows][N]
  uint32_t* amax;        // GEMM1 per-row max |h| (binary32 bits)
  uint16_t* y;           // GEMM2 output [rows][N] bf16
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& w, const v8i& x, const v4f& c) {
  // scale operands 0: the plain (unscaled) fp8 x fp8 product
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, c, 0, 0, 0, 0, 0, 0);
}

// e8m0 value of 2^0 for the token side of the block-scaled product.
constexpr int kE8m0One = 127;

__device__ __forceinline__ v4f mfma_fp4w(const v8i& w, const v8i& x, const v4f& c, int wscale) {
  // A = e2m1 weights (format 4) with a per-lane e8m0 block scale,
  // B = e4m3 tokens (format 0) with scale 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, c, 4, 0, 0, wscale, 0, kE8m0One);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Workgroup b < total -> logical tile; each XCD gets a contiguous range.
__device__ __forceinline__ long xcd_remap(long b, long total) {
  const long q = total >> 3, r = total & 7;
  const long x = b & 7, slot = b >> 3;
  return x * q + (x < r ? x : r) + slot;
}

struct TileInfo {
  int g;      // group
  int wi;     // 0 routed, 1 shared
  long eg;    // expert index within the weight array
  int row0;   // first row of the tile
  int row1;   // one past the last row of the group
  int nt;     // channel tile
};

// Locates tile L: group g is the largest with tile_prefix[g] * ntiles <= L.
__device__ __forceinline__ TileInfo find_tile(const GemmParams& p, const int* s_tp, long L, int bm) {
  int lo = 0, hi = p.n_groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long)s_tp[mid] * p.ntiles <= L) lo = mid; else hi = mid - 1;
  }
  TileInfo ti;
  ti.g = lo;
  const long local = L - (long)s_tp[lo] * p.ntiles;
  const int mcount = s_tp[lo + 1] - s_tp[lo];
  ti.nt = (int)(local / mcount);
  const int mt = (int)(local - (long)ti.nt * mcount);
  const int seg0 = p.offsets[lo];
  ti.row1 = p.offsets[lo + 1];
  ti.row0 = seg0 + mt * bm;
  ti.wi = (lo < p.n_routed) ? 0 : 1;
  ti.eg = ti.wi ? 0 : lo;
  return ti;
}

// ============================================================================
// large variant (fp8)
// ============================================================================

constexpr int kLgRows = 128;      // token rows per tile
constexpr int kLgCh = 256;        // channel rows per tile (GEMM1: 128 gate + 128 up)
constexpr int kLgTokBytes = kLgRows * 128;
constexpr int kLgStage = (kLgRows + kLgCh) * 128;   // 48 KiB

template <bool GEMM1>
__global__ __launch_bounds__(256, 1) void gemm_large_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kLgStage];
  __shared__ int s_tp[kMaxExperts + 2];

  const int tid = threadIdx.x;
  const long total = (long)p.tile_prefix[p.n_groups] * p.ntiles;
  if ((long)blockIdx.x >= total) return;
  for (int i = tid; i <= p.n_groups; i += 256) s_tp[i] = p.tile_prefix[i];
  __syncthreads();
  const TileInfo ti = find_tile(p, s_tp, xcd_remap(blockIdx.x, total), kLgRows);

  const int K = p.K;
  const int nk = K >> 7;
  const int chPerMat = GEMM1 ? (kLgCh / 2) : kLgCh;
  const int n0 = ti.nt * chPerMat;
  const uint8_t* Wa = p.wa[ti.wi] + ti.eg * (long)p.N * K;
  const uint8_t* Wb = GEMM1 ? (p.wb[ti.wi] + ti.eg * (long)p.N * K) : nullptr;

  // ---- global -> register -> LDS staging assignment ----
  // tokens: 1024 chunks of 16 B (128 rows x 8), 4 per thread
  // channels: 2048 chunks (256 rows x 8), 8 per thread
  const uint8_t* tsrc[4];
  int tdst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    const int row = q >> 3, c = q & 7;
    int grow = ti.row0 + row;
    if (grow >= ti.row1) grow = ti.row1 - 1;
    tsrc[i] = p.a[ti.wi] + (grow - (ti.wi ? p.shared_row0 : 0)) * (long)K + c * 16;
    tdst[i] = row * 128 + ((c ^ (row & 7)) << 4);
  }
  const uint8_t* csrc[8];
  int cdst[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + 256 * i;
    const int row = q >> 3, c = q & 7;
    const uint8_t* base;
    if (GEMM1) base = (row < 128) ? (Wa + (long)(n0 + row) * K) : (Wb + (long)(n0 + row - 128) * K);
    else base = Wa + (long)(n0 + row) * K;
    csrc[i] = base + c * 16;
    cdst[i] = kLgTokBytes + row * 128 + ((c ^ (row & 7)) << 4);
  }

  uint4 rt[4], rc[8];
  auto gload = [&](int ks) {
    const long ko = (long)ks << 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) rt[i] = *reinterpret_cast<const uint4*>(tsrc[i] + ko);
#pragma unroll
    for (int i = 0; i < 8; ++i) rc[i] = *reinterpret_cast<const uint4*>(csrc[i] + ko);
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * kLgStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(base + tdst[i]) = rt[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(base + cdst[i]) = rc[i];
  };

  // ---- per-lane fragment addressing ----
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lg = lane >> 4;
  const int so0 = l16 * 128 + (((2 * lg) ^ (lane & 7)) << 4);
  const int so1 = l16 * 128 + (((2 * lg + 1) ^ (lane & 7)) << 4);
  int chrow[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    if (GEMM1) chrow[f] = (f < 4) ? (wn * 64 + f * 16) : (128 + wn * 64 + (f - 4) * 16);
    else chrow[f] = wn * 128 + f * 16;
  }

  v4f acc[8][4];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[f][t] = v4f{0.f, 0.f, 0.f, 0.f};

  auto frag = [&](const uint8_t* base, int rowbase) -> v8i {
    const uint8_t* r = base + rowbase * 128;
    const uint4 x0 = *reinterpret_cast<const uint4*>(r + so0);
    const uint4 x1 = *reinterpret_cast<const uint4*>(r + so1);
    return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const bool more = (ks + 1) < nk;
    if (more) gload(ks + 1);
    const uint8_t* stage = smem + (ks & 1) * kLgStage;
    v8i xt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) xt[t] = frag(stage, wm * 64 + t * 16);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const v8i wf = frag(stage + kLgTokBytes, chrow[f]);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[f][t] = mfma_fp8(wf, xt[t], acc[f][t]);
    }
    if (more) lstore((ks + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue ----
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int grow = ti.row0 + wm * 64 + t * 16 + l16;
    const bool valid = grow < ti.row1;
    const float xs = valid ? p.a_scale[ti.wi][grow - (ti.wi ? p.shared_row0 : 0)] : 0.0f;
    if (GEMM1) {
      const float* S1 = reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N;
      const float* S3 = reinterpret_cast<const float*>(p.sb[ti.wi]) + ti.eg * p.N;
      float rmax = 0.0f;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int ch = n0 + wn * 64 + f * 16 + 4 * lg;
        const float4 s1 = *reinterpret_cast<const float4*>(S1 + ch);
        const float4 s3 = *reinterpret_cast<const float4*>(S3 + ch);
        const float sg[4] = {s1.x, s1.y, s1.z, s1.w};
        const float su[4] = {s3.x, s3.y, s3.z, s3.w};
        float hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float g = acc[f][t][v] * xs * sg[v];
          const float u = acc[f + 4][t][v] * xs * su[v];
          hv[v] = silu(g) * u;
          rmax = fmaxf(rmax, fabsf(hv[v]));
        }
        if (valid)
          *reinterpret_cast<float4*>(p.h + (long)grow * p.N + ch) = make_float4(hv[0], hv[1], hv[2], hv[3]);
      }
      rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
      rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
      if (valid && lg == 0) atomicMax(p.amax + grow, __float_as_uint(rmax));
    } else {
      const float* S2 = reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N;
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int ch = n0 + wn * 128 + f * 16 + 4 * lg;
        const float4 s2 = *reinterpret_cast<const float4*>(S2 + ch);
        const float sw[4] = {s2.x, s2.y, s2.z, s2.w};
        uint32_t b[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) b[v] = bf16_rne(acc[f][t][v] * xs * sw[v]);
        if (valid)
          *reinterpret_cast<uint2*>(p.y + (long)grow * p.N + ch) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      }
    }
  }
}

// ============================================================================
// small variant (fp8 or MXFP4 weights)
// ============================================================================

constexpr int kSmRows = 32;   // token rows per tile: 2 fragments
constexpr int kSmCh = 64;     // channel rows per tile: 4 fragments (GEMM1: 2 gate + 2 up)

template <bool GEMM1, int FMT>
__global__ __launch_bounds__(256) void gemm_small_kernel(GemmParams p) {
  __shared__ v4f red[4][8][64];                 // 32 KiB: per-wave partial sums
  __shared__ int s_tp[kMaxExperts + 2];

  const int tid = threadIdx.x;
  const long total = (long)p.tile_prefix[p.n_groups] * p.ntiles;
  if ((long)blockIdx.x >= total) return;
  for (int i = tid; i <= p.n_groups; i += 256) s_tp[i] = p.tile_prefix[i];
  __syncthreads();
  const TileInfo ti = find_tile(p, s_tp, xcd_remap(blockIdx.x, total), kSmRows);

  const int K = p.K;
  const int nk = K >> 7;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const bool fp4 = (FMT == kMxfp4) && ti.wi == 0;   // the shared group is fp8
  const long rowBytes = fp4 ? (K >> 1) : K;
  const int chPerMat = GEMM1 ? (kSmCh / 2) : kSmCh;
  const int n0 = ti.nt * chPerMat;
  const uint8_t* Wa = p.wa[ti.wi] + ti.eg * (long)p.N * rowBytes;
  const uint8_t* Wb = GEMM1 ? (p.wb[ti.wi] + ti.eg * (long)p.N * rowBytes) : nullptr;

  const uint8_t* tp[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int grow = ti.row0 + t * 16 + l16;
    if (grow >= ti.row1) grow = ti.row1 - 1;
    tp[t] = p.a[ti.wi] + (grow - (ti.wi ? p.shared_row0 : 0)) * (long)K + lg * 32;
  }
  const uint8_t* wp[4];
  const uint8_t* sp[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    long crow;
    const uint8_t* W;
    const uint8_t* S;
    if (GEMM1) {
      const int m = f >> 1;                          // 0 gate, 1 up
      crow = n0 + (f & 1) * 16 + l16;
      W = m ? Wb : Wa;
      S = reinterpret_cast<const uint8_t*>(m ? p.sb[ti.wi] : p.sa[ti.wi]);
    } else {
      crow = n0 + f * 16 + l16;
      W = Wa;
      S = reinterpret_cast<const uint8_t*>(p.sa[ti.wi]);
    }
    wp[f] = W + crow * rowBytes + (fp4 ? lg * 16 : lg * 32);
    // MXFP4 block scales of this channel row: K/32 bytes, 4 per K step
    sp[f] = fp4 ? (S + (ti.eg * (long)p.N + crow) * (K >> 5)) : nullptr;
  }

  v4f acc[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[f][t] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int ks = wave; ks < nk; ks += 4) {
    v8i x[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(tp[t] + ((long)ks << 7));
      const uint4 a1 = *reinterpret_cast<const uint4*>(tp[t] + ((long)ks << 7) + 16);
      x[t] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    }
    if (fp4) {
      v8i w[4];
      int sc[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint4 b0 = *reinterpret_cast<const uint4*>(wp[f] + ((long)ks << 6));
        w[f] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
        const uint32_t s4 = *reinterpret_cast<const uint32_t*>(sp[f] + ks * 4);
        sc[f] = (int)((s4 >> (8 * lg)) & 0xFFu);
      }
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[f][t] = mfma_fp4w(w[f], x[t], acc[f][t], sc[f]);
    } else {
      v8i w[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint4 b0 = *reinterpret_cast<const uint4*>(wp[f] + ((long)ks << 7));
        const uint4 b1 = *reinterpret_cast<const uint4*>(wp[f] + ((long)ks << 7) + 16);
        w[f] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      }
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[f][t] = mfma_fp8(w[f], x[t], acc[f][t]);
    }
  }

  // ---- reduce the 4 waves' partial sums ----
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 2; ++t) red[wave][f * 2 + t][lane] = acc[f][t];
  __syncthreads();

  const bool per_channel = !fp4;   // fp8 weights carry one scale per channel
  if (GEMM1) {
    // wave w: gate fragment f = w >> 1 (up fragment f + 2), token fragment t = w & 1
    const int f = wave >> 1, t = wave & 1;
    v4f gsum = red[0][f * 2 + t][lane], usum = red[0][(f + 2) * 2 + t][lane];
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      gsum += red[q][f * 2 + t][lane];
      usum += red[q][(f + 2) * 2 + t][lane];
    }
    const int grow = ti.row0 + t * 16 + l16;
    const bool valid = grow < ti.row1;
    const float xs = valid ? p.a_scale[ti.wi][grow - (ti.wi ? p.shared_row0 : 0)] : 0.0f;
    const int ch = n0 + f * 16 + 4 * lg;
    float sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
    if (per_channel) {
      const float4 s1 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N + ch);
      const float4 s3 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.sb[ti.wi]) + ti.eg * p.N + ch);
      sg[0] = s1.x; sg[1] = s1.y; sg[2] = s1.z; sg[3] = s1.w;
      su[0] = s3.x; su[1] = s3.y; su[2] = s3.z; su[3] = s3.w;
    }
    float hv[4], rmax = 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float g = gsum[v] * xs * sg[v];
      const float u = usum[v] * xs * su[v];
      hv[v] = silu(g) * u;
      rmax = fmaxf(rmax, fabsf(hv[v]));
    }
    if (valid) *reinterpret_cast<float4*>(p.h + (long)grow * p.N + ch) = make_float4(hv[0], hv[1], hv[2], hv[3]);
    rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
    if (valid && lg == 0) atomicMax(p.amax + grow, __float_as_uint(rmax));
  } else {
    // wave w: channel fragment f = w, both token fragments
    const int f = wave;
    const int ch = n0 + f * 16 + 4 * lg;
    float sw[4] = {1.f, 1.f, 1.f, 1.f};
    if (per_channel) {
      const float4 s2 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N + ch);
      sw[0] = s2.x; sw[1] = s2.y; sw[2] = s2.z; sw[3] = s2.w;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      v4f s = red[0][f * 2 + t][lane];
#pragma unroll
      for (int q = 1; q < 4; ++q) s += red[q][f * 2 + t][lane];
      const int grow = ti.row0 + t * 16 + l16;
      if (grow < ti.row1) {
        const float hs = p.a_scale[ti.wi][grow - (ti.wi ? p.shared_row0 : 0)];
        uint32_t b[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) b[v] = bf16_rne(s[v] * hs * sw[v]);
        *reinterpret_cast<uint2*>(p.y + (long)grow * p.N + ch) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      }
    }
  }
}

// ============================================================================
// tile prefix, quantisation of h
// ============================================================================

// Block 0 (1024 threads) scans the per-group tile counts; all blocks zero amax.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int* __restrict__ offsets, int G, int bm,
                                                           int* __restrict__ tile_prefix,
                                                           uint32_t* __restrict__ amax, long n_rows) {
  const long stride = (long)gridDim.x * 1024;
  for (long i = (long)blockIdx.x * 1024 + threadIdx.x; i < n_rows; i += stride) amax[i] = 0u;
  if (blockIdx.x != 0) return;
  __shared__ int cnt[kMaxExperts + 1];
  __shared__ int tmp[16];
  const int g = threadIdx.x;
  if (g < G) {
    const int rows = offsets[g + 1] - offsets[g];
    cnt[g] = rows > 0 ? (rows + bm - 1) / bm : 0;
  }
  __syncthreads();
  const int total = block_exclusive_scan_1024(cnt, tmp, G);
  if (g < G) tile_prefix[g] = cnt[g];
  if (g == 0) tile_prefix[G] = total;
}

// One block per row; I / 8 chunks of 8 floats, 256 threads.
__global__ __launch_bounds__(256) void quant_h_kernel(const float* __restrict__ h,
                                                      const uint32_t* __restrict__ amax, int I,
                                                      uint8_t* __restrict__ hq, float* __restrict__ hs) {
  const long r = blockIdx.x;
  const float a = __uint_as_float(amax[r]);
  const float s = (a == 0.0f) ? 1.0f : a / kE4M3Max;
  if (threadIdx.x == 0) hs[r] = s;
  const float4* src = reinterpret_cast<const float4*>(h + r * I);
  uint2* dst = reinterpret_cast<uint2*>(hq + r * I);
  for (int c = threadIdx.x; c < (I >> 3); c += 256) {
    const float4 v0 = src[2 * c], v1 = src[2 * c + 1];
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w0 |= e4m3_encode(v[i] / s) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) w1 |= e4m3_encode(v[4 + i] / s) << (8 * i);
    dst[c] = make_uint2(w0, w1);
  }
}

// ============================================================================
// launchers
// ============================================================================

long max_row_tiles(long n_rows, int n_groups, int bm) { return (n_rows + bm - 1) / bm + n_groups; }

int choose_variant(const FfnGroups& g, long n_rows) {
  const bool large_ok = g.fmt == kFp8 && (g.hidden % kLgCh) == 0 && (g.inter % (kLgCh / 2)) == 0;
  const long avg = n_rows / (g.n_groups > 0 ? g.n_groups : 1);
  return (large_ok && avg >= 64) ? kVariantLarge : kVariantSmall;
}

hipError_t launch_tile_prefix(const int* offsets, int n_groups, int bm, int* tile_prefix,
                              uint32_t* amax, long n_rows, hipStream_t s) {
  long blocks = (n_rows + 1024 * 8 - 1) / (1024 * 8);
  if (blocks < 1) blocks = 1;
  if (blocks > 256) blocks = 256;
  tile_prefix_kernel<<<(int)blocks, 1024, 0, s>>>(offsets, n_groups, bm, tile_prefix, amax, n_rows);
  return hipGetLastError();
}

static void set_rows(GemmParams& p, const RowOperand& x) {
  p.a[0] = x.q[0];
  p.a[1] = x.q[1];
  p.a_scale[0] = x.s[0];
  p.a_scale[1] = x.s[1];
  p.shared_row0 = x.shared_row0;
}

static GemmParams base_params(const FfnGroups& g, const int* tile_prefix) {
  GemmParams p{};
  p.fmt = g.fmt;
  p.n_groups = g.n_groups;
  p.n_routed = g.n_routed;
  p.offsets = g.offsets;
  p.tile_prefix = tile_prefix;
  return p;
}

hipError_t launch_gemm1(int variant, const FfnGroups& g, const RowOperand& x,
                        const int* tile_prefix, long n_rows, float* h, uint32_t* amax,
                        hipStream_t s) {
  GemmParams p = base_params(g, tile_prefix);
  p.K = g.hidden;
  p.N = g.inter;
  set_rows(p, x);
  for (int i = 0; i < 2; ++i) {
    p.wa[i] = g.w1[i];
    p.wb[i] = g.w3[i];
    p.sa[i] = g.s1[i];
    p.sb[i] = g.s3[i];
  }
  p.h = h;
  p.amax = amax;
  if (variant == kVariantLarge) {
    p.ntiles = g.inter / (kLgCh / 2);
    const long grid = max_row_tiles(n_rows, g.n_groups, kLgRows) * p.ntiles;
    gemm_large_kernel<true><<<(unsigned)grid, 256, 0, s>>>(p);
  } else {
    p.ntiles = g.inter / (kSmCh / 2);
    const long grid = max_row_tiles(n_rows, g.n_groups, kSmRows) * p.ntiles;
    if (g.fmt == kMxfp4) gemm_small_kernel<true, kMxfp4><<<(unsigned)grid, 256, 0, s>>>(p);
    else gemm_small_kernel<true, kFp8><<<(unsigned)grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_quant_h(const float* h, const uint32_t* amax, long n_rows, int I, uint8_t* hq,
                          float* hs, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  quant_h_kernel<<<(unsigned)n_rows, 256, 0, s>>>(h, amax, I, hq, hs);
  return hipGetLastError();
}

hipError_t launch_gemm2(int variant, const FfnGroups& g, const RowOperand& hq,
                        const int* tile_prefix, long n_rows, uint16_t* y, hipStream_t s) {
  GemmParams p = base_params(g, tile_prefix);
  p.K = g.inter;
  p.N = g.hidden;
  set_rows(p, hq);
  for (int i = 0; i < 2; ++i) {
    p.wa[i] = g.w2[i];
    p.sa[i] = g.s2[i];
  }
  p.y = y;
  if (variant == kVariantLarge) {
    p.ntiles = g.hidden / kLgCh;
    const long grid = max_row_tiles(n_rows, g.n_groups, kLgRows) * p.ntiles;
    gemm_large_kernel<false><<<(unsigned)grid, 256, 0, s>>>(p);
  } else {
    p.ntiles = g.hidden / kSmCh;
    const long grid = max_row_tiles(n_rows, g.n_groups, kSmRows) * p.ntiles;
    if (g.fmt == kMxfp4) gemm_small_kernel<false, kMxfp4><<<(unsigned)grid, 256, 0, s>>>(p);
    else gemm_small_kernel<false, kFp8><<<(unsigned)grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace moe
