// Grouped expert GEMMs on gfx950 matrix cores.
//
// The Ling-2.6-1T page, §2 (table: the matrix unit runs the W1/W3 gate-up
// and W2 down projections, the vector unit the SiLU, gate multiply and scale
// multiplies) and §5 (per-channel direct_scaled_dot: fp8 tokens and fp8
// weights go straight into the matrix unit over the full K with fp32
// partials; per-token and per-channel scales are applied after the
// reduction).  MXFP4 weights (sglang-jax gap list §4; Kimi K3 page §2.5) use
// the block-scaled form of the fp8 instruction: e2m1 codes with one e8m0
// scale per 32 contraction elements enter each partial product.
//
// GEMM1 (gate-up) is e4m3 tokens x e4m3 (or e2m1) weights on the f8f6f4
// MFMA.  Its SiLU * gate epilogue rounds h to bf16.  GEMM2 (down) is
// bf16 h x W2 on the bf16 MFMA, with W2's e4m3 / e2m1 codes converted
// exactly to bf16 in registers; its fp32 output rows are rounded only once,
// by the combine.
//
// Operand roles: the MFMA "A" operand is a weight fragment (output channels
// as rows) and "B" a token fragment, so each lane ends up holding 4
// consecutive channels of one token: for 16x16 tiles lane l holds
// D[4*(l/16) + v][l%16]; for 32x32 tiles D[8*(j/4) + 4*(l/32) + j%4][l%32],
// j = 0..15.  When both operands have the same element type, both take the
// same per-lane slice of the K step, so whatever K order the instruction
// uses is the same on both sides.  The e2m1 x e4m3 form is the exception
// (see gemm1_small_kernel).
//
// Work decomposition: a tile is (group, channel tile, row tile).  Row tiles
// never straddle two groups; tile_prefix[g] counts the row tiles before group
// g, so a launch covers ragged, skewed groups with uniform tiles without
// host knowledge of the per-expert counts.  Tiles are ordered group, channel
// tile, row tile (the row tiles that share a weight tile are consecutive) and
// dealt out to the 8 XCDs in contiguous ranges (workgroup b runs on XCD
// b % 8), so tiles that share weights run together on one XCD's L2.
//
// Two variants:
//   large: BM rows x 256 channel rows per workgroup, 4 waves in a 2 x 2
//          layout, 32x32 MFMA fragments.  Tiles stream through a ring of
//          LDS stages filled by direct-to-LDS loads (global_load_lds), issued
//          STAGES-1 steps ahead; waits and barriers are explicit.  fp8
//          weights.
//   small: 32 rows x 64 channel rows, the 4 waves split the K steps and read
//          their fragments straight from memory into registers, then reduce
//          through LDS.  For decode-sized groups, where the weight stream is
//          the bound; fp8 and MXFP4 weights.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace moe {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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
  // group's rows from a[1] (row index r - shared_row0).  GEMM1: e4m3 codes
  // with per-row scales a_scale; GEMM2: bf16 h (no scale).
  const void* a[2];
  const float* a_scale[2];
  long shared_row0;
  const uint8_t* wa[2];  // GEMM1: W1 (gate), GEMM2: W2 -- [0] routed, [1] shared
  const uint8_t* wb[2];  // GEMM1: W3 (up)
  const void* sa[2];
  const void* sb[2];
  uint16_t* h;           // GEMM1 output [rows][N] bf16
  float* y;              // GEMM2 output [rows][N] fp32
};

// ---- MFMA wrappers ---------------------------------------------------------

__device__ __forceinline__ v4f mfma16_fp8(const v8i& w, const v8i& x, const v4f& c) {
  // scale operands 0: the plain (unscaled) e4m3 x e4m3 product
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma32_fp8(const v8i& w, const v8i& x, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, c, 0, 0, 0, 0, 0, 0);
}

// e8m0 value of 2^0 (the scale operands are OCP e8m0: 2^(s - 127)).
constexpr int kE8m0One = 127;

__device__ __forceinline__ v4f mfma16_fp4w(const v8i& w, const v8i& x, const v4f& c, int wscale) {
  // A = e2m1 weights (format 4) with a per-lane e8m0 block scale,
  // B = e4m3 tokens (format 0) with scale 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, c, 4, 0, 0, wscale, 0, kE8m0One);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// 32 e4m3 codes (8 words) -> 4 x 8 bf16, exact.
__device__ __forceinline__ void fp8x32_to_bf16(const uint32_t (&w)[8], v8bf (&out)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * i], 1.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * i], 1.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * i + 1], 1.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * i + 1], 1.0f, true);
    out[i] = v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
}

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


// ---- tile lookup -----------------------------------------------------------

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
  ti.row1 = p.offsets[lo + 1];
  ti.row0 = p.offsets[lo] + mt * bm;
  ti.wi = (lo < p.n_routed) ? 0 : 1;
  ti.eg = ti.wi ? 0 : lo;
  return ti;
}

// Row r of the row operand (bytes per row `rb`).
__device__ __forceinline__ const uint8_t* row_ptr(const GemmParams& p, const TileInfo& ti, int r, long rb) {
  return reinterpret_cast<const uint8_t*>(p.a[ti.wi]) + (r - (ti.wi ? p.shared_row0 : 0)) * rb;
}

// Common prologue: exits surplus workgroups, loads the tile prefix, finds the tile.
#define MOE_TILE_PROLOGUE(BMROWS)                                                 \
  const long total_ = (long)p.tile_prefix[p.n_groups] * p.ntiles;               \
  if ((long)blockIdx.x >= total_) return;                                        \
  for (int i_ = threadIdx.x; i_ <= p.n_groups; i_ += blockDim.x) s_tp[i_] = p.tile_prefix[i_]; \
  __syncthreads();                                                               \
  const TileInfo ti = find_tile(p, s_tp, xcd_remap(blockIdx.x, total_), BMROWS)

// ============================================================================
// large GEMM1: e4m3 tokens x e4m3 W1/W3 -> h = SiLU(g) * u (bf16)
// ============================================================================
//
// LDS stage: BM token rows then 256 channel rows (W1 rows n0.., then W3 rows
// n0..), each 64 bytes of the K step, as 4 16-byte slots (swz64).  One dma16
// fills 16 rows.  Each K step issues this stage's successor STAGES-1 steps
// ahead, one pair of dma16 after each group of MFMAs, so the loads drain
// while the matrix cores work instead of stalling the wave in one burst.

constexpr int kLgCh = 256;    // channel rows per tile
#ifndef MOE_LARGE_WN
#define MOE_LARGE_WN 4
#endif
constexpr int kLgWN = MOE_LARGE_WN;   // waves along the channel rows (2 x kLgWN waves)

// fast SiLU for the epilogue (h is rounded to bf16 afterwards): g * 1/(1 + 2^(-g log2 e))
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// Waves form a 2 x WN grid: wave (wm, wn) owns tokens [wm * BM/2, +BM/2) and,
// of the 128 gate and 128 up channel rows, the slice [wn * 128/WN, +128/WN)
// of each (so gate and up of one channel meet in the same lane).  WN = 4
// gives 8 waves, two per SIMD: while one waits on its loads or the barrier,
// the other keeps the matrix core busy.
template <int BM, int WN, int STAGES>
__global__ __launch_bounds__(128 * WN, 1) void gemm1_large_kernel(GemmParams p) {
  constexpr int NW = 2 * WN;                // waves
  constexpr int kRows = BM + kLgCh;
  constexpr int kStage = kRows * 64;
  constexpr int kDma = kRows / 16;          // dma16 per stage
  constexpr int kPer = kDma / NW;           // per wave
  static_assert(kDma % NW == 0, "dma split");
  constexpr int TF = BM / 64;               // token fragments per wave (32 rows each)
  constexpr int CF = 4 / WN;                // gate fragments per wave (= up fragments)
  constexpr int NF = 2 * CF;
  constexpr int kHRow = 128 * 2 + 16;       // padded LDS row of the h tile (bytes)
  static_assert(STAGES * kStage >= BM * kHRow, "h staging fits in the ring");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * kStage];
  __shared__ int s_tp[kMaxExperts + 2];
  MOE_TILE_PROLOGUE(BM);

  const int K = p.K;
  const int nk = K >> 6;
  const int n0 = ti.nt * (kLgCh / 2);
  const uint8_t* W1 = p.wa[ti.wi] + ti.eg * (long)p.N * K;
  const uint8_t* W3 = p.wb[ti.wi] + ti.eg * (long)p.N * K;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // this lane's source of each of the wave's dma16 per stage
  const uint8_t* src[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int row = (wave * kPer + i) * 16 + (lane >> 2);
    const int chunk = swz64(row, lane & 3);
    const uint8_t* base;
    if (row < BM) {
      int r = ti.row0 + row;
      if (r >= ti.row1) r = ti.row1 - 1;
      base = row_ptr(p, ti, r, K);
    } else {
      const int c = row - BM;
      base = (c < kLgCh / 2) ? (W1 + (long)(n0 + c) * K) : (W3 + (long)(n0 + c - kLgCh / 2) * K);
    }
    src[i] = base + chunk * 16;
  }
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int ks, int i0, int i1) {
    const uint32_t st = lds0 + (ks % STAGES) * kStage;
#pragma unroll
    for (int i = i0; i < i1; ++i) dma16(src[i] + ((long)ks << 6), st + (wave * kPer + i) * 1024);
  };

  // fragment addressing: lane reads row (base + l%32), bytes [32h, 32h + 32);
  // fragment bases are multiples of 32 rows, so the swizzle depends on l%32
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hh = lane >> 5;
  const int fo0 = l32 * 64 + (swz64(l32, 2 * hh) << 4);
  const int fo1 = l32 * 64 + (swz64(l32, 2 * hh + 1) << 4);
  int chbase[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
    chbase[f] = (BM + (f < CF ? 0 : kLgCh / 2) + wn * (128 / WN) + (f % CF) * 32) * 64;

  v16f acc[NF][TF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < TF; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[f][t][j] = 0.0f;

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s, 0, kPer);

  constexpr int kDmaPerGroup = (kPer + NF - 1) / NF;
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + STAGES - 2 < nk) wait_barrier<(STAGES - 2) * kPer>();
    else wait_barrier<0>();
    const bool more = ks + STAGES - 1 < nk;
    const uint8_t* st = smem + (ks % STAGES) * kStage;
    v8i x[TF];
#pragma unroll
    for (int t = 0; t < TF; ++t) {
      const uint8_t* r = st + (wm * (BM / 2) + t * 32) * 64;
      x[t] = as_v8i(*reinterpret_cast<const uint4*>(r + fo0), *reinterpret_cast<const uint4*>(r + fo1));
    }
    v8i w = as_v8i(*reinterpret_cast<const uint4*>(st + chbase[0] + fo0),
                   *reinterpret_cast<const uint4*>(st + chbase[0] + fo1));
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      v8i wnext = w;
      if (f + 1 < NF)
        wnext = as_v8i(*reinterpret_cast<const uint4*>(st + chbase[f + 1] + fo0),
                       *reinterpret_cast<const uint4*>(st + chbase[f + 1] + fo1));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < TF; ++t) acc[f][t] = mfma32_fp8(w, x[t], acc[f][t]);
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
        const int i0 = f * kDmaPerGroup, i1 = (f + 1) * kDmaPerGroup < kPer ? (f + 1) * kDmaPerGroup : kPer;
        if (i0 < i1) issue(ks + STAGES - 1, i0, i1);
      }
      __builtin_amdgcn_sched_barrier(0);
      w = wnext;
    }
  }

  // ---- epilogue.  Lane holds token l%32 of each token fragment and, per
  // group q of 4 accumulator entries, channels 8q + 4h .. +3 of the fragment.
  // h = bf16(SiLU(g) * u) goes through a padded LDS tile [BM][128 channels]
  // so that the global stores are whole 256-byte rows.
  const float* S1 = reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N;
  const float* S3 = reinterpret_cast<const float*>(p.sb[ti.wi]) + ti.eg * p.N;
  float4 s1v[CF][4], s3v[CF][4];
#pragma unroll
  for (int c = 0; c < CF; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = n0 + wn * (128 / WN) + c * 32 + 8 * q + 4 * hh;
      s1v[c][q] = *reinterpret_cast<const float4*>(S1 + ch);
      s3v[c][q] = *reinterpret_cast<const float4*>(S3 + ch);
    }
  float xs[TF];
#pragma unroll
  for (int t = 0; t < TF; ++t) {
    int grow = ti.row0 + wm * (BM / 2) + t * 32 + l32;
    if (grow >= ti.row1) grow = ti.row1 - 1;
    xs[t] = p.a_scale[ti.wi][grow - (ti.wi ? p.shared_row0 : 0)];
  }
  wait_barrier<0>();     // every wave is done reading the stage ring
#pragma unroll
  for (int t = 0; t < TF; ++t) {
    uint8_t* hrow = smem + (wm * (BM / 2) + t * 32 + l32) * kHRow;
#pragma unroll
    for (int c = 0; c < CF; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sg[4] = {s1v[c][q].x, s1v[c][q].y, s1v[c][q].z, s1v[c][q].w};
        const float su[4] = {s3v[c][q].x, s3v[c][q].y, s3v[c][q].z, s3v[c][q].w};
        uint32_t b[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float g = acc[c][t][4 * q + v] * xs[t] * sg[v];
          const float u = acc[CF + c][t][4 * q + v] * xs[t] * su[v];
          b[v] = bf16_rne(silu_fast(g) * u);
        }
        const int col = wn * (128 / WN) + c * 32 + 8 * q + 4 * hh;
        *reinterpret_cast<uint2*>(hrow + col * 2) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      }
  }
  __syncthreads();
  // BM rows x 256 bytes: 16 threads per row, 16 bytes each
  constexpr int kRowsPerPass = 128 * WN / 16;
#pragma unroll
  for (int r0 = 0; r0 < BM; r0 += kRowsPerPass) {
    const int r = r0 + (int)(threadIdx.x >> 4), c = threadIdx.x & 15;
    const int grow = ti.row0 + r;
    if (grow < ti.row1)
      *reinterpret_cast<uint4*>(p.h + (long)grow * p.N + n0 + c * 8) =
          *reinterpret_cast<const uint4*>(smem + r * kHRow + c * 16);
  }
}

// ============================================================================
// large GEMM2: bf16 h x W2 (e4m3 -> bf16) -> y (fp32)
// ============================================================================
//
// LDS stage: BM h rows of 64 bf16 (128 bytes, 8 slots, swz128) then 256 W2
// rows of 64 e4m3 codes (64 bytes, swz64).  Waves form a 2 x WN grid: wave
// (wm, wn) owns tokens [wm * BM/2, +BM/2) and W2 rows [wn * 256/WN, +256/WN).
// DMA issue is interleaved with the MFMA groups as in GEMM1.

template <int BM, int WN, int STAGES>
__global__ __launch_bounds__(128 * WN, 1) void gemm2_large_kernel(GemmParams p) {
  constexpr int NW = 2 * WN;
  constexpr int kTokBytes = BM * 128;
  constexpr int kStage = kTokBytes + kLgCh * 64;
  constexpr int kDmaT = BM / 8;             // dma16 for h rows (8 rows each)
  constexpr int kDmaW = kLgCh / 16;         // dma16 for W2 rows (16 rows each)
  constexpr int kPer = (kDmaT + kDmaW) / NW;
  static_assert((kDmaT + kDmaW) % NW == 0, "dma split");
  constexpr int TF = BM / 64;
  constexpr int NF = 8 / WN;                // W2 fragments per wave
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * kStage];
  __shared__ int s_tp[kMaxExperts + 2];
  MOE_TILE_PROLOGUE(BM);

  const int K = p.K;                        // = I
  const int nk = K >> 6;
  const int n0 = ti.nt * kLgCh;
  const uint8_t* W2 = p.wa[ti.wi] + ti.eg * (long)p.N * K;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const uint8_t* src[kPer];
  long step[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = wave * kPer + i;
    if (q < kDmaT) {
      const int row = q * 8 + (lane >> 3);
      const int chunk = swz128(row, lane & 7);
      int r = ti.row0 + row;
      if (r >= ti.row1) r = ti.row1 - 1;
      src[i] = row_ptr(p, ti, r, 2L * K) + chunk * 16;
      step[i] = 128;
    } else {
      const int row = (q - kDmaT) * 16 + (lane >> 2);
      const int chunk = swz64(row, lane & 3);
      src[i] = W2 + (long)(n0 + row) * K + chunk * 16;
      step[i] = 64;
    }
  }
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int ks, int i0, int i1) {
    const uint32_t st = lds0 + (ks % STAGES) * kStage;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int q = wave * kPer + i;
      const uint32_t dst = (q < kDmaT) ? st + q * 1024 : st + kTokBytes + (q - kDmaT) * 1024;
      dma16(src[i] + step[i] * ks, dst);
    }
  };

  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hh = lane >> 5;
  // h fragment: row l32, bf16 elements [32h, 32h + 32) = chunks 4h .. 4h+3
  int ho[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ho[i] = l32 * 128 + (swz128(l32, 4 * hh + i) << 4);
  // W2 fragment: row l32, codes [32h, 32h + 32) = chunks 2h, 2h+1
  const int wo0 = l32 * 64 + (swz64(l32, 2 * hh) << 4);
  const int wo1 = l32 * 64 + (swz64(l32, 2 * hh + 1) << 4);

  v16f acc[NF][TF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < TF; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[f][t][j] = 0.0f;

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s, 0, kPer);

  constexpr int kDmaPerGroup = (kPer + NF - 1) / NF;
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + STAGES - 2 < nk) wait_barrier<(STAGES - 2) * kPer>();
    else wait_barrier<0>();
    const bool more = ks + STAGES - 1 < nk;
    const uint8_t* st = smem + (ks % STAGES) * kStage;
    v8bf x[TF][4];
#pragma unroll
    for (int t = 0; t < TF; ++t) {
      const uint8_t* r = st + (wm * (BM / 2) + t * 32) * 128;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[t][i] = as_v8bf(*reinterpret_cast<const uint4*>(r + ho[i]));
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint8_t* r = st + kTokBytes + (wn * (256 / WN) + f * 32) * 64;
      const uint4 c0 = *reinterpret_cast<const uint4*>(r + wo0);
      const uint4 c1 = *reinterpret_cast<const uint4*>(r + wo1);
      const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      v8bf w[4];
      fp8x32_to_bf16(cw, w);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < TF; ++t)
          acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[i], x[t][i], acc[f][t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
        const int i0 = f * kDmaPerGroup, i1 = (f + 1) * kDmaPerGroup < kPer ? (f + 1) * kDmaPerGroup : kPer;
        if (i0 < i1) issue(ks + STAGES - 1, i0, i1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  const float* S2 = reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N;
  float4 s2v[NF][4];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      s2v[f][q] = *reinterpret_cast<const float4*>(S2 + n0 + wn * (256 / WN) + f * 32 + 8 * q + 4 * hh);
#pragma unroll
  for (int t = 0; t < TF; ++t) {
    const int grow = ti.row0 + wm * (BM / 2) + t * 32 + l32;
    if (grow >= ti.row1) continue;
    float* yrow = p.y + (long)grow * p.N;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = n0 + wn * (256 / WN) + f * 32 + 8 * q + 4 * hh;
        const float4 s2 = s2v[f][q];
        *reinterpret_cast<float4*>(yrow + ch) =
            make_float4(acc[f][t][4 * q] * s2.x, acc[f][t][4 * q + 1] * s2.y, acc[f][t][4 * q + 2] * s2.z,
                        acc[f][t][4 * q + 3] * s2.w);
      }
  }
}

// ============================================================================
// small variants (decode-sized groups; fp8 or MXFP4 weights)
// ============================================================================

constexpr int kSmRows = 32;   // token rows per tile: 2 fragments of 16
constexpr int kSmCh = 64;     // channel rows per tile: 4 fragments (GEMM1: 2 gate + 2 up)

// GEMM1: 16x16x128 MFMA on e4m3 x e4m3, or e2m1 x e4m3 with block scales.
template <int FMT>
__global__ __launch_bounds__(256) void gemm1_small_kernel(GemmParams p) {
  __shared__ v4f red[4][8][64];                 // per-wave partial sums
  __shared__ int s_tp[kMaxExperts + 2];
  MOE_TILE_PROLOGUE(kSmRows);

  const int K = p.K;
  const int nk = K >> 7;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const bool fp4 = (FMT == kMxfp4) && ti.wi == 0;   // the shared group is fp8
  const long rowBytes = fp4 ? (K >> 1) : K;
  const int n0 = ti.nt * (kSmCh / 2);
  const uint8_t* Wa = p.wa[ti.wi] + ti.eg * (long)p.N * rowBytes;
  const uint8_t* Wb = p.wb[ti.wi] + ti.eg * (long)p.N * rowBytes;

  // Token fragment bytes [0,16) and [16,32) of lane group lg.  Against e4m3
  // weights both operands take bytes [32*lg, 32*lg + 32) of the K step.
  // Against e2m1 weights the operands differ: an e2m1 lane group holds K
  // [32*lg, 32*lg + 32) contiguously (one 32-element scale block) while an
  // e4m3 lane group holds K [16*lg, 16*lg + 16) in its first 16 bytes and
  // K [64 + 16*lg, 64 + 16*lg + 16) in its last 16, so the token bytes are
  // fetched from those positions to pair each product with the right K.
  const int tok_off0 = fp4 ? lg * 16 : lg * 32;
  const int tok_off1 = fp4 ? 64 + lg * 16 : lg * 32 + 16;
  const uint8_t* tp[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int r = ti.row0 + t * 16 + l16;
    if (r >= ti.row1) r = ti.row1 - 1;
    tp[t] = row_ptr(p, ti, r, K);
  }
  const uint8_t* wp[4];
  const uint8_t* sp[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int m = f >> 1;                          // 0 gate, 1 up
    const long crow = n0 + (f & 1) * 16 + l16;
    const uint8_t* W = m ? Wb : Wa;
    const uint8_t* S = reinterpret_cast<const uint8_t*>(m ? p.sb[ti.wi] : p.sa[ti.wi]);
    wp[f] = W + crow * rowBytes + (fp4 ? lg * 16 : lg * 32);
    sp[f] = fp4 ? (S + (ti.eg * (long)p.N + crow) * (K >> 5)) : nullptr;  // K/32 e8m0 per row
  }

  v4f acc[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[f][t] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int ks = wave; ks < nk; ks += 4) {
    v8i x[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      x[t] = as_v8i(*reinterpret_cast<const uint4*>(tp[t] + ((long)ks << 7) + tok_off0),
                    *reinterpret_cast<const uint4*>(tp[t] + ((long)ks << 7) + tok_off1));
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
        for (int t = 0; t < 2; ++t) acc[f][t] = mfma16_fp4w(w[f], x[t], acc[f][t], sc[f]);
    } else {
      v8i w[4];
#pragma unroll
      for (int f = 0; f < 4; ++f)
        w[f] = as_v8i(*reinterpret_cast<const uint4*>(wp[f] + ((long)ks << 7)),
                      *reinterpret_cast<const uint4*>(wp[f] + ((long)ks << 7) + 16));
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[f][t] = mfma16_fp8(w[f], x[t], acc[f][t]);
    }
  }

#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 2; ++t) red[wave][f * 2 + t][lane] = acc[f][t];
  __syncthreads();

  // wave w: gate fragment f = w >> 1 (up fragment f + 2), token fragment t = w & 1
  const int f = wave >> 1, t = wave & 1;
  v4f gsum = red[0][f * 2 + t][lane], usum = red[0][(f + 2) * 2 + t][lane];
#pragma unroll
  for (int q = 1; q < 4; ++q) {
    gsum += red[q][f * 2 + t][lane];
    usum += red[q][(f + 2) * 2 + t][lane];
  }
  const int grow = ti.row0 + t * 16 + l16;
  if (grow >= ti.row1) return;
  const float xs = p.a_scale[ti.wi][grow - (ti.wi ? p.shared_row0 : 0)];
  const int ch = n0 + f * 16 + 4 * lg;
  float sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
  if (!fp4) {   // e4m3 weights carry one scale per channel
    const float4 s1 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N + ch);
    const float4 s3 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.sb[ti.wi]) + ti.eg * p.N + ch);
    sg[0] = s1.x; sg[1] = s1.y; sg[2] = s1.z; sg[3] = s1.w;
    su[0] = s3.x; su[1] = s3.y; su[2] = s3.z; su[3] = s3.w;
  }
  uint32_t b[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float g = gsum[v] * xs * sg[v];
    const float u = usum[v] * xs * su[v];
    b[v] = bf16_rne(silu(g) * u);
  }
  *reinterpret_cast<uint2*>(p.h + (long)grow * p.N + ch) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
}

// GEMM2: 16x16x32 bf16 MFMA; W2 codes converted to bf16 in registers.  Lane
// group lg takes elements [32*lg, 32*lg + 32) of the 128-wide K step on both
// operands; sub-step i of the 4 instructions uses elements [8i, 8i + 8).
template <int FMT>
__global__ __launch_bounds__(256) void gemm2_small_kernel(GemmParams p) {
  __shared__ v4f red[4][8][64];
  __shared__ int s_tp[kMaxExperts + 2];
  MOE_TILE_PROLOGUE(kSmRows);

  const int K = p.K;                          // = I
  const int nk = K >> 7;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const bool fp4 = (FMT == kMxfp4) && ti.wi == 0;
  const long rowBytes = fp4 ? (K >> 1) : K;
  const int n0 = ti.nt * kSmCh;
  const uint8_t* W2 = p.wa[ti.wi] + ti.eg * (long)p.N * rowBytes;

  const uint8_t* tp[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int r = ti.row0 + t * 16 + l16;
    if (r >= ti.row1) r = ti.row1 - 1;
    tp[t] = row_ptr(p, ti, r, 2L * K) + lg * 64;
  }
  const uint8_t* wp[4];
  const uint8_t* sp[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const long crow = n0 + f * 16 + l16;
    wp[f] = W2 + crow * rowBytes + (fp4 ? lg * 16 : lg * 32);
    sp[f] = fp4 ? (reinterpret_cast<const uint8_t*>(p.sa[0]) + (ti.eg * (long)p.N + crow) * (K >> 5)) : nullptr;
  }

  v4f acc[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[f][t] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int ks = wave; ks < nk; ks += 4) {
    v8bf x[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[t][i] = as_v8bf(*reinterpret_cast<const uint4*>(tp[t] + ((long)ks << 8) + 16 * i));
    v8bf w[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (fp4) {
        const uint4 b0 = *reinterpret_cast<const uint4*>(wp[f] + ((long)ks << 6));
        const uint32_t cw[4] = {b0.x, b0.y, b0.z, b0.w};
        const uint32_t s = sp[f][ks * 4 + lg];
        fp4x32_to_bf16(cw, e8m0_to_f32(s), w[f]);
      } else {
        const uint4 b0 = *reinterpret_cast<const uint4*>(wp[f] + ((long)ks << 7));
        const uint4 b1 = *reinterpret_cast<const uint4*>(wp[f] + ((long)ks << 7) + 16);
        const uint32_t cw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        fp8x32_to_bf16(cw, w[f]);
      }
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[f][i], x[t][i], acc[f][t], 0, 0, 0);
  }

#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 2; ++t) red[wave][f * 2 + t][lane] = acc[f][t];
  __syncthreads();

  // wave w: channel fragment f = w, both token fragments
  const int f = wave;
  const int ch = n0 + f * 16 + 4 * lg;
  float s2v[4] = {1.f, 1.f, 1.f, 1.f};
  if (!fp4) {
    const float4 s2 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N + ch);
    s2v[0] = s2.x; s2v[1] = s2.y; s2v[2] = s2.z; s2v[3] = s2.w;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    v4f s = red[0][f * 2 + t][lane];
#pragma unroll
    for (int q = 1; q < 4; ++q) s += red[q][f * 2 + t][lane];
    const int grow = ti.row0 + t * 16 + l16;
    if (grow < ti.row1)
      *reinterpret_cast<float4*>(p.y + (long)grow * p.N + ch) =
          make_float4(s[0] * s2v[0], s[1] * s2v[1], s[2] * s2v[2], s[3] * s2v[3]);
  }
}

// ============================================================================
// tile prefix
// ============================================================================

// One block of 1024 threads scans the per-group row-tile counts.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int* __restrict__ offsets, int G, int bm,
                                                           int* __restrict__ tile_prefix) {
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

// ============================================================================
// launchers
// ============================================================================

long max_row_tiles(long n_rows, int n_groups, int bm) { return (n_rows + bm - 1) / bm + n_groups; }

int choose_variant(const FfnGroups& g, long n_rows) {
  const bool large_ok = g.fmt == kFp8 && (g.hidden % kLgCh) == 0 && (g.inter % (kLgCh / 2)) == 0;
  const long avg = n_rows / (g.n_groups > 0 ? g.n_groups : 1);
  if (!large_ok || avg < 64) return kVariantSmall;
  return avg >= 384 ? kVariantLarge256 : kVariantLarge128;
}

int variant_rows(int variant) {
  return variant == kVariantLarge256 ? 256 : variant == kVariantLarge128 ? 128 : kSmRows;
}

const char* variant_name(int variant) {
  return variant == kVariantLarge256 ? "large256" : variant == kVariantLarge128 ? "large128" : "small32";
}

hipError_t launch_tile_prefix(const int* offsets, int n_groups, int bm, int* tile_prefix, hipStream_t s) {
  tile_prefix_kernel<<<1, 1024, 0, s>>>(offsets, n_groups, bm, tile_prefix);
  return hipGetLastError();
}

static GemmParams base_params(const FfnGroups& g, const RowOperand& x, const int* tile_prefix) {
  GemmParams p{};
  p.fmt = g.fmt;
  p.n_groups = g.n_groups;
  p.n_routed = g.n_routed;
  p.offsets = g.offsets;
  p.tile_prefix = tile_prefix;
  p.a[0] = x.q[0];
  p.a[1] = x.q[1];
  p.a_scale[0] = x.s[0];
  p.a_scale[1] = x.s[1];
  p.shared_row0 = x.shared_row0;
  return p;
}

hipError_t launch_gemm1(int variant, const FfnGroups& g, const RowOperand& x, const int* tile_prefix,
                        long n_rows, uint16_t* h, hipStream_t s) {
  GemmParams p = base_params(g, x, tile_prefix);
  p.K = g.hidden;
  p.N = g.inter;
  for (int i = 0; i < 2; ++i) {
    p.wa[i] = g.w1[i];
    p.wb[i] = g.w3[i];
    p.sa[i] = g.s1[i];
    p.sb[i] = g.s3[i];
  }
  p.h = h;
  const int bm = variant_rows(variant);
  if (variant == kVariantSmall) {
    p.ntiles = g.inter / (kSmCh / 2);
    const long grid = max_row_tiles(n_rows, g.n_groups, bm) * p.ntiles;
    if (g.fmt == kMxfp4) gemm1_small_kernel<kMxfp4><<<(unsigned)grid, 256, 0, s>>>(p);
    else gemm1_small_kernel<kFp8><<<(unsigned)grid, 256, 0, s>>>(p);
  } else {
    p.ntiles = g.inter / (kLgCh / 2);
    const long grid = max_row_tiles(n_rows, g.n_groups, bm) * p.ntiles;
    if (variant == kVariantLarge256) gemm1_large_kernel<256, kLgWN, 4><<<(unsigned)grid, 128 * kLgWN, 0, s>>>(p);
    else gemm1_large_kernel<128, kLgWN, 4><<<(unsigned)grid, 128 * kLgWN, 0, s>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_gemm2(int variant, const FfnGroups& g, const RowOperand& h, const int* tile_prefix,
                        long n_rows, float* y, hipStream_t s) {
  GemmParams p = base_params(g, h, tile_prefix);
  p.K = g.inter;
  p.N = g.hidden;
  for (int i = 0; i < 2; ++i) {
    p.wa[i] = g.w2[i];
    p.sa[i] = g.s2[i];
  }
  p.y = y;
  const int bm = variant_rows(variant);
  if (variant == kVariantSmall) {
    p.ntiles = g.hidden / kSmCh;
    const long grid = max_row_tiles(n_rows, g.n_groups, bm) * p.ntiles;
    if (g.fmt == kMxfp4) gemm2_small_kernel<kMxfp4><<<(unsigned)grid, 256, 0, s>>>(p);
    else gemm2_small_kernel<kFp8><<<(unsigned)grid, 256, 0, s>>>(p);
  } else {
    p.ntiles = g.hidden / kLgCh;
    const long grid = max_row_tiles(n_rows, g.n_groups, bm) * p.ntiles;
    if (variant == kVariantLarge256) gemm2_large_kernel<256, kLgWN, 3><<<(unsigned)grid, 128 * kLgWN, 0, s>>>(p);
    else gemm2_large_kernel<128, kLgWN, 4><<<(unsigned)grid, 128 * kLgWN, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace moe
