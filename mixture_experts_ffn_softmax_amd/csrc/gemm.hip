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
//          STAGES-1 steps ahead; waits and barriers are explicit.
//          Per-channel fp8 weights, and per-block fp8 in the down GEMM.
//   small: 32 rows x 64 channel rows, the 4 waves split the K steps and read
//          their fragments straight from memory into registers, then reduce
//          through LDS.  For decode-sized groups, where the weight stream is
//          the bound; fp8, per-block fp8 and MXFP4 weights (64-row tiles:
//          the medium variant, for per-block fp8 batches with many rows).
#include <math.h>

#include <type_traits>

#include <hip/hip_ext.h>

#include "device_common.h"
#include "internal.h"
#include "mfma_common.h"


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
  // group's rows from a[1] (row index r - shared_row0).  GEMM1: e4m3 codes
  // with per-row scales a_scale; GEMM2: bf16 h (no scale).
  const void* a[2];
  const float* a_scale[2];
  long shared_row0;
  const int* gather;     // GEMM1, optional: routed row r reads a[0] row gather[r] / gather_k
  int gather_k;
  Operand ta[2];         // byte addressing of a[0] / a[1]
  const uint8_t* wa[2];  // GEMM1: W1 (gate), GEMM2: W2 -- [0] routed, [1] shared
  const uint8_t* wb[2];  // GEMM1: W3 (up)
  const void* sa[2];
  const void* sb[2];
  Operand wd[2];         // byte addressing of one expert's weight matrix (codes)
  Operand sd[2];         // byte addressing of one expert's e8m0 scales (MXFP4)
  int act[2];            // GEMM1: gate Activation of the routed / shared group
  float beta[2];         // GEMM1: SiTU's beta per group
  uint16_t* h;           // GEMM1 output: bf16, K-blocked (kHChunk-byte chunks)
  long h_cs;             // its chunk stride in bytes (rows * kHChunk)
  float* y;              // GEMM2 output [rows][N] fp32
};

// Byte offset of contraction byte k of row r (see Operand).
__device__ __forceinline__ long op_off(const Operand& d, long r, long k) {
  return r * d.row_pitch + (k >> d.kc_shift) * d.chunk_stride + (k & ((1L << d.kc_shift) - 1));
}
// Byte advance of every row's pointer per contraction step of `step` bytes:
// K-blocked operands have chunks of exactly one step.
__device__ __forceinline__ long op_step(const Operand& d, int step) {
  return (d.kc_shift < 31) ? d.chunk_stride : step;
}
// Element offset (bf16 units) of channel ch of row r in the K-blocked h.
__device__ __forceinline__ long h_off(long h_cs, long r, int ch) {
  return (ch >> 5) * (h_cs >> 1) + r * (kHChunk >> 1) + (ch & 31);
}

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


// 16 e4m3 codes (4 words) -> 2 x 8 bf16, exact.
__device__ __forceinline__ void fp8x16_to_bf16(const uint32_t (&w)[4], v8bf (&out)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * i], 1.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * i], 1.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * i + 1], 1.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * i + 1], 1.0f, true);
    out[i] = v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
}

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





// ---- tile lookup -----------------------------------------------------------


struct TileInfo {
  int g;      // group
  int wi;     // 0 routed, 1 shared
  long eg;    // expert index within the weight array
  int row0;   // first row of the tile
  int row1;   // one past the last row of the group
  int nt;     // channel tile
};

// Locates tile L: group g is the largest with tile_prefix[g] * ntiles <= L.
__device__ __forceinline__ TileInfo find_tile(const GemmParams& p, const int* s_tp, const int* s_off, long L, int bm) {
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
  ti.row1 = s_off[lo + 1];
  ti.row0 = s_off[lo] + mt * bm;
  ti.wi = (lo < p.n_routed) ? 0 : 1;
  ti.eg = ti.wi ? 0 : lo;
  // the tile is the workgroup's: keep its fields in scalar registers
  ti.g = __builtin_amdgcn_readfirstlane(ti.g);
  ti.nt = __builtin_amdgcn_readfirstlane(ti.nt);
  ti.row0 = __builtin_amdgcn_readfirstlane(ti.row0);
  ti.row1 = __builtin_amdgcn_readfirstlane(ti.row1);
  ti.wi = __builtin_amdgcn_readfirstlane(ti.wi);
  ti.eg = __builtin_amdgcn_readfirstlane((int)ti.eg);
  return ti;
}

// Row of a[ti.wi] (and a_scale[ti.wi]) that tile row r reads: the shared
// group's rows start at shared_row0; routed rows are stored in row order
// (G = kRowsStored), gathered from the token-order rows through row_to_pair / k
// (G = kRowsGathered, p.gather set), or either, as p.gather says (kRowsAny).
enum RowSource { kRowsStored = 0, kRowsGathered = 1, kRowsAny = 2 };
template <int G = kRowsAny>
__device__ __forceinline__ long a_row(const GemmParams& p, const TileInfo& ti, int r) {
  if (ti.wi) return r - p.shared_row0;
  if constexpr (G == kRowsStored) return r;
  else if constexpr (G == kRowsGathered) return p.gather[r] / p.gather_k;
  else return p.gather ? p.gather[r] / p.gather_k : r;
}
// Start of row r of the row operand (contraction byte 0).
template <int G = kRowsAny>
__device__ __forceinline__ const uint8_t* row_ptr(const GemmParams& p, const TileInfo& ti, int r) {
  return reinterpret_cast<const uint8_t*>(p.a[ti.wi]) + a_row<G>(p, ti, r) * p.ta[ti.wi].row_pitch;
}

// Common prologue: loads the tile prefix and the group offsets into s_tp
// (kTileLds ints: the prefix, then the offsets at kOffLds) in one round
// trip, exits surplus workgroups, finds the tile.
constexpr int kOffLds = kMaxExperts + 2;
constexpr int kTileLds = 2 * kOffLds;
#define MOE_TILE_PROLOGUE(BMROWS)                                                 \
  for (int i_ = threadIdx.x; i_ <= p.n_groups; i_ += blockDim.x) {               \
    s_tp[i_] = p.tile_prefix[i_];                                                \
    s_tp[kOffLds + i_] = p.offsets[i_];                                          \
  }                                                                              \
  __syncthreads();                                                               \
  const long total_ = (long)s_tp[p.n_groups] * p.ntiles;                         \
  if ((long)blockIdx.x >= total_) return;                                        \
  const TileInfo ti = find_tile(p, s_tp, s_tp + kOffLds, xcd_remap(blockIdx.x, total_), BMROWS)

constexpr int kLgCh = 256;    // channel rows per tile

// The SiTU epilogue takes tanh(z) = 1 - 2 / (1 + e^(2z)), which saturates
// cleanly at +-1 when the exponential overflows or underflows.


// ============================================================================
// large variants: 4 waves, one per SIMD, pipelined through an LDS ring
// ============================================================================
//
// Each wave owns a 128 x 128 output tile (256 accumulator registers, possible
// with one wave per SIMD), so fragment reads per K step stay at 1/64 byte per
// flop.  With one wave per SIMD nothing hides LDS latency, so the fragments of
// step k+1 are read into a second register set while the MFMAs of step k run.
// The LDS ring holds the stage being read into registers plus STAGES-1 stages
// in flight: the DMA issued during step k fills step k+STAGES into the slot
// that step k-1's reads released.
//
// Token fragments are interleaved between the two wave rows: fragment t of
// wave row wm covers tile rows [(2t + wm) * 32, +32).  A row tile that ends
// inside a group (the last tile of a ragged group) has a valid prefix of
// rows; fragments wholly past it are skipped (the main loop is instantiated
// for each count TV of valid fragments), and the interleave keeps the two wave
// rows' shares of the remaining work equal.

// 32-byte LDS rows (2 slots): conflict-free for 8 or 16 lanes per cycle when
// 32 lanes read one slot of 32 consecutive rows.
__device__ __forceinline__ int swz32(int r, int c) { return c ^ ((r >> 2) & 1) ^ ((r >> 3) & 1); }

// Wait for this wave's loads of the stage to be read next (at most N of its
// DMAs outstanding), then barrier: that stage is complete for every wave and
// every wave's reads of the slot about to be refilled are done.
template <int N, int STAGES, int PER>
__device__ __forceinline__ void pp_wait(int ks, int nk) {
  if (ks + STAGES - 1 < nk) wait_barrier<N>();
  else wait_barrier<0>();
}

// Ring depth for a short tile's body: as many stages of `stage` bytes as the
// kernel's ring of `ring` bytes holds, at most 8, and such that the direct-to-
// LDS loads in flight stay within the vmcnt range (`per` per wave per stage).
constexpr int short_stages(int ring, int stage, int per) {
  int n = ring / stage;
  if (n > 8) n = 8;
  while ((n - 1) * per >= 64) --n;
  return n;
}

// Valid token fragments of wave row wm in a tile with `vr` valid rows.
template <int TF>
__device__ __forceinline__ int valid_frags(int vr, int wm) {
  const int v = (vr - wm * 32 + 63) >> 6;
  return v < 0 ? 0 : (v > TF ? TF : v);
}

// GEMM1 large epilogue.  Lane holds token l32 of each token fragment and, per
// group q of 4 accumulator entries, channels 8q + 4hh .. +3 of the fragment.
// The gate and up sums are scaled by the token and channel scales and
// h = bf16(act(g) * u) goes straight to the K-blocked h: a 32-channel
// fragment is one 64-byte chunk row, so the four q stores of a fragment fill
// 32 consecutive chunk rows (2 KB).
// BLK: per-block fp8 weights; the accumulators hold the sums in units of
// the last K block's scale mantissas mg / mu (see gemm1_pp_body), which
// replace the per-channel scales.
template <int TV, int TA, bool BLK = false, typename Act>
__device__ __forceinline__ void gemm1_pp_epilogue(const GemmParams& p, const TileInfo& ti, int n0, int wm, int wn,
                                                  int l32, int hh, const v16f (&acc)[4][TA], Act act,
                                                  float mg = 1.0f, float mu = 1.0f) {
  const float* S1 = reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N;
  const float* S3 = reinterpret_cast<const float*>(p.sb[ti.wi]) + ti.eg * p.N;
  float xs[TV];
#pragma unroll
  for (int t = 0; t < TV; ++t) {
    int grow = ti.row0 + (2 * t + wm) * 32 + l32;
    if (grow >= ti.row1) grow = ti.row1 - 1;
    xs[t] = p.a_scale[ti.wi][a_row(p, ti, grow)];
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ch0 = n0 + wn * 64 + c * 32;
    float4 s1v[4], s3v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s1v[q] = BLK ? make_float4(mg, mg, mg, mg) : *reinterpret_cast<const float4*>(S1 + ch0 + 8 * q + 4 * hh);
      s3v[q] = BLK ? make_float4(mu, mu, mu, mu) : *reinterpret_cast<const float4*>(S3 + ch0 + 8 * q + 4 * hh);
    }
#pragma unroll
    for (int t = 0; t < TV; ++t) {
      const int grow = ti.row0 + (2 * t + wm) * 32 + l32;
      if (grow >= ti.row1) continue;
      uint16_t* hrow = p.h + h_off(p.h_cs, grow, ch0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sg[4] = {s1v[q].x, s1v[q].y, s1v[q].z, s1v[q].w};
        const float su[4] = {s3v[q].x, s3v[q].y, s3v[q].z, s3v[q].w};
        uint32_t b[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float g = acc[c][t][4 * q + v] * xs[t] * sg[v];
          const float u = acc[2 + c][t][4 * q + v] * xs[t] * su[v];
          b[v] = bf16_rne(act(g) * u);
        }
        *reinterpret_cast<uint2*>(hrow + 8 * q + 4 * hh) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      }
    }
  }
}

// GEMM1: wave (wm, wn) owns the interleaved token fragments of wave row wm
// and channels [wn * 64, +64) of both the gate (fragments 0, 1) and the up
// rows (2, 3).  LDS stage: BM token rows then 256 channel rows (W1 rows
// n0.., then W3 rows n0..), 64 bytes of the K step each (swz64).  SITU:
// some group uses SiTU (a separate instantiation, so that the SiLU-only
// kernel carries no second epilogue and its register allocation is unchanged).
// BLK: per-block fp8 weights (the routed group of the per-block format).
// The workgroup's 128 gate (and 128 up) channels are one channel block, so a
// K block (two steps) has one gate and one up scale s = m * 2^e (m in [1, 2)).
// The exponent enters the MFMA as its e8m0 weight scale (exact); the
// mantissa cannot, so the accumulators are kept in units of the current
// block's mantissa: at each block start they are multiplied by
// m_previous / m_current, and the epilogue multiplies by the last block's m.
// (A zero or subnormal scale gives e8m0 0, i.e. 2^-127, with the mantissa of
// the block before: its products fall below binary32's range.)
template <int BM, int STAGES, int TV, bool SITU, bool BLK = false>
__device__ __forceinline__ void gemm1_pp_body(const GemmParams& p, const TileInfo& ti, uint8_t* smem) {
  constexpr int kRows = BM + kLgCh;
  constexpr int kStage = kRows * 64;
  constexpr int kDma = kRows / 16;
  constexpr int kPer = kDma / 4;
  static_assert(kDma % 4 == 0, "dma split");
  constexpr int NF = 4;
  constexpr int kGrp = (kPer + NF - 1) / NF;     // DMAs issued after each MFMA group
  constexpr int TA = TV > 0 ? TV : 1;
  static_assert((STAGES - 1) * kPer < 64, "vmcnt range");

  const int K = p.K;
  const int nk = K >> 6;
  const int n0 = ti.nt * (kLgCh / 2);
  const uint8_t* W1 = p.wa[ti.wi] + ti.eg * (long)p.N * K;
  const uint8_t* W3 = p.wb[ti.wi] + ti.eg * (long)p.N * K;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // per-block scales of the gate and up channel blocks (at most 128 K
  // blocks): lane l holds those of K blocks l and l + 64, loaded and waited
  // for before any direct-to-LDS load is issued
  const int nkb = K >> 7;
  float sg0 = 1.0f, sg1 = 1.0f, su0 = 1.0f, su1 = 1.0f;
  if constexpr (BLK) {
    const long base = (ti.eg * (long)(p.N >> 7) + (n0 >> 7)) * nkb;
    const float* S1b = reinterpret_cast<const float*>(p.sa[ti.wi]) + base;
    const float* S3b = reinterpret_cast<const float*>(p.sb[ti.wi]) + base;
    if (lane < nkb) {
      sg0 = S1b[lane];
      su0 = S3b[lane];
    }
    if (lane + 64 < nkb) {
      sg1 = S1b[lane + 64];
      su1 = S3b[lane + 64];
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  }
  auto lane_pick = [&](float v0, float v1, int kb) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kb < 64 ? v0 : v1), kb & 63));
  };
  // e8m0 exponent and mantissa of a block scale
  auto blk_exp = [](float sc) { return (int)((__float_as_uint(sc) >> 23) & 0xFFu); };
  auto blk_mant = [](float sc, float prev) {
    const uint32_t b = __float_as_uint(sc);
    const float m = ((b >> 23) & 0xFFu) ? __uint_as_float((b & 0x807FFFFFu) | 0x3F800000u) : sc * 0x1p127f;
    return m != 0.0f ? m : prev;
  };
  float mg = 1.0f, mu = 1.0f;   // mantissas of the current K block
  int eg8 = 127, eu8 = 127;     // e8m0 exponents of the current K block

  // this lane's source of each of the wave's dma16 per stage, advanced by one
  // K step after every issue (stages are issued in order)
  const uint8_t* src[kPer];
  long inc[kPer];
  const Operand& wd = p.wd[ti.wi];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int row = (wave * kPer + i) * 16 + (lane >> 2);
    const int chunk = swz64(row, lane & 3);
    if (row < BM) {
      int r = ti.row0 + row;
      if (r >= ti.row1) r = ti.row1 - 1;
      src[i] = row_ptr(p, ti, r) + chunk * 16;
      inc[i] = op_step(p.ta[ti.wi], 64);
    } else {
      const int c = row - BM;
      const uint8_t* W = (c < kLgCh / 2) ? W1 : W3;
      src[i] = W + (long)(n0 + (c & (kLgCh / 2 - 1))) * wd.row_pitch + chunk * 16;
      inc[i] = op_step(wd, 64);
    }
  }
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int ks, int i0, int i1) {
    const uint32_t st = lds0 + (ks % STAGES) * kStage;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      dma16(src[i], st + (wave * kPer + i) * 1024);
      src[i] += inc[i];
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;
  const int fo0 = l32 * 64 + (swz64(l32, 2 * hh) << 4);
  const int fo1 = l32 * 64 + (swz64(l32, 2 * hh + 1) << 4);
  auto xoff = [&](int t) { return (2 * t + wm) * 32 * 64; };
  auto woff = [&](int f) { return (BM + (f < 2 ? 0 : kLgCh / 2) + wn * 64 + (f & 1) * 32) * 64; };
  auto rd = [&](const uint8_t* at) {
    return as_v8i(*reinterpret_cast<const uint4*>(at + fo0), *reinterpret_cast<const uint4*>(at + fo1));
  };

  v16f acc[NF][TA];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < TA; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[f][t][j] = 0.0f;

#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nk) issue(s, 0, kPer);
  if (STAGES <= nk) wait_barrier<(STAGES - 1) * kPer>();
  else wait_barrier<0>();

  v8i xa[TA], wa[NF], xb[TA], wb[NF];
  if constexpr (TV > 0) {
#pragma unroll
    for (int t = 0; t < TV; ++t) xa[t] = rd(smem + xoff(t));
#pragma unroll
    for (int f = 0; f < NF; ++f) wa[f] = rd(smem + woff(f));
  }

  // one K step on register set (xc, wc), reading step ks+1 into (xn, wn_).
  // steady = true: step ks+1 exists and step ks+STAGES is to be loaded.
  // Per-block: an even step starts a K block (nk is even: K is a multiple
  // of 256 for these kernels).
  auto step = [&](auto steady, int ks, const v8i (&xc)[TA], const v8i (&wc)[NF], v8i (&xn)[TA],
                  v8i (&wn_)[NF]) {
    constexpr bool kSteady = decltype(steady)::value;
    float rg = 1.0f, ru = 1.0f;
    if constexpr (BLK) {
      if ((ks & 1) == 0) {
        const int kb = ks >> 1;
        const float sg = lane_pick(sg0, sg1, kb), su = lane_pick(su0, su1, kb);
        const float mg2 = blk_mant(sg, mg), mu2 = blk_mant(su, mu);
        rg = mg / mg2;
        ru = mu / mu2;
        mg = mg2;
        mu = mu2;
        eg8 = blk_exp(sg);
        eu8 = blk_exp(su);
      }
    }
    if (kSteady) wait_barrier<(STAGES - 2) * kPer>();
    else pp_wait<(STAGES - 2) * kPer, STAGES, kPer>(ks, nk);
    const bool next = kSteady || ks + 1 < nk;
    const bool more = kSteady || ks + STAGES < nk;
    const uint8_t* stn = smem + ((ks + 1) % STAGES) * kStage;
    static_for<NF>([&](auto fc) {
      constexpr int f = decltype(fc)::value;
      __builtin_amdgcn_sched_barrier(0);
      // the next step's fragment reads and this group's MFMAs in one
      // scheduling region, one read after each MFMA
      if constexpr (TV > 0) {
        if (next) {
          wn_[f] = rd(stn + woff(f));
          if (f < TV) xn[f] = rd(stn + xoff(f));
        }
      }
      if constexpr (BLK) {
        // at a block start (r != 1 only there) the sums so far move to the
        // new block's mantissa; the block's exponent scales the weights
        const float r = f < 2 ? rg : ru;
        const int e8 = f < 2 ? eg8 : eu8;
#pragma unroll
        for (int t = 0; t < TV; ++t) {
          if ((ks & 1) == 0) acc[f][t] = acc[f][t] * r;
          acc[f][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wc[f], xc[t], acc[f][t], 0, 0, 0, e8, 0,
                                                                      kE8m0One);
        }
      } else {
#pragma unroll
        for (int t = 0; t < TV; ++t) acc[f][t] = mfma32_fp8(wc[f], xc[t], acc[f][t]);
      }
      if constexpr (TV > 0) {
        constexpr int kReads = 2 + (f < TV ? 2 : 0);
        static_for<(TV > kReads ? TV : kReads)>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (i < TV) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if constexpr (i < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
        constexpr int i0 = f * kGrp, i1 = (f + 1) * kGrp < kPer ? (f + 1) * kGrp : kPer;
        if constexpr (i0 < i1) issue(ks + STAGES, i0, i1);
      }
    });
  };
  const std::true_type steady;
  const std::false_type tail;
  int ks = 0;
  for (; ks + 1 + STAGES < nk; ks += 2) {
    step(steady, ks, xa, wa, xb, wb);
    step(steady, ks + 1, xb, wb, xa, wa);
  }
  for (; ks + 1 < nk; ks += 2) {
    step(tail, ks, xa, wa, xb, wb);
    step(tail, ks + 1, xb, wb, xa, wa);
  }
  if (ks < nk) step(tail, ks, xa, wa, xb, wb);

  // ---- epilogue
  if constexpr (TV > 0) {
    if constexpr (SITU) {
      // one epilogue for both activations (a second copy spills): SiLU is
      // the product with the linear factor g instead of beta tanh(g / beta)
      const bool use_situ = p.act[ti.wi] == kActSitu;
      const float beta = p.beta[ti.wi], rbeta = 1.0f / beta;
      gemm1_pp_epilogue<TV, TA, BLK>(p, ti, n0, wm, wn, l32, hh, acc, [=](float g) {
        const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
        const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(2.8853900817779268f * g * rbeta));
        return (use_situ ? beta * th : g) * sig;
      }, mg, mu);
    } else {
      gemm1_pp_epilogue<TV, TA, BLK>(p, ti, n0, wm, wn, l32, hh, acc, [](float g) { return silu_fast(g); }, mg, mu);
    }
  }
}

// BLKK: the routed group has per-block fp8 weights (the shared group is
// always per-channel).  The tile dispatch is written out in the kernel (a
// macro), as in the down GEMM, so that the per-channel kernel's code is
// that of the plain dispatch.
#define MOE_G1_TILE(B)                                                                          \
  if (BM > 64 && vr <= 64) {                                                                    \
    if (valid_frags<1>(vr, wm) == 0) gemm1_pp_body<64, S64, 0, SITU, B>(p, ti, smem);           \
    else gemm1_pp_body<64, S64, 1, SITU, B>(p, ti, smem);                                       \
    return;                                                                                     \
  }                                                                                             \
  if (BM > 128 && vr <= 128) {                                                                  \
    switch (valid_frags<2>(vr, wm)) {                                                           \
      case 0: gemm1_pp_body<128, S128, 0, SITU, B>(p, ti, smem); break;                         \
      case 1: gemm1_pp_body<128, S128, 1, SITU, B>(p, ti, smem); break;                         \
      default: gemm1_pp_body<128, S128, 2, SITU, B>(p, ti, smem); break;                        \
    }                                                                                           \
    return;                                                                                     \
  }                                                                                             \
  switch (valid_frags<TF>(vr, wm)) {                                                            \
    case 0: gemm1_pp_body<BM, STAGES, 0, SITU, B>(p, ti, smem); break;                          \
    case 1: gemm1_pp_body<BM, STAGES, 1, SITU, B>(p, ti, smem); break;                          \
    case 2: gemm1_pp_body<BM, STAGES, 2, SITU, B>(p, ti, smem); break;                          \
    case 3: if constexpr (TF >= 3) gemm1_pp_body<BM, STAGES, 3, SITU, B>(p, ti, smem); break;   \
    default: if constexpr (TF >= 4) gemm1_pp_body<BM, STAGES, 4, SITU, B>(p, ti, smem); break;  \
  }                                                                                             \
  return

template <int BM, int STAGES, bool SITU, bool BLKK = false>
__global__ __launch_bounds__(256, 1) void gemm1_pp_kernel(GemmParams p) {
  constexpr int kStage = (BM + kLgCh) * 64;
  constexpr int TF = BM / 64;
  // the tile-prefix table and offsets live in the ring until the first DMA is issued
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * kStage];
  static_assert(STAGES * kStage >= kTileLds * 4, "tile prefix and offsets fit in the ring");
  int* s_tp = reinterpret_cast<int*>(smem);
  MOE_TILE_PROLOGUE(BM);
  __syncthreads();   // every thread has its tile: the ring is free
  const int vr = min(BM, ti.row1 - ti.row0);
  const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 7);
  // a short tile (the last of a ragged group) stages only the rows it has:
  // 64 or 128 token rows per stage instead of BM, so that fewer direct-to-LDS
  // loads are in flight (their throughput falls as more are outstanding)
  // and, its stages being smaller, as deep a ring as the LDS holds (its
  // loop is bound by the weight stream's latency, not by the MFMAs)
  constexpr int S64 = short_stages(STAGES * kStage, (64 + kLgCh) * 64, 5);
  constexpr int S128 = short_stages(STAGES * kStage, (128 + kLgCh) * 64, 6);
  if constexpr (BLKK) {
    if (ti.wi == 0) {
      MOE_G1_TILE(true);
    }
  }
  MOE_G1_TILE(false);
}
#undef MOE_G1_TILE

// 32 e4m3 codes (4 words, 16 per half-lane K slice) -> the two bf16 halves
// of a 32x32x16 fragment pair, exact.
struct BfPair { v8bf a, b; };
__device__ __forceinline__ BfPair fp8x16_to_bf16(const uint4& w) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
  const v2bf e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.z, 1.0f, false);
  const v2bf g = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.z, 1.0f, true);
  const v2bf h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.w, 1.0f, false);
  const v2bf k = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.w, 1.0f, true);
  return BfPair{v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]},
                v8bf{e[0], e[1], g[0], g[1], h[0], h[1], k[0], k[1]}};
}

// The same 16 codes times a per-block scale s, each product rounded once to
// bf16 (the code widened exactly to binary32, multiplied in binary32, then
// rounded to nearest even).
__device__ __forceinline__ BfPair fp8x16_to_bf16_scaled(const uint4& w, float s) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  __bf16 o[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[i], false);
    const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[i], true);
    o[4 * i] = (__bf16)(lo[0] * s);
    o[4 * i + 1] = (__bf16)(lo[1] * s);
    o[4 * i + 2] = (__bf16)(hi[0] * s);
    o[4 * i + 3] = (__bf16)(hi[1] * s);
  }
  return BfPair{v8bf{o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]},
                v8bf{o[8], o[9], o[10], o[11], o[12], o[13], o[14], o[15]}};
}

// GEMM2: K step of 32 elements.  LDS stage: BM h rows of 32 bf16 (64 bytes,
// swz64) then 256 W2 rows of 32 codes (32 bytes, swz32).  Wave (wm, wn) owns
// the interleaved token fragments of wave row wm and output channels
// [wn * 128, +128).  W2 fragments are widened to bf16 one step ahead: the
// conversions of step k+1 run between the MFMAs of step k, which do not
// depend on them, so the vector unit works while the matrix core does.
// BLK: per-block fp8 W2 (the routed group of the per-block format).  A
// wave's 128 channels are one channel block, so the scale of a K block (four
// steps) is one number per wave; it is applied to the codes as they are
// widened (each product rounded once to bf16, a relative error of at most
// 2^-9 per weight, the size of h's own rounding) rather than to partial sums,
// for which a 128 x 128 wave tile has no registers left.
template <int BM, int STAGES, int TV, bool BLK>
__device__ __forceinline__ void gemm2_pp_body(const GemmParams& p, const TileInfo& ti, uint8_t* smem) {
  constexpr int kTokBytes = BM * 64;
  constexpr int kStage = kTokBytes + kLgCh * 32;
  constexpr int kDmaT = BM / 16;            // 16 h rows per dma16
  constexpr int kDmaW = kLgCh / 32;         // 32 W2 rows per dma16
  constexpr int kPer = (kDmaT + kDmaW) / 4;
  static_assert((kDmaT + kDmaW) % 4 == 0, "dma split");
  static_assert((STAGES - 1) * kPer < 64, "vmcnt range");
  constexpr int NF = 4;
  constexpr int kGrp = (kPer + NF - 1) / NF;
  constexpr int TA = TV > 0 ? TV : 1;

  const int K = p.K;                        // = I
  const int nk = K >> 5;
  const int n0 = ti.nt * kLgCh;
  const uint8_t* W2 = p.wa[ti.wi] + ti.eg * (long)p.N * K;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // per-block scales of this wave's channel block, one per K block (at most
  // 128): lane l holds those of K blocks l and l + 64, loaded before any
  // direct-to-LDS load is issued and waited for at once, so that no later
  // wait for them drains the ring's loads; a step takes its scale with a
  // lane read
  const int nkb = K >> 7;
  float sv0 = 1.0f, sv1 = 1.0f;
  if constexpr (BLK) {
    const float* sbw =
        reinterpret_cast<const float*>(p.sa[ti.wi]) + (ti.eg * (long)(p.N >> 7) + (n0 >> 7) + (wave & 1)) * nkb;
    if (lane < nkb) sv0 = sbw[lane];
    if (lane + 64 < nkb) sv1 = sbw[lane + 64];
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  }
  auto scale_of = [&](int kb) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kb < 64 ? sv0 : sv1), kb & 63));
  };
  auto widen = [&](const uint4& raw, float sc) { return BLK ? fp8x16_to_bf16_scaled(raw, sc) : fp8x16_to_bf16(raw); };

  const uint8_t* src[kPer];
  const Operand& wd = p.wd[ti.wi];
  const long inc_t = op_step(p.ta[ti.wi], 64);
  const long inc_w = op_step(wd, 32);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = wave * kPer + i;
    if (q < kDmaT) {
      const int row = q * 16 + (lane >> 2);
      int r = ti.row0 + row;
      if (r >= ti.row1) r = ti.row1 - 1;
      src[i] = row_ptr<kRowsStored>(p, ti, r) + swz64(row, lane & 3) * 16;
    } else {
      const int row = (q - kDmaT) * 32 + (lane >> 1);
      src[i] = W2 + (long)(n0 + row) * wd.row_pitch + swz32(row, lane & 1) * 16;
    }
  }
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int ks, int i0, int i1) {
    const uint32_t st = lds0 + (ks % STAGES) * kStage;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int q = wave * kPer + i;
      const bool tok = q < kDmaT;
      dma16(src[i], st + (tok ? q * 1024 : kTokBytes + (q - kDmaT) * 1024));
      src[i] += tok ? inc_t : inc_w;
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;
  // h fragment: row l32, bf16 elements [16h, 16h + 16) = 64-byte-row slots 2h, 2h+1
  const int ho0 = l32 * 64 + (swz64(l32, 2 * hh) << 4);
  const int ho1 = l32 * 64 + (swz64(l32, 2 * hh + 1) << 4);
  // W2 fragment: row l32, codes [16h, 16h + 16) = 32-byte-row slot h
  const int wo = kTokBytes + wn * 128 * 32 + l32 * 32 + (swz32(l32, hh) << 4);
  auto xoff = [&](int t) { return (2 * t + wm) * 32 * 64; };

  auto rdx = [&](const uint8_t* at) {
    return BfPair{as_v8bf(*reinterpret_cast<const uint4*>(at + ho0)), as_v8bf(*reinterpret_cast<const uint4*>(at + ho1))};
  };
  auto rdw = [&](const uint8_t* st, int f) { return *reinterpret_cast<const uint4*>(st + wo + f * 32 * 32); };

  v16f acc[NF][TA];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < TA; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[f][t][j] = 0.0f;

#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nk) issue(s, 0, kPer);
  if (STAGES <= nk) wait_barrier<(STAGES - 1) * kPer>();
  else wait_barrier<0>();

  BfPair xa[TA], xb[TA], wa[NF], wb[NF];
  if constexpr (TV > 0) {
    const float sc0 = BLK ? scale_of(0) : 1.0f;
#pragma unroll
    for (int t = 0; t < TV; ++t) xa[t] = rdx(smem + xoff(t));
#pragma unroll
    for (int f = 0; f < NF; ++f) wa[f] = widen(rdw(smem, f), sc0);
  }

  auto step = [&](auto steady, int ks, const BfPair (&xc)[TA], const BfPair (&wc)[NF], BfPair (&xn)[TA],
                  BfPair (&wn_)[NF]) {
    constexpr bool kSteady = decltype(steady)::value;
    if (kSteady) wait_barrier<(STAGES - 2) * kPer>();
    else pp_wait<(STAGES - 2) * kPer, STAGES, kPer>(ks, nk);
    const bool next = kSteady || ks + 1 < nk;
    const bool more = kSteady || ks + STAGES < nk;
    const uint8_t* stn = smem + ((ks + 1) % STAGES) * kStage;
    // the scale of step ks+1's K block (the last step reads a valid entry it does not use)
    float scn = 1.0f;
    if constexpr (BLK && TV > 0) scn = scale_of(min((ks + 1) >> 2, nkb - 1));
    uint4 raw[NF];
    static_for<NF>([&](auto fc) {
      constexpr int f = decltype(fc)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (TV > 0) {
        if (next) {
          if (f == 0) {
#pragma unroll
            for (int g = 0; g < NF; ++g) raw[g] = rdw(stn, g);
          }
          if (f < TV) xn[f] = rdx(stn + xoff(f));
        }
      }
      // MFMAs of this group, the conversions of the next step's W2 fragments
      // (f - 1 and, in the last group, f) and the fragment reads in one
      // scheduling region, one read and a few conversions after each MFMA
      // the two K halves of each accumulator TV instructions apart
#pragma unroll
      for (int t = 0; t < TV; ++t)
        acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wc[f].a, xc[t].a, acc[f][t], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < TV; ++t)
        acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wc[f].b, xc[t].b, acc[f][t], 0, 0, 0);
      if constexpr (TV > 0) {
        if (next && f > 0) {
          wn_[f - 1] = widen(raw[f - 1], scn);
          if (f == NF - 1) wn_[f] = widen(raw[f], scn);
        }
      }
      if constexpr (TV > 0) {
        // per group: 2*TV MFMAs; DS reads: the 4 raw W2 fragments (group 0)
        // and one token fragment (2 reads); 8 conversions per W2 fragment
        constexpr int kReads = (f == 0 ? NF : 0) + (f < TV ? 2 : 0);
        constexpr int kCvtF = BLK ? 32 : 8;    // vector instructions per widened fragment
        constexpr int kCvt = (f == 0) ? 0 : (f == NF - 1 ? 2 * kCvtF : kCvtF);
        constexpr int kCvtPer = (kCvt + 2 * TV - 1) / (2 * TV);
        static_for<2 * TV>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if constexpr (i < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if constexpr (kCvtPer > 0) __builtin_amdgcn_sched_group_barrier(0x002, kCvtPer, 0);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
        constexpr int i0 = f * kGrp, i1 = (f + 1) * kGrp < kPer ? (f + 1) * kGrp : kPer;
        if constexpr (i0 < i1) issue(ks + STAGES, i0, i1);
      }
    });
  };
  const std::true_type steady;
  const std::false_type tail;
  int ks = 0;
  for (; ks + 1 + STAGES < nk; ks += 2) {
    step(steady, ks, xa, wa, xb, wb);
    step(steady, ks + 1, xb, wb, xa, wa);
  }
  for (; ks + 1 < nk; ks += 2) {
    step(tail, ks, xa, wa, xb, wb);
    step(tail, ks + 1, xb, wb, xa, wa);
  }
  if (ks < nk) step(tail, ks, xa, wa, xb, wb);

  // ---- epilogue: y = acc * s2 in fp32 (per-block: the scales are in acc
  // already).  Lane holds token l32 of each token fragment and channels
  // 8q + 4hh .. +3 of each channel fragment.
  if constexpr (TV > 0) {
    const float* S2 = reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N + n0 + wn * 128;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      float4 s2v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        s2v[q] = BLK ? make_float4(1.f, 1.f, 1.f, 1.f) : *reinterpret_cast<const float4*>(S2 + f * 32 + 8 * q + 4 * hh);
#pragma unroll
      for (int t = 0; t < TV; ++t) {
        const int grow = ti.row0 + (2 * t + wm) * 32 + l32;
        if (grow >= ti.row1) continue;
        float* yrow = p.y + (long)grow * p.N + n0 + wn * 128 + f * 32 + 4 * hh;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(yrow + 8 * q) =
              make_float4(acc[f][t][4 * q] * s2v[q].x, acc[f][t][4 * q + 1] * s2v[q].y,
                          acc[f][t][4 * q + 2] * s2v[q].z, acc[f][t][4 * q + 3] * s2v[q].w);
      }
    }
  }
}

// BLKK: the routed group has per-block fp8 weights (the shared group is
// always per-channel).  A tile takes the body for its valid rows; a short
// tile stages only the rows it has (as in the gate-up GEMM).  The dispatch is
// written out in the kernel (a macro, not a helper function, which changed
// the register allocation of the per-channel kernel's tile set-up).
#define MOE_G2_TILE(B)                                                                  \
  if (BM > 64 && vr <= 64) {                                                            \
    if (valid_frags<1>(vr, wm) == 0) gemm2_pp_body<64, S64, 0, B>(p, ti, smem);         \
    else gemm2_pp_body<64, S64, 1, B>(p, ti, smem);                                     \
    return;                                                                             \
  }                                                                                     \
  if (BM > 128 && vr <= 128) {                                                          \
    switch (valid_frags<2>(vr, wm)) {                                                   \
      case 0: gemm2_pp_body<128, S128, 0, B>(p, ti, smem); break;                       \
      case 1: gemm2_pp_body<128, S128, 1, B>(p, ti, smem); break;                       \
      default: gemm2_pp_body<128, S128, 2, B>(p, ti, smem); break;                      \
    }                                                                                   \
    return;                                                                             \
  }                                                                                     \
  switch (valid_frags<TF>(vr, wm)) {                                                    \
    case 0: gemm2_pp_body<BM, STAGES, 0, B>(p, ti, smem); break;                        \
    case 1: gemm2_pp_body<BM, STAGES, 1, B>(p, ti, smem); break;                        \
    case 2: gemm2_pp_body<BM, STAGES, 2, B>(p, ti, smem); break;                        \
    case 3: if constexpr (TF >= 3) gemm2_pp_body<BM, STAGES, 3, B>(p, ti, smem); break; \
    default: if constexpr (TF >= 4) gemm2_pp_body<BM, STAGES, 4, B>(p, ti, smem); break; \
  }                                                                                     \
  return

template <int BM, int STAGES, bool BLKK>
__global__ __launch_bounds__(256, 1) void gemm2_pp_kernel(GemmParams p) {
  constexpr int kStage = BM * 64 + kLgCh * 32;
  constexpr int TF = BM / 64;
  // the tile-prefix table and offsets live in the ring until the first DMA is issued
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * kStage];
  static_assert(STAGES * kStage >= kTileLds * 4, "tile prefix and offsets fit in the ring");
  int* s_tp = reinterpret_cast<int*>(smem);
  MOE_TILE_PROLOGUE(BM);
  __syncthreads();   // every thread has its tile: the ring is free
  const int vr = min(BM, ti.row1 - ti.row0);
  const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 7);
  constexpr int S64 = short_stages(STAGES * kStage, 64 * 64 + kLgCh * 32, 3);
  constexpr int S128 = short_stages(STAGES * kStage, 128 * 64 + kLgCh * 32, 4);
  if constexpr (BLKK) {
    if (ti.wi == 0) {
      MOE_G2_TILE(true);
    }
  }
  MOE_G2_TILE(false);
}
#undef MOE_G2_TILE
// ============================================================================
// small variants (decode-sized groups; fp8 or MXFP4 weights)
// ============================================================================
//
// The weight stream is the bound: every weight byte of a touched expert is
// read once per row tile, and a decode-sized group fits in one row tile.  The
// 4 waves of a workgroup take the K steps round-robin and reduce through LDS
// at the end.  GEMM1 keeps the loads of a wave's next K step in flight (a
// second register set) while the MFMAs of the current one run; GEMM2 (short
// K) spends the registers on a wider channel tile instead.  A tile with at
// most 16 valid rows skips its second token fragment (loads and MFMAs).

constexpr int kSmRows = 32;   // token rows per tile: 2 fragments of 16
constexpr int kMdRows = 64;   // the medium variant's: 4 fragments of 16
constexpr int kSmCh = 64;     // GEMM1 channel rows per tile: 4 fragments (2 gate + 2 up)
constexpr int kSmCh2 = 128;   // GEMM2 output channels per tile: 8 fragments
constexpr int kMdCh2 = 64;    // the medium variant's: 4 fragments
// per-block fp8 groups averaging at least this many rows take the medium
// variant: 64-row tiles halve the weight fragments loaded per flop (on the
// 2048-token prefill share the gate-up GEMM runs 508 us instead of 575; the
// down GEMM is unchanged)
constexpr long kMdMinAvgRows = 48;

// Steps ks = wave, wave + 4, ... < nk of this wave through D register sets:
// load(ks, set) fills a set, compute(set) consumes it; the loads of the next
// D - 1 steps are in flight while a step computes.
// K steps wave, wave + 4, ... of a small-variant tile, D in flight.  The
// first D steps' weight loads are issued before `rows` runs (it locates the
// tile's rows, which may take a dependent load of the gather table) and
// before their row-operand loads, so the weight stream starts one round
// trip earlier.
template <int D, class St, class LoadW, class Rows, class LoadX, class Compute>
__device__ __forceinline__ void small_pipeline(int wave, int nk, LoadW&& load_w, Rows&& rows, LoadX&& load_x,
                                               Compute&& compute) {
  const int n = nk > wave ? (nk - wave + 3) >> 2 : 0;
  St st[D];
  static_for<D>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if (j < n) load_w(wave + 4 * j, st[j]);
  });
  rows();
  static_for<D>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if (j < n) load_x(wave + 4 * j, st[j]);
  });
  for (int i = 0; i < n; i += D) {
    static_for<D>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if (i + j < n) {
        compute(st[j]);
        if (i + j + D < n) {
          load_x(wave + 4 * (i + j + D), st[j]);
          load_w(wave + 4 * (i + j + D), st[j]);
        }
      }
    });
  }
}

// GEMM1: 16x16x128 MFMA on e4m3 x e4m3, or e2m1 x e4m3 with block scales.
// NT: weights loaded non-temporally (see load_w16).
// TVM: token fragments of the kernel's row tile (2 or 4); TV <= TVM of them
// hold rows of this tile.
template <int WF, int TV, int G, bool NT, int TVM>
__device__ __forceinline__ void gemm1_small_body(const GemmParams& p, const TileInfo& ti, v4f (*red)[4 * TVM][64]) {
  constexpr int kSmallDepth1 = 2;
  const int K = p.K;
  const int nk = K >> 7;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  constexpr bool fp4 = WF == kMxfp4;
  constexpr bool blk = WF == kFp8Block;       // per-tile scales inside the reduction
  const long rowBytes = fp4 ? (K >> 1) : K;
  const int n0 = ti.nt * (kSmCh / 2);
  const uint8_t* Wa = p.wa[ti.wi] + ti.eg * (long)p.N * rowBytes;
  const uint8_t* Wb = p.wb[ti.wi] + ti.eg * (long)p.N * rowBytes;
  // per-block fp8: the scales of this tile's channel block for K block ks
  // (one 128-wide step) are sb1[ks] (gate) and sb3[ks] (up)
  const float* sb1 = nullptr;
  const float* sb3 = nullptr;
  if constexpr (blk) {
    const long base = (ti.eg * (long)(p.N >> 7) + (n0 >> 7)) * (K >> 7);
    sb1 = reinterpret_cast<const float*>(p.sa[ti.wi]) + base;
    sb3 = reinterpret_cast<const float*>(p.sb[ti.wi]) + base;
  }

  // Token fragment bytes [0,16) and [16,32) of lane group lg.  Against e4m3
  // weights both operands take bytes [32*lg, 32*lg + 32) of the K step.
  // Against e2m1 weights the operands differ: an e2m1 lane group holds K
  // [32*lg, 32*lg + 32) contiguously (one 32-element scale block) while an
  // e4m3 lane group holds K [16*lg, 16*lg + 16) in its first 16 bytes and
  // K [64 + 16*lg, 64 + 16*lg + 16) in its last 16, so the token bytes are
  // fetched from those positions to pair each product with the right K.
  //
  // The contraction is a sum over K, so any assignment of K elements to lane
  // groups serves as long as both operands use the same one.  Against e4m3
  // weights lane group lg takes K [16*lg, +16) and [64 + 16*lg, +16) of the
  // step as well: one load instruction then reads 16 weight rows x 64
  // contiguous bytes, a whole K-blocked chunk row block, instead of half of
  // two.
  const int tok_off0 = lg * 16;
  const int tok_off1 = 64 + lg * 16;
  // 16-byte pieces never straddle a K chunk of either layout, so each piece
  // is addressed through its operand's layout
  const Operand& td = p.ta[ti.wi];
  const Operand& wd = p.wd[ti.wi];
  const uint8_t* tp[TV];
  auto rows = [&]() {
#pragma unroll
    for (int t = 0; t < TV; ++t) {
      int r = ti.row0 + t * 16 + l16;
      if (r >= ti.row1) r = ti.row1 - 1;
      tp[t] = row_ptr<G>(p, ti, r);
    }
  };
  const uint8_t* wp[4];
  const uint8_t* sp[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int m = f >> 1;                          // 0 gate, 1 up
    const long crow = n0 + (f & 1) * 16 + l16;
    const uint8_t* W = m ? Wb : Wa;
    const uint8_t* S = reinterpret_cast<const uint8_t*>(m ? p.sb[ti.wi] : p.sa[ti.wi]);
    // MXFP4: this lane's codes [16*lg, 16*lg + 16) and the 4 scales of a K
    // step, addressed through the (row-major or K-blocked) operands
    wp[f] = fp4 ? W + op_off(wd, crow, lg * 16) : W + crow * wd.row_pitch;
    sp[f] = fp4 ? S + ti.eg * (long)p.N * (K >> 5) + op_off(p.sd[ti.wi], crow, 0) : nullptr;
  }
  auto tok = [&](int t, long k) {
    return *reinterpret_cast<const uint4*>(tp[t] + ((k >> td.kc_shift) * td.chunk_stride + (k & ((1L << td.kc_shift) - 1))));
  };
  auto wgt = [&](int f, long k) {
    return load_w16<NT>(wp[f] + ((k >> wd.kc_shift) * wd.chunk_stride + (k & ((1L << wd.kc_shift) - 1))));
  };

  v4f acc[4][TV];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < TV; ++t) acc[f][t] = v4f{0.f, 0.f, 0.f, 0.f};

  struct St {
    v8i x[TV];
    v8i w[4];
    int sc[4];
    float bs[2];
  };
  auto load_x = [&](int ks, St& st) {
    const long kb = (long)ks << 7;
#pragma unroll
    for (int t = 0; t < TV; ++t) st.x[t] = as_v8i(tok(t, kb + tok_off0), tok(t, kb + tok_off1));
  };
  auto load_w = [&](int ks, St& st) {
    const long kb = (long)ks << 7;
    if constexpr (blk) {
      st.bs[0] = sb1[ks];
      st.bs[1] = sb3[ks];
    }
    if constexpr (fp4) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint4 b0 = load_w16<NT>(wp[f] + (long)ks * op_step(wd, 64));
        st.w[f] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
        st.sc[f] = (int)*reinterpret_cast<const uint32_t*>(sp[f] + (long)ks * op_step(p.sd[ti.wi], 4));
      }
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f) st.w[f] = as_v8i(wgt(f, kb + tok_off0), wgt(f, kb + tok_off1));
    }
  };
  auto compute = [&](const St& st) {
    if constexpr (fp4) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int sc = (st.sc[f] >> (8 * lg)) & 0xFF;
#pragma unroll
        for (int t = 0; t < TV; ++t) acc[f][t] = mfma16_fp4w(st.w[f], st.x[t], acc[f][t], sc);
      }
    } else if constexpr (blk) {
      // one K step is one K block: its partial sum times its scale
      const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < TV; ++t) acc[f][t] += st.bs[f >> 1] * mfma16_fp8(st.w[f], st.x[t], zero);
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < TV; ++t) acc[f][t] = mfma16_fp8(st.w[f], st.x[t], acc[f][t]);
    }
  };
  small_pipeline<kSmallDepth1, St>(wave, nk, load_w, rows, load_x, compute);

#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < TV; ++t) red[wave][f * TVM + t][lane] = acc[f][t];
  __syncthreads();

  // wave w: gate fragment f = w >> 1 (up fragment f + 2), token fragments
  // t = (w & 1) + 2j
  const int f = wave >> 1;
  const int ch = n0 + f * 16 + 4 * lg;
  float sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
  if (!fp4 && !blk && (wave & 1) < TV) {   // per-channel e4m3 weights carry one scale per channel
    const float4 s1 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N + ch);
    const float4 s3 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.sb[ti.wi]) + ti.eg * p.N + ch);
    sg[0] = s1.x; sg[1] = s1.y; sg[2] = s1.z; sg[3] = s1.w;
    su[0] = s3.x; su[1] = s3.y; su[2] = s3.z; su[3] = s3.w;
  }
  const bool use_situ = p.act[ti.wi] == kActSitu;
  const float beta = p.beta[ti.wi];
#pragma unroll
  for (int t = wave & 1; t < TV; t += 2) {
    v4f gsum = red[0][f * TVM + t][lane], usum = red[0][(f + 2) * TVM + t][lane];
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      gsum += red[q][f * TVM + t][lane];
      usum += red[q][(f + 2) * TVM + t][lane];
    }
    const int grow = ti.row0 + t * 16 + l16;
    if (grow >= ti.row1) continue;
    const float xs = p.a_scale[ti.wi][a_row<G>(p, ti, grow)];
    uint32_t b[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float g = gsum[v] * xs * sg[v];
      const float u = usum[v] * xs * su[v];
      b[v] = bf16_rne((use_situ ? situ(g, beta) : silu(g)) * u);
    }
    *reinterpret_cast<uint2*>(p.h + h_off(p.h_cs, grow, ch)) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
  }
}

// G: where the routed rows come from (RowSource: stored, or gathered)
// ROWS: rows per tile, 32 (small variant) or 64 (medium variant: twice the
// rows per weight byte, for batches where many row tiles re-read each
// expert's weights).
template <int FMT, int G, bool NT, int ROWS = kSmRows>
__global__ __launch_bounds__(256) void gemm1_small_kernel(GemmParams p) {
  constexpr int TVM = ROWS / 16;
  __shared__ v4f red[4][4 * TVM][64];           // per-wave partial sums
  __shared__ int s_tp[kTileLds];
  MOE_TILE_PROLOGUE(ROWS);
  const int vr = ti.row1 - ti.row0;
  // the routed group takes FMT; the shared group is always per-channel fp8
  auto run = [&](auto fc) {
    constexpr int F = decltype(fc)::value;
    if (TVM > 2 && vr > 48) gemm1_small_body<F, TVM, G, NT, TVM>(p, ti, red);
    else if (TVM > 2 && vr > 32) gemm1_small_body<F, (TVM > 2 ? 3 : 2), G, NT, TVM>(p, ti, red);
    else if (vr > 16) gemm1_small_body<F, 2, G, NT, TVM>(p, ti, red);
    else gemm1_small_body<F, 1, G, NT, TVM>(p, ti, red);
  };
  if (FMT != kFp8 && ti.wi == 0) run(std::integral_constant<int, FMT>{});
  else run(std::integral_constant<int, kFp8>{});
}

// GEMM2: 16x16x32 bf16 MFMA; W2 codes converted to bf16 in registers.  Lane
// group lg takes a quarter of each K step on both operands (the sum over K
// does not care which, as long as both agree); sub-step i of the step's
// instructions uses 8 of them.  MXFP4, 128-wide steps: elements [32*lg, +32)
// (16 bytes of a 64-byte chunk, so a load reads 16 rows x 64 contiguous
// bytes); sub-step i of 4: [32*lg + 8i, +8).  e4m3, 64-wide steps: elements
// [16*lg, +16) (lane groups 0-1 and 2-3 read 16 rows of one 32-byte chunk
// each, whole); sub-step i of 2: [16*lg + 8i, +8).
// A tile is kSmCh2 = 128 output channels (8 fragments): with K = I the
// shortest contraction of the layer, wider tiles keep the launch to about
// one workgroup per two SIMD pairs.
// CH: output channels of the kernel's tile (kSmCh2 or kMdCh2); TVM, TV as
// in the gate-up body.
template <int WF, int TV, bool NT, int TVM, int CH>
__device__ __forceinline__ void gemm2_small_body(const GemmParams& p, const TileInfo& ti, v4f (*red)[TVM * CH / 16][64]) {
  constexpr bool fp4 = WF == kMxfp4;
  constexpr bool blk = WF == kFp8Block;
  // K elements per step: e4m3 steps of 64 (16 code bytes per lane and
  // fragment) keep two steps in flight in the registers one 128-wide step
  // would take; MXFP4 steps of 128 (16 bytes of codes per lane), one in flight
  constexpr int KS = fp4 ? 128 : 64;
  constexpr int XS = KS / 32;                 // 16-byte h pieces per token fragment and step
  constexpr int kSmallDepth2 = fp4 ? 1 : 2;
  constexpr int NF = CH / 16;                 // channel fragments
  const int K = p.K;                          // = I
  const int nk = K / KS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const long rowBytes = fp4 ? (K >> 1) : K;
  const int n0 = ti.nt * CH;
  const uint8_t* W2 = p.wa[ti.wi] + ti.eg * (long)p.N * rowBytes;
  // per-block fp8: the 128 channels of the tile form one channel block; the
  // scale of the K block of step ks (two 64-wide steps per block) is sb2[ks / 2]
  const float* sb2 = nullptr;
  if constexpr (blk)
    sb2 = reinterpret_cast<const float*>(p.sa[ti.wi]) + (ti.eg * (long)(p.N >> 7) + (n0 >> 7)) * (K >> 7);

  const Operand& td = p.ta[ti.wi];
  const Operand& wd = p.wd[ti.wi];
  // wave w's share of the epilogue: channel fragments (NF / 4) w + ff; the
  // per-channel scales are fetched with the rows
  float4 es2[NF / 4];
#pragma unroll
  for (int ff = 0; ff < NF / 4; ++ff) es2[ff] = make_float4(1.f, 1.f, 1.f, 1.f);
  const uint8_t* tp[TV];
  auto rows = [&]() {
#pragma unroll
    for (int t = 0; t < TV; ++t) {
      int r = ti.row0 + t * 16 + l16;
      if (r >= ti.row1) r = ti.row1 - 1;
      tp[t] = row_ptr<kRowsStored>(p, ti, r);
    }
    if (!fp4 && !blk)
#pragma unroll
      for (int ff = 0; ff < NF / 4; ++ff)
        es2[ff] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.sa[ti.wi]) + ti.eg * p.N + n0 +
                                                   (wave * (NF / 4) + ff) * 16 + 4 * lg);
  };
  const uint8_t* wp[NF];
  const uint8_t* sp[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const long crow = n0 + f * 16 + l16;
    wp[f] = fp4 ? W2 + op_off(wd, crow, lg * 16) : W2 + crow * wd.row_pitch;
    sp[f] = fp4 ? (reinterpret_cast<const uint8_t*>(p.sa[0]) + ti.eg * (long)p.N * (K >> 5) +
                   op_off(p.sd[0], crow, lg))
                : nullptr;
  }
  auto hpiece = [&](int t, long k) {
    return *reinterpret_cast<const uint4*>(tp[t] + ((k >> td.kc_shift) * td.chunk_stride + (k & ((1L << td.kc_shift) - 1))));
  };
  auto wgt = [&](int f, long k) {
    return load_w16<NT>(wp[f] + ((k >> wd.kc_shift) * wd.chunk_stride + (k & ((1L << wd.kc_shift) - 1))));
  };

  v4f acc[NF][TV];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < TV; ++t) acc[f][t] = v4f{0.f, 0.f, 0.f, 0.f};

  struct St {
    uint4 x[TV][XS];
    uint4 w[NF];
    uint32_t sc[NF];
    float bs;
  };
  auto load_x = [&](int ks, St& st) {
#pragma unroll
    for (int t = 0; t < TV; ++t)
#pragma unroll
      for (int i = 0; i < XS; ++i)   // byte offsets of the bf16 elements of sub-step i
        st.x[t][i] = hpiece(t, (long)ks * (2 * KS) + (fp4 ? lg * 64 + 16 * i : 32 * lg + 16 * i));
  };
  auto load_w = [&](int ks, St& st) {
    if constexpr (blk) st.bs = sb2[ks >> 1];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if constexpr (fp4) {
        st.w[f] = load_w16<NT>(wp[f] + (long)ks * op_step(wd, 64));
        st.sc[f] = sp[f][(long)ks * op_step(p.sd[0], 4)];
      } else {
        st.w[f] = wgt(f, (long)ks * KS + lg * 16);
      }
    }
  };
  auto compute = [&](const St& st) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      v8bf w[XS];
      const uint32_t cw[4] = {st.w[f].x, st.w[f].y, st.w[f].z, st.w[f].w};
      if constexpr (fp4) fp4x32_to_bf16(cw, e8m0_to_f32(st.sc[f]), w);
      else fp8x16_to_bf16(cw, w);
      if constexpr (blk) {
        // a K step lies inside one K block: its partial sum times the block's scale
#pragma unroll
        for (int t = 0; t < TV; ++t) {
          v4f part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < XS; ++i)
            part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[i], as_v8bf(st.x[t][i]), part, 0, 0, 0);
          acc[f][t] += st.bs * part;
        }
      } else {
#pragma unroll
        for (int i = 0; i < XS; ++i)
#pragma unroll
          for (int t = 0; t < TV; ++t)
            acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[i], as_v8bf(st.x[t][i]), acc[f][t], 0, 0, 0);
      }
    }
  };
  small_pipeline<kSmallDepth2, St>(wave, nk, load_w, rows, load_x, compute);

#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < TV; ++t) red[wave][f * TVM + t][lane] = acc[f][t];
  __syncthreads();

  // wave w: channel fragments 2w and 2w + 1, every valid token fragment
#pragma unroll
  for (int ff = 0; ff < NF / 4; ++ff) {
    const int f = wave * (NF / 4) + ff;
    const int ch = n0 + f * 16 + 4 * lg;
    const float s2v[4] = {es2[ff].x, es2[ff].y, es2[ff].z, es2[ff].w};
#pragma unroll
    for (int t = 0; t < TV; ++t) {
      v4f s = red[0][f * TVM + t][lane];
#pragma unroll
      for (int q = 1; q < 4; ++q) s += red[q][f * TVM + t][lane];
      const int grow = ti.row0 + t * 16 + l16;
      if (grow < ti.row1)
        *reinterpret_cast<float4*>(p.y + (long)grow * p.N + ch) =
            make_float4(s[0] * s2v[0], s[1] * s2v[1], s[2] * s2v[2], s[3] * s2v[3]);
    }
  }
}

// ROWS, CH: rows and output channels per tile: 32 x 128 (small variant) or
// 64 x 64 (medium variant).
template <int FMT, bool NT, int ROWS = kSmRows, int CH = kSmCh2>
__global__ __launch_bounds__(256) void gemm2_small_kernel(GemmParams p) {
  constexpr int TVM = ROWS / 16;
  __shared__ v4f red[4][TVM * CH / 16][64];
  __shared__ int s_tp[kTileLds];
  MOE_TILE_PROLOGUE(ROWS);
  const int vr = ti.row1 - ti.row0;
  // the routed group takes FMT; the shared group is always per-channel fp8
  auto run = [&](auto fc) {
    constexpr int F = decltype(fc)::value;
    if (TVM > 2 && vr > 48) gemm2_small_body<F, TVM, NT, TVM, CH>(p, ti, red);
    else if (TVM > 2 && vr > 32) gemm2_small_body<F, (TVM > 2 ? 3 : 2), NT, TVM, CH>(p, ti, red);
    else if (vr > 16) gemm2_small_body<F, 2, NT, TVM, CH>(p, ti, red);
    else gemm2_small_body<F, 1, NT, TVM, CH>(p, ti, red);
  };
  if (FMT != kFp8 && ti.wi == 0) run(std::integral_constant<int, FMT>{});
  else run(std::integral_constant<int, kFp8>{});
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
// weight layout
// ============================================================================

// dst[e][c][n][0 .. C) = src[e][n][c*C .. c*C + C): one thread per 16 bytes of
// dst (consecutive threads write consecutive bytes).
__global__ __launch_bounds__(256) void pack_kblocked_kernel(const uint8_t* __restrict__ src,
                                                            uint8_t* __restrict__ dst, int N, int K, int C,
                                                            long total16) {
  const long per_e = (long)N * K, per_c = (long)N * C;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total16; i += (long)gridDim.x * blockDim.x) {
    const long byte = i * 16;
    const long e = byte / per_e;
    const long r1 = byte - e * per_e;
    const long c = r1 / per_c;
    const long r2 = r1 - c * per_c;
    const long n = r2 / C;
    const long off = r2 - n * C;
    *reinterpret_cast<uint4*>(dst + byte) =
        *reinterpret_cast<const uint4*>(src + e * per_e + n * K + c * C + off);
  }
}

// The same with chunks of 4 bytes: one thread per 4 bytes of dst.
__global__ __launch_bounds__(256) void pack_kblocked4_kernel(const uint32_t* __restrict__ src,
                                                             uint32_t* __restrict__ dst, int N, int K4,
                                                             long total4) {
  const long per_e = (long)N * K4;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total4; i += (long)gridDim.x * blockDim.x) {
    const long e = i / per_e;
    const long r1 = i - e * per_e;
    const long c = r1 / N;
    const long n = r1 - c * N;
    dst[i] = src[e * per_e + n * K4 + c];
  }
}

hipError_t launch_pack_kblocked4(const uint8_t* src, uint8_t* dst, int E, int N, int K, hipStream_t s) {
  const long total4 = (long)E * N * (K / 4);
  if (total4 == 0) return hipSuccess;
  long blocks = (total4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  pack_kblocked4_kernel<<<(unsigned)blocks, 256, 0, s>>>(reinterpret_cast<const uint32_t*>(src),
                                                         reinterpret_cast<uint32_t*>(dst), N, K / 4, total4);
  return hipGetLastError();
}

hipError_t launch_pack_kblocked(const uint8_t* src, uint8_t* dst, int E, int N, int K, int C, hipStream_t s) {
  const long total16 = (long)E * N * K / 16;
  if (total16 == 0) return hipSuccess;
  long blocks = (total16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  pack_kblocked_kernel<<<(unsigned)blocks, 256, 0, s>>>(src, dst, N, K, C, total16);
  return hipGetLastError();
}

// ============================================================================
// launchers
// ============================================================================

long max_row_tiles(long n_rows, int n_groups, int bm) { return (n_rows + bm - 1) / bm + n_groups; }

int choose_variant(const FfnGroups& g, long n_rows) {
  const bool shapes_ok = (g.hidden % kLgCh) == 0 && (g.inter % (kLgCh / 2)) == 0;
  const long avg = n_rows / (g.n_groups > 0 ? g.n_groups : 1);
  if (g.fmt == kFp8Block) {
    // the large gate-up kernel's per-block form: 128-row tiles (its
    // accumulator rescaling needs the registers the 256-row tile uses), a
    // wave's K-block scales held in two lanes' registers
    if (shapes_ok && g.hidden <= 128 * 128 && avg >= 64) return kVariantLarge128;
    return avg >= kMdMinAvgRows ? kVariantMedium : kVariantSmall;
  }
  if (g.fmt != kFp8 || !shapes_ok) return kVariantSmall;
  if (avg < 64) return kVariantSmall;
  return avg >= 384 ? kVariantLarge256 : kVariantLarge128;
}

// The down GEMM's variant: as the gate-up GEMM's, except for per-block fp8
// weights, which take the 256-row large kernel too (their block scale is
// one number per wave and K block there, applied as the codes are widened;
// the gate-up kernel's per-block form runs 128-row tiles only).
int choose_down_variant(const FfnGroups& g, long n_rows) {
  if (g.fmt != kFp8Block) return choose_variant(g, n_rows);
  // the large kernel holds a wave's K-block scales in two lanes' registers
  const bool large_ok = (g.hidden % kLgCh) == 0 && (g.inter % (kLgCh / 2)) == 0 && g.inter <= 128 * 128;
  const long avg = n_rows / (g.n_groups > 0 ? g.n_groups : 1);
  if (large_ok && avg >= 64) return avg >= 384 ? kVariantLarge256 : kVariantLarge128;
  return avg >= kMdMinAvgRows ? kVariantMedium : kVariantSmall;
}

int shared_gate_up_variant(const FfnGroups& g, long n_rows, long shared_rows) {
  if (g.fmt != kFp8Block || g.n_groups <= g.n_routed || !variant_in_registers(choose_variant(g, n_rows))) return -1;
  if ((g.hidden % kLgCh) != 0 || (g.inter % (kLgCh / 2)) != 0 || shared_rows < 64) return -1;
  // 256-row tiles only when they alone fill the chip (a launch of one group
  // has no other groups' tiles beside it)
  const long tiles256 = (shared_rows + 255) / 256 * (g.inter / (kLgCh / 2));
  return tiles256 >= kNumCUs ? kVariantLarge256 : kVariantLarge128;
}

bool small_streams_weights(const FfnGroups& g, long n_rows) {
  return n_rows <= (long)kSmRows * (g.n_groups > 0 ? g.n_groups : 1);
}

int variant_rows(int variant) {
  return variant == kVariantLarge256 ? 256 : variant == kVariantLarge128 ? 128 : variant == kVariantMedium ? kMdRows : kSmRows;
}

const char* variant_name(int variant) {
  return variant == kVariantLarge256 ? "large256"
         : variant == kVariantLarge128 ? "large128"
         : variant == kVariantMedium   ? "medium64"
                                       : "small32";
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
  for (int i = 0; i < 2; ++i) {
    p.a[i] = x.q[i];
    p.a_scale[i] = x.s[i];
    p.ta[i] = x.d[i];
  }
  p.shared_row0 = x.shared_row0;
  p.gather = x.gather;
  p.gather_k = x.gather_k;
  return p;
}

hipError_t launch_gemm1(int variant, const FfnGroups& g, const RowOperand& x, const int* tile_prefix,
                        long n_rows, uint16_t* h, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop,
                        long grid_rows) {
  if (grid_rows < 0) grid_rows = n_rows;
  GemmParams p = base_params(g, x, tile_prefix);
  p.K = g.hidden;
  p.N = g.inter;
  for (int i = 0; i < 2; ++i) {
    p.wa[i] = g.w1[i];
    p.wb[i] = g.w3[i];
    p.sa[i] = g.s1[i];
    p.sb[i] = g.s3[i];
    const bool fp4 = i == 0 && g.fmt == kMxfp4;
    p.wd[i] = g.blocked[i] ? k_blocked_operand(g.inter, fp4 ? kFp4Chunk : kW13Chunk)
                           : row_major_operand(fp4 ? g.hidden / 2 : g.hidden);
    p.sd[i] = g.blocked[i] ? k_blocked_operand(g.inter, kFp4ScaleChunk) : row_major_operand(g.hidden / 32);
    p.act[i] = g.act[i];
    p.beta[i] = g.beta[i];
  }
  p.h = h;
  p.h_cs = n_rows * kHChunk;
  const int bm = variant_rows(variant);
  if (variant_in_registers(variant)) {
    p.ntiles = g.inter / (kSmCh / 2);
    const long grid = max_row_tiles(grid_rows, g.n_groups, bm) * p.ntiles;
    auto pick = [&](auto nt, auto rows) {
      constexpr bool NT = decltype(nt)::value;
      constexpr int R = decltype(rows)::value;
      return x.gather ? (g.fmt == kMxfp4      ? gemm1_small_kernel<kMxfp4, kRowsGathered, NT, R>
                         : g.fmt == kFp8Block ? gemm1_small_kernel<kFp8Block, kRowsGathered, NT, R>
                                              : gemm1_small_kernel<kFp8, kRowsGathered, NT, R>)
                      : (g.fmt == kMxfp4      ? gemm1_small_kernel<kMxfp4, kRowsStored, NT, R>
                         : g.fmt == kFp8Block ? gemm1_small_kernel<kFp8Block, kRowsStored, NT, R>
                                              : gemm1_small_kernel<kFp8, kRowsStored, NT, R>);
    };
    using Sm = std::integral_constant<int, kSmRows>;
    using Md = std::integral_constant<int, kMdRows>;
    auto kern = variant == kVariantMedium ? pick(std::false_type{}, Md{})
                : small_streams_weights(g, n_rows) ? pick(std::true_type{}, Sm{}) : pick(std::false_type{}, Sm{});
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, ev_start, ev_stop, 0, p);
  } else {
    p.ntiles = g.inter / (kLgCh / 2);
    const long grid = max_row_tiles(grid_rows, g.n_groups, bm) * p.ntiles;
    const bool situ = g.act[0] == kActSitu || (g.n_groups > g.n_routed && g.act[1] == kActSitu);
    // per-block fp8 takes the 128-row kernel only (choose_variant)
    const bool blk = g.fmt == kFp8Block;
    auto kern = variant == kVariantLarge256 ? (situ ? gemm1_pp_kernel<256, 4, true> : gemm1_pp_kernel<256, 4, false>)
                : blk ? (situ ? gemm1_pp_kernel<128, 6, true, true> : gemm1_pp_kernel<128, 6, false, true>)
                      : (situ ? gemm1_pp_kernel<128, 6, true> : gemm1_pp_kernel<128, 6, false>);
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, ev_start, ev_stop, 0, p);
  }
  return hipGetLastError();
}

hipError_t launch_gemm2(int variant, const FfnGroups& g, const uint16_t* h, const int* tile_prefix,
                        long n_rows, float* y, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  // every group's rows index the one K-blocked h directly
  const Operand hd = k_blocked_operand(n_rows, kHChunk);
  const RowOperand hr{{h, h}, {nullptr, nullptr}, 0, {hd, hd}};
  GemmParams p = base_params(g, hr, tile_prefix);
  p.K = g.inter;
  p.N = g.hidden;
  for (int i = 0; i < 2; ++i) {
    p.wa[i] = g.w2[i];
    p.sa[i] = g.s2[i];
    const bool fp4 = i == 0 && g.fmt == kMxfp4;
    p.wd[i] = g.blocked[i] ? k_blocked_operand(g.hidden, fp4 ? kFp4Chunk : kW2Chunk)
                           : row_major_operand(fp4 ? g.inter / 2 : g.inter);
    p.sd[i] = g.blocked[i] ? k_blocked_operand(g.hidden, kFp4ScaleChunk) : row_major_operand(g.inter / 32);
  }
  p.y = y;
  const int bm = variant_rows(variant);
  if (variant_in_registers(variant)) {
    const bool md = variant == kVariantMedium;
    p.ntiles = g.hidden / (md ? kMdCh2 : kSmCh2);
    const long grid = max_row_tiles(n_rows, g.n_groups, bm) * p.ntiles;
    auto pick = [&](auto nt, auto rows, auto ch) {
      constexpr bool NT = decltype(nt)::value;
      constexpr int R = decltype(rows)::value, C = decltype(ch)::value;
      return g.fmt == kMxfp4      ? gemm2_small_kernel<kMxfp4, NT, R, C>
             : g.fmt == kFp8Block ? gemm2_small_kernel<kFp8Block, NT, R, C>
                                  : gemm2_small_kernel<kFp8, NT, R, C>;
    };
    using Sm = std::integral_constant<int, kSmRows>;
    using Md = std::integral_constant<int, kMdRows>;
    using SmC = std::integral_constant<int, kSmCh2>;
    using MdC = std::integral_constant<int, kMdCh2>;
    auto kern = md ? pick(std::false_type{}, Md{}, MdC{})
                : small_streams_weights(g, n_rows) ? pick(std::true_type{}, Sm{}, SmC{})
                                                   : pick(std::false_type{}, Sm{}, SmC{});
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, ev_start, ev_stop, 0, p);
  } else {
    p.ntiles = g.hidden / kLgCh;
    const long grid = max_row_tiles(n_rows, g.n_groups, bm) * p.ntiles;
    const bool blk = g.fmt == kFp8Block;
    auto kern = variant == kVariantLarge256 ? (blk ? gemm2_pp_kernel<256, 4, true> : gemm2_pp_kernel<256, 4, false>)
                                            : (blk ? gemm2_pp_kernel<128, 8, true> : gemm2_pp_kernel<128, 8, false>);
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, ev_start, ev_stop, 0, p);
  }
  return hipGetLastError();
}

}  // namespace moe
