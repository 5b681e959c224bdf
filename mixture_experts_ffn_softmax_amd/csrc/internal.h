// Internal launch interface between the C ABI layer (moe_api.cpp) and the
// kernels.  Every launcher enqueues on `stream`, never synchronises, and
// returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kNumCUs = 256;        // gfx950: 8 XCDs x 32 CUs
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kPermuteChunk = 1024;  // pairs per counting / ranking chunk
constexpr int kMetaMaxPairs = 16384; // pairs handled by the single-workgroup metadata kernel
// ... for at most this many experts: its ballot ranking visits every expert
// present among a wave's 256 pairs, so its cost grows with E
constexpr int kMetaMaxE = 64;
constexpr int kMetaRouteMaxE = 32;   // experts the one-workgroup router handles (bit masks) ...
constexpr int kMetaRouteMaxT = 4096; // ... for batches of at most this many tokens ...
constexpr int kMetaRouteMaxPairs = 16384;  // ... and pairs; the same launch quantises
constexpr int kMetaQuantMaxH = 32768;      // tokens of at most this many elements

// Byte addressing of a matrix operand with rows of K contraction bytes: byte k
// of row r sits at r * row_pitch + (k >> kc_shift) * chunk_stride +
// (k & ((1 << kc_shift) - 1)).  Row-major: row_pitch = K, kc_shift = 31.
// K-blocked in C-byte chunks over R rows: row_pitch = C, kc_shift = log2 C,
// chunk_stride = R * C (every chunk holds all R rows).
struct Operand {
  long row_pitch;
  long chunk_stride;
  int kc_shift;
};
inline Operand row_major_operand(long k_bytes) { return Operand{k_bytes, 0, 31}; }
inline Operand k_blocked_operand(long rows, int chunk_bytes) {
  int sh = 0;
  while ((1 << sh) < chunk_bytes) ++sh;
  return Operand{chunk_bytes, rows * chunk_bytes, sh};
}
// K-blocked chunk sizes: quantised tokens and W1/W3 in 64-byte chunks (one
// gate-up MFMA step), h (bf16) in 64-byte chunks of 32 elements and W2 in
// 32-byte chunks (one down-projection step of 32 elements).
constexpr int kTokChunk = 64;
constexpr int kW13Chunk = 64;
constexpr int kHChunk = 64;
constexpr int kW2Chunk = 32;
// MXFP4 weights K-blocked: codes in 64-byte chunks (128 elements, one MFMA
// step of either GEMM) and e8m0 scales in 4-byte chunks (the same 128).
constexpr int kFp4Chunk = 64;
constexpr int kFp4ScaleChunk = 4;

// ---- router ---------------------------------------------------------------
// sigmoid: scores 1 / (1 + e^-l) instead of the softmax; same selection.
// ev_start (optional): stamped by the router's dispatch when it begins.
hipError_t launch_route(const float* logits, int T, int E, int k, bool sigmoid, int* ids, float* w,
                        hipStream_t s, hipEvent_t ev_start = nullptr);

// ---- counts, offsets, ranks, quantise + scatter ---------------------------
inline int permute_chunks(long pairs) { return (int)((pairs + kPermuteChunk - 1) / kPermuteChunk); }

// chunk_hist / chunk_base: int [chunks][E] each.  extra_rows > 0 appends one
// group of that many rows after the E expert segments: offsets[E+1] =
// offsets[E] + extra_rows (offsets must then hold E+2 ints).
hipError_t launch_counts(const int* ids, int pairs, int E, int* chunk_hist, int* chunk_base,
                         int* counts, int* offsets, int extra_rows, hipStream_t s);
hipError_t launch_rank(const int* ids, int pairs, int E, const int* chunk_base, int* pair_to_row,
                       int* row_to_pair, hipStream_t s);
// Quantise each token and write its codes / scale to rows pair_to_row[t][*]
// (skipped when negative) and, when xq_tok is non-NULL, to xq_tok[t] / xs_tok[t].
// blocked = false: row-major [rows][H]; true: K-blocked in kTokChunk-byte
// chunks, xq_rows over T*k rows and xq_tok over T rows.  xq_copy, when
// non-NULL, also receives xq_rows row-major.
hipError_t launch_quant_scatter(const uint16_t* x, int T, int H, int k, const int* pair_to_row,
                                uint8_t* xq_rows, float* xs_rows, uint8_t* xq_tok, float* xs_tok,
                                bool blocked, uint8_t* xq_copy, hipStream_t s);
// For T * k <= kMetaMaxPairs: counts, offsets (+ the extra group), ranks and,
// when tile_prefix is non-NULL, the tile prefix of the groups for row tiles
// of bm, from the expert ids, in one launch of one workgroup (16 waves).
hipError_t launch_meta(int T, int E, int k, const int* ids, int* counts, int* offsets, int extra_rows,
                       int* pair_to_row, int* row_to_pair, int* tile_prefix, int bm, hipStream_t s);
// Routing from the logits (ids / w; T <= kMetaRouteMaxT, E <= kMetaRouteMaxE,
// T * k <= kMetaRouteMaxPairs, H <= kMetaQuantMaxH, else
// hipErrorInvalidValue), the metadata of launch_meta, and the per-token
// quantisation into token order (xq_tok K-blocked in kTokChunk-byte chunks,
// xs_tok [T]) in one launch: workgroup 0 routes and builds the metadata,
// workgroup 1 + i quantises tokens 2i and 2i + 1.  The two parts read and
// write disjoint buffers.
hipError_t launch_meta_quant(const float* logits, bool sigmoid, const uint16_t* x, int T, int H, int E, int k,
                             int* ids, float* w, int* counts, int* offsets, int extra_rows, int* pair_to_row,
                             int* row_to_pair, int* tile_prefix, int bm, uint8_t* xq_tok, float* xs_tok,
                             hipStream_t s, hipEvent_t ev_start = nullptr);
// Row-major, expert-ordered copy (xq_rows [T*k][H], xs_rows [T*k]; either may
// be NULL) of the K-blocked token-order quantised rows: row r holds token
// row_to_pair[r] / k.
hipError_t launch_rows_from_tokens(const uint8_t* xq_tok, const float* xs_tok, const int* row_to_pair, int T,
                                   int k, int H, uint8_t* xq_rows, float* xs_rows, hipStream_t s);
// The same rows K-blocked (kTokChunk-byte chunks over T*k rows, as the
// grouped GEMMs read them), with their scales; both outputs required.
hipError_t launch_rows_kblocked(const uint8_t* xq_tok, const float* xs_tok, const int* row_to_pair, int T, int k,
                                int H, uint8_t* xq_rows, float* xs_rows, hipStream_t s);

// ---- grouped expert FFN ---------------------------------------------------
// kFp8Block: e4m3 codes with one fp32 scale per 128 x 128 tile (channel
// block x K block); only the small GEMM variants take it.
enum WeightFormat { kFp8 = 0, kMxfp4 = 1, kFp8Block = 3 };
enum Activation { kActSilu = 0, kActSitu = 1 };   // gate activation of an expert group

// One grouped GEMM launch covers groups 0..n_groups-1.  Rows of group g are
// offsets[g] .. offsets[g+1]-1 of the row operand.  Groups g < n_routed take
// their weights from the routed base pointers (expert g); group n_routed (if
// n_groups > n_routed) from the shared base pointers.
struct FfnGroups {
  int fmt;            // WeightFormat (routed); the shared group is always fp8
  int n_groups;
  int n_routed;
  int hidden;         // H
  int inter;          // I
  const int* offsets; // device [n_groups + 1]
  // routed / shared weights (index 0 / 1)
  const uint8_t* w1[2];
  const uint8_t* w3[2];
  const uint8_t* w2[2];
  const void* s1[2];
  const void* s3[2];
  const void* s2[2];
  bool blocked[2];    // weights K-blocked (moe_pack_weights) rather than row-major
  int act[2];         // Activation of the routed / shared group
  float beta[2];      // SiTU's beta of the routed / shared group
};

// Row operand of a grouped GEMM: GEMM1 reads e4m3 codes q with per-row
// scales s, GEMM2 reads bf16 h (s unused).  Rows below shared_row0 are read
// from q[0]/s[0] at their row index; the shared group's rows from q[1]/s[1]
// at (row - shared_row0).
struct RowOperand {
  const void* q[2];
  const float* s[2];
  long shared_row0;
  Operand d[2];       // byte addressing of q[0] / q[1]
  // optional gather of the routed rows: row r < shared_row0 reads row
  // gather[r] / gather_k of q[0] / s[0] (gather = row_to_pair, q[0] the
  // token-order rows), so that no expert-ordered copy is needed
  const int* gather = nullptr;
  int gather_k = 1;
};

// small: 32-row tiles, operands straight into registers (weight streaming);
// medium: the same kernels with 64-row tiles, for per-block fp8 batches with
// many rows per group but too few for the large kernels;
// large: 128- or 256-row tiles staged through an LDS ring (per-channel fp8;
// per-block fp8 in 128-row gate-up tiles and in the down GEMM).
enum GemmVariant { kVariantSmall = 0, kVariantLarge128 = 1, kVariantLarge256 = 2, kVariantMedium = 3 };
// The variants whose kernels read their row fragments straight into registers.
inline bool variant_in_registers(int v) { return v == kVariantSmall || v == kVariantMedium; }

int choose_variant(const FfnGroups& g, long n_rows);
// The down GEMM's variant: choose_variant's, except that per-block fp8
// weights may take the 256-row large kernel (the gate-up GEMM's 128 only).
int choose_down_variant(const FfnGroups& g, long n_rows);
// With per-block fp8 routed weights the gate-up GEMM runs the register-fed
// kernels; the shared group (per-channel fp8, shared_rows rows) then takes a
// launch of its own on the large kernel: its variant, or -1 (one launch).
int shared_gate_up_variant(const FfnGroups& g, long n_rows, long shared_rows);
// The small variant streams its weights with non-temporal loads when the
// groups average at most one row tile (kSmRows rows): each weight tile is then
// read by about one workgroup.  With more rows per group several row tiles
// re-read each weight tile, and ordinary (cached) loads serve them.
bool small_streams_weights(const FfnGroups& g, long n_rows);
int variant_rows(int variant);          // rows per tile
const char* variant_name(int variant);
long max_row_tiles(long n_rows, int n_groups, int bm);

// tile_prefix[g] = sum over g' < g of ceil(rows(g') / bm), g = 0..n_groups.
hipError_t launch_tile_prefix(const int* offsets, int n_groups, int bm, int* tile_prefix, hipStream_t s);
// GEMM1: h[r][n] = bf16(SiLU(g) * u) for the gate/up pair of channel n.  h is
// K-blocked for GEMM2: kHChunk-byte chunks (32 channels) over n_rows rows.
// ev_start / ev_stop (may be NULL): stamped by the GEMM1 dispatch itself.
// grid_rows (>= 0): the rows the launch's groups hold, when fewer than
// n_rows (a launch over some of the groups); sizes the grid only.
hipError_t launch_gemm1(int variant, const FfnGroups& g, const RowOperand& x, const int* tile_prefix,
                        long n_rows, uint16_t* h, hipStream_t s, hipEvent_t ev_start = nullptr,
                        hipEvent_t ev_stop = nullptr, long grid_rows = -1);
// GEMM2: y[r][j] = (h_r . W2[j]) * s2[j] in fp32; h as GEMM1 writes it.
hipError_t launch_gemm2(int variant, const FfnGroups& g, const uint16_t* h, const int* tile_prefix,
                        long n_rows, float* y, hipStream_t s, hipEvent_t ev_start = nullptr,
                        hipEvent_t ev_stop = nullptr);

// ---- weight layout ------------------------------------------------------------
// Copies E matrices of [N][K] bytes into the K-blocked layout with C-byte chunks.
hipError_t launch_pack_kblocked(const uint8_t* src, uint8_t* dst, int E, int N, int K, int C,
                                hipStream_t s);
// The same for chunks of 4 bytes (C = 4; K a multiple of 4).
hipError_t launch_pack_kblocked4(const uint8_t* src, uint8_t* dst, int E, int N, int K, hipStream_t s);

// ---- fixed scratch (moe_forward_noalloc) -----------------------------------
// Device address of the library's scratch array on device `dev`, which must
// be the current device: looked up with hipGetSymbolAddress on the first
// call for that device and kept for the rest of the process.
hipError_t noalloc_scratch(int dev, void** ptr);

// ---- combine --------------------------------------------------------------
hipError_t launch_combine(const float* y_rows, const int* pair_to_row, const float* w, int T,
                          int H, int k, const float* y_shared, const float* gamma, float eps,
                          uint16_t* out, hipStream_t s, hipEvent_t ev_start = nullptr,
                          hipEvent_t ev_stop = nullptr);

// ---- dense GEMMs (LatentMoE projections and shared experts) --------------
// C[M][N] = epilogue(A[M][K] x B[N][K]^T): A bf16 row-major with row pitch
// lda elements; B bf16 [N][K] (bfmt kBf16W) or MXFP4 codes [N][K/2] + e8m0
// [N][K/32] (bfmt kMxfp4).  K % 64 == 0; N % 128 == 0 (N % 64 in kDnGateUp,
// where b is W1 and b3 is W3, and the output h[m][n] = bf16(act(g) * u)).
enum DenseMode { kDnStoreBf16 = 0, kDnStoreF32 = 1, kDnAddBf16 = 2, kDnGateUp = 3 };
constexpr int kBf16W = 2;   // bf16 weights (beside kFp8 / kMxfp4)
struct DenseParams {
  const uint16_t* a;
  long lda;
  int M, N, K;
  int bfmt;
  const void* b;        // W (or W1 in kDnGateUp)
  const uint8_t* bs;    // its e8m0 scales (MXFP4)
  const void* b3;       // W3 (kDnGateUp)
  const uint8_t* bs3;
  int mode;             // DenseMode
  const float* addend;  // kDnAddBf16: fp32 [M][ldc], added before the rounding
  void* c;              // bf16 or fp32 [M][ldc]
  long ldc;
  int act;              // kDnGateUp: Activation and beta
  float beta;
  int tiles_n;          // set by launch_dense
  int ksplit;           // set by launch_dense_splitk: workgroups per tile, each a K range
};
hipError_t launch_dense(const DenseParams& p, hipStream_t s, hipEvent_t ev_start = nullptr,
                        hipEvent_t ev_stop = nullptr);
// kDnStoreBf16 with K split over `ksplit` workgroups per tile: each writes an
// fp32 partial into part[z][M][N] (ksplit * M * N floats), then one pass sums
// the partials in order z = 0, 1, ... and rounds once into p.c.  K must be a
// multiple of 64 * ksplit.
hipError_t launch_dense_splitk(const DenseParams& p, int ksplit, float* part, hipStream_t s,
                               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

}  // namespace moe
