// Routing metadata and the scatter of token rows to experts.
//
// The Ling-2.6-1T page (§1: scatter tokens -> local expert FFN -> gather
// results; §6: the metadata block of token-to-expert map, per-expert
// offsets/counts and scatter/gather indices) and its §5 (tokens quantised to
// fp8 per token before the scatter).
//
// Pairs p = t*k + j are cut into chunks of kPermuteChunk.  Kernels:
//   hist_kernel    per-chunk expert histograms (LDS atomics: counts only, so
//                  the result does not depend on their order)
//   scan_kernel    per-expert totals, exclusive offsets, and per-(chunk,
//                  expert) starting rows, expert-major then chunk-minor
//   rank_kernel    stable rank of each pair inside its chunk, by wave ballots
//                  in pair order -> pair_to_row / row_to_pair
//   quant_scatter  per token: amax, scale, e4m3 codes, written to each of the
//                  token's rows (and optionally in token order)
//   meta_kernel    one workgroup doing all of the above but the quantisation
//                  (and the grouped GEMMs' tile prefix) when there are at
//                  most kMetaMaxPairs pairs: one launch instead of four
//   meta_quant_kernel  the same plus the routing, in one workgroup, for at
//                  most kMetaRouteMaxT tokens and kMetaRouteMaxE experts,
//                  with the quantisation into token order in the same launch
//                  (the other workgroups); the gate-up GEMM then gathers the
//                  routed rows through row_to_pair
// Rows are ordered by expert and, inside an expert, by pair index; this order
// is unique, so the result is deterministic.  Expert ids outside [0, E) are
// skipped (their pairs get row -1) so that no access leaves its buffer.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "internal.h"

namespace moe {

__global__ __launch_bounds__(256) void hist_kernel(const int* __restrict__ ids, int pairs, int E,
                                                   int* __restrict__ chunk_hist) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const long base = (long)blockIdx.x * kPermuteChunk;
  for (int i = threadIdx.x; i < kPermuteChunk; i += 256) {
    const long p = base + i;
    if (p < pairs) {
      const int e = ids[p];
      if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_hist[(long)blockIdx.x * E + e] = h[e];
}

// One block of 1024 threads.  Thread t works on expert t % E and on the
// (t / E)-th of P = min(1024 / E, chunks) contiguous ranges of chunks, so that
// with few experts most threads still have loads in flight; each pass keeps
// eight chunk loads of a thread in flight.  The bases come out as if one
// thread per expert walked its chunks in order.
__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ chunk_hist, int chunks,
                                                    int E, int* __restrict__ chunk_base,
                                                    int* __restrict__ counts,
                                                    int* __restrict__ offsets, int extra_rows) {
  __shared__ int off[kMaxExperts];
  __shared__ int part[1024];
  __shared__ int tmp[16];
  const int t = threadIdx.x;
  const int Eg = E > 0 ? E : 1;
  const int P = max(1, min(1024 / Eg, chunks));
  const int cpp = (chunks + P - 1) / P;
  const int e = t % Eg, p = t / Eg;
  const bool act = E > 0 && p < P;
  const int c0 = act ? min(p * cpp, chunks) : 0;
  const int c1 = act ? min(c0 + cpp, chunks) : 0;
  int sum = 0;
  int c = c0;
  for (; c + 8 <= c1; c += 8) {
    int a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = chunk_hist[(long)(c + i) * E + e];
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += a[i];
  }
  for (; c < c1; ++c) sum += chunk_hist[(long)c * E + e];
  if (act) part[t] = sum;                     // part[p * E + e]
  __syncthreads();
  int total = 0;
  if (t < E) {
    for (int q = 0; q < P; ++q) total += part[q * E + t];
    off[t] = total;
  }
  __syncthreads();
  const int all = block_exclusive_scan_1024(off, tmp, E);
  if (t < E) {
    counts[t] = total;
    offsets[t] = off[t];
  }
  if (act) {
    int run = off[e];
    for (int q = 0; q < p; ++q) run += part[q * E + e];
    c = c0;
    for (; c + 8 <= c1; c += 8) {
      int a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = chunk_hist[(long)(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        chunk_base[(long)(c + i) * E + e] = run;
        run += a[i];
      }
    }
    for (; c < c1; ++c) {
      const int n = chunk_hist[(long)c * E + e];
      chunk_base[(long)c * E + e] = run;
      run += n;
    }
  }
  if (t == 0) {
    offsets[E] = all;
    if (extra_rows > 0) offsets[E + 1] = all + extra_rows;
  }
}

// Block of 256 threads = 4 waves per chunk of 1024 pairs; wave w ranks pairs
// [w*256, w*256+256) of the chunk in four windows of 64, in order: a pair's
// rank is its expert's count so far in the wave plus the number of earlier
// lanes of the window with the same expert (found by matching the expert id
// bit by bit with ballots, so the cost does not grow with the number of
// distinct experts in the window).
__global__ __launch_bounds__(256) void rank_kernel(const int* __restrict__ ids, int pairs, int E,
                                                   const int* __restrict__ chunk_base,
                                                   int* __restrict__ pair_to_row,
                                                   int* __restrict__ row_to_pair) {
  __shared__ int cnt[4][kMaxExperts];
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const long cbase = (long)blockIdx.x * kPermuteChunk;
  for (int i = threadIdx.x; i < 4 * E; i += 256) cnt[i / E][i % E] = 0;
  __syncthreads();
  int my_e[4];
#pragma unroll
  for (int win = 0; win < 4; ++win) {
    const long p = cbase + w * 256 + win * 64 + lane;
    int e = -1;
    if (p < pairs) {
      e = ids[p];
      if ((unsigned)e >= (unsigned)E) e = -1;
    }
    my_e[win] = e;
    if (e >= 0) atomicAdd(&cnt[w][e], 1);
  }
  __syncthreads();
  // per-wave starting rows: chunk base plus the counts of the earlier waves
  for (int e = threadIdx.x; e < E; e += 256) {
    int run = chunk_base[(long)blockIdx.x * E + e];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = cnt[q][e];
      cnt[q][e] = run;
      run += n;
    }
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint64_t gt_mask = ~lt_mask & ~(1ull << lane);
  // id bits to match: E - 1 fits in nbits bits
  const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
#pragma unroll
  for (int win = 0; win < 4; ++win) {
    const long p = cbase + w * 256 + win * 64 + lane;
    const int e = my_e[win];
    // the window's lanes with this lane's expert: one ballot per id bit
    // (lanes without an expert are outside the first mask)
    uint64_t same = __ballot(e >= 0);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    int row = -1;
    const int before = (int)__popcll(same & lt_mask);
    if (e >= 0) row = cnt[w][e] + before;
    // every lane's read of its expert's count precedes the update (one
    // wave's LDS operations complete in order); the expert's last lane in
    // the window advances it past the window's pairs
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && (same & gt_mask) == 0) cnt[w][e] += before + 1;
    __builtin_amdgcn_wave_barrier();
    if (p < pairs) {
      pair_to_row[p] = row;
      if (row >= 0) row_to_pair[row] = (int)p;
    }
  }
}

// Byte offset of the 8 codes idx*8 .. idx*8+7 of row r: row-major (cs = 0)
// or K-blocked in kTokChunk-byte chunks with chunk stride cs.
__device__ __forceinline__ long code_offset(long r, int idx, int H, long cs) {
  return cs ? (long)(idx >> 3) * cs + r * kTokChunk + (idx & 7) * 8 : r * H + (long)idx * 8;
}

// One block per token.  The row is nchk chunks of 8 bf16; thread i handles
// chunks i, i + blockDim, ..., (CPT of them, some possibly past nchk).
// blockDim is a multiple of 64 so that the wave reductions see full waves.
// rows_cs / tok_cs: chunk strides of the K-blocked xq_rows / xq_tok (0 =
// row-major); xq_copy: optional row-major copy of the xq_rows writes.
template <int CPT>
__device__ __forceinline__ void quant_token(const uint16_t* __restrict__ x, long t, int H, int k,
                                            const int* __restrict__ pair_to_row, uint8_t* __restrict__ xq_rows,
                                            float* __restrict__ xs_rows, uint8_t* __restrict__ xq_tok,
                                            float* __restrict__ xs_tok, long rows_cs, long tok_cs,
                                            uint8_t* __restrict__ xq_copy) {
  __shared__ float red[16];
  __shared__ int s_rows[kMaxTopK];
  const int nchk = H >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * H);
  // the token's rows, fetched first so that their latency overlaps the row's;
  // a barrier after the amax reduction publishes them to every lane
  if (threadIdx.x < k) s_rows[threadIdx.x] = pair_to_row[t * k + threadIdx.x];
  uint4 in[CPT];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = threadIdx.x + c * blockDim.x;
    in[c] = (idx < nchk) ? src[idx] : make_uint4(0, 0, 0, 0);
    const uint32_t wds[4] = {in[c].x, in[c].y, in[c].z, in[c].w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(wds[q])), fabsf(bf16_hi(wds[q]))));
  }
  amax = block_max(amax, red);
  // block_max has barriers only when the block has more than one wave
  if (blockDim.x <= 64) __syncthreads();
  const float s = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
  const float r = e4m3_recip(s);
  uint2 q8[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const uint32_t wds[4] = {in[c].x, in[c].y, in[c].z, in[c].w};
    q8[c] = e4m3_encode8(wds, s, r);
  }
  for (int j = 0; j < k; ++j) {
    const int r = s_rows[j];
    if (r < 0) continue;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = threadIdx.x + c * blockDim.x;
      if (idx < nchk) {
        *reinterpret_cast<uint2*>(xq_rows + code_offset(r, idx, H, rows_cs)) = q8[c];
        if (xq_copy) *reinterpret_cast<uint2*>(xq_copy + (long)r * H + (long)idx * 8) = q8[c];
      }
    }
    if (threadIdx.x == 0) xs_rows[r] = s;
  }
  if (xq_tok) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = threadIdx.x + c * blockDim.x;
      if (idx < nchk) *reinterpret_cast<uint2*>(xq_tok + code_offset(t, idx, H, tok_cs)) = q8[c];
    }
    if (threadIdx.x == 0) xs_tok[t] = s;
  }
}

template <int CPT>
__global__ __launch_bounds__(1024) void quant_scatter_kernel(
    const uint16_t* __restrict__ x, int H, int k, const int* __restrict__ pair_to_row,
    uint8_t* __restrict__ xq_rows, float* __restrict__ xs_rows, uint8_t* __restrict__ xq_tok,
    float* __restrict__ xs_tok, long rows_cs, long tok_cs, uint8_t* __restrict__ xq_copy) {
  quant_token<CPT>(x, blockIdx.x, H, k, pair_to_row, xq_rows, xs_rows, xq_tok, xs_tok, rows_cs, tok_cs, xq_copy);
}

// ---------------------------------------------------------------------------
// meta_kernel: one workgroup of 1024 threads (16 waves).
//   1. ids read from `ids` into LDS.
//   2. counts (LDS atomics: counts only), exclusive offsets, the optional
//      extra group, and the tile prefix of the groups for row tiles of bm.
//   3. ranks, chunk by chunk of 1024 pairs in pair order: each wave ranks its
//      64 pairs by ballots, a per-expert scan over the 16 waves turns the
//      wave counts into starting rows.
constexpr int kMetaWaves = 16;
constexpr int kMetaChunk = kMetaWaves * 256;   // pairs per rank chunk: 4 per lane

// Expert ids of pairs p0 .. p0+3 from LDS; -1 past the end or out of range.
__device__ __forceinline__ void load_chunk_ids(const int* s_ids, int R, int E, int p0, int (&e)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int x = (p0 + i < R) ? s_ids[p0 + i] : -1;
    e[i] = ((unsigned)x < (unsigned)E) ? x : -1;
  }
}

// Visits each expert present among the wave's 256 pairs (lane l holds pairs
// 4l .. 4l+3 in order) once: fn(expert, pairs of that expert in the wave,
// rank[4]) where rank[i] counts the wave's earlier pairs of that expert
// (valid where e[i] is that expert).
template <class Fn>
__device__ __forceinline__ void wave_match4(const int (&e)[4], uint64_t lt_mask, Fn&& fn) {
  const int lane = threadIdx.x & 63;
  bool pend[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pend[i] = e[i] >= 0;
  while (true) {
    int mine = -1;
#pragma unroll
    for (int i = 3; i >= 0; --i)
      if (pend[i]) mine = e[i];
    const uint64_t any = __ballot(mine >= 0);
    if (!any) break;
    const int leader = __ffsll((unsigned long long)any) - 1;
    const int el = __builtin_amdgcn_readlane(mine, leader);
    uint64_t m[4];
    int n = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[i] = __ballot(e[i] == el);
      n += __popcll(m[i]);
    }
    int before = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) before += __popcll(m[i] & lt_mask);
    int r[4];
    int own = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = before + own;
      if (e[i] == el) {
        ++own;
        pend[i] = false;
      }
    }
    fn(el, n, r);
  }
}

__global__ __launch_bounds__(1024) void meta_kernel(int T, int E, int k, const int* __restrict__ ids,
                                                    int* __restrict__ counts, int* __restrict__ offsets,
                                                    int extra_rows, int* __restrict__ pair_to_row,
                                                    int* __restrict__ row_to_pair, int* __restrict__ tile_prefix,
                                                    int bm) {
  __shared__ int s_ids[kMetaMaxPairs];
  __shared__ int s_cnt[kMetaWaves * kMaxExperts];
  __shared__ int s_tot[kMaxExperts + 1];
  __shared__ int s_run[kMaxExperts];
  __shared__ int s_tmp[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int R = T * k;

  for (int x = tid; x < E; x += 1024) s_tot[x] = 0;
  for (int p = tid; p < R; p += 1024) s_ids[p] = ids[p];
  __syncthreads();

  // ---- counts, offsets, tile prefix.  Counts come from the same wave-level
  // matching as the ranks (one LDS add per wave and expert present).
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < R; c0 += kMetaChunk) {
    int e[4];
    load_chunk_ids(s_ids, R, E, c0 + wv * 256 + 4 * lane, e);
    wave_match4(e, lt_mask, [&](int el, int n, const int*) {
      if (lane == 0) atomicAdd(&s_tot[el], n);
    });
  }
  __syncthreads();
  const int cnt_e = (tid < E) ? s_tot[tid] : 0;
  const int total = block_exclusive_scan_1024(s_tot, s_tmp, E);
  if (tid < E) {
    counts[tid] = cnt_e;
    offsets[tid] = s_tot[tid];
    s_run[tid] = s_tot[tid];
  }
  if (tid == 0) {
    offsets[E] = total;
    if (extra_rows > 0) offsets[E + 1] = total + extra_rows;
  }
  if (tile_prefix) {
    const int G = E + (extra_rows > 0 ? 1 : 0);
    __syncthreads();                     // s_tot is reused for the tile counts
    const int rows = (tid < E) ? cnt_e : (tid == E ? extra_rows : 0);
    if (tid < G) s_tot[tid] = rows > 0 ? (rows + bm - 1) / bm : 0;
    __syncthreads();
    const int tiles = block_exclusive_scan_1024(s_tot, s_tmp, G);
    if (tid < G) tile_prefix[tid] = s_tot[tid];
    if (tid == 0) tile_prefix[G] = tiles;
  }
  __syncthreads();

  // ---- ranks, chunk by chunk of kMetaChunk pairs in pair order.  Lane l of
  // wave w owns pairs c0 + 256 w + 4 l + i (i < 4); inside the wave a pair's
  // rank among its expert's pairs comes from ballots, the per-expert wave
  // counts become starting rows by a scan over the 16 waves (16 lanes per
  // expert, shuffles), carried across chunks in s_run.
  int* my_cnt = s_cnt + wv * E;
  for (int c0 = 0; c0 < R; c0 += kMetaChunk) {
    for (int x = lane; x < E; x += 64) my_cnt[x] = 0;
    const int p0 = c0 + wv * 256 + 4 * lane;
    int e[4], rank[4] = {0, 0, 0, 0};
    load_chunk_ids(s_ids, R, E, p0, e);
    wave_match4(e, lt_mask, [&](int el, int n, const int* r) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e[i] == el) rank[i] = r[i];
      if (lane == 0) my_cnt[el] = n;
    });
    __syncthreads();
    for (int base = 0; base < E * kMetaWaves; base += 1024) {
      const int idx = base + tid;
      const int x = idx >> 4, q = idx & 15;    // expert, wave
      const int v = (x < E) ? s_cnt[q * E + x] : 0;
      int inc = v;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const int o = __shfl_up(inc, d, 16);
        if (q >= d) inc += o;
      }
      if (x < E) {
        const int run = s_run[x];
        s_cnt[q * E + x] = run + inc - v;
        if (q == 15) s_run[x] = run + inc;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + i;
      if (p < R) {
        const int row = e[i] >= 0 ? my_cnt[e[i]] + rank[i] : -1;
        pair_to_row[p] = row;
        if (row >= 0) row_to_pair[row] = p;
      }
    }
    __syncthreads();
  }
}

// meta_route_body: the same results as meta_kernel with routing, for at
// most kMetaRouteMaxT tokens, kMetaRouteMaxE experts and kMetaRouteMaxPairs
// pairs, in one workgroup of kMetaQuantThreads threads.  Tokens are cut into
// chunks of 64; wave w routes chunks w, w + W, ... one token per lane, and
// keeps each token's expert set as a bit mask.  A token picks distinct
// experts, so the rank of pair (t, j) among the pairs of its expert e is the
// number of earlier tokens that picked e: the pairs of e in the chunks
// before t's (a scan over the chunks) plus a popcount of the ballot of e
// over t's chunk below lane t % 64.
constexpr int kMetaQuantThreads = 1024;
constexpr int kMetaWavesR = kMetaQuantThreads / 64;
constexpr int kMetaRouteChunks = kMetaRouteMaxT / 64;
static_assert(kMetaRouteChunks <= 64, "one lane per token chunk in the chunk scan");

// Token t's logits, loaded without branches: a token past T reads the last
// row and an index past E reads the last logit (neither is used: the caller
// skips t >= T and the selection masks experts >= E).
template <int NE>
__device__ __forceinline__ void load_logits(const float* __restrict__ logits, int t, int T, int E, float (&v)[NE]) {
  const float* row = logits + (long)(t < T ? t : T - 1) * E;
#pragma unroll
  for (int i = 0; i < NE; ++i) v[i] = row[i < E ? i : E - 1];
}

// Routes D tokens per lane at once (t[d], live[d]: t[d] < T), the same
// selection and weight arithmetic as route_kernel: descending logit, equal
// logits by lower index, NaN below every number; w_j = e^(l_j - l_0) / sum
// (softmax) or sigmoid(l_j) / sum.  The D tokens' chains are independent, so
// their instructions interleave: one token's selection is a serial chain of
// compares and selects, latency-bound on its own.  Writes ids, w and the
// picks to s_ids for live tokens; returns each token's expert set as a mask.
template <int NE, int D>
__device__ __forceinline__ void route_tokens(const float (&raw)[D][NE], bool sigmoid, const int (&t)[D],
                                             const bool (&live)[D], int E, int k, int* __restrict__ ids,
                                             float* __restrict__ w, uint8_t* s_ids, uint32_t (&set)[D]) {
  float v[D][NE];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int i = 0; i < NE; ++i) v[d][i] = (raw[d][i] == raw[d][i]) ? raw[d][i] : -INFINITY;
  const uint32_t all = (E >= 32) ? 0xFFFFFFFFu : ((1u << E) - 1u);
  uint32_t avail[D];
  float vmax[D], sum[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    avail[d] = all;
    vmax[d] = 0.0f;
    sum[d] = 0.0f;
  }
  // the picks and the sum of their scores (ascending scan: a strictly larger
  // value replaces the pick, so equal values keep the lower index; the first
  // available expert is taken whatever its value, as every value may be
  // -inf); bitwise, without branches, so that the scan compiles to selects.
  // The loops over picks stay rolled: k is up to 32.
#pragma unroll 1
  for (int j = 0; j < k; ++j) {
    float bv[D];
    int bi[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      bv[d] = -INFINITY;
      bi[d] = -1;
    }
#pragma unroll
    for (int i = 0; i < NE; ++i)
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const bool take = (((avail[d] >> i) & 1u) != 0u) & ((v[d][i] > bv[d]) | (bi[d] < 0));
        bv[d] = take ? v[d][i] : bv[d];
        bi[d] = take ? i : bi[d];
      }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      avail[d] &= ~(1u << bi[d]);
      if (j == 0) vmax[d] = bv[d];
      sum[d] += sigmoid ? 1.0f / (1.0f + expf(-bv[d])) : expf(bv[d] - vmax[d]);
      if (live[d]) {
        ids[(long)t[d] * k + j] = bi[d];
        s_ids[t[d] * k + j] = (uint8_t)bi[d];
      }
    }
  }
  // the weights: each pick's value fetched again by its index
#pragma unroll 1
  for (int j = 0; j < k; ++j) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (!live[d]) continue;
      const int bi = s_ids[t[d] * k + j];
      float bv = v[d][0];
#pragma unroll
      for (int i = 1; i < NE; ++i) bv = (i == bi) ? v[d][i] : bv;
      const float ex = sigmoid ? 1.0f / (1.0f + expf(-bv)) : expf(bv - vmax[d]);
      w[(long)t[d] * k + j] = ex / sum[d];
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) set[d] = live[d] ? (all & ~avail[d]) : 0u;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// The LDS of the routing metadata: each pair's expert, each expert's ballot
// per token chunk, each expert's first row per chunk (relative to the
// expert's first row), and each expert's count and first row.
struct MetaRouteLds {
  uint8_t ids[kMetaRouteMaxPairs];
  uint64_t m[kMetaRouteMaxE][kMetaRouteChunks];
  int base[kMetaRouteMaxE][kMetaRouteChunks];
  int tot[kMetaRouteMaxE];
  int off[kMetaRouteMaxE];
};

// Routes chunks wave, wave + W, ... (D of them at a time, interleaved) and
// records each expert's ballot per chunk.
template <int NE, int D>
__device__ __forceinline__ void route_chunks(const float* __restrict__ logits, bool sigmoid, int T, int E, int k,
                                             int* __restrict__ ids, float* __restrict__ w, MetaRouteLds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = (T + 63) >> 6;
  constexpr int kCPW = kMetaRouteChunks / kMetaWavesR;   // chunks per wave, at most
#pragma unroll 1
  for (int i0 = 0; i0 < kCPW && wave + i0 * kMetaWavesR < nch; i0 += D) {
    float raw[D][NE];
    int t[D];
    bool live[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      t[d] = (wave + (i0 + d) * kMetaWavesR) * 64 + lane;
      live[d] = t[d] < T;
      load_logits<NE>(logits, t[d], T, E, raw[d]);
    }
    uint32_t set[D];
    route_tokens<NE, D>(raw, sigmoid, t, live, E, k, ids, w, L.ids, set);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int c = wave + (i0 + d) * kMetaWavesR;
      if (c < nch)
        for (int e = 0; e < E; ++e) {
          const uint64_t m = __ballot((set[d] >> e) & 1u);
          if (lane == 0) L.m[e][c] = m;
        }
    }
  }
}

// Run by all kMetaQuantThreads threads of a workgroup (it holds barriers).
__device__ __forceinline__ void meta_route_body(const float* __restrict__ logits, bool sigmoid, int T, int E, int k,
                                                int* __restrict__ ids, float* __restrict__ w,
                                                int* __restrict__ counts, int* __restrict__ offsets, int extra_rows,
                                                int* __restrict__ pair_to_row, int* __restrict__ row_to_pair,
                                                int* __restrict__ tile_prefix, int bm, MetaRouteLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (T + 63) >> 6;

  // ---- route; each expert's ballot over each chunk.  Up to one chunk per
  // wave one token per lane; beyond, several chunks interleaved per lane
  if (nch <= kMetaWavesR) {
    if (E <= 8) route_chunks<8, 1>(logits, sigmoid, T, E, k, ids, w, L);
    else if (E <= 16) route_chunks<16, 1>(logits, sigmoid, T, E, k, ids, w, L);
    else route_chunks<kMetaRouteMaxE, 1>(logits, sigmoid, T, E, k, ids, w, L);
  } else {
    if (E <= 8) route_chunks<8, 2>(logits, sigmoid, T, E, k, ids, w, L);
    else if (E <= 16) route_chunks<16, 2>(logits, sigmoid, T, E, k, ids, w, L);
    else route_chunks<kMetaRouteMaxE, 1>(logits, sigmoid, T, E, k, ids, w, L);
  }
  __syncthreads();

  // ---- per expert (one wave each): the chunk scan, lane c = chunk c
  for (int e = wave; e < E; e += kMetaWavesR) {
    const int v = (lane < nch) ? (int)__popcll(L.m[e][lane]) : 0;
    const int incl = wave_inclusive_scan(v);
    L.base[e][lane] = incl - v;
    if (lane == 63) L.tot[e] = incl;
  }
  __syncthreads();

  // ---- wave 0, lane e: count, offset (a scan over the lanes), tile prefix
  if (wave == 0) {
    const int cnt = (lane < E) ? L.tot[lane] : 0;
    const int incl = wave_inclusive_scan(cnt);
    const int total = __shfl(incl, E - 1, 64);
    if (lane < E) {
      counts[lane] = cnt;
      offsets[lane] = incl - cnt;
      L.off[lane] = incl - cnt;
    }
    if (lane == 0) {
      offsets[E] = total;
      if (extra_rows > 0) offsets[E + 1] = total + extra_rows;
    }
    if (tile_prefix) {
      const int G = E + (extra_rows > 0 ? 1 : 0);
      const int rows = (lane < E) ? cnt : (lane == E ? extra_rows : 0);
      const int tiles = (lane < G && rows > 0) ? (rows + bm - 1) / bm : 0;
      const int tincl = wave_inclusive_scan(tiles);
      if (lane < G) tile_prefix[lane] = tincl - tiles;
      if (lane == G - 1) tile_prefix[G] = tincl;
    }
  }
  __syncthreads();

  // ---- rows, in pair order (coalesced pair_to_row)
  const int R = T * k;
  for (int p = tid; p < R; p += kMetaQuantThreads) {
    const int t = p / k;
    const int e = L.ids[p];
    const int c = t >> 6, tl = t & 63;
    const uint64_t below = (tl == 0) ? 0ull : (~0ull >> (64 - tl));
    const int row = L.off[e] + L.base[e][c] + (int)__popcll(L.m[e][c] & below);
    pair_to_row[p] = row;
    row_to_pair[row] = p;
  }
}

// Quantises tokens t0 and t0 + 1 (if < T) into the K-blocked token-order
// rows with one workgroup of kMetaQuantThreads threads.  Piece q (8
// elements) of the pair: token (q >> 3) & 1, 64-byte chunk q >> 4, piece
// q & 7 of the chunk, so the 16 lanes writing one chunk of both tokens write
// one whole 128-byte line (the two tokens' chunks are adjacent).  A thread
// serves one token: its lanes' token bit does not change with the step j.
template <int CPT>
__device__ __forceinline__ void quant_token_pair(const uint16_t* __restrict__ x, int t0, int T, int H,
                                                 uint8_t* __restrict__ xq_tok, float* __restrict__ xs_tok,
                                                 long tok_cs) {
  __shared__ float red[2][kMetaQuantThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tt = (tid >> 3) & 1;
  const int t = t0 + tt;
  const bool live = t < T;
  const int nchk = H >> 3;                    // pieces per token
  uint4 in[CPT];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int q = tid + j * kMetaQuantThreads;
    const int idx = (q >> 4) * 8 + (q & 7);
    in[j] = (live && idx < nchk) ? *reinterpret_cast<const uint4*>(x + (long)t * H + (long)idx * 8)
                                 : make_uint4(0, 0, 0, 0);
    const uint32_t wds[4] = {in[j].x, in[j].y, in[j].z, in[j].w};
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(wds[qq])), fabsf(bf16_hi(wds[qq]))));
  }
  // the two tokens' maxima: lanes of token 0 and 1 alternate in groups of 8
  float m0 = wave_max(tt == 0 ? amax : 0.0f);
  float m1 = wave_max(tt == 1 ? amax : 0.0f);
  if (lane == 0) {
    red[0][wv] = m0;
    red[1][wv] = m1;
  }
  __syncthreads();
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < kMetaQuantThreads / 64; ++i) a = fmaxf(a, red[tt][i]);
  const float s = (a == 0.0f) ? 1.0f : a / kE4M3Max;
  const float r = e4m3_recip(s);
  if (!live) return;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int q = tid + j * kMetaQuantThreads;
    const int idx = (q >> 4) * 8 + (q & 7);
    if (idx >= nchk) continue;
    const uint32_t wds[4] = {in[j].x, in[j].y, in[j].z, in[j].w};
    *reinterpret_cast<uint2*>(xq_tok + code_offset(t, idx, H, tok_cs)) = e4m3_encode8(wds, s, r);
  }
  if ((tid & 15) == 8 * tt && tid < 16) xs_tok[t] = s;
}

// meta_quant_kernel: workgroup 0 computes the routing and its metadata
// (meta_route_body), workgroup 1 + i quantises tokens 2i and 2i + 1 into
// token order (quant_token_pair).  The
// metadata reads only the logits and the quantisation only x, so nothing
// waits across workgroups.  kMetaQuantThreads (1024) threads per workgroup:
// sixteen routing waves, four per SIMD to hide each other's dependent
// chains, with at most two chunks interleaved per lane so that a routing
// lane fits the 128 registers that many waves leave it (64 used).
template <int CPT>
__global__ __launch_bounds__(kMetaQuantThreads) void meta_quant_kernel(const float* __restrict__ logits, bool sigmoid,
                                                          const uint16_t* __restrict__ x, int T, int H, int E,
                                                          int k, int* __restrict__ ids, float* __restrict__ w,
                                                          int* __restrict__ counts, int* __restrict__ offsets,
                                                          int extra_rows, int* __restrict__ pair_to_row,
                                                          int* __restrict__ row_to_pair,
                                                          int* __restrict__ tile_prefix, int bm,
                                                          uint8_t* __restrict__ xq_tok, float* __restrict__ xs_tok,
                                                          long tok_cs) {
  if (blockIdx.x == 0) {
    __shared__ MetaRouteLds L;
    meta_route_body(logits, sigmoid, T, E, k, ids, w, counts, offsets, extra_rows, pair_to_row, row_to_pair,
                    tile_prefix, bm, L);
    return;
  }
  quant_token_pair<CPT>(x, 2 * ((int)blockIdx.x - 1), T, H, xq_tok, xs_tok, tok_cs);
}

// Expert-ordered, row-major copy of quantised rows from the token-order rows
// (K-blocked, tok_cs): row r holds token row_to_pair[r] / k.  One block per row.
__global__ __launch_bounds__(256) void rows_from_tokens_kernel(const uint8_t* __restrict__ xq_tok,
                                                               const float* __restrict__ xs_tok,
                                                               const int* __restrict__ row_to_pair, int k, int H,
                                                               long tok_cs, uint8_t* __restrict__ xq_rows,
                                                               float* __restrict__ xs_rows) {
  const long r = blockIdx.x;
  const long t = row_to_pair[r] / k;
  if (xq_rows)
    for (int idx = threadIdx.x; idx < (H >> 3); idx += blockDim.x)
      *reinterpret_cast<uint2*>(xq_rows + r * H + (long)idx * 8) =
          *reinterpret_cast<const uint2*>(xq_tok + code_offset(t, idx, H, tok_cs));
  if (xs_rows && threadIdx.x == 0) xs_rows[r] = xs_tok[t];
}

// K-blocked expert-ordered rows from the K-blocked token-order rows: 16
// bytes per thread, consecutive threads on consecutive bytes of the
// destination (chunk c of rows 0..R-1 is contiguous there), so the writes
// coalesce; each 64-byte chunk row of a token is read by 4 threads.
__global__ __launch_bounds__(256) void rows_kblocked_kernel(const uint8_t* __restrict__ xq_tok,
                                                            const float* __restrict__ xs_tok,
                                                            const int* __restrict__ row_to_pair, int k, long R,
                                                            long tok_cs, long n16, uint8_t* __restrict__ xq_rows,
                                                            float* __restrict__ xs_rows) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (long)gridDim.x * blockDim.x) {
    const long q = i & 3;                // 16-byte piece of the 64-byte chunk row
    const long rc = i >> 2;              // chunk c of row r: rc = c * R + r
    const long c = rc / R;
    const long r = rc - c * R;
    const long t = row_to_pair[r] / k;
    *reinterpret_cast<uint4*>(xq_rows + (rc << 6) + (q << 4)) =
        *reinterpret_cast<const uint4*>(xq_tok + c * tok_cs + (t << 6) + (q << 4));
    if (c == 0 && q == 0) xs_rows[r] = xs_tok[t];
  }
}

hipError_t launch_rows_kblocked(const uint8_t* xq_tok, const float* xs_tok, const int* row_to_pair, int T, int k,
                                int H, uint8_t* xq_rows, float* xs_rows, hipStream_t s) {
  const long R = (long)T * k;
  if (R == 0) return hipSuccess;
  const long n16 = R * (H / kTokChunk) * 4;
  long blocks = (n16 + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  rows_kblocked_kernel<<<(unsigned)blocks, 256, 0, s>>>(xq_tok, xs_tok, row_to_pair, k, R, (long)T * kTokChunk, n16,
                                                        xq_rows, xs_rows);
  return hipGetLastError();
}

hipError_t launch_rows_from_tokens(const uint8_t* xq_tok, const float* xs_tok, const int* row_to_pair, int T,
                                   int k, int H, uint8_t* xq_rows, float* xs_rows, hipStream_t s) {
  const long R = (long)T * k;
  if (R == 0 || (!xq_rows && !xs_rows)) return hipSuccess;
  rows_from_tokens_kernel<<<(unsigned)R, 256, 0, s>>>(xq_tok, xs_tok, row_to_pair, k, H, (long)T * kTokChunk,
                                                       xq_rows, xs_rows);
  return hipGetLastError();
}

// Threads per token-quantising workgroup and chunks of 8 elements per thread
// for a row of H elements (H a multiple of 128): at most max_threads, a
// multiple of 64.
static void quant_shape(int H, int max_threads, int* threads, int* cpt) {
  const int chunks = H / 8;
  int c = 1;
  while (chunks > max_threads * c) c *= 2;
  const int t = (chunks + c - 1) / c;
  *threads = ((t + 63) / 64) * 64;
  *cpt = c;
}

hipError_t launch_meta_quant(const float* logits, bool sigmoid, const uint16_t* x, int T, int H, int E, int k,
                             int* ids, float* w, int* counts, int* offsets, int extra_rows, int* pair_to_row,
                             int* row_to_pair, int* tile_prefix, int bm, uint8_t* xq_tok, float* xs_tok,
                             hipStream_t s, hipEvent_t ev_start) {
  if (T == 0) return hipSuccess;
  if (!logits || T > kMetaRouteMaxT || E > kMetaRouteMaxE || (long)T * k > kMetaRouteMaxPairs ||
      H > kMetaQuantMaxH)
    return hipErrorInvalidValue;
  // every workgroup has kMetaQuantThreads threads: the metadata workgroup
  // needs all of them, the quantising ones take CPT pieces of 8 elements of
  // a token pair per thread
  int threads = 64, cpt = 1;
  quant_shape(2 * H, kMetaQuantThreads, &threads, &cpt);
  threads = kMetaQuantThreads;
  const long tok_cs = (long)T * kTokChunk;
  const unsigned grid = 1 + (unsigned)((T + 1) / 2);
#define MOE_MQ(C)                                                                                           \
  hipExtLaunchKernelGGL(meta_quant_kernel<C>, dim3(grid), dim3(threads), 0, s, ev_start, nullptr, 0, logits, \
                        sigmoid, x, T, H, E, k, ids, w, counts, offsets, extra_rows, pair_to_row, row_to_pair,  \
                        tile_prefix, bm, xq_tok, xs_tok, tok_cs)
  static_assert(2 * kMetaQuantMaxH / 8 <= 8 * kMetaQuantThreads, "a token pair takes at most 8 pieces per thread");
  switch (cpt) {
    case 1: MOE_MQ(1); break;
    case 2: MOE_MQ(2); break;
    case 4: MOE_MQ(4); break;
    default: MOE_MQ(8); break;   // H up to kMetaQuantMaxH
  }
#undef MOE_MQ
  return hipGetLastError();
}

hipError_t launch_counts(const int* ids, int pairs, int E, int* chunk_hist, int* chunk_base,
                         int* counts, int* offsets, int extra_rows, hipStream_t s) {
  const int chunks = permute_chunks(pairs);
  if (chunks > 0) hist_kernel<<<chunks, 256, 0, s>>>(ids, pairs, E, chunk_hist);
  scan_kernel<<<1, 1024, 0, s>>>(chunk_hist, chunks, E, chunk_base, counts, offsets, extra_rows);
  return hipGetLastError();
}

hipError_t launch_rank(const int* ids, int pairs, int E, const int* chunk_base, int* pair_to_row,
                       int* row_to_pair, hipStream_t s) {
  const int chunks = permute_chunks(pairs);
  if (chunks > 0)
    rank_kernel<<<chunks, 256, 0, s>>>(ids, pairs, E, chunk_base, pair_to_row, row_to_pair);
  return hipGetLastError();
}

hipError_t launch_quant_scatter(const uint16_t* x, int T, int H, int k, const int* pair_to_row,
                                uint8_t* xq_rows, float* xs_rows, uint8_t* xq_tok, float* xs_tok,
                                bool blocked, uint8_t* xq_copy, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const long rows_cs = blocked ? (long)T * k * kTokChunk : 0;
  const long tok_cs = blocked ? (long)T * kTokChunk : 0;
  int threads = 64, cpt = 1;
  quant_shape(H, 1024, &threads, &cpt);
#define MOE_QS(C)                                                                          \
  quant_scatter_kernel<C><<<T, threads, 0, s>>>(x, H, k, pair_to_row, xq_rows, xs_rows, xq_tok, \
                                                xs_tok, rows_cs, tok_cs, xq_copy)
  switch (cpt) {
    case 1: MOE_QS(1); break;
    case 2: MOE_QS(2); break;
    case 4: MOE_QS(4); break;
    default: MOE_QS(8); break;
  }
#undef MOE_QS
  return hipGetLastError();
}

hipError_t launch_meta(int T, int E, int k, const int* ids, int* counts, int* offsets, int extra_rows,
                       int* pair_to_row, int* row_to_pair, int* tile_prefix, int bm, hipStream_t s) {
  meta_kernel<<<1, 1024, 0, s>>>(T, E, k, ids, counts, offsets, extra_rows, pair_to_row, row_to_pair,
                                 tile_prefix, bm);
  return hipGetLastError();
}

}  // namespace moe
