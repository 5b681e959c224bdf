// C ABI of the routed MoE layer: argument validation, workspace carve-up and
// launch sequencing.  Validation runs on the host before anything is
// enqueued and touches no device state, so every error path can be exercised
// without a GPU.  See include/moe.h for the contract of each entry point.
// the C ABI is the library's only exported interface (built with hidden
// visibility otherwise)
#pragma GCC visibility push(default)
#include "../../include/moe.h"
#pragma GCC visibility pop

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status_t ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status_t device_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxDim = 65536;

// Validation helpers return MOE_OK or the first failing status.
#define MOE_CHECK(expr)                 \
  do {                                  \
    const moe_status_t st_ = (expr);    \
    if (st_ != MOE_OK) return st_;      \
  } while (0)

moe_status_t need(const void* p, const char* name) {
  if (!p) return fail(MOE_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

moe_status_t opt(const void* p, const char* name) {
  if (p && !aligned16(p)) return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

moe_status_t check_route_shape(int32_t T, int32_t E, int32_t k) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T = %d < 0", T);
  if (E < 1 || E > moe::kMaxExperts) return fail(MOE_ERR_SHAPE, "E = %d outside [1, %d]", E, moe::kMaxExperts);
  if (k < 1 || k > E || k > moe::kMaxTopK)
    return fail(MOE_ERR_SHAPE, "top_k = %d outside [1, min(E=%d, %d)]", k, E, moe::kMaxTopK);
  if ((int64_t)T * k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "T * top_k overflows int32");
  return MOE_OK;
}

moe_status_t check_score(int32_t score) {
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_UNSUPPORTED, "unknown router score function %d", score);
  return MOE_OK;
}

moe_status_t check_dim(int32_t v, const char* name) {
  if (v < 128 || v > kMaxDim || v % 128 != 0)
    return fail(MOE_ERR_SHAPE, "%s = %d is not a multiple of 128 in [128, %d]", name, v, kMaxDim);
  return MOE_OK;
}

moe_status_t check_weights(const moe_weights_t* w, const char* name) {
  if (!w) return fail(MOE_ERR_NULL, "%s is NULL", name);
  if (w->fmt != MOE_W_FP8_E4M3_PERCHANNEL && w->fmt != MOE_W_MXFP4_E2M1_E8M0_G32 &&
      w->fmt != MOE_W_FP8_E4M3_BLOCK128)
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown weight format %d", name, w->fmt);
  if (w->n_experts < 1 || w->n_experts > moe::kMaxExperts)
    return fail(MOE_ERR_SHAPE, "%s: n_experts = %d outside [1, %d]", name, w->n_experts, moe::kMaxExperts);
  MOE_CHECK(check_dim(w->hidden, "hidden"));
  MOE_CHECK(check_dim(w->inter, "inter"));
  if (w->layout != MOE_LAYOUT_ROW_MAJOR && w->layout != MOE_LAYOUT_K_BLOCKED)
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown weight layout %d", name, w->layout);
  if (w->reserved != 0) return fail(MOE_ERR_SHAPE, "%s: reserved field must be 0", name);
  if (w->activation != MOE_ACT_SILU && w->activation != MOE_ACT_SITU)
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown activation %d", name, w->activation);
  if (w->activation == MOE_ACT_SITU && !(w->act_beta > 0.0f && w->act_beta <= 3.0e38f))
    return fail(MOE_ERR_SHAPE, "%s: SiTU needs a finite act_beta > 0", name);
  MOE_CHECK(need(w->w1, "w1"));
  MOE_CHECK(need(w->w3, "w3"));
  MOE_CHECK(need(w->w2, "w2"));
  MOE_CHECK(need(w->s1, "s1"));
  MOE_CHECK(need(w->s3, "s3"));
  MOE_CHECK(need(w->s2, "s2"));
  return MOE_OK;
}

// Bump allocator over the caller's workspace: 256-byte aligned slices.
struct Carve {
  uint8_t* base;
  size_t used = 0;
  explicit Carve(void* b) : base(static_cast<uint8_t*>(b)) {}
  template <class T>
  T* take(size_t count) {
    used = (used + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

// tile_prefix[0..n_groups] serves the gate-up GEMM, the next n_groups + 1
// entries the down GEMM when it takes another row-tile height, the last two a
// gate-up launch of the shared group alone.
size_t ffn_ws(Carve& c, long n_rows, int n_groups, int inter, int32_t** tile_prefix, uint16_t** h) {
  *tile_prefix = c.take<int32_t>(2 * (n_groups + 1) + 2);
  *h = c.take<uint16_t>((size_t)n_rows * inter);
  return c.used;
}

moe::FfnGroups make_groups(const moe_weights_t* r, const moe_weights_t* sh, const int32_t* offsets) {
  moe::FfnGroups g{};
  g.fmt = r->fmt == MOE_W_MXFP4_E2M1_E8M0_G32 ? moe::kMxfp4
          : r->fmt == MOE_W_FP8_E4M3_BLOCK128   ? moe::kFp8Block
                                                : moe::kFp8;
  g.n_routed = r->n_experts;
  g.n_groups = r->n_experts + (sh ? 1 : 0);
  g.hidden = r->hidden;
  g.inter = r->inter;
  g.offsets = offsets;
  const moe_weights_t* src[2] = {r, sh ? sh : r};
  for (int i = 0; i < 2; ++i) {
    g.act[i] = src[i]->activation == MOE_ACT_SITU ? moe::kActSitu : moe::kActSilu;
    g.beta[i] = src[i]->act_beta;
    g.w1[i] = src[i]->w1;
    g.w3[i] = src[i]->w3;
    g.w2[i] = src[i]->w2;
    g.s1[i] = src[i]->s1;
    g.s3[i] = src[i]->s3;
    g.s2[i] = src[i]->s2;
    g.blocked[i] = src[i]->layout == MOE_LAYOUT_K_BLOCKED;
  }
  return g;
}

// GEMM1 -> GEMM2 over the groups of `g`.
// tile_prefix_ready: the tile prefix for this variant is already in place
// (the metadata kernel computed it).
moe_status_t run_ffn(const moe::FfnGroups& g, const moe::RowOperand& x, long n_rows, float* y,
                     int32_t* tile_prefix, uint16_t* h, hipStream_t s, void* const* events,
                     char* variant_out, size_t variant_len, bool tile_prefix_ready = false,
                     void* const* gemm1_events = nullptr, void* const* gemm2_events = nullptr) {
  const int variant = moe::choose_variant(g, n_rows);
  const int variant2 = moe::choose_down_variant(g, n_rows);
  const long shared_rows = g.n_groups > g.n_routed ? n_rows - x.shared_row0 : 0;
  const int variant_sh = moe::shared_gate_up_variant(g, n_rows, shared_rows);
  // the down GEMM's tile prefix, when its tiles have another height, and
  // that of the shared group's own gate-up launch
  int32_t* tile_prefix2 = variant2 == variant ? tile_prefix : tile_prefix + g.n_groups + 1;
  int32_t* tile_prefix_sh = tile_prefix + 2 * (g.n_groups + 1);
  if (variant_out) {
    snprintf(variant_out, variant_len, "%s/%s", moe::variant_name(variant), g.fmt == moe::kMxfp4 ? "mxfp4" : "fp8");
    size_t used = strlen(variant_out);
    if (variant2 != variant)
      snprintf(variant_out + used, variant_len - used, "/down:%s", moe::variant_name(variant2));
    used = strlen(variant_out);
    if (variant_sh >= 0)
      snprintf(variant_out + used, variant_len - used, "/shared:%s", moe::variant_name(variant_sh));
  }
  hipError_t e = hipSuccess;
  if (!tile_prefix_ready) {
    e = moe::launch_tile_prefix(g.offsets, g.n_groups, moe::variant_rows(variant), tile_prefix, s);
    if (e != hipSuccess) return device_status(e, "tile_prefix");
  }
  if (variant2 != variant) {
    e = moe::launch_tile_prefix(g.offsets, g.n_groups, moe::variant_rows(variant2), tile_prefix2, s);
    if (e != hipSuccess) return device_status(e, "tile_prefix");
  }
  // the shared group alone: group 0 of a launch whose offsets start at its own
  moe::FfnGroups g_sh = g;
  if (variant_sh >= 0) {
    g_sh.offsets = g.offsets + g.n_routed;
    g_sh.n_groups = 1;
    g_sh.n_routed = 0;
    e = moe::launch_tile_prefix(g_sh.offsets, 1, moe::variant_rows(variant_sh), tile_prefix_sh, s);
    if (e != hipSuccess) return device_status(e, "tile_prefix");
  }
  if (events && events[MOE_STAGE_GEMM1]) hipEventRecord((hipEvent_t)events[MOE_STAGE_GEMM1], s);
  hipEvent_t g1_start = gemm1_events ? (hipEvent_t)gemm1_events[0] : nullptr;
  hipEvent_t g1_stop = gemm1_events ? (hipEvent_t)gemm1_events[1] : nullptr;
  if (variant_sh >= 0) {
    moe::FfnGroups g_routed = g;
    g_routed.n_groups = g.n_routed;
    e = moe::launch_gemm1(variant, g_routed, x, tile_prefix, n_rows, h, s, g1_start, nullptr, x.shared_row0);
    if (e == hipSuccess)
      e = moe::launch_gemm1(variant_sh, g_sh, x, tile_prefix_sh, n_rows, h, s, nullptr, g1_stop, shared_rows);
  } else {
    e = moe::launch_gemm1(variant, g, x, tile_prefix, n_rows, h, s, g1_start, g1_stop);
  }
  if (e != hipSuccess) return device_status(e, "gemm1");
  if (events && events[MOE_STAGE_GEMM2]) hipEventRecord((hipEvent_t)events[MOE_STAGE_GEMM2], s);
  e = moe::launch_gemm2(variant2, g, h, tile_prefix2, n_rows, y, s,
                        gemm2_events ? (hipEvent_t)gemm2_events[0] : nullptr,
                        gemm2_events ? (hipEvent_t)gemm2_events[1] : nullptr);
  if (e != hipSuccess) return device_status(e, "gemm2");
  return ok();
}

}  // namespace

extern "C" {

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "the workspace is too small";
    case MOE_ERR_UNSUPPORTED: return "no kernel exists for this case";
    case MOE_ERR_DEVICE: return "the HIP runtime reported an error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------
moe_status_t moe_route(const float* logits, int32_t T, int32_t E, int32_t top_k, int32_t score,
                       int32_t* topk_ids, float* topk_w, void* stream) {
  MOE_CHECK(check_route_shape(T, E, top_k));
  MOE_CHECK(check_score(score));
  if (T == 0) return ok();
  MOE_CHECK(need(logits, "logits"));
  MOE_CHECK(need(topk_ids, "topk_ids"));
  MOE_CHECK(need(topk_w, "topk_w"));
  return device_status(moe::launch_route(logits, T, E, top_k, score == MOE_SCORE_SIGMOID, topk_ids, topk_w,
                                         (hipStream_t)stream),
                       "route");
}

// ---------------------------------------------------------------------------
size_t moe_permute_workspace_size(int32_t T, int32_t top_k, int32_t E) {
  if (T < 0 || top_k < 1 || E < 1) return 0;
  Carve c(nullptr);
  const long chunks = moe::permute_chunks((long)T * top_k);
  c.take<int32_t>(chunks * E);
  c.take<int32_t>(chunks * E);
  return c.used + 256;
}

moe_status_t moe_permute(const uint16_t* x, int32_t T, int32_t H, const int32_t* topk_ids,
                         int32_t top_k, int32_t E, int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* pair_to_row, int32_t* row_to_pair, uint8_t* xq_rows, float* xs_rows,
                         uint8_t* xq_tok, float* xs_tok, void* ws, size_t ws_bytes, void* stream) {
  MOE_CHECK(check_route_shape(T, E, top_k));
  MOE_CHECK(check_dim(H, "H"));
  MOE_CHECK(need(expert_counts, "expert_counts"));
  MOE_CHECK(need(expert_offsets, "expert_offsets"));
  if ((xq_tok == nullptr) != (xs_tok == nullptr))
    return fail(MOE_ERR_NULL, "xq_tok and xs_tok must both be set or both be NULL");
  if (T > 0) {
    MOE_CHECK(need(x, "x"));
    MOE_CHECK(need(topk_ids, "topk_ids"));
    MOE_CHECK(need(pair_to_row, "pair_to_row"));
    MOE_CHECK(need(row_to_pair, "row_to_pair"));
    MOE_CHECK(need(xq_rows, "xq_rows"));
    MOE_CHECK(need(xs_rows, "xs_rows"));
    MOE_CHECK(opt(xq_tok, "xq_tok"));
    MOE_CHECK(opt(xs_tok, "xs_tok"));
  }
  const size_t need_ws = moe_permute_workspace_size(T, top_k, E);
  if (!ws || ws_bytes < need_ws)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu B < %zu B", ws ? ws_bytes : 0, need_ws);
  MOE_CHECK(need(ws, "ws"));
  hipStream_t s = (hipStream_t)stream;
  const long pairs = (long)T * top_k;
  const long chunks = moe::permute_chunks(pairs);
  Carve c(ws);
  int32_t* hist = c.take<int32_t>(chunks * E);
  int32_t* base = c.take<int32_t>(chunks * E);
  hipError_t e;
  if (T > 0 && pairs <= moe::kMetaMaxPairs && E <= moe::kMetaMaxE) {
    // reads topk_ids only (no logits): the const is not written through
    e = moe::launch_meta(T, E, top_k, topk_ids, expert_counts, expert_offsets, 0, pair_to_row, row_to_pair, nullptr,
                         0, s);
    if (e != hipSuccess) return device_status(e, "meta");
  } else {
    e = moe::launch_counts(topk_ids, (int)pairs, E, hist, base, expert_counts, expert_offsets, 0, s);
    if (e != hipSuccess) return device_status(e, "counts");
    if (T == 0) return ok();
    e = moe::launch_rank(topk_ids, (int)pairs, E, base, pair_to_row, row_to_pair, s);
    if (e != hipSuccess) return device_status(e, "rank");
  }
  e = moe::launch_quant_scatter(x, T, H, top_k, pair_to_row, xq_rows, xs_rows, xq_tok, xs_tok, false,
                                nullptr, s);
  return device_status(e, "quant_scatter");
}

// ---------------------------------------------------------------------------
size_t moe_expert_ffn_workspace_size(int32_t n_rows, const moe_weights_t* w) {
  if (!w || n_rows < 0 || w->n_experts < 1 || w->inter < 1) return 0;
  Carve c(nullptr);
  int32_t* tp;
  uint16_t* h;
  return ffn_ws(c, n_rows, w->n_experts, w->inter, &tp, &h) + 256;
}

moe_status_t moe_expert_ffn(const uint8_t* xq_rows, const float* xs_rows, int32_t n_rows,
                            const int32_t* expert_offsets, const moe_weights_t* w, float* y_rows,
                            void* ws, size_t ws_bytes, void* stream) {
  MOE_CHECK(check_weights(w, "weights"));
  if (n_rows < 0) return fail(MOE_ERR_SHAPE, "n_rows = %d < 0", n_rows);
  if (n_rows == 0) return ok();
  MOE_CHECK(need(xq_rows, "xq_rows"));
  MOE_CHECK(need(xs_rows, "xs_rows"));
  MOE_CHECK(need(expert_offsets, "expert_offsets"));
  MOE_CHECK(need(y_rows, "y_rows"));
  const size_t need_ws = moe_expert_ffn_workspace_size(n_rows, w);
  if (!ws || ws_bytes < need_ws)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu B < %zu B", ws ? ws_bytes : 0, need_ws);
  MOE_CHECK(need(ws, "ws"));
  Carve c(ws);
  int32_t* tp;
  uint16_t* h;
  ffn_ws(c, n_rows, w->n_experts, w->inter, &tp, &h);
  const moe::FfnGroups g = make_groups(w, nullptr, expert_offsets);
  const moe::Operand rm = moe::row_major_operand(w->hidden);
  moe::RowOperand x{{xq_rows, xq_rows}, {xs_rows, xs_rows}, (long)n_rows, {rm, rm}};
  return run_ffn(g, x, n_rows, y_rows, tp, h, (hipStream_t)stream, nullptr, nullptr, 0);
}

// ---------------------------------------------------------------------------
moe_status_t moe_combine(const float* y_rows, const int32_t* pair_to_row, const float* topk_w,
                         int32_t T, int32_t H, int32_t top_k, const float* y_shared,
                         const float* norm_gamma, float norm_eps, uint16_t* out, void* stream) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T = %d < 0", T);
  if (top_k < 1 || top_k > moe::kMaxTopK) return fail(MOE_ERR_SHAPE, "top_k = %d outside [1, %d]", top_k, moe::kMaxTopK);
  MOE_CHECK(check_dim(H, "H"));
  if (norm_gamma && !(norm_eps >= 0.0f)) return fail(MOE_ERR_SHAPE, "norm_eps must be >= 0");
  if (T == 0) return ok();
  MOE_CHECK(need(y_rows, "y_rows"));
  MOE_CHECK(need(pair_to_row, "pair_to_row"));
  MOE_CHECK(need(topk_w, "topk_w"));
  MOE_CHECK(need(out, "out"));
  MOE_CHECK(opt(y_shared, "y_shared"));
  MOE_CHECK(opt(norm_gamma, "norm_gamma"));
  return device_status(moe::launch_combine(y_rows, pair_to_row, topk_w, T, H, top_k, y_shared, norm_gamma,
                                           norm_eps, out, (hipStream_t)stream),
                       "combine");
}

// ---------------------------------------------------------------------------
struct ForwardLayout {
  int32_t *ids, *counts, *offsets, *p2r, *r2p, *hist, *base, *tile_prefix;
  float *w, *xs_rows, *xs_tok;
  uint8_t *xq_rows, *xq_tok;
  uint16_t* h;
  float* y_rows;
  size_t bytes;
};

// Up to kMetaMaxPairs pairs and kMetaMaxE experts, one workgroup computes
// the whole routing metadata.  For at most kMetaRouteMaxE experts (each
// token's expert set is a 32-bit mask), kMetaRouteMaxT tokens and
// kMetaRouteMaxPairs pairs it also routes, in the same launch as the
// quantisation (beyond that one CU's routing takes longer than a grid-wide
// router launch).  Beyond kMetaMaxPairs pairs or kMetaMaxE experts, route /
// counts / ranks run as grid-wide kernels.
static bool meta_path(int32_t T, int32_t k, int32_t E) {
  return (long)T * k <= moe::kMetaMaxPairs && E <= moe::kMetaMaxE;
}
// The one-launch path's gate-up GEMM reads token-order rows: gathered
// through row_to_pair by the register-fed kernels up to kGatherSmallMaxT
// tokens, beyond that (and always for the large kernels) from an
// expert-ordered copy.
constexpr int32_t kGatherSmallMaxT = 256;
static bool fused_route_path(int32_t T, int32_t k, const moe_weights_t* routed) {
  const int32_t E = routed->n_experts, H = routed->hidden;
  return meta_path(T, k, E) && E <= moe::kMetaRouteMaxE && T <= moe::kMetaRouteMaxT &&
         (long)T * k <= moe::kMetaRouteMaxPairs && H <= moe::kMetaQuantMaxH;
}
// On the one-launch routing path the large kernels read expert-ordered rows
// that a copy kernel writes from the token-order rows: their direct-to-LDS
// loads of gathered rows fetch scattered 64-byte half lines, which cost the
// 256-row gate-up GEMM about 40 us on the 2048-token prefill share, against
// about 10 us for the copy.  The register-fed kernels gather their token
// fragments for little cost at decode sizes but not beyond (+100 us on the
// 2048-token per-block fp8 share), so past kGatherSmallMaxT tokens they too
// read the copy.
static bool fused_rows_copied(int32_t T, int32_t k, const moe_weights_t* routed, bool shared) {
  if (!fused_route_path(T, k, routed)) return false;
  if (T > kGatherSmallMaxT) return true;
  const moe::FfnGroups g = make_groups(routed, shared ? routed : nullptr, nullptr);
  return !moe::variant_in_registers(moe::choose_variant(g, (long)T * k + (shared ? T : 0)));
}

static ForwardLayout forward_layout(void* ws, int32_t T, int32_t k, const moe_weights_t* routed, bool shared) {
  ForwardLayout L{};
  Carve c(ws);
  const int32_t E = routed->n_experts, H = routed->hidden, I = routed->inter;
  const long R = (long)T * k;
  // the fused routing path keeps the quantised tokens in token order only
  // (the gate-up GEMM gathers each routed row's token); the other paths
  // scatter them to expert-ordered rows, and keep token order for the
  // shared expert
  const bool fused = fused_route_path(T, k, routed);
  const bool rows_needed = !fused || fused_rows_copied(T, k, routed, shared);
  const long rows = R + (shared ? T : 0);
  const long chunks = moe::permute_chunks(R);
  L.ids = c.take<int32_t>(R);
  L.w = c.take<float>(R);
  L.counts = c.take<int32_t>(E);
  L.offsets = c.take<int32_t>(E + 2);
  L.p2r = c.take<int32_t>(R);
  L.r2p = c.take<int32_t>(R);
  L.hist = c.take<int32_t>(chunks * E);
  L.base = c.take<int32_t>(chunks * E);
  L.xq_rows = rows_needed ? c.take<uint8_t>((size_t)R * H) : nullptr;
  L.xs_rows = rows_needed ? c.take<float>(R) : nullptr;
  L.xq_tok = (shared || fused) ? c.take<uint8_t>((size_t)T * H) : nullptr;
  L.xs_tok = (shared || fused) ? c.take<float>(T) : nullptr;
  L.y_rows = c.take<float>((size_t)rows * H);
  ffn_ws(c, rows, E + (shared ? 1 : 0), I, &L.tile_prefix, &L.h);
  L.bytes = c.used + 256;
  return L;
}

size_t moe_forward_workspace_size(int32_t T, int32_t top_k, const moe_weights_t* routed, int32_t use_shared) {
  if (!routed || T < 0 || top_k < 1 || routed->n_experts < 1) return 0;
  return forward_layout(nullptr, T, top_k, routed, use_shared != 0)
      .bytes;
}

}  // extern "C"

// moe_forward's argument checks other than the workspace (host only).
static moe_status_t check_forward(const uint16_t* x, const float* logits, int32_t T, int32_t top_k, int32_t score,
                                  const moe_weights_t* routed, int32_t use_shared, const moe_weights_t* shared,
                                  const float* norm_gamma, float norm_eps, uint16_t* out, const moe_debug_t* dbg) {
  MOE_CHECK(check_weights(routed, "routed"));
  const int32_t E = routed->n_experts, H = routed->hidden, I = routed->inter;
  MOE_CHECK(check_route_shape(T, E, top_k));
  MOE_CHECK(check_score(score));
  if (use_shared) {
    MOE_CHECK(check_weights(shared, "shared"));
    if (shared->n_experts != 1) return fail(MOE_ERR_SHAPE, "shared expert must have n_experts = 1");
    if (shared->hidden != H || shared->inter != I)
      return fail(MOE_ERR_UNSUPPORTED, "shared expert shape %dx%d differs from routed %dx%d",
                  shared->hidden, shared->inter, H, I);
    if (shared->fmt != MOE_W_FP8_E4M3_PERCHANNEL)
      return fail(MOE_ERR_UNSUPPORTED, "shared expert must use per-channel fp8 weights");
    if (E + 1 > moe::kMaxExperts)
      return fail(MOE_ERR_UNSUPPORTED, "with a shared expert E must be at most %d", moe::kMaxExperts - 1);
  }
  if (norm_gamma && !(norm_eps >= 0.0f)) return fail(MOE_ERR_SHAPE, "norm_eps must be >= 0");
  if (T == 0) return ok();
  MOE_CHECK(need(x, "x"));
  MOE_CHECK(need(logits, "logits"));
  MOE_CHECK(need(out, "out"));
  MOE_CHECK(opt(norm_gamma, "norm_gamma"));
  if (dbg) {
    MOE_CHECK(opt(dbg->topk_ids, "dbg.topk_ids"));
    MOE_CHECK(opt(dbg->topk_w, "dbg.topk_w"));
    MOE_CHECK(opt(dbg->expert_counts, "dbg.expert_counts"));
    MOE_CHECK(opt(dbg->expert_offsets, "dbg.expert_offsets"));
    MOE_CHECK(opt(dbg->pair_to_row, "dbg.pair_to_row"));
    MOE_CHECK(opt(dbg->row_to_pair, "dbg.row_to_pair"));
    MOE_CHECK(opt(dbg->xq_rows, "dbg.xq_rows"));
    MOE_CHECK(opt(dbg->xs_rows, "dbg.xs_rows"));
  }
  return ok();
}

extern "C" {

moe_status_t moe_forward(const uint16_t* x, const float* logits, int32_t T, int32_t top_k,
                         int32_t score, const moe_weights_t* routed, int32_t use_shared, const moe_weights_t* shared,
                         const float* norm_gamma, float norm_eps, uint16_t* out, moe_debug_t* dbg,
                         void* ws, size_t ws_bytes, void* stream) {
  MOE_CHECK(check_forward(x, logits, T, top_k, score, routed, use_shared, shared, norm_gamma, norm_eps, out, dbg));
  if (T == 0) return ok();
  const int32_t E = routed->n_experts, H = routed->hidden;
  const bool sigmoid = score == MOE_SCORE_SIGMOID;
  const bool sh = use_shared != 0;
  const size_t need_ws = moe_forward_workspace_size(T, top_k, routed, use_shared);
  if (!ws || ws_bytes < need_ws)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu B < %zu B", ws ? ws_bytes : 0, need_ws);
  MOE_CHECK(need(ws, "ws"));

  ForwardLayout L = forward_layout(ws, T, top_k, routed, sh);
  void* const* ev = dbg ? dbg->events : nullptr;
  if (dbg) {
    if (dbg->topk_ids) L.ids = dbg->topk_ids;
    if (dbg->topk_w) L.w = dbg->topk_w;
    if (dbg->expert_counts) L.counts = dbg->expert_counts;
    if (dbg->expert_offsets) L.offsets = dbg->expert_offsets;
    if (dbg->pair_to_row) L.p2r = dbg->pair_to_row;
    if (dbg->row_to_pair) L.r2p = dbg->row_to_pair;
    if (dbg->xs_rows && L.xs_rows) L.xs_rows = dbg->xs_rows;
  }
  hipStream_t s = (hipStream_t)stream;
  const long R = (long)T * top_k;
  hipError_t e;

  const moe::FfnGroups g = make_groups(routed, sh ? shared : nullptr, L.offsets);
  const long rows = R + (sh ? T : 0);
  const bool meta = meta_path(T, top_k, E);
  const bool fused_route = fused_route_path(T, top_k, routed);
  if (ev && ev[MOE_STAGE_ROUTE]) hipEventRecord((hipEvent_t)ev[MOE_STAGE_ROUTE], s);
  // the layer's first dispatch (router, or the fused routing + quantisation
  // kernel) and its last (combine) stamp the optional layer events
  const hipEvent_t lev0 = dbg ? (hipEvent_t)dbg->layer_events[0] : nullptr;
  const hipEvent_t lev1 = dbg ? (hipEvent_t)dbg->layer_events[1] : nullptr;
  const moe::Operand rows_d = moe::k_blocked_operand(R, moe::kTokChunk);
  const moe::Operand tok_d = moe::k_blocked_operand(T, moe::kTokChunk);
  moe::RowOperand xr{{L.xq_rows, sh ? L.xq_tok : L.xq_rows}, {L.xs_rows, sh ? L.xs_tok : L.xs_rows}, R,
                     {rows_d, sh ? tok_d : rows_d}};
  if (fused_route) {
    // routing, metadata and the token-order quantisation in one launch; the
    // gate-up GEMM gathers each routed row's token through row_to_pair
    if (ev && ev[MOE_STAGE_PERMUTE]) hipEventRecord((hipEvent_t)ev[MOE_STAGE_PERMUTE], s);
    const int bm = moe::variant_rows(moe::choose_variant(g, rows));
    e = moe::launch_meta_quant(logits, sigmoid, x, T, H, E, top_k, L.ids, L.w, L.counts, L.offsets, sh ? T : 0,
                               L.p2r, L.r2p, L.tile_prefix, bm, L.xq_tok, L.xs_tok, s, lev0);
    if (e != hipSuccess) return device_status(e, "meta_quant");
    if (dbg && (dbg->xq_rows || dbg->xs_rows)) {   // the expert-ordered rows, for inspection
      e = moe::launch_rows_from_tokens(L.xq_tok, L.xs_tok, L.r2p, T, top_k, H, dbg->xq_rows, dbg->xs_rows, s);
      if (e != hipSuccess) return device_status(e, "rows_from_tokens");
    }
    if (fused_rows_copied(T, top_k, routed, sh)) {
      e = moe::launch_rows_kblocked(L.xq_tok, L.xs_tok, L.r2p, T, top_k, H, L.xq_rows, L.xs_rows, s);
      if (e != hipSuccess) return device_status(e, "rows_kblocked");
      xr = moe::RowOperand{{L.xq_rows, sh ? L.xq_tok : L.xq_rows}, {L.xs_rows, sh ? L.xs_tok : L.xs_rows}, R,
                           {rows_d, sh ? tok_d : rows_d}};
    } else {
      xr = moe::RowOperand{{L.xq_tok, L.xq_tok}, {L.xs_tok, L.xs_tok}, R, {tok_d, tok_d}};
      xr.gather = L.r2p;
      xr.gather_k = top_k;
    }
  } else {
    e = moe::launch_route(logits, T, E, top_k, sigmoid, L.ids, L.w, s, lev0);
    if (e != hipSuccess) return device_status(e, "route");
    if (ev && ev[MOE_STAGE_PERMUTE]) hipEventRecord((hipEvent_t)ev[MOE_STAGE_PERMUTE], s);
    if (meta) {
      const int bm = moe::variant_rows(moe::choose_variant(g, rows));
      e = moe::launch_meta(T, E, top_k, L.ids, L.counts, L.offsets, sh ? T : 0, L.p2r, L.r2p, L.tile_prefix, bm, s);
      if (e != hipSuccess) return device_status(e, "meta");
    } else {
      e = moe::launch_counts(L.ids, (int)R, E, L.hist, L.base, L.counts, L.offsets, sh ? T : 0, s);
      if (e != hipSuccess) return device_status(e, "counts");
      e = moe::launch_rank(L.ids, (int)R, E, L.base, L.p2r, L.r2p, s);
      if (e != hipSuccess) return device_status(e, "rank");
    }
    // the layer keeps the quantised rows K-blocked (64-byte chunks); the
    // debug capture receives a row-major copy
    e = moe::launch_quant_scatter(x, T, H, top_k, L.p2r, L.xq_rows, L.xs_rows, L.xq_tok, L.xs_tok, true,
                                  dbg ? dbg->xq_rows : nullptr, s);
    if (e != hipSuccess) return device_status(e, "quant_scatter");
  }
  char* vout = dbg ? dbg->variant : nullptr;
  MOE_CHECK(run_ffn(g, xr, rows, L.y_rows, L.tile_prefix, L.h, s, ev, vout,
                    dbg ? sizeof(dbg->variant) : 0, meta, dbg ? dbg->gemm1_events : nullptr,
                    dbg ? dbg->gemm2_events : nullptr));

  if (ev && ev[MOE_STAGE_COMBINE]) hipEventRecord((hipEvent_t)ev[MOE_STAGE_COMBINE], s);
  e = moe::launch_combine(L.y_rows, L.p2r, L.w, T, H, top_k, sh ? L.y_rows + (size_t)R * H : nullptr,
                          norm_gamma, norm_eps, out, s, nullptr, lev1);
  if (e != hipSuccess) return device_status(e, "combine");
  if (ev && ev[MOE_N_STAGES]) hipEventRecord((hipEvent_t)ev[MOE_N_STAGES], s);
  return ok();
}

moe_status_t moe_forward_noalloc(const uint16_t* x, const float* logits, int32_t T, int32_t top_k, int32_t score,
                                 const moe_weights_t* routed, int32_t use_shared, const moe_weights_t* shared,
                                 const float* norm_gamma, float norm_eps, uint16_t* out, moe_debug_t* dbg,
                                 void* stream) {
  MOE_CHECK(check_forward(x, logits, T, top_k, score, routed, use_shared, shared, norm_gamma, norm_eps, out, dbg));
  if (T == 0) return ok();
  const size_t need_ws = moe_forward_workspace_size(T, top_k, routed, use_shared);
  if (need_ws > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "this call needs %zu B of scratch; moe_forward_noalloc holds %zu B per device "
                "(use moe_forward with a workspace of that size)",
                need_ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return device_status(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(MOE_ERR_UNSUPPORTED, "the stream belongs to device %d but device %d is current", sdev, dev);
  }
  void* scratch = nullptr;
  e = moe::noalloc_scratch(dev, &scratch);
  if (e != hipSuccess) return device_status(e, "scratch address (hipGetSymbolAddress)");
  return moe_forward(x, logits, T, top_k, score, routed, use_shared, shared, norm_gamma, norm_eps, out, dbg,
                     scratch, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

// ---------------------------------------------------------------------------
moe_status_t moe_pack_weights(const moe_weights_t* src, const moe_weights_t* dst, void* stream) {
  MOE_CHECK(check_weights(src, "src"));
  MOE_CHECK(check_weights(dst, "dst"));
  if (src->layout != MOE_LAYOUT_ROW_MAJOR) return fail(MOE_ERR_SHAPE, "src must be row-major");
  if (dst->layout != MOE_LAYOUT_K_BLOCKED) return fail(MOE_ERR_SHAPE, "dst must be K-blocked");
  if (dst->fmt != src->fmt || dst->n_experts != src->n_experts || dst->hidden != src->hidden ||
      dst->inter != src->inter)
    return fail(MOE_ERR_SHAPE, "dst shape differs from src");
  const bool fp4 = src->fmt == MOE_W_MXFP4_E2M1_E8M0_G32;
  const int E = src->n_experts, H = src->hidden, I = src->inter;
  // the buffers written (codes, and the scales for MXFP4) must not overlap
  // what is read or each other
  const size_t code_bytes = (size_t)E * I * H / (fp4 ? 2 : 1);
  const size_t scale_bytes = (size_t)E * I * H / 32;
  struct Buf { const void* p; size_t n; };
  const Buf rd[6] = {{src->w1, code_bytes}, {src->w3, code_bytes}, {src->w2, code_bytes},
                     {src->s1, fp4 ? scale_bytes : 0}, {src->s3, fp4 ? scale_bytes : 0},
                     {src->s2, fp4 ? scale_bytes : 0}};
  const Buf wr[6] = {{dst->w1, code_bytes}, {dst->w3, code_bytes}, {dst->w2, code_bytes},
                     {dst->s1, fp4 ? scale_bytes : 0}, {dst->s3, fp4 ? scale_bytes : 0},
                     {dst->s2, fp4 ? scale_bytes : 0}};
  auto overlap = [](const Buf& a, const Buf& b) {
    const uint8_t* pa = static_cast<const uint8_t*>(a.p);
    const uint8_t* pb = static_cast<const uint8_t*>(b.p);
    return a.n && b.n && pa < pb + b.n && pb < pa + a.n;
  };
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(wr[i], rd[j])) return fail(MOE_ERR_SHAPE, "dst weight buffers overlap src's");
    for (int j = i + 1; j < 6; ++j)
      if (overlap(wr[i], wr[j])) return fail(MOE_ERR_SHAPE, "dst weight buffers overlap each other");
  }
  hipStream_t s = (hipStream_t)stream;
  auto u8 = [](const void* p) { return const_cast<uint8_t*>(static_cast<const uint8_t*>(p)); };
  hipError_t e;
  if (!fp4) {
    e = moe::launch_pack_kblocked(src->w1, u8(dst->w1), E, I, H, moe::kW13Chunk, s);
    if (e == hipSuccess) e = moe::launch_pack_kblocked(src->w3, u8(dst->w3), E, I, H, moe::kW13Chunk, s);
    if (e == hipSuccess) e = moe::launch_pack_kblocked(src->w2, u8(dst->w2), E, H, I, moe::kW2Chunk, s);
    return device_status(e, "pack_weights");
  }
  e = moe::launch_pack_kblocked(src->w1, u8(dst->w1), E, I, H / 2, moe::kFp4Chunk, s);
  if (e == hipSuccess) e = moe::launch_pack_kblocked(src->w3, u8(dst->w3), E, I, H / 2, moe::kFp4Chunk, s);
  if (e == hipSuccess) e = moe::launch_pack_kblocked(src->w2, u8(dst->w2), E, H, I / 2, moe::kFp4Chunk, s);
  if (e == hipSuccess) e = moe::launch_pack_kblocked4(u8(src->s1), u8(dst->s1), E, I, H / 32, s);
  if (e == hipSuccess) e = moe::launch_pack_kblocked4(u8(src->s3), u8(dst->s3), E, I, H / 32, s);
  if (e == hipSuccess) e = moe::launch_pack_kblocked4(u8(src->s2), u8(dst->s2), E, H, I / 32, s);
  return device_status(e, "pack_weights");
}

// ---------------------------------------------------------------------------
// LatentMoE block
// ---------------------------------------------------------------------------

}  // extern "C"

namespace {

moe_status_t check_linear(const moe_linear_t* w, const char* name) {
  if (!w) return fail(MOE_ERR_NULL, "%s is NULL", name);
  if (w->fmt != MOE_LIN_MXFP4 && w->fmt != MOE_LIN_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown projection format %d", name, w->fmt);
  if (w->reserved != 0) return fail(MOE_ERR_SHAPE, "%s: reserved field must be 0", name);
  MOE_CHECK(check_dim(w->n_out, "n_out"));
  if (w->n_in < 64 || w->n_in > kMaxDim || w->n_in % 64 != 0)
    return fail(MOE_ERR_SHAPE, "%s: n_in = %d is not a multiple of 64 in [64, %d]", name, w->n_in, kMaxDim);
  MOE_CHECK(need(w->w, "w"));
  if (w->fmt == MOE_LIN_MXFP4) {
    if (!w->s) return fail(MOE_ERR_NULL, "%s: MXFP4 scales are NULL", name);
  } else if (w->s) {
    return fail(MOE_ERR_SHAPE, "%s: bf16 weights take no scales", name);
  }
  return MOE_OK;
}

moe::DenseParams dense_params(const uint16_t* a, int M, const moe_linear_t* w) {
  moe::DenseParams p{};
  p.a = a;
  p.lda = w->n_in;
  p.M = M;
  p.N = w->n_out;
  p.K = w->n_in;
  p.bfmt = w->fmt == MOE_LIN_MXFP4 ? moe::kMxfp4 : moe::kBf16W;
  p.b = w->w;
  p.bs = static_cast<const uint8_t*>(w->s);
  return p;
}

moe_status_t check_latent(const moe_latent_t* lw, const moe_weights_t* routed) {
  if (!lw) return fail(MOE_ERR_NULL, "latent weights are NULL");
  MOE_CHECK(check_linear(&lw->down, "down"));
  MOE_CHECK(check_linear(&lw->up, "up"));
  const int32_t Hm = lw->down.n_in, L = lw->down.n_out;
  if (lw->up.n_in != L || lw->up.n_out != Hm)
    return fail(MOE_ERR_SHAPE, "up-projection %d -> %d does not invert down-projection %d -> %d", lw->up.n_in,
                lw->up.n_out, Hm, L);
  if (routed->hidden != L)
    return fail(MOE_ERR_SHAPE, "routed experts' hidden %d differs from the latent %d", routed->hidden, L);
  if (lw->reserved != 0) return fail(MOE_ERR_SHAPE, "latent: reserved field must be 0");
  if (lw->shared_inter != 0) {
    MOE_CHECK(check_dim(lw->shared_inter, "shared_inter"));
    if (lw->shared_activation != MOE_ACT_SILU && lw->shared_activation != MOE_ACT_SITU)
      return fail(MOE_ERR_UNSUPPORTED, "shared experts: unknown activation %d", lw->shared_activation);
    if (lw->shared_activation == MOE_ACT_SITU && !(lw->shared_beta > 0.0f && lw->shared_beta <= 3.0e38f))
      return fail(MOE_ERR_SHAPE, "shared experts: SiTU needs a finite beta > 0");
    MOE_CHECK(need(lw->sw1, "sw1"));
    MOE_CHECK(need(lw->sw3, "sw3"));
    MOE_CHECK(need(lw->sw2, "sw2"));
  }
  return MOE_OK;
}

struct LatentLayout {
  uint16_t *lat, *core, *h;
  float* up;
  void* core_ws;
  size_t core_bytes, bytes;
};

LatentLayout latent_layout(void* ws, int32_t T, int32_t k, const moe_weights_t* routed, const moe_latent_t* lw) {
  LatentLayout L{};
  Carve c(ws);
  const int32_t Hm = lw->down.n_in, Lt = lw->down.n_out, Is = lw->shared_inter;
  L.lat = c.take<uint16_t>((size_t)T * Lt);
  L.core = c.take<uint16_t>((size_t)T * Lt);
  L.up = Is ? c.take<float>((size_t)T * Hm) : nullptr;
  L.h = Is ? c.take<uint16_t>((size_t)T * Is) : nullptr;
  L.core_bytes = moe_forward_workspace_size(T, k, routed, 0);
  L.core_ws = c.take<uint8_t>(L.core_bytes);
  L.bytes = c.used + 256;
  return L;
}

}  // namespace

extern "C" {

moe_status_t moe_linear(const uint16_t* a, int32_t M, const moe_linear_t* w, const float* addend,
                        uint16_t* out_bf16, float* out_f32, void* stream) {
  MOE_CHECK(check_linear(w, "w"));
  if (M < 0) return fail(MOE_ERR_SHAPE, "M = %d < 0", M);
  if ((out_bf16 != nullptr) == (out_f32 != nullptr))
    return fail(MOE_ERR_SHAPE, "exactly one of out_bf16 and out_f32 must be given");
  if (addend && !out_bf16) return fail(MOE_ERR_SHAPE, "addend needs out_bf16");
  if (M == 0) return ok();
  MOE_CHECK(need(a, "a"));
  MOE_CHECK(opt(addend, "addend"));
  MOE_CHECK(opt(out_bf16, "out_bf16"));
  MOE_CHECK(opt(out_f32, "out_f32"));
  moe::DenseParams p = dense_params(a, M, w);
  p.mode = out_f32 ? moe::kDnStoreF32 : (addend ? moe::kDnAddBf16 : moe::kDnStoreBf16);
  p.addend = addend;
  p.c = out_f32 ? static_cast<void*>(out_f32) : static_cast<void*>(out_bf16);
  p.ldc = w->n_out;
  return device_status(moe::launch_dense(p, (hipStream_t)stream), "linear");
}

size_t moe_latent_forward_workspace_size(int32_t T, int32_t top_k, const moe_weights_t* routed,
                                         const moe_latent_t* lw) {
  if (!routed || !lw || T < 0 || top_k < 1 || routed->n_experts < 1) return 0;
  return latent_layout(nullptr, T, top_k, routed, lw).bytes;
}

moe_status_t moe_latent_forward(const uint16_t* x, const float* logits, int32_t T, int32_t top_k,
                                int32_t score, const moe_latent_t* lw, const moe_weights_t* routed,
                                const float* norm_gamma, float norm_eps, uint16_t* out, moe_debug_t* dbg,
                                void* ws, size_t ws_bytes, void* stream) {
  MOE_CHECK(check_weights(routed, "routed"));
  MOE_CHECK(check_latent(lw, routed));
  MOE_CHECK(check_route_shape(T, routed->n_experts, top_k));
  MOE_CHECK(check_score(score));
  if (norm_gamma && !(norm_eps >= 0.0f)) return fail(MOE_ERR_SHAPE, "norm_eps must be >= 0");
  if (T == 0) return ok();
  MOE_CHECK(need(x, "x"));
  MOE_CHECK(need(logits, "logits"));
  MOE_CHECK(need(out, "out"));
  if (dbg) {
    MOE_CHECK(opt(dbg->latent, "dbg.latent"));
    MOE_CHECK(opt(dbg->core_out, "dbg.core_out"));
  }
  const size_t need_ws = moe_latent_forward_workspace_size(T, top_k, routed, lw);
  if (!ws || ws_bytes < need_ws)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu B < %zu B", ws ? ws_bytes : 0, need_ws);
  MOE_CHECK(need(ws, "ws"));
  const LatentLayout L = latent_layout(ws, T, top_k, routed, lw);
  hipStream_t s = (hipStream_t)stream;
  const int32_t Hm = lw->down.n_in, Lt = lw->down.n_out, Is = lw->shared_inter;
  const hipEvent_t lev0 = dbg ? (hipEvent_t)dbg->layer_events[0] : nullptr;
  const hipEvent_t lev1 = dbg ? (hipEvent_t)dbg->layer_events[1] : nullptr;
  uint16_t* lat = (dbg && dbg->latent) ? dbg->latent : L.lat;
  uint16_t* core = (dbg && dbg->core_out) ? dbg->core_out : L.core;

  // down-projection -> latent (bf16).  When even 64-row tiles leave CUs
  // idle (512 tokens: 224 tiles), two workgroups per tile each contract half
  // of K into fp32 partials, which the routed core's workspace holds until
  // they are summed (the core's kernels come after on the same stream).
  moe::DenseParams dp = dense_params(x, T, &lw->down);
  dp.mode = moe::kDnStoreBf16;
  dp.c = lat;
  dp.ldc = Lt;
  const long tiles64 = (long)((T + 63) / 64) * (Lt / 128);
  const bool split = tiles64 < moe::kNumCUs && Hm % (2 * 64) == 0 && L.core_bytes >= (size_t)2 * T * Lt * sizeof(float);
  hipError_t e = split ? moe::launch_dense_splitk(dp, 2, static_cast<float*>(L.core_ws), s, lev0, nullptr)
                       : moe::launch_dense(dp, s, lev0, nullptr);
  if (e != hipSuccess) return device_status(e, "down-projection");

  // the routed core over the latent, with its RMSNorm, no shared expert
  moe_debug_t inner{};
  if (dbg) {
    inner = *dbg;
    inner.layer_events[0] = inner.layer_events[1] = nullptr;
  }
  MOE_CHECK(moe_forward(lat, logits, T, top_k, score, routed, 0, nullptr, norm_gamma, norm_eps, core,
                        dbg ? &inner : nullptr, L.core_ws, L.core_bytes, stream));
  if (dbg) std::memcpy(dbg->variant, inner.variant, sizeof(dbg->variant));

  // up-projection (+ shared experts on the hidden stream)
  moe::DenseParams up = dense_params(core, T, &lw->up);
  up.ldc = Hm;
  if (Is == 0) {
    up.mode = moe::kDnStoreBf16;
    up.c = out;
    e = moe::launch_dense(up, s, nullptr, lev1);
    return device_status(e, "up-projection");
  }
  up.mode = moe::kDnStoreF32;
  up.c = L.up;
  e = moe::launch_dense(up, s);
  if (e != hipSuccess) return device_status(e, "up-projection");
  const moe_linear_t w13{MOE_LIN_BF16, Is, Hm, 0, lw->sw1, nullptr};
  moe::DenseParams gu = dense_params(x, T, &w13);
  gu.mode = moe::kDnGateUp;
  gu.b3 = lw->sw3;
  gu.c = L.h;
  gu.ldc = Is;
  gu.act = lw->shared_activation == MOE_ACT_SITU ? moe::kActSitu : moe::kActSilu;
  gu.beta = lw->shared_beta;
  e = moe::launch_dense(gu, s);
  if (e != hipSuccess) return device_status(e, "shared gate-up");
  const moe_linear_t w2{MOE_LIN_BF16, Hm, Is, 0, lw->sw2, nullptr};
  moe::DenseParams dn = dense_params(L.h, T, &w2);
  dn.mode = moe::kDnAddBf16;
  dn.addend = L.up;
  dn.c = out;
  dn.ldc = Hm;
  e = moe::launch_dense(dn, s, nullptr, lev1);
  return device_status(e, "shared down");
}

}  // extern "C"
