/*
 * moe.h -- C ABI of the routed mixture-of-experts layer on one MI355X (gfx950).
 *
 * The layer is the one described on the page "Optimising Ling-2.6-1T on TPU
 * with SGLang-JAX: hiding MoE data movement behind compute with one Pallas
 * kernel" (cited below as [Ling]):
 *
 *   route (softmax, top-k, renormalise)
 *     -> per-token fp8 e4m3 activation quantisation        [Ling] §5, activation quantisation
 *     -> per-expert counts / offsets and a stable scatter  [Ling] §1 and §6 (routing metadata)
 *     -> grouped gate-up GEMM with a SiLU * gate epilogue  [Ling] §2 table, §5 direct_scaled_dot
 *     -> grouped down GEMM
 *     -> top-k weighted combine (+ shared expert)          [Ling] §1, §5 in-kernel shared expert
 *
 * Weights are per-output-channel fp8 e4m3 ([Ling] §5) or MXFP4: e2m1 codes two
 * per byte with one e8m0 scale per 32 contiguous contraction elements (page
 * "Implementation gaps: advanced optimisations" of the sglang-jax wiki, §4
 * MXFP4; page "Feasibility of porting Kimi K3 to the Google TPU ecosystem",
 * §2.5).  The optional RMSNorm of the routed sum is the LatentMoE
 * routed_expert_norm of that Kimi K3 page, §2.4.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Tensor pointers are DEVICE pointers to row-major, contiguous arrays
 *    (expert weights may instead use the K-blocked layout of
 *    moe_pack_weights).
 *    bf16 is passed as uint16_t bit patterns; fp8 e4m3 (OCP E4M3FN), packed
 *    e2m1 pairs and e8m0 scales as uint8_t.  `stream` is a hipStream_t
 *    (NULL = the default stream).
 *  - Ownership: the caller allocates and owns every buffer, including the
 *    workspace sized by the *_workspace_size functions.  The library never
 *    allocates or frees device memory, never synchronises the device, never
 *    copies device data to the host and never reads device data on the
 *    host.  All work is enqueued on `stream`, so every call can be captured
 *    into a HIP graph.  No global mutable state: calls on different streams
 *    with distinct workspaces may run concurrently.  The one exception is
 *    moe_forward_noalloc, whose workspace is a per-device scratch array the
 *    library holds (see there).
 *  - Errors: arguments are validated on the host before anything is enqueued;
 *    on a non-OK return nothing has been enqueued or written.  A launch
 *    failure reported by the runtime returns MOE_ERR_DEVICE (work enqueued
 *    before it may have run).  Faults inside kernels surface at the caller's
 *    next synchronisation.  moe_last_error() gives a thread-local message
 *    for the last non-OK return on the calling thread.
 *  - T = 0 is valid and does nothing.  Inputs holding NaN or Inf give
 *    undefined values, with one exception: the routing ranks a NaN logit
 *    as -Inf (below every number; equal values by expert index), so that
 *    every expert id stays in [0, E).
 *  - Limits: 1 <= E <= 1024; 1 <= top_k <= min(E, 32); T * top_k < 2^31;
 *    H and I multiples of 128 (one MFMA contraction step) and at most 65536;
 *    pointers 16-byte aligned.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                          */
  MOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent              */
  MOE_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                    */
  MOE_ERR_WORKSPACE = 4,   /* the workspace is smaller than *_workspace_size()   */
  MOE_ERR_UNSUPPORTED = 5, /* valid, but no kernel exists for this case           */
  MOE_ERR_DEVICE = 6       /* the HIP runtime reported an error                   */
} moe_status_t;

typedef enum {
  MOE_W_FP8_E4M3_PERCHANNEL = 0, /* e4m3 codes + one fp32 scale per output channel */
  MOE_W_MXFP4_E2M1_E8M0_G32 = 1, /* e2m1 pairs + one e8m0 scale per 32 K-elements   */
  MOE_W_FP8_E4M3_BLOCK128 = 2    /* e4m3 codes + one fp32 scale per 128x128 tile    */
} moe_wfmt_t;

/*
 * Byte layout of each expert's weight matrix [N][K] (N output channels, K
 * contraction bytes).  ROW_MAJOR: byte k of channel n at n*K + k.  K_BLOCKED
 * (written by moe_pack_weights): the matrix is cut into K chunks of C bytes,
 * stored chunk after chunk, each chunk holding all N channels: byte k of
 * channel n at (k / C) * N * C + n * C + k % C.  FP8: C = 64 for W1 and W3,
 * C = 32 for W2, the per-channel scales unchanged.  MXFP4: C = 64 for the
 * codes of W1, W3 and W2 (128 elements) and the e8m0 scales K-blocked too,
 * with C = 4 (the 4 scales of the same 128 elements).  One contraction step
 * of a GEMM tile then reads one contiguous block instead of N short pieces
 * K bytes apart.  Experts stay contiguous ([E][...]).
 */
typedef enum {
  MOE_LAYOUT_ROW_MAJOR = 0,
  MOE_LAYOUT_K_BLOCKED = 1
} moe_wlayout_t;

/*
 * Gate activation of an expert group: h = act(g) * u.  SILU: g * sigmoid(g)
 * (the Ling-2.6-1T page, §2: SiLU on the gate).  SITU: beta * tanh(g / beta)
 * * sigmoid(g) (the Kimi K3 page, §2.6, with beta = 4).
 */
typedef enum {
  MOE_ACT_SILU = 0,
  MOE_ACT_SITU = 1
} moe_act_t;

/*
 * Router score function.  SOFTMAX: p = softmax(logits[t]) (the default).
 * SIGMOID: p = 1 / (1 + e^-l) per expert (the Kimi K3 page, §2.4; its
 * noaux_tc selection bias is not defined there and not provided).  Both are
 * increasing in the logit, so both select the k largest logits; the weights
 * are p renormalised over the k chosen.
 */
typedef enum {
  MOE_SCORE_SOFTMAX = 0,
  MOE_SCORE_SIGMOID = 1
} moe_score_t;

/*
 * A group of experts that share one shape.  Host struct holding device
 * pointers; caller-owned.  W1 is the gate projection (through the
 * activation), W3 the up projection, W2 the down projection; the contraction
 * index is last ("K contiguous").
 *
 *   fmt = FP8:   w1, w3  uint8 [E][I][H]      s1, s3  float [E][I]
 *                w2      uint8 [E][H][I]      s2      float [E][H]
 *                (w* in `layout`: row-major as written, or K-blocked)
 *   fmt = FP8 BLOCK128: w1, w3, w2 as for FP8;  s1, s3  float [E][I/128][H/128]
 *                                               s2      float [E][H/128][I/128]
 *                one scale per tile of 128 output channels x 128 K elements,
 *                applied to that tile's partial sum inside the reduction:
 *                out[n] = sum_kb s[n/128][kb] * sum_{k in kb} a[k] W[n][k]
 *                ([Ling] §5, per-block scaling; the [128, 128] block-wise
 *                format of the Kimi K3 page, §3.7).  Routed experts only.
 *                Small batches run the register-fed kernels, which sum each
 *                K block and scale the fp32 partial.  From 64 rows per
 *                expert on average the LDS-staged kernels run: the gate-up
 *                GEMM takes the scale's power of two in the MFMA and its
 *                mantissa by rescaling the fp32 accumulators at each K
 *                block; the down GEMM applies the scale to each weight as
 *                it is widened (bf16(code * s), one rounding of at most
 *                2^-9 relative, the size of h's own bf16 rounding).
 *   fmt = MXFP4: w1, w3  uint8 [E][I][H/2]    s1, s3  uint8 [E][I][H/32]
 *                w2      uint8 [E][H][I/2]    s2      uint8 [E][H][I/32]
 *                (element 2i in the low nibble of byte i; scale 255 = NaN is
 *                 not allowed; w* and s* in `layout`)
 */
typedef struct {
  int32_t fmt;       /* moe_wfmt_t */
  int32_t n_experts; /* E */
  int32_t hidden;    /* H: model dimension (FFN input and output width) */
  int32_t inter;     /* I: intermediate dimension */
  int32_t layout;    /* moe_wlayout_t of w1, w3, w2 */
  int32_t activation;/* moe_act_t (0 = SiLU) */
  float act_beta;    /* SiTU's beta, finite and > 0; ignored for SiLU */
  int32_t reserved;  /* must be 0 */
  const uint8_t* w1;
  const uint8_t* w3;
  const uint8_t* w2;
  const void* s1;
  const void* s3;
  const void* s2;
} moe_weights_t;

/* Stage boundaries at which moe_forward records the events of a moe_debug_t. */
enum {
  MOE_STAGE_ROUTE = 0,   /* router                                            */
  MOE_STAGE_PERMUTE = 1, /* counts, offsets, ranks, quantise+scatter, GEMM
                            tile prefix                                       */
  MOE_STAGE_GEMM1 = 2,   /* gate-up grouped GEMM + SiLU * gate (one kernel)   */
  MOE_STAGE_GEMM2 = 3,   /* down grouped GEMM (one kernel)                    */
  MOE_STAGE_COMBINE = 4, /* weighted gather (+ RMSNorm) (+ shared)            */
  MOE_N_STAGES = 5
};

/*
 * Optional capture of intermediates and stage timing for moe_forward.  Every
 * non-NULL device pointer receives the named intermediate (and is used in
 * place of the corresponding workspace slice).  events[i], when non-NULL, is
 * a hipEvent_t recorded on `stream` just before stage i; events[MOE_N_STAGES]
 * after the last stage (each such record is one more packet on the stream,
 * a few microseconds of command-processor time).  `variant` receives a
 * NUL-terminated name of the kernel variants chosen.  gemm1_events[0] / [1]
 * and gemm2_events[0] / [1], when non-NULL, are hipEvent_t stamped by the
 * gate-up / down GEMM's own dispatch (hipExtLaunchKernel) at its start and
 * end: its duration with no extra packets on the stream.  layer_events[0] /
 * [1], when non-NULL, are stamped the same way by the layer's first dispatch
 * (the router, or the routing + quantisation kernel) at its start and by its
 * last (the combine) at its end: the whole layer's duration (moe_forward
 * only).  A dispatch that stamps events costs the stream a little more than
 * one that does not: time the layer and the GEMMs in separate calls.
 */
typedef struct {
  int32_t* topk_ids;       /* [T][k]   */
  float* topk_w;           /* [T][k]   */
  int32_t* expert_counts;  /* [E]      */
  int32_t* expert_offsets; /* [E+1]; [E+2] with a shared expert, whose token-order
                              rows are the extra group T*k .. T*k+T-1 */
  int32_t* pair_to_row;    /* [T][k]   */
  int32_t* row_to_pair;    /* [T*k]    */
  uint8_t* xq_rows;        /* [T*k][H] row-major copy of the quantised rows (the
                              layer itself keeps them K-blocked, 64-byte chunks) */
  float* xs_rows;          /* [T*k]    */
  void* events[MOE_N_STAGES + 1];
  char variant[96];
  void* gemm1_events[2];
  void* gemm2_events[2];
  void* layer_events[2];
  uint16_t* latent;     /* moe_latent_forward: bf16 [T][L] down-projection output */
  uint16_t* core_out;   /* moe_latent_forward: bf16 [T][L] routed core output */
} moe_debug_t;

/* ------------------------------------------------------------------------ */

/*
 * moe_route -- router with top-k selection.
 *   logits    float [T][E]   router logits (|l| <= 80: beyond, fp32 sigmoid
 *                            scores underflow and the weights are undefined)
 *   score     moe_score_t
 *   topk_ids  int32 [T][k]   out: chosen experts, slot order = descending
 *                            logit, equal logits by ascending expert index
 *                            (-0.0 equals +0.0); the raw fp32 logits decide
 *   topk_w    float [T][k]   out: w_j = p[id_j] / sum_j' p[id_j'] with p the
 *                            score (routed scaling 1.0)
 * [Ling] overview and §1 (top-8 of 256 routed experts); renormalised weights
 * and the sigmoid score as in the Kimi K3 page, §2.4.
 */
moe_status_t moe_route(const float* logits, int32_t T, int32_t E, int32_t top_k, int32_t score,
                       int32_t* topk_ids, float* topk_w, void* stream);

/*
 * moe_permute -- per-token fp8 quantisation, per-expert counts and offsets,
 * and the stable scatter of quantised token rows into expert order.
 *   x              bf16  [T][H]   activations
 *   topk_ids       int32 [T][k]   from moe_route
 *   expert_counts  int32 [E]      out: rows per expert
 *   expert_offsets int32 [E+1]    out: exclusive prefix sum, [0] = 0, [E] = T*k
 *   pair_to_row    int32 [T][k]   out: row of pair (t, j)
 *   row_to_pair    int32 [T*k]    out: pair index t*k + j of each row
 *   xq_rows        uint8 [T*k][H] out: e4m3 codes of token t at row pair_to_row[t][j]
 *   xs_rows        float [T*k]    out: its scale
 *   xq_tok, xs_tok uint8 [T][H], float [T]  out, optional (NULL = skip): the
 *                  same quantised tokens in token order
 * Quantisation: a = max|x[t]|, s = a/448 (IEEE binary32 division; s = 1 if
 * a = 0), q = e4m3(x/s) with round-half-even, saturation at +-448 and signed
 * zero ([Ling] §5, activation quantisation before the scatter).  Rows are
 * ordered by expert, and within an expert by pair index (t*k + j): the
 * permutation is unique and deterministic.
 */
size_t moe_permute_workspace_size(int32_t T, int32_t top_k, int32_t E);
moe_status_t moe_permute(const uint16_t* x, int32_t T, int32_t H, const int32_t* topk_ids,
                         int32_t top_k, int32_t E, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* pair_to_row, int32_t* row_to_pair,
                         uint8_t* xq_rows, float* xs_rows, uint8_t* xq_tok, float* xs_tok,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn -- gated FFN of expert-grouped rows.
 *   xq_rows        uint8 [n_rows][H]  e4m3 rows grouped by expert
 *   xs_rows        float [n_rows]     per-row scales
 *   expert_offsets int32 [E+1]        device; rows of expert e are
 *                                     offsets[e] .. offsets[e+1]-1, offsets[E] = n_rows
 *   y_rows         float [n_rows][H]  out (fp32: the output is rounded only once,
 *                                     by the combine)
 * For row r of expert e ([Ling] §5, per-channel direct_scaled_dot: scales
 * applied after the full-K reduction; fp32 accumulation):
 *   g = (sum_k q_r[k] W1[e][n][k]) * xs_r * s1[e][n];  u likewise with W3, s3
 *   h = bf16( act(g) * u )   act = SiLU or SiTU (w->activation)
 *   y_r[j] = (sum_n h_r[n] W2[e][j][n]) * s2[e][j]
 * GEMM1 runs e4m3 x e4m3 on the matrix cores; GEMM2 runs bf16 h x W2 with
 * W2's codes converted exactly to bf16.
 * For MXFP4 the e8m0 block scales enter each 32-element partial sum and
 * s1/s3/s2 are not per-channel.  A shared expert is a call with E = 1 and
 * offsets {0, T} over token-order rows.
 */
size_t moe_expert_ffn_workspace_size(int32_t n_rows, const moe_weights_t* w);
moe_status_t moe_expert_ffn(const uint8_t* xq_rows, const float* xs_rows, int32_t n_rows,
                            const int32_t* expert_offsets, const moe_weights_t* w,
                            float* y_rows, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine -- weighted gather back into token order.
 *   y_rows      float [T*k][H]  expert outputs
 *   pair_to_row int32 [T][k]
 *   topk_w      float [T][k]
 *   y_shared    float [T][H]    optional (NULL = none): shared expert output
 *   norm_gamma  float [H]       optional (NULL = no RMSNorm)
 *   out         bf16  [T][H]    out
 * o = sum_{j<k} w[t][j] * y_rows[pair_to_row[t][j]] in fp32, slot order;
 * with norm_gamma: o = o / sqrt(mean(o^2) + norm_eps) * gamma (the LatentMoE
 * routed_expert_norm, Kimi K3 page §2.4); then o += y_shared[t];
 * out = bf16(o), round-half-even.  [Ling] §1 (gather results) and the
 * SparseCore gather-reduce of the sglang-jax gap list, §8.
 */
moe_status_t moe_combine(const float* y_rows, const int32_t* pair_to_row, const float* topk_w,
                         int32_t T, int32_t H, int32_t top_k, const float* y_shared,
                         const float* norm_gamma, float norm_eps, uint16_t* out, void* stream);

/*
 * moe_forward -- the whole layer: route -> permute -> expert FFN (routed
 * experts and, if use_shared, the shared expert on every token) -> combine.
 *   x       bf16  [T][H]         logits float [T][E] (E = routed->n_experts)
 *   score   moe_score_t of the router (see moe_route)
 *   routed  the routed experts; shared: one expert of the same H and I, fp8
 *           (required iff use_shared)
 *   out     bf16  [T][H]
 *   dbg     optional (NULL = none), see moe_debug_t
 * The shared expert reads the same quantised tokens as the routed experts
 * and is added with weight 1 after the routed sum (and after the RMSNorm)
 * ([Ling] §5, in-kernel shared expert).
 */
size_t moe_forward_workspace_size(int32_t T, int32_t top_k, const moe_weights_t* routed,
                                  int32_t use_shared);
moe_status_t moe_forward(const uint16_t* x, const float* logits, int32_t T, int32_t top_k,
                         int32_t score, const moe_weights_t* routed, int32_t use_shared,
                         const moe_weights_t* shared, const float* norm_gamma, float norm_eps,
                         uint16_t* out, moe_debug_t* dbg, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * moe_forward_noalloc -- moe_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The arguments and results are moe_forward's, without the
 * workspace: the call uses a scratch array of MOE_NOALLOC_SCRATCH_BYTES that
 * the library holds on each device (a file-scope device array, allocated when
 * the library's code is loaded on that device and kept until the process
 * ends).  The call itself allocates and frees nothing.
 *   - Limit: a call whose moe_forward_workspace_size exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE with nothing
 *     enqueued.  64 MiB holds, for instance, the 8-expert decode share
 *     (H 8192, I 2048, top-2, shared expert) up to about 560 tokens.
 *   - The stream must belong to the current device (else
 *     MOE_ERR_UNSUPPORTED).  The scratch address of a device is looked up
 *     (hipGetSymbolAddress) on the first call with that device current.
 *   - Every call on a device shares that device's scratch, and the scratch
 *     keeps the last call's contents (every buffer the layer carves from it
 *     is fully written before it is read).  Calls that overlap in time on
 *     one device -- on different streams, or from different threads --
 *     race on the scratch: order them on one stream.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_forward_noalloc(const uint16_t* x, const float* logits, int32_t T, int32_t top_k,
                                 int32_t score, const moe_weights_t* routed, int32_t use_shared,
                                 const moe_weights_t* shared, const float* norm_gamma, float norm_eps,
                                 uint16_t* out, moe_debug_t* dbg, void* stream);

/*
 * moe_pack_weights -- copy row-major expert weights into the K-blocked
 * layout (see moe_wlayout_t), once, when the weights are loaded.
 *   src  layout ROW_MAJOR, device pointers
 *   dst  the same fmt, n_experts, hidden and inter, layout K_BLOCKED;
 *        dst->w1, w3, w2 are caller buffers of the sizes of src's, disjoint
 *        from them and from each other.  FP8: dst->s1, s3, s2 are not
 *        written (the per-channel scales are the same in both layouts and may
 *        alias src's).  MXFP4: dst->s1, s3, s2 receive the K-blocked scales
 *        (caller buffers of the sizes of src's, disjoint like the codes)
 * The codes are only moved, never changed: the layer computes the same
 * values from either layout.  The per-step weight tile of the gate-up and
 * down GEMMs becomes one contiguous block, which the direct-to-LDS loads
 * stream at about twice the rate of the row-major pieces.  The pages do the
 * corresponding layout work for the TPU's vector unit inside the kernel
 * ([Ling] §7: fp8 packing and lane shuffles remain the bottleneck); here it
 * is paid once per weight load.
 */
moe_status_t moe_pack_weights(const moe_weights_t* src, const moe_weights_t* dst, void* stream);

/* ------------------------------------------------------------------------ */
/* The LatentMoE block ([K3] §2.4: down-projection hidden -> latent before the
 * routed experts, their RMSNorm, up-projection latent -> hidden, shared
 * experts on the hidden stream; §2.5: the projections are MXFP4, the shared
 * experts keep bf16 weights).  All pointers are caller-owned device memory. */

typedef enum { MOE_LIN_MXFP4 = 0, MOE_LIN_BF16 = 1 } moe_lin_fmt_t;

/* One dense projection y = a W^T with W [n_out][n_in].
 *   MXFP4: w uint8 [n_out][n_in/2] (two e2m1 per byte, element 2i in the low
 *          nibble), s uint8 e8m0 [n_out][n_in/32]
 *   BF16:  w uint16 bf16 [n_out][n_in], s NULL
 * n_out a multiple of 128, n_in of 64. */
typedef struct {
  int32_t fmt;     /* moe_lin_fmt_t */
  int32_t n_out;
  int32_t n_in;
  int32_t reserved;  /* must be 0 */
  const void* w;
  const void* s;
} moe_linear_t;

/* The block's own weights around the routed experts (hidden Hm, latent L). */
typedef struct {
  moe_linear_t down;        /* Hm -> L, MXFP4 */
  moe_linear_t up;          /* L -> Hm, MXFP4 */
  int32_t shared_inter;     /* Is of the shared experts (a multiple of 64); 0 = none */
  int32_t shared_activation;/* moe_act_t of the shared experts */
  float shared_beta;        /* SiTU's beta (shared_activation == MOE_ACT_SITU) */
  int32_t reserved;         /* must be 0 */
  const uint16_t* sw1;      /* bf16 [Is][Hm] gate */
  const uint16_t* sw3;      /* bf16 [Is][Hm] up */
  const uint16_t* sw2;      /* bf16 [Hm][Is] down */
} moe_latent_t;

/*
 * moe_linear -- out = a W^T on the bf16 MFMA, fp32 accumulation.
 *   a       bf16  [M][n_in] row-major
 *   out_bf16 bf16 [M][n_out] (rounded to nearest even), or NULL
 *   out_f32  float [M][n_out], or NULL (exactly one of the two)
 *   addend  optional float [M][n_out] added before the bf16 rounding
 *           (only with out_bf16)
 * The MXFP4 weights are widened exactly to bf16 inside the kernel.
 */
moe_status_t moe_linear(const uint16_t* a, int32_t M, const moe_linear_t* w, const float* addend,
                        uint16_t* out_bf16, float* out_f32, void* stream);

/*
 * moe_latent_forward -- the LatentMoE block:
 *   lat  = bf16( x down^T )                      [T][L]
 *   core = moe_forward(lat, logits, routed experts over L, RMSNorm(norm_gamma,
 *          norm_eps), no shared expert)          bf16 [T][L]
 *   out  = bf16( core up^T + shared(x) )         [T][Hm]
 *   shared(x) = bf16( act(x sw1^T) * (x sw3^T) ) sw2^T   (absent if Is = 0)
 * x bf16 [T][Hm]; logits float [T][E]; routed->hidden == L.  dbg: as for
 * moe_forward (its routing captures describe the core); dbg->latent and
 * dbg->core_out (bf16 [T][L]) receive the two intermediates; layer_events
 * bracket the whole block.  The latent and the core's output are rounded to
 * bf16 (the activation dtype between steps); the up-projection and the
 * shared experts' output are summed in fp32 and rounded once.
 */
size_t moe_latent_forward_workspace_size(int32_t T, int32_t top_k, const moe_weights_t* routed,
                                         const moe_latent_t* lw);
moe_status_t moe_latent_forward(const uint16_t* x, const float* logits, int32_t T, int32_t top_k,
                                int32_t score, const moe_latent_t* lw, const moe_weights_t* routed,
                                const float* norm_gamma, float norm_eps, uint16_t* out, moe_debug_t* dbg,
                                void* ws, size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* moe_status_string(moe_status_t s);

/* Thread-local detail of the last non-OK return on this thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
