"""The routed MoE layer, step by step, in float64 (plain definition).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Steps and where the pages describe them:

1. ``route``            -- softmax (or sigmoid) router, top-k, renormalised weights.
   *Ling-2.6-1T on TPU*: overview (256 routed experts, top-8 plus one shared
   expert) and §1 cost model; *Kimi K3 on TPU*, §2.4 LatentMoE
   (renormalised top-k weights, routed scaling factor 1.0).
2. ``quantize_tokens``  -- dynamic per-token fp8 quantisation of the bf16
   activations before the scatter.  *Ling-2.6-1T on TPU*, §5 "activation
   quantisation".
3. ``expert_counts_offsets`` and ``permute_rows`` -- routing metadata
   (token-to-expert map, per-expert counts and offsets, scatter/gather
   indices) and the scatter of token rows to experts.  *Ling-2.6-1T on TPU*,
   §1 ("scatter tokens -> local expert FFN -> gather results") and §6 (the
   metadata block).
4. ``expert_ffn``       -- gated expert FFN: W1/W3 gate-up projection, SiLU
   (or SiTU, *Kimi K3 on TPU* §2.6), gate multiply, scale multiply, W2 down
   projection, with per-channel scales applied after the full-K reduction.
   *Ling-2.6-1T on TPU*, §2 (table of hardware units and the MoE work each
   does) and §5 "per-channel direct_scaled_dot".
5. ``combine``          -- weighted gather back into token order, optional
   per-token RMSNorm of the routed sum (*Kimi K3 on TPU*, §2.4
   routed_expert_norm), plus the shared expert's output (*Ling-2.6-1T on TPU*,
   §1 and §5 "in-kernel shared expert").

Readings where the pages are silent (each listed in the design notes):
top-k compares the raw fp32 logits with ties to the lower expert index and
keeps slots in that order; fp8 is OCP E4M3FN with round-half-even and
saturation; scales are amax/448 by IEEE binary32 division (1 when amax is 0);
W1 is the gate and W3 the up projection; the FFN intermediate h stays in the
activation dtype, bf16 (only the tokens are quantised, before the scatter);
the shared expert reads
the same quantised tokens and is added with weight 1 after the routed sum
(after the RMSNorm when there is one); the output is bfloat16.
"""

import numpy as np

from .codecs import (
    e4m3_decode,
    e4m3_encode,
    bf16_decode,
    bf16_encode,
    mxfp4_decode,
    E4M3_MAX,
)


# ----------------------------------------------------------------------------
# 1. Router
# ----------------------------------------------------------------------------


def route(logits, top_k, score="softmax"):
    """Top-k experts per token and their renormalised weights.

    logits: float32 [T][E].  Returns (topk_ids int32 [T][k], topk_w float64
    [T][k]).  Experts are ordered by descending logit, equal logits by
    ascending expert index; that order is both the selection and the slot
    order.  score "softmax": p = softmax(logits[t]) in float64 (max
    subtracted); score "sigmoid" (the *Kimi K3 on TPU* router, §2.4, without
    its selection bias, which the pages do not define): p = 1 / (1 + e^-l).
    Both are increasing in the logit, so they select the same experts.  Then
    w_j = p[id_j] / sum_j' p[id_j'] (renormalised, routed scaling factor 1).
    """
    if score not in ("softmax", "sigmoid"):
        raise ValueError(score)
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k out of range")
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    index = np.arange(E)
    for t in range(T):
        row = logits[t].astype(np.float64)
        # np.lexsort sorts by the last key first: primary -logit, then index.
        order = np.lexsort((index, -row))
        sel = order[:top_k]
        ids[t] = sel
        if score == "softmax":
            p = np.exp(row - row.max())
            p = p / p.sum()
        else:
            p = 1.0 / (1.0 + np.exp(-row))
        w[t] = p[sel] / p[sel].sum()
    return ids, w


# ----------------------------------------------------------------------------
# 2. Per-token fp8 quantisation
# ----------------------------------------------------------------------------


def quantize_rows_f32(values):
    """Per-row e4m3 quantisation of binary32 values.

    a = max|v|; s = a / 448 as an IEEE binary32 division (s = 1 when a = 0);
    q = e4m3(v / s) with the division again in binary32.  Returns
    (codes uint8 [N][D], scales float32 [N]).
    """
    v = np.asarray(values, dtype=np.float32)
    a = np.max(np.abs(v), axis=1)
    s = a / np.float32(E4M3_MAX)                      # binary32 division
    s = np.where(a == 0, np.float32(1.0), s).astype(np.float32)
    q = e4m3_encode(v / s[:, None])                   # binary32 division
    return q, s


def quantize_tokens(x_bf16):
    """bf16 activations [T][H] (uint16 bits) -> (xq uint8 [T][H], xs float32 [T])."""
    x = bf16_decode(x_bf16).astype(np.float32)        # exact
    return quantize_rows_f32(x)


# ----------------------------------------------------------------------------
# 3. Routing metadata and the scatter
# ----------------------------------------------------------------------------


def expert_counts_offsets(topk_ids, n_experts):
    """counts[e] = number of (t, j) with topk_ids[t][j] == e; offsets is the
    exclusive prefix sum with offsets[0] = 0 and offsets[E] = T*k."""
    ids = np.asarray(topk_ids).ravel()
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in ids:
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    return counts.astype(np.int32), offsets.astype(np.int32)


def permute_rows(topk_ids, offsets, xq, xs):
    """Stable scatter of token rows into expert-grouped rows.

    Pairs (t, j) are visited in row-major order; each takes the next free row
    of its expert's segment.  Returns (pair_to_row int32 [T][k], row_to_pair
    int32 [R], xq_rows uint8 [R][H], xs_rows float32 [R]) with R = T*k and
    pair index p = t*k + j.
    """
    ids = np.asarray(topk_ids)
    T, k = ids.shape
    R = T * k
    cursor = np.array(offsets[:-1], dtype=np.int64).copy()
    pair_to_row = np.empty((T, k), dtype=np.int32)
    row_to_pair = np.empty(R, dtype=np.int32)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            r = cursor[e]
            cursor[e] += 1
            pair_to_row[t, j] = r
            row_to_pair[r] = t * k + j
    tok = row_to_pair // k
    xq_rows = np.asarray(xq)[tok]
    xs_rows = np.asarray(xs, dtype=np.float32)[tok]
    return pair_to_row, row_to_pair, xq_rows, xs_rows


# ----------------------------------------------------------------------------
# 4. Expert FFN
# ----------------------------------------------------------------------------


class ExpertWeights:
    """Weights of a group of experts in one of the two formats.

    fmt "fp8":   w1, w3 uint8 [E][I][H]; w2 uint8 [E][H][I] (e4m3 codes, the
                 contraction index last); s1, s3 float32 [E][I], s2 float32
                 [E][H] (one scale per output channel).
    fmt "mxfp4": w1, w3 uint8 [E][I][H/2]; w2 uint8 [E][H][I/2] (two e2m1 per
                 byte, element 2i in the low nibble); s1, s3 uint8
                 [E][I][H/32], s2 uint8 [E][H][I/32] (e8m0 per 32 consecutive
                 contraction elements of one output channel).
    fmt "fp8_block": w1, w3, w2 as for "fp8"; s1, s3 float32 [E][I/128][H/128],
                 s2 float32 [E][H/128][I/128]: one scale per block of 128
                 output channels x 128 contraction elements, so that
                 out[n] = sum_k a[k] W[n][k] scale[n // 128][k // 128]
                 (*Ling-2.6-1T on TPU*, §5, per-block scaling: the scale
                 depends on the K block and cannot leave the reduction; the
                 [128, 128] block shape is the block-wise fp8 format the
                 *Kimi K3 on TPU* page, §3.7, names).
    W1 is the gate projection and W3 the up projection.  The six stacks may
    be any objects with a ``shape`` whose ``[e]`` gives expert e as a NumPy
    array (so very large stacks can be fetched one expert at a time).
    activation: "silu" (SiLU(g) * u) or "situ" (SiTU with parameter beta).
    """

    def __init__(self, fmt, w1, w3, w2, s1, s3, s2, activation="silu", beta=4.0):
        if fmt not in ("fp8", "mxfp4", "fp8_block"):
            raise ValueError(fmt)
        if activation not in ("silu", "situ") or not beta > 0:
            raise ValueError(activation)
        self.fmt = fmt
        self.activation = activation
        self.beta = float(beta)
        wrap = lambda a: a if hasattr(a, "shape") and not isinstance(a, (list, tuple)) else np.asarray(a)  # noqa: E731
        self.w1, self.w3, self.w2 = (wrap(a) for a in (w1, w3, w2))
        self.s1, self.s3, self.s2 = (wrap(a) for a in (s1, s3, s2))
        self.n_experts = self.w1.shape[0]
        self.inter = self.w1.shape[1]
        self.hidden = self.w2.shape[1]

    def decode(self, e):
        """Expert e as float64 matrices and per-channel scales:
        (W1 [I][H], W3 [I][H], W2 [H][I], c1 [I], c3 [I], c2 [H])."""
        if self.fmt == "fp8":
            return (e4m3_decode(self.w1[e]), e4m3_decode(self.w3[e]),
                    e4m3_decode(self.w2[e]),
                    np.asarray(self.s1[e], dtype=np.float64), np.asarray(self.s3[e], dtype=np.float64),
                    np.asarray(self.s2[e], dtype=np.float64))
        ones_i = np.ones(self.inter)
        if self.fmt == "fp8_block":
            return (block_scaled(e4m3_decode(self.w1[e]), self.s1[e]),
                    block_scaled(e4m3_decode(self.w3[e]), self.s3[e]),
                    block_scaled(e4m3_decode(self.w2[e]), self.s2[e]),
                    ones_i, ones_i, np.ones(self.hidden))
        return (mxfp4_decode(self.w1[e], self.s1[e]),
                mxfp4_decode(self.w3[e], self.s3[e]),
                mxfp4_decode(self.w2[e], self.s2[e]),
                ones_i, ones_i, np.ones(self.hidden))


def block_scaled(W, scales, block=128):
    """W [N][K] times scale[n // block][k // block] for every element: the
    per-block weights as the float64 matrix whose plain product with a row
    gives sum over K blocks of (block dot product) x (block scale), exactly."""
    sc = np.asarray(scales, dtype=np.float64)
    return W * np.repeat(np.repeat(sc, block, axis=0), block, axis=1)


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def situ(z, beta):
    """SiTU(z) = beta * tanh(z / beta) * sigmoid(z) (*Kimi K3 on TPU*, §2.6,
    with beta = 4): SiLU with its linear factor z bounded to (-beta, beta)."""
    with np.errstate(over="ignore"):
        return beta * np.tanh(z / beta) / (1.0 + np.exp(-z))


def activate(g, weights):
    """The expert group's gate activation."""
    return silu(g) if weights.activation == "silu" else situ(g, weights.beta)


def expert_ffn(xq_rows, xs_rows, offsets, weights):
    """Gated FFN of every routed row with its expert's weights.

    For row r in expert e's segment (rows offsets[e] .. offsets[e+1]-1):
      g = (sum_k q_r[k] W1[e][n][k]) * xs_r * s1[e][n]
      u = (sum_k q_r[k] W3[e][n][k]) * xs_r * s3[e][n]
      h = bf16( act(g) * u )                   (the activation dtype;
                                                act = SiLU, or SiTU)
      y[r][j] = (sum_n h_r[n] W2[e][j][n]) * s2[e][j]
    The sums of fp8 (or e2m1 * 2^k) products, and of bf16 x fp8 products,
    are exact in float64.  Returns (y float64 [R][H], h uint16 bf16 bits [R][I]).
    """
    xq_rows = np.asarray(xq_rows)
    xs_rows = np.asarray(xs_rows, dtype=np.float64)
    R = xq_rows.shape[0]
    H, I = weights.hidden, weights.inter
    y = np.zeros((R, H), dtype=np.float64)
    h_all = np.zeros((R, I), dtype=np.uint16)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        W1, W3, W2, c1, c3, c2 = weights.decode(e)
        a = e4m3_decode(xq_rows[r0:r1])
        g = (a @ W1.T) * xs_rows[r0:r1, None] * c1[None, :]
        u = (a @ W3.T) * xs_rows[r0:r1, None] * c3[None, :]
        h = bf16_encode(activate(g, weights) * u)
        y[r0:r1] = (bf16_decode(h) @ W2.T) * c2[None, :]
        h_all[r0:r1] = h
    return y, h_all


# ----------------------------------------------------------------------------
# 5. Combine
# ----------------------------------------------------------------------------


def rms_norm(o, gamma, eps):
    """Per-row RMSNorm: o / sqrt(mean(o^2) + eps) * gamma."""
    return o / np.sqrt(np.mean(o * o, axis=1, keepdims=True) + eps) * gamma[None, :]


def combine(y_rows, pair_to_row, topk_w, y_shared=None, norm_gamma=None, norm_eps=1e-6,
            rounded=True):
    """out[t] = bf16( [RMSNorm]( sum_j w[t][j] * y_rows[pair_to_row[t][j]] ) + y_shared[t] ).

    The routed sum runs over slots j = 0..k-1 in order.  Returns uint16 bf16
    bits, or with rounded=False the float64 value before the bf16 rounding.
    """
    p2r = np.asarray(pair_to_row)
    w = np.asarray(topk_w, dtype=np.float64)
    T, k = p2r.shape
    o = np.zeros((T, y_rows.shape[1]), dtype=np.float64)
    for j in range(k):
        o += w[:, j, None] * y_rows[p2r[:, j]]
    if norm_gamma is not None:
        o = rms_norm(o, np.asarray(norm_gamma, dtype=np.float64), norm_eps)
    if y_shared is not None:
        o = o + y_shared
    return bf16_encode(o) if rounded else o


# ----------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------


def forward(x_bf16, logits, top_k, routed, shared=None, norm_gamma=None, norm_eps=1e-6,
            score="softmax"):
    """Route -> quantise -> count/offset -> permute -> expert FFN -> combine.

    x_bf16 uint16 [T][H]; logits float32 [T][E]; routed/shared ExpertWeights
    (shared has one expert and runs on every token in token order); score as
    in ``route``.  Returns a dict with every intermediate and ``out`` (uint16
    bf16 [T][H]).
    """
    ids, w = route(logits, top_k, score)
    xq, xs = quantize_tokens(x_bf16)
    counts, offsets = expert_counts_offsets(ids, routed.n_experts)
    pair_to_row, row_to_pair, xq_rows, xs_rows = permute_rows(ids, offsets, xq, xs)
    y_rows, h = expert_ffn(xq_rows, xs_rows, offsets, routed)
    y_shared = None
    if shared is not None:
        T = xq.shape[0]
        y_shared = expert_ffn(xq, xs, np.array([0, T]), shared)[0]
    exact = combine(y_rows, pair_to_row, w, y_shared, norm_gamma, norm_eps, rounded=False)
    return dict(topk_ids=ids, topk_w=w, xq=xq, xs=xs, counts=counts, offsets=offsets,
                pair_to_row=pair_to_row, row_to_pair=row_to_pair, xq_rows=xq_rows,
                xs_rows=xs_rows, h=h, y_rows=y_rows, y_shared=y_shared,
                out_exact=exact, out=bf16_encode(exact))


def forward_sampled(x_bf16, logits, top_k, routed, tokens, shared=None,
                    norm_gamma=None, norm_eps=1e-6, routing=None, score="softmax"):
    """The layer's output for a subset of tokens only (rows are independent).

    Routing runs for all tokens (or is taken from ``routing`` = (topk_ids,
    topk_w) as returned by ``route``); quantisation, permutation, FFN and
    combine run only for the pairs of ``tokens``.  Returns the float64 output
    before its bf16 rounding, shape [len(tokens)][H] (row i is token
    tokens[i]).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    ids, w = route(logits, top_k, score) if routing is None else routing
    xq, xs = quantize_tokens(np.asarray(x_bf16)[tokens])
    sub_ids = ids[tokens]
    _, sub_off = expert_counts_offsets(sub_ids, routed.n_experts)
    sub_p2r, _, sub_q, sub_s = permute_rows(sub_ids, sub_off, xq, xs)
    y_sub = expert_ffn(sub_q, sub_s, sub_off, routed)[0]
    y_shared = None
    if shared is not None:
        y_shared = expert_ffn(xq, xs, np.array([0, len(tokens)]), shared)[0]
    return combine(y_sub, sub_p2r, w[tokens], y_shared, norm_gamma, norm_eps, rounded=False)
