"""The LatentMoE block around the routed expert core, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

*Kimi K3 on TPU*, §2.4 "LatentMoE" gives the block's three parts, and §2.5
says which of their weights are MXFP4:

  hidden x [T][Hm]
    -> routed_expert_down_proj   Hm -> L  (MXFP4 weights)        -> latent
    -> routed experts, top-k of E, each L -> I -> L, and
       routed_expert_norm (RMSNorm on the weighted routed sum)
    -> routed_expert_up_proj     L -> Hm  (MXFP4 weights)
  + shared experts on the hidden stream, Hm -> Is -> Hm (bf16 weights: the
    quantisation's ignore list names them)

The routed core between the projections is ``moe.forward`` with RMSNorm and
no shared expert.

Readings (the page gives the wiring, not the number formats between steps):
  * the projections are weight-only MXFP4: their input stays bf16, the
    weights decode exactly to e2m1 * 2^e, the products are summed exactly;
  * the latent is rounded once to bf16 (the dtype of activations between
    operations) and is the core's bf16 token input (quantised per token to
    fp8 inside the core, as in the plain layer);
  * the core's output (the normalised routed sum) is rounded to bf16 before
    the up-projection;
  * the shared experts' gated FFN reads the bf16 hidden x with bf16 weights
    (nothing quantised), rounds h to bf16, and its output is added to the
    up-projection in float64, then rounded once to bf16.
"""

import numpy as np

from . import moe
from .codecs import bf16_decode, bf16_encode, mxfp4_decode


class LinearWeights:
    """One dense projection y = a W^T with W [N][K].

    fmt "mxfp4": w uint8 [N][K/2] (two e2m1 per byte, element 2i in the low
                 nibble), s uint8 [N][K/32] (e8m0 per 32 consecutive inputs).
    fmt "bf16":  w uint16 [N][K] (bfloat16 bits), s None.
    """

    def __init__(self, fmt, w, s=None):
        if fmt not in ("mxfp4", "bf16"):
            raise ValueError(fmt)
        self.fmt = fmt
        self.w = np.asarray(w)
        self.s = None if s is None else np.asarray(s)
        self.n_out = self.w.shape[0]
        self.n_in = self.w.shape[1] * (2 if fmt == "mxfp4" else 1)

    def decode(self):
        """W as float64 [N][K]."""
        if self.fmt == "mxfp4":
            return mxfp4_decode(self.w, self.s)
        return bf16_decode(self.w)


def linear(a, weights):
    """a [M][K] float64 times W^T: the exact float64 sums of the products."""
    return np.asarray(a, dtype=np.float64) @ weights.decode().T


class DenseFFN:
    """The shared experts as one gated FFN with bf16 weights: w1 (gate), w3
    (up) uint16 [Is][Hm], w2 uint16 [Hm][Is]; activation as for the routed
    experts ("silu" or "situ" with beta)."""

    def __init__(self, w1, w3, w2, activation="silu", beta=4.0):
        if activation not in ("silu", "situ") or not beta > 0:
            raise ValueError(activation)
        self.w1, self.w3, self.w2 = (LinearWeights("bf16", w) for w in (w1, w3, w2))
        self.activation = activation
        self.beta = float(beta)


def dense_ffn(x, ffn):
    """x float64 [T][Hm] (bf16 values): g = x W1^T, u = x W3^T,
    h = bf16(act(g) * u), y = h W2^T.  Returns (y float64, h uint16 bits)."""
    g = linear(x, ffn.w1)
    u = linear(x, ffn.w3)
    h = bf16_encode(moe.activate(g, ffn) * u)
    return linear(bf16_decode(h), ffn.w2), h


def latent_forward(x_bf16, logits, top_k, down, routed, up, shared=None, norm_gamma=None,
                   norm_eps=1e-6, score="softmax"):
    """The whole block.  x_bf16 uint16 [T][Hm]; logits float32 [T][E];
    down / up LinearWeights (Hm -> L, L -> Hm); routed ExpertWeights over L;
    shared DenseFFN or None; norm_gamma float [L] (the core's RMSNorm).
    Returns a dict with the latent (bf16 bits), the core's result dict, the
    up-projection and shared outputs (float64), ``out_exact`` (float64) and
    ``out`` (uint16 bf16)."""
    X = bf16_decode(x_bf16)
    lat = bf16_encode(linear(X, down))
    core = moe.forward(lat, logits, top_k, routed, None, norm_gamma, norm_eps, score)
    y_up = linear(bf16_decode(core["out"]), up)
    y_shared = dense_ffn(X, shared)[0] if shared is not None else None
    exact = y_up if y_shared is None else y_up + y_shared
    return dict(lat=lat, core=core, up=y_up, y_shared=y_shared, out_exact=exact, out=bf16_encode(exact))


def latent_forward_sampled(x_bf16, logits, top_k, down, routed, up, tokens, shared=None,
                           norm_gamma=None, norm_eps=1e-6, score="softmax", routing=None):
    """The block's float64 output (before the final bf16 rounding) for a
    subset of tokens (every step is per token once routing is done).
    Routing runs on all tokens, or is taken from ``routing`` = (ids, w)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    ids, w = moe.route(logits, top_k, score) if routing is None else routing
    X = bf16_decode(np.asarray(x_bf16)[tokens])
    lat = bf16_encode(linear(X, down))
    n = len(tokens)
    core = moe.forward_sampled(lat, None, top_k, routed, np.arange(n), norm_gamma=norm_gamma,
                               norm_eps=norm_eps, routing=(ids[tokens], w[tokens]))
    y = linear(bf16_decode(bf16_encode(core)), up)
    if shared is not None:
        y = y + dense_ffn(X, shared)[0]
    return y
