"""Planted mistakes in the oracle must each fail at least one pin.

Each case patches one plausible error into the oracle (on the CPU only) and
runs the pin that should catch it.  A pin that still passes under the
mutation would be too weak to trust.
"""

import numpy as np
import pytest

import oracle
from oracle import codecs, moe

import test_oracle_codecs as pc
import test_oracle_layer as pl


def route_high_index_ties(logits, k):
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k))
    for t in range(T):
        row = logits[t].astype(np.float64)
        order = np.lexsort((-np.arange(E), -row))[:k]        # wrong tie-break
        ids[t] = order
        p = np.exp(row - row.max())
        w[t] = p[order] / p[order].sum()
    return ids, w


def route_no_renorm(logits, k):
    ids, _ = oracle.route(logits, k)
    l = np.asarray(logits, np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)   # dropped renormalisation


def quantize_fnuz_max(x):
    xv = codecs.bf16_decode(x).astype(np.float32)
    s = (np.abs(xv).max(axis=1) / np.float32(240.0)).astype(np.float32)   # wrong fp8 max
    return codecs.e4m3_encode(xv / s[:, None]), s


def permute_unstable(ids, offsets, xq, xs):
    p2r, r2p, _, _ = oracle.permute_rows(ids, offsets, xq, xs)
    k = ids.shape[1]
    for e in range(len(offsets) - 1):                   # reverse rows inside each segment
        r2p[offsets[e]:offsets[e + 1]] = r2p[offsets[e]:offsets[e + 1]][::-1].copy()
    p2r = np.empty_like(p2r).ravel()
    p2r[r2p] = np.arange(len(r2p))
    tok = r2p // k
    return p2r.reshape(ids.shape), r2p, np.asarray(xq)[tok], np.asarray(xs)[tok]


def decode_swapped_gate_up(self, e):
    W1, W3, W2, c1, c3, c2 = ORIG_DECODE(self, e)
    return W3, W1, W2, c3, c1, c2


def decode_transposed_scale(self, e):
    W1, W3, W2, c1, c3, c2 = ORIG_DECODE(self, e)
    return W1, W3, W2, c1[::-1].copy(), c3, c2


ORIG_DECODE = moe.ExpertWeights.decode


def e4m3_decode_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8)
    v = codecs.e4m3_decode(c) / 2.0                    # exponent bias 8 instead of 7
    return v


def unpack_high_first(p):
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p >> 4                             # nibble order swapped
    out[..., 1::2] = p & 0x0F
    return out


def silu_wrong_sign(z):
    return z / (1.0 + np.exp(z))


def combine_unweighted(y_rows, pair_to_row, topk_w, *a, **kw):
    return ORIG_COMBINE(y_rows, pair_to_row, np.ones_like(topk_w), *a, **kw)


ORIG_COMBINE = moe.combine


def expert_ffn_no_token_scale(xq_rows, xs_rows, offsets, weights):
    return ORIG_FFN(xq_rows, np.ones_like(xs_rows), offsets, weights)


ORIG_FFN = moe.expert_ffn


def bf16_truncate(values):
    f32 = np.asarray(values, dtype=np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)   # truncation, not RNE


CASES = [
    ("route ties to higher index", lambda mp: None, lambda: pl.check_route_brute_force(route_high_index_ties)),
    ("route without renormalisation", lambda mp: None, lambda: pl.check_route_brute_force(route_no_renorm)),
    ("fp8 max 240 instead of 448", lambda mp: None, lambda: pl.check_quantize(quantize_fnuz_max)),
    ("unstable permutation", lambda mp: None,
     lambda: pl.check_permutation(permute=permute_unstable)),
    ("gate and up swapped", lambda mp: mp.setattr(moe.ExpertWeights, "decode", decode_swapped_gate_up),
     pl.check_closed_form),
    ("gate scale reversed", lambda mp: mp.setattr(moe.ExpertWeights, "decode", decode_transposed_scale),
     pl.check_dense_reduction),
    ("e4m3 exponent bias 8", lambda mp: None, lambda: pc.check_e4m3_decode(e4m3_decode_bias8)),
    ("nibble order swapped", lambda mp: None, lambda: pc.check_nibble_order(unpack_high_first)),
    ("SiLU sign error", lambda mp: mp.setattr(moe, "silu", silu_wrong_sign), pl.check_closed_form),
    ("combine ignores routing weights", lambda mp: mp.setattr(moe, "combine", combine_unweighted),
     pl.check_per_token_brute_force),
    ("token scale dropped", lambda mp: mp.setattr(moe, "expert_ffn", expert_ffn_no_token_scale),
     pl.check_dense_reduction),
    ("bf16 by truncation", lambda mp: None, lambda: pc.check_bf16_encode(bf16_truncate)),
]


@pytest.mark.parametrize("name,patch,check", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, patch, check):
    patch(monkeypatch)
    with pytest.raises(AssertionError):
        check()


def test_unmutated_checks_pass():
    pl.check_closed_form()
    pl.check_dense_reduction()
    pl.check_per_token_brute_force()
