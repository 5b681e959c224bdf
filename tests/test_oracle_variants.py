"""Pins of the oracle's router and activation variants.

The Kimi K3 page (§2.4 LatentMoE routing: sigmoid scores, top-k,
renormalised, routed scaling factor 1.0; §2.6 the SiTU activation
beta * tanh(gate / beta) * sigmoid(gate) * up with beta = 4).  Each check
uses a closed form worked by hand, brute force, a library routine (scipy's
expit, torch's tanh / sigmoid / linear), or a limit of the definition; none
compares the oracle with itself.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import codecs, moe
from oracle.moe import ExpertWeights

from test_oracle_layer import bf16_bits, random_fp8_weights, rng, small_case

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ----------------------------------------------------------------------------
# sigmoid router
# ----------------------------------------------------------------------------


def check_sigmoid_route_closed_form(route=oracle.route):
    """logits (ln 3, 0, -5), top-2: sigmoid gives 3/4 and 1/2, renormalised
    3/5 and 2/5; top-1 gives weight 1."""
    logits = np.array([[math.log(3.0), 0.0, -5.0]], np.float32)
    ids, w = route(logits, 2, "sigmoid")
    assert list(ids[0]) == [0, 1]
    l0 = float(np.float32(math.log(3.0)))                    # the binary32 logit the router sees
    s0 = 1.0 / (1.0 + math.exp(-l0))
    assert w[0, 0] == pytest.approx(s0 / (s0 + 0.5), rel=1e-15)
    assert w[0, 0] == pytest.approx(0.6, rel=1e-7) and w[0, 1] == pytest.approx(0.4, rel=1e-7)
    ids1, w1 = route(logits, 1, "sigmoid")
    assert list(ids1[0]) == [0] and w1[0, 0] == 1.0


def test_sigmoid_route_closed_form():
    check_sigmoid_route_closed_form()


def check_sigmoid_route_brute_force(route=oracle.route):
    """Same selection as brute-force sorting; weights = scipy's expit of the
    selected logits, renormalised; they sum to one."""
    r = rng(8)
    for E, k in ((4, 1), (6, 3), (9, 9), (16, 4)):
        logits = np.concatenate([r.integers(-3, 3, (20, E)), r.standard_normal((20, E)) * 3]).astype(np.float32)
        ids, w = route(logits, k, "sigmoid")
        for t in range(logits.shape[0]):
            order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
            assert list(ids[t]) == order
            p = scipy.special.expit(logits[t, order].astype(np.float64))
            assert np.allclose(w[t], p / p.sum(), rtol=1e-13, atol=0)
        assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-14)


def test_sigmoid_route_brute_force():
    check_sigmoid_route_brute_force()


def test_sigmoid_and_softmax_select_alike_but_weigh_differently():
    r = rng(9)
    logits = r.standard_normal((50, 12)).astype(np.float32)
    ids_s, w_s = oracle.route(logits, 4, "softmax")
    ids_g, w_g = oracle.route(logits, 4, "sigmoid")
    assert (ids_s == ids_g).all()
    assert np.abs(w_s - w_g).max() > 1e-3
    # equal logits: both give 1/k
    ids_e, w_e = oracle.route(np.zeros((3, 8), np.float32), 4, "sigmoid")
    assert (ids_e == np.arange(4)).all() and (w_e == 0.25).all()


# ----------------------------------------------------------------------------
# SiTU
# ----------------------------------------------------------------------------


def check_situ_closed_form(situ=moe.situ):
    """g = 2 ln 3, beta = 4: tanh(ln(3) / 2) = 1/2, sigmoid(2 ln 3) = 9/10,
    so SiTU = 4 * 1/2 * 9/10 = 1.8; SiTU(0) = 0; SiTU is odd in its tanh
    factor: SiTU(-g) = -beta tanh(g/beta) sigmoid(-g); for large g it tends
    to beta."""
    g = 2.0 * math.log(3.0)
    assert situ(np.array([g]), 4.0)[0] == pytest.approx(1.8, rel=1e-14)
    assert situ(np.array([0.0]), 4.0)[0] == 0.0
    assert situ(np.array([-g]), 4.0)[0] == pytest.approx(-4.0 * 0.5 * 0.1, rel=1e-13)
    assert situ(np.array([60.0]), 4.0)[0] == pytest.approx(4.0, rel=1e-12)
    # beta -> infinity: tanh(g / beta) * beta -> g, SiTU -> SiLU
    z = np.linspace(-6, 6, 25)
    assert np.allclose(situ(z, 1e7), z * scipy.special.expit(z), rtol=1e-9, atol=1e-12)


def test_situ_closed_form():
    check_situ_closed_form()


def situ_weights(W, beta=4.0):
    return ExpertWeights(W.fmt, W.w1, W.w3, W.w2, W.s1, W.s3, W.s2, activation="situ", beta=beta)


def check_situ_dense_reduction(forward=oracle.forward):
    """E = 1, k = 1 with SiTU: a dense FFN built from torch library calls
    (linear, tanh, sigmoid) in float64, the intermediate cast to bfloat16."""
    x, _, W, _ = small_case(T=9, H=64, I=48, E=1, k=1, seed=13)
    W = situ_weights(W)
    res = forward(x, np.zeros((9, 1), np.float32), 1, W)
    xq, xs = oracle.quantize_tokens(x)
    A = torch.from_numpy(codecs.e4m3_decode(xq))
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64)  # noqa: E731
    W1, W3, W2 = dec(W.w1[0]), dec(W.w3[0]), dec(W.w2[0])
    xs_t = torch.from_numpy(xs.astype(np.float64))[:, None]
    g = torch.nn.functional.linear(A, W1) * xs_t * torch.from_numpy(W.s1[0].astype(np.float64))
    u = torch.nn.functional.linear(A, W3) * xs_t * torch.from_numpy(W.s3[0].astype(np.float64))
    act = 4.0 * torch.tanh(g / 4.0) * torch.sigmoid(g)
    h = (act * u).to(torch.float32).to(torch.bfloat16).to(torch.float64)
    y = torch.nn.functional.linear(h, W2) * torch.from_numpy(W.s2[0].astype(np.float64))
    ref = y.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    diff = np.abs(res["out"].astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1 and (diff == 0).mean() > 0.97


def test_situ_dense_reduction():
    check_situ_dense_reduction()


def test_situ_differs_from_silu_where_the_gate_is_large():
    """Same weights, SiLU vs SiTU: the outputs differ (SiTU bounds the linear
    factor at beta), and agree as beta grows."""
    x, logits, W, k = small_case(seed=17)
    x = bf16_bits(codecs.bf16_decode(x) * 8.0)          # large gates
    a = oracle.forward(x, logits, k, W)["out_exact"]
    b = oracle.forward(x, logits, k, situ_weights(W))["out_exact"]
    c = oracle.forward(x, logits, k, situ_weights(W, beta=1e7))["out_exact"]
    assert np.abs(a - b).max() > 1e-2 * np.abs(a).max()
    assert np.allclose(a, c, rtol=1e-6, atol=1e-9 * np.abs(a).max())


# ----------------------------------------------------------------------------
# planted mistakes
# ----------------------------------------------------------------------------


def route_sigmoid_no_renorm(logits, k, score="softmax"):
    ids, _ = oracle.route(logits, k, score)
    p = 1.0 / (1.0 + np.exp(-np.asarray(logits, np.float64)))
    return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)   # dropped renormalisation


def route_sigmoid_as_softmax(logits, k, score="softmax"):
    return oracle.route(logits, k, "softmax")                         # ignores the score function


def situ_unscaled_tanh(z, beta):
    return beta * np.tanh(z) / (1.0 + np.exp(-z))                     # tanh(z), not tanh(z / beta)


def situ_without_beta(z, beta):
    return np.tanh(z / beta) / (1.0 + np.exp(-z))                     # missing the beta factor


CASES = [
    ("sigmoid route without renormalisation", lambda mp: None,
     lambda: check_sigmoid_route_closed_form(route_sigmoid_no_renorm)),
    ("sigmoid route computed as softmax", lambda mp: None,
     lambda: check_sigmoid_route_brute_force(route_sigmoid_as_softmax)),
    ("SiTU tanh argument not divided by beta", lambda mp: mp.setattr(moe, "situ", situ_unscaled_tanh),
     check_situ_dense_reduction),
    ("SiTU missing its beta factor", lambda mp: None, lambda: check_situ_closed_form(situ_without_beta)),
]


@pytest.mark.parametrize("name,patch,check", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, patch, check):
    patch(monkeypatch)
    with pytest.raises(AssertionError):
        check()
