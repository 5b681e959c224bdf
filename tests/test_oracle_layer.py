"""Pins of the oracle's layer steps against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check uses brute force,
a textbook or library routine (scipy softmax, NumPy stable argsort, torch's
silu / linear / float8 cast), a closed form worked by hand, or an invariant
of the method (token-permutation equivariance, zero routing weights,
power-of-two linearity, the MXFP4 / fp8 cross-format identity).
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import codecs
from oracle.moe import ExpertWeights


def rng(seed=0):
    return np.random.default_rng(seed)


def bf16_bits(values):
    t = torch.from_numpy(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def random_fp8_weights(E, H, I, seed=0):
    r = rng(seed)

    def mat(n, k):
        w = (r.standard_normal((E, n, k)) * 0.02).astype(np.float32)
        s = (np.abs(w).max(axis=2) / 448.0).astype(np.float32)
        q = torch.from_numpy(w / s[..., None]).clamp(-448, 448).to(torch.float8_e4m3fn)
        return q.view(torch.uint8).numpy(), s

    w1, s1 = mat(I, H)
    w3, s3 = mat(I, H)
    w2, s2 = mat(H, I)
    return ExpertWeights("fp8", w1, w3, w2, s1, s3, s2)


def small_case(T=24, H=64, I=32, E=5, k=2, seed=0):
    r = rng(seed)
    x = bf16_bits(r.standard_normal((T, H)))
    logits = r.standard_normal((T, E)).astype(np.float32)
    return x, logits, random_fp8_weights(E, H, I, seed + 1), k


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------


def check_route_brute_force(route=oracle.route):
    r = rng(3)
    for E, k in ((4, 1), (6, 3), (9, 9), (16, 4)):
        # small integers make exact ties frequent
        logits = r.integers(-3, 3, (40, E)).astype(np.float32)
        ids, w = route(logits, k)
        for t in range(logits.shape[0]):
            order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
            assert list(ids[t]) == order
            sel = logits[t, order].astype(np.float64)
            assert np.allclose(w[t], scipy.special.softmax(sel), rtol=1e-13, atol=0)
        assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-14)


def test_route_brute_force():
    check_route_brute_force()


def check_route_full_softmax(route=oracle.route):
    # k = E: the weights are the textbook softmax over all experts
    logits = rng(4).standard_normal((10, 7)).astype(np.float32)
    ids, w = route(logits, 7)
    ref = scipy.special.softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(ref, ids.astype(np.int64), axis=1), rtol=1e-13, atol=0)
    assert (np.diff(np.take_along_axis(logits, ids.astype(np.int64), axis=1), axis=1) <= 0).all()


def test_route_full_softmax():
    check_route_full_softmax()


def check_route_ties(route=oracle.route):
    # all equal -> ids 0..k-1, weights exactly 1/k
    ids, w = route(np.zeros((3, 8), dtype=np.float32), 4)
    assert (ids == np.arange(4)).all() and (w == 0.25).all()
    # -0.0 and +0.0 tie; the lower index comes first in either sign arrangement
    l = np.array([[-1.0, 0.0, -0.0, -2.0], [-1.0, -0.0, 0.0, -2.0]], dtype=np.float32)
    ids, _ = route(l, 2)
    assert ids.tolist() == [[1, 2], [1, 2]]


def test_route_ties():
    check_route_ties()


# ----------------------------------------------------------------------------
# activation quantisation
# ----------------------------------------------------------------------------


def check_quantize(quantize=oracle.quantize_tokens):
    r = rng(5)
    xf = r.standard_normal((32, 96)).astype(np.float32)
    x = bf16_bits(xf)
    q, s = quantize(x)
    xv = codecs.bf16_decode(x).astype(np.float32)
    # the amax element always encodes to +-448 (0x7E / 0xFE)
    i = np.argmax(np.abs(xv), axis=1)
    amax_codes = q[np.arange(32), i]
    assert set(amax_codes.tolist()) <= {0x7E, 0xFE}
    # codes agree with torch's float8 cast of x / s (binary32 division)
    s_ref = (np.abs(xv).max(axis=1) / np.float32(448.0)).astype(np.float32)
    assert (s == s_ref).all()
    ref = torch.from_numpy(xv / s_ref[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
    assert (q == ref.view(torch.uint8).numpy()).all()
    # scaling a row by 2^j leaves the codes and scales s by exactly 2^j
    for j in (-5, 3):
        q2, s2 = quantize(bf16_bits(xv * np.float32(2.0 ** j)))
        assert (q2 == q).all() and (s2 == s * np.float32(2.0 ** j)).all()
    # a zero row: s = 1 and codes are signed zeros
    z = bf16_bits(np.array([[0.0, -0.0, 0.0]], dtype=np.float32))
    qz, sz = quantize(z)
    assert sz[0] == 1.0 and qz[0].tolist() == [0x00, 0x80, 0x00]


def test_quantize():
    check_quantize()


# ----------------------------------------------------------------------------
# counts, offsets, permutation
# ----------------------------------------------------------------------------


def check_permutation(counts_offsets=oracle.expert_counts_offsets, permute=oracle.permute_rows):
    r = rng(6)
    T, E, k, H = 50, 7, 3, 16
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[:5] = ids[0]                                   # repeated routing pattern
    xq = r.integers(0, 256, (T, H)).astype(np.uint8)
    xs = r.random(T).astype(np.float32)
    counts, offsets = counts_offsets(ids, E)
    assert counts.tolist() == np.bincount(ids.ravel(), minlength=E).tolist()
    assert offsets[0] == 0 and offsets[-1] == T * k and (np.diff(offsets) == counts).all()
    p2r, r2p, xq_rows, xs_rows = permute(ids, offsets, xq, xs)
    # rows in expert order, within an expert by pair index: NumPy's stable argsort
    assert (r2p == np.argsort(ids.ravel(), kind="stable")).all()
    assert (p2r.ravel()[r2p] == np.arange(T * k)).all()      # inverse
    for t in range(T):                                    # position by position
        for j in range(k):
            rr = p2r[t, j]
            assert offsets[ids[t, j]] <= rr < offsets[ids[t, j] + 1]
            assert (xq_rows[rr] == xq[t]).all() and xs_rows[rr] == xs[t]


def test_permutation():
    check_permutation()


def test_permutation_empty_experts_and_one_expert():
    ids = np.full((6, 1), 3, dtype=np.int32)
    counts, offsets = oracle.expert_counts_offsets(ids, 5)
    assert counts.tolist() == [0, 0, 0, 6, 0] and offsets.tolist() == [0, 0, 0, 0, 6, 6]


# ----------------------------------------------------------------------------
# expert FFN and combine
# ----------------------------------------------------------------------------


def check_closed_form(forward=oracle.forward):
    """One token, H=2, I=1, one expert, worked by hand.

    x = [448, 224] -> s = 1, codes exact.  W1 = [2^-8, 0] -> g = 1.75;
    W3 = [0, 2^-7] with s3 = 2 -> u = 3.5.  h = bf16(SiLU(1.75) * 3.5) and
    W2 = [1, -0.5] gives y = [h, -h/2].  A swapped gate/up would give
    SiLU(3.5) * 1.75 instead.
    """
    x = bf16_bits(np.array([[448.0, 224.0]]))
    w1 = np.array([[[0x02, 0x00]]], dtype=np.uint8)          # 2 * 2^-9, 0
    w3 = np.array([[[0x00, 0x04]]], dtype=np.uint8)          # 0, 4 * 2^-9
    w2 = np.array([[[0x38], [0xB0]]], dtype=np.uint8)        # 1.0, -0.5
    W = ExpertWeights("fp8", w1, w3, w2, np.array([[1.0]], np.float32),
                      np.array([[2.0]], np.float32), np.array([[1.0, 1.0]], np.float32))
    out = forward(x, np.zeros((1, 1), np.float32), 1, W)["out"]
    h = 1.75 / (1.0 + math.exp(-1.75)) * 3.5
    got = codecs.bf16_decode(out)[0]
    assert got[0] == pytest.approx(h, rel=2 ** -8) and got[1] == pytest.approx(-h / 2, rel=2 ** -8)


def test_closed_form():
    check_closed_form()


def check_dense_reduction(forward=oracle.forward):
    """E = 1, k = 1: the layer is a dense gated FFN on the quantised tokens.

    Reference built from torch library calls in float64: linear, silu, and the
    bfloat16 cast of the intermediate.
    """
    x, _, W, _ = small_case(T=9, H=64, I=48, E=1, k=1, seed=11)
    res = forward(x, np.zeros((9, 1), np.float32), 1, W)
    xq, xs = oracle.quantize_tokens(x)
    A = torch.from_numpy(codecs.e4m3_decode(xq))
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64)  # noqa: E731
    W1, W3, W2 = dec(W.w1[0]), dec(W.w3[0]), dec(W.w2[0])
    xs_t = torch.from_numpy(xs.astype(np.float64))[:, None]
    g = torch.nn.functional.linear(A, W1) * xs_t * torch.from_numpy(W.s1[0].astype(np.float64))
    u = torch.nn.functional.linear(A, W3) * xs_t * torch.from_numpy(W.s3[0].astype(np.float64))
    h = (torch.nn.functional.silu(g) * u).to(torch.float32).to(torch.bfloat16).to(torch.float64)
    y = torch.nn.functional.linear(h, W2) * torch.from_numpy(W.s2[0].astype(np.float64))
    ref = y.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # the oracle rounds float64 -> bf16 once; torch goes via binary32: allow 1 ulp
    diff = np.abs(res["out"].astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1 and (diff == 0).mean() > 0.97


def test_dense_reduction():
    check_dense_reduction()


def brute_force_per_token(x, logits, k, W):
    """Per token, per slot: run the token through its expert directly."""
    ids, w = oracle.route(logits, k)
    xq, xs = oracle.quantize_tokens(x)
    out = np.zeros((x.shape[0], W.hidden))
    for t in range(x.shape[0]):
        for j in range(k):
            e = int(ids[t, j])
            off = np.zeros(W.n_experts + 1, dtype=np.int64)
            off[e + 1:] = 1
            y = oracle.expert_ffn(xq[t:t + 1], xs[t:t + 1], off, W)[0]
            out[t] += w[t, j] * y[0]
    return codecs.bf16_encode(out)


def check_per_token_brute_force(forward=oracle.forward):
    x, logits, W, k = small_case(seed=21)
    assert (forward(x, logits, k, W)["out"] == brute_force_per_token(x, logits, k, W)).all()


def test_per_token_brute_force():
    check_per_token_brute_force()


def check_token_permutation(forward=oracle.forward):
    x, logits, W, k = small_case(seed=31)
    out = forward(x, logits, k, W)["out"]
    perm = rng(9).permutation(x.shape[0])
    out_p = forward(x[perm], logits[perm], k, W)["out"]
    assert (out_p == out[perm]).all()


def test_token_permutation():
    check_token_permutation()


def test_zero_routing_weights_give_zero():
    x, logits, W, k = small_case(seed=41)
    res = oracle.forward(x, logits, k, W)
    out = oracle.combine(res["y_rows"], res["pair_to_row"], np.zeros_like(res["topk_w"]))
    assert (codecs.bf16_decode(out) == 0).all()


def check_power_of_two_linearity(expert_ffn=oracle.expert_ffn):
    x, logits, W, k = small_case(seed=51)
    res = oracle.forward(x, logits, k, W)
    y1 = expert_ffn(res["xq_rows"], res["xs_rows"], res["offsets"], W)[0]
    W2x = ExpertWeights("fp8", W.w1, W.w3, W.w2, W.s1, W.s3, W.s2 * np.float32(2.0))
    y2 = expert_ffn(res["xq_rows"], res["xs_rows"], res["offsets"], W2x)[0]
    assert (y2 == 2.0 * y1).all()


def test_power_of_two_linearity():
    check_power_of_two_linearity()


def check_mxfp4_matches_fp8(forward=oracle.forward):
    """With every e8m0 scale = 127 (2^0) an MXFP4 expert equals an fp8 expert
    holding the same values (e2m1 values are exactly representable in e4m3)
    with per-channel scales 1."""
    r = rng(61)
    T, H, I, E, k = 12, 64, 64, 3, 2
    x = bf16_bits(r.standard_normal((T, H)))
    logits = r.standard_normal((T, E)).astype(np.float32)

    def nib(n, kk):
        return r.integers(0, 16, (E, n, kk)).astype(np.uint8)

    c1, c3, c2 = nib(I, H), nib(I, H), nib(H, I)
    pack = lambda c: (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)  # noqa: E731
    ones = lambda n, kk: np.full((E, n, kk // 32), 127, np.uint8)           # noqa: E731
    Wm = ExpertWeights("mxfp4", pack(c1), pack(c3), pack(c2), ones(I, H), ones(I, H), ones(H, I))
    enc = lambda c: codecs.e4m3_encode(codecs.e2m1_decode(c))                # noqa: E731
    f1 = lambda n: np.ones((E, n), np.float32)                              # noqa: E731
    Wf = ExpertWeights("fp8", enc(c1), enc(c3), enc(c2), f1(I), f1(I), f1(H))
    assert (forward(x, logits, k, Wm)["out"] == forward(x, logits, k, Wf)["out"]).all()
    # and a block scale of 2^1 on W2 doubles y exactly
    Wm2 = ExpertWeights("mxfp4", Wm.w1, Wm.w3, Wm.w2, Wm.s1, Wm.s3, Wm.s2 + np.uint8(1))
    res1 = forward(x, logits, k, Wm)
    res2 = forward(x, logits, k, Wm2)
    assert (res2["y_rows"] == 2.0 * res1["y_rows"]).all()


def test_mxfp4_matches_fp8():
    check_mxfp4_matches_fp8()


def test_rmsnorm_closed_form_and_scale_invariance():
    eps = 1e-6
    c = np.array([[0.5] * 8, [-3.0] * 8])
    out = oracle.moe.rms_norm(c, np.ones(8), eps)
    expect = np.sign(c[:, :1]) / np.sqrt(1.0 + eps / c[:, :1] ** 2)
    assert np.allclose(out, expect, rtol=1e-15)
    r = rng(71).standard_normal((4, 32))
    a = oracle.moe.rms_norm(r, np.ones(32), 0.0)
    b = oracle.moe.rms_norm(37.0 * r, np.ones(32), 0.0)
    assert np.allclose(a, b, rtol=1e-14)
    assert np.allclose(np.mean(a * a, axis=1), 1.0, rtol=1e-14)


def test_shared_expert_added_with_unit_weight():
    x, logits, W, k = small_case(seed=81)
    Ws = random_fp8_weights(1, W.hidden, W.inter, seed=82)
    with_sh = oracle.forward(x, logits, k, W, shared=Ws)
    xq, xs = oracle.quantize_tokens(x)
    y_sh = oracle.expert_ffn(xq, xs, np.array([0, x.shape[0]]), Ws)[0]
    res = oracle.forward(x, logits, k, W)
    o = np.zeros_like(y_sh)
    for j in range(k):
        o += res["topk_w"][:, j, None] * res["y_rows"][res["pair_to_row"][:, j]]
    assert (with_sh["out"] == codecs.bf16_encode(o + y_sh)).all()


def test_forward_sampled_matches_forward():
    x, logits, W, k = small_case(T=30, seed=91)
    Ws = random_fp8_weights(1, W.hidden, W.inter, seed=92)
    full = oracle.forward(x, logits, k, W, shared=Ws)
    toks = np.array([3, 17, 0, 29])
    samp = oracle.moe.forward_sampled(x, logits, k, W, toks, shared=Ws)
    assert (samp == full["out_exact"][toks]).all()
