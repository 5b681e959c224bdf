"""Pins of the oracle's LatentMoE block (*Kimi K3 on TPU*, §2.4 LatentMoE:
down-projection to the latent, routed experts with routed_expert_norm,
up-projection back to the hidden size, shared experts on the hidden stream;
§2.5: the projections are MXFP4, the shared experts bf16).

Each check uses exactly representable weights chosen so the result follows
from the definition by hand (selection matrices, a closed form through scipy's
expit), a library routine (torch's linear in float64), an exact invariance, or
the already pinned routed core; none compares the oracle with itself.
"""

import numpy as np
import pytest
import scipy.special
import torch

import moe_synth
from oracle import codecs, latent, moe
from oracle.latent import DenseFFN, LinearWeights
from oracle.moe import ExpertWeights

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mx(w):
    """float [N][K] -> MXFP4 LinearWeights through the input generator's
    quantiser (exact for the values used here)."""
    q, s = moe_synth.mxfp4_rows(torch.as_tensor(np.asarray(w, np.float32)))
    return LinearWeights("mxfp4", q.numpy(), s.numpy())


def bf16_bits(v):
    return codecs.bf16_encode(np.asarray(v, np.float64))


def rng(seed):
    return np.random.default_rng(seed)


def exact_mx_matrix(r, N, K):
    """Values of e2m1 x 2^j with every 32-block holding a +-4 or +-6, so the
    quantiser's block scale is 2^j and every element is exact."""
    W = r.choice(E2M1, (N, K)) * r.choice([-1.0, 1.0], (N, K))
    W[:, ::32] = r.choice([4.0, -4.0, 6.0, -6.0], (N, K // 32))
    j = r.integers(-6, 3, (N, K // 32))
    return W * np.repeat(np.ldexp(1.0, j), 32, axis=1)


# ----------------------------------------------------------------------------
# projections
# ----------------------------------------------------------------------------


def check_linear_exact(linear_fn=latent.linear):
    """An MXFP4 projection of exactly representable weights equals the float64
    product a @ W^T (W [N][K]: N outputs, K inputs; N != K so that a
    transposed operand cannot pass)."""
    r = rng(1)
    W = exact_mx_matrix(r, 48, 96)
    a = codecs.bf16_decode(bf16_bits(r.standard_normal((5, 96))))
    got = linear_fn(a, mx(W))
    assert got.shape == (5, 48)
    assert np.array_equal(got, a @ W.T)


def test_linear_exact():
    check_linear_exact()


def test_linear_bf16_weights_against_torch():
    r = rng(2)
    Wb = bf16_bits(r.standard_normal((40, 64)) * 0.1)
    a = codecs.bf16_decode(bf16_bits(r.standard_normal((7, 64))))
    got = latent.linear(a, LinearWeights("bf16", Wb))
    ref = torch.nn.functional.linear(torch.from_numpy(a),
                                     torch.from_numpy(Wb.view(np.int16)).view(torch.bfloat16).double()).numpy()
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------
# shared experts (bf16 gated FFN)
# ----------------------------------------------------------------------------


def selection(n_out, n_in, cols, scale=1.0):
    """[n_out][n_in] with row i holding `scale` at column cols[i] (rows past
    len(cols) zero)."""
    W = np.zeros((n_out, n_in))
    W[np.arange(len(cols)), cols] = scale
    return W


def check_shared_closed_form(forward=latent.latent_forward, activation="silu"):
    """Shared experts W1 = 2*[I|0], W3 = [I|0], W2 = [I;0] over Is = 32 of the
    Hm = 128 hidden units, and an all-zero up-projection: out_exact[t][i] for
    i < 32 is bf16(act(2 x) * x) (h rounded once to bf16), 0 beyond."""
    T, Hm, L, I, E, k, Is = 6, 128, 64, 64, 4, 2, 32
    r = rng(3)
    x = bf16_bits(r.standard_normal((T, Hm)) * 2.0)
    inp = moe_synth.custom_inputs(T, L, I, E, k, fmt="mxfp4", seed=3, norm=True)
    routed = ExpertWeights("mxfp4", *(inp["routed"][n].numpy() for n in ("w1", "w3", "w2", "s1", "s3", "s2")))
    cols = np.arange(Is)
    sh = DenseFFN(bf16_bits(selection(Is, Hm, cols, 2.0)), bf16_bits(selection(Is, Hm, cols)),
                  bf16_bits(selection(Hm, Is, cols)), activation=activation)
    down = mx(selection(L, Hm, np.arange(L)))
    up = mx(np.zeros((Hm, L)))
    res = forward(x, inp["logits"].numpy(), k, down, routed, up, sh, np.ones(L), 1e-6)
    X = codecs.bf16_decode(x)
    g = 2.0 * X[:, :Is]
    act = g * scipy.special.expit(g) if activation == "silu" else 4.0 * np.tanh(g / 4.0) * scipy.special.expit(g)
    want = np.zeros((T, Hm))
    want[:, :Is] = codecs.bf16_decode(bf16_bits(act * X[:, :Is]))
    assert np.array_equal(res["out_exact"], want)


@pytest.mark.parametrize("activation", ["silu", "situ"])
def test_shared_closed_form(activation):
    check_shared_closed_form(activation=activation)


def test_dense_ffn_against_torch():
    """The shared FFN against torch's float64 linear / sigmoid / tanh with h
    rounded to bf16 by torch (via binary32: a double rounding that can move
    an h by one bf16 step, rarely)."""
    r = rng(4)
    Hm, Is, T = 96, 64, 9
    w1, w3 = (bf16_bits(r.standard_normal((Is, Hm)) * 0.05) for _ in range(2))
    w2 = bf16_bits(r.standard_normal((Hm, Is)) * 0.05)
    X = codecs.bf16_decode(bf16_bits(r.standard_normal((T, Hm))))
    for act in ("silu", "situ"):
        y, h = latent.dense_ffn(X, DenseFFN(w1, w3, w2, activation=act))
        t = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double()  # noqa: E731
        F = torch.nn.functional
        xt = torch.from_numpy(X)
        g, u = F.linear(xt, t(w1)), F.linear(xt, t(w3))
        a = g * torch.sigmoid(g) if act == "silu" else 4.0 * torch.tanh(g / 4.0) * torch.sigmoid(g)
        ht = (a * u).float().bfloat16()
        hb = ht.view(torch.int16).numpy().view(np.uint16)
        diff = np.abs(h.astype(np.int32) - hb.astype(np.int32))
        assert diff.max() <= 1 and (diff == 0).mean() > 0.99
        ok = (diff == 0).all(axis=1)
        yt = F.linear(ht.double(), t(w2)).numpy()
        assert ok.any() and np.allclose(y[ok], yt[ok], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# the block's wiring
# ----------------------------------------------------------------------------


def wiring_case(seed=5):
    T, Hm, L, I, E, k = 24, 128, 64, 64, 4, 2
    r = rng(seed)
    x = bf16_bits(r.standard_normal((T, Hm)))
    inp = moe_synth.custom_inputs(T, L, I, E, k, fmt="mxfp4", seed=seed, norm=True)
    routed = ExpertWeights("mxfp4", *(inp["routed"][n].numpy() for n in ("w1", "w3", "w2", "s1", "s3", "s2")))
    perm = r.permutation(Hm)[:L]          # the latent unit i reads hidden unit perm[i]
    q = r.permutation(Hm)[:L]             # latent unit i lands on hidden unit q[i]
    down = mx(selection(L, Hm, perm))
    up_w = np.zeros((Hm, L))
    up_w[q, np.arange(L)] = 1.0
    gamma = 1.0 + 0.25 * r.integers(-2, 3, L)
    return x, inp["logits"].numpy(), k, down, routed, mx(up_w), gamma, perm, q


def check_wiring_by_selection(forward=latent.latent_forward):
    """Selection-matrix projections: the block's output on hidden unit q[i] is
    the routed core's (RMS-normalised) output i for the latent x[:, perm],
    bit for bit; every other hidden unit is 0."""
    x, logits, k, down, routed, up, gamma, perm, q = wiring_case()
    res = forward(x, logits, k, down, routed, up, None, gamma, 1e-6)
    core = moe.forward(np.ascontiguousarray(x[:, perm]), logits, k, routed, None, gamma, 1e-6)["out"]
    assert np.array_equal(res["out"][:, q], core)
    rest = np.setdiff1d(np.arange(x.shape[1]), q)
    assert (res["out_exact"][:, rest] == 0).all()


def test_wiring_by_selection():
    check_wiring_by_selection()


def test_power_of_two_scalings():
    """Without shared experts and with eps = 0: doubling every routed W2 block
    scale changes nothing (the routed sum doubles exactly and the RMSNorm,
    which sits before the up-projection, removes the factor); doubling every
    up-projection block scale doubles the output exactly (the up-projection is
    the last, linear step)."""
    T, Hm, L, I, E, k = 16, 256, 128, 64, 4, 2
    blk = moe_synth.latent_block_inputs(T, Hm, L, I, E, k, 0, cfg=7)
    down, up = (LinearWeights("mxfp4", blk[n]["w"].numpy(), blk[n]["s"].numpy()) for n in ("down", "up"))
    rw = {n: blk["routed"][n].numpy() for n in ("w1", "w3", "w2", "s1", "s3", "s2")}
    routed = ExpertWeights("mxfp4", *(rw[n] for n in ("w1", "w3", "w2", "s1", "s3", "s2")))
    routed2 = ExpertWeights("mxfp4", rw["w1"], rw["w3"], rw["w2"], rw["s1"], rw["s3"], rw["s2"] + 1)
    up2 = LinearWeights("mxfp4", up.w, up.s + 1)
    x = blk["x"].view(torch.int16).numpy().view(np.uint16)
    lg = blk["logits"].numpy()
    a = latent.latent_forward(x, lg, k, down, routed, up, None, np.ones(L), 0.0)
    b = latent.latent_forward(x, lg, k, down, routed2, up, None, np.ones(L), 0.0)
    c = latent.latent_forward(x, lg, k, down, routed, up2, None, np.ones(L), 0.0)
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(c["out_exact"], 2.0 * a["out_exact"])


def test_sampled_matches_full():
    T, Hm, L, I, E, k, Is = 20, 128, 64, 64, 8, 3, 64
    blk = moe_synth.latent_block_inputs(T, Hm, L, I, E, k, Is, cfg=8)
    down, up = (LinearWeights("mxfp4", blk[n]["w"].numpy(), blk[n]["s"].numpy()) for n in ("down", "up"))
    routed = ExpertWeights("mxfp4", *(blk["routed"][n].numpy() for n in ("w1", "w3", "w2", "s1", "s3", "s2")))
    sh = DenseFFN(*(blk["shared"][n].view(torch.int16).numpy().view(np.uint16) for n in ("w1", "w3", "w2")))
    x = blk["x"].view(torch.int16).numpy().view(np.uint16)
    full = latent.latent_forward(x, blk["logits"].numpy(), k, down, routed, up, sh, np.ones(L), 1e-6)
    tok = np.array([0, 3, 7, 19])
    part = latent.latent_forward_sampled(x, blk["logits"].numpy(), k, down, routed, up, tok, sh,
                                         np.ones(L), 1e-6)
    assert np.allclose(part, full["out_exact"][tok], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# planted mistakes
# ----------------------------------------------------------------------------


def forward_norm_after_up(x, logits, k, down, routed, up, shared=None, gamma=None, eps=1e-6, score="softmax"):
    """RMSNorm moved from the latent core to after the up-projection."""
    X = codecs.bf16_decode(x)
    lat = codecs.bf16_encode(latent.linear(X, down))
    core = moe.forward(lat, logits, k, routed, None, None, eps, score)["out"]
    y = latent.linear(codecs.bf16_decode(core), up)
    y = moe.rms_norm(y, np.ones(y.shape[1]), eps)
    if shared is not None:
        y = y + latent.dense_ffn(X, shared)[0]
    return dict(out_exact=y, out=codecs.bf16_encode(y))


def forward_skip_down(x, logits, k, down, routed, up, shared=None, gamma=None, eps=1e-6, score="softmax"):
    """The core reads the first L hidden units instead of the down-projection."""
    L = down.n_out
    core = moe.forward(np.ascontiguousarray(x[:, :L]), logits, k, routed, None, gamma, eps, score)["out"]
    y = latent.linear(codecs.bf16_decode(core), up)
    if shared is not None:
        y = y + latent.dense_ffn(codecs.bf16_decode(x), shared)[0]
    return dict(out_exact=y, out=codecs.bf16_encode(y))


def linear_transposed_blocks(a, weights):
    """Scales applied along the wrong axis: each e8m0 scale of row n used for
    column block n's elements instead (a plausible layout slip)."""
    vals = codecs.e2m1_decode(codecs.e2m1_unpack(weights.w))
    sc = codecs.e8m0_decode(weights.s)
    W = vals * np.repeat(sc, 32, axis=1)[:, ::-1]
    return np.asarray(a, np.float64) @ W.T


def dense_ffn_unrounded_h(x, ffn):
    g = latent.linear(x, ffn.w1)
    u = latent.linear(x, ffn.w3)
    h = moe.activate(g, ffn) * u                                       # h kept in float64
    return latent.linear(h, ffn.w2), codecs.bf16_encode(h)


CASES = [
    ("RMSNorm after the up-projection", lambda mp: None,
     lambda: check_wiring_by_selection(forward_norm_after_up)),
    ("down-projection skipped", lambda mp: None, lambda: check_wiring_by_selection(forward_skip_down)),
    ("block scales along the wrong axis", lambda mp: None, lambda: check_linear_exact(linear_transposed_blocks)),
    ("shared h not rounded to bf16", lambda mp: mp.setattr(latent, "dense_ffn", dense_ffn_unrounded_h),
     check_shared_closed_form),
]


@pytest.mark.parametrize("name,patch,check", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, patch, check):
    patch(monkeypatch)
    with pytest.raises(AssertionError):
        check()
