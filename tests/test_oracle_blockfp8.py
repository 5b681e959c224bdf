"""Pins of the oracle's per-block fp8 weights (*Ling-2.6-1T on TPU*, §5:
per-block scaling, out[m,n] = sum_k A[m,k] W[k,n] scale[block(k), n]; block
shape 128 x 128 as in the block-wise fp8 format of *Kimi K3 on TPU*, §3.7).

Checks: a hand-worked closed form with two K blocks and two channel blocks,
the reduction to per-channel fp8 when every channel block has one scale for
all its K blocks, a per-element brute-force loop of the definition, and
planted mistakes in the block indexing.
"""

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from oracle import codecs, moe
from oracle.moe import ExpertWeights

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

ONE = 0x38       # e4m3 code of 1.0


def closed_form_expert():
    """H = I = 256 (2 x 2 blocks), all weight codes 1.0.
    s1 = [[1, 2], [4, 8]] (channel block x K block), s3 = 1, s2 = [[3, 1], [3, 1]]."""
    w = np.full((1, 256, 256), ONE, np.uint8)
    s1 = np.array([[[1.0, 2.0], [4.0, 8.0]]], np.float32)
    s3 = np.ones((1, 2, 2), np.float32)
    s2 = np.array([[[3.0, 1.0], [3.0, 1.0]]], np.float32)
    return ExpertWeights("fp8_block", w, w, w, s1, s3, s2)


def check_closed_form(forward=oracle.forward):
    """One token x = [1]*128 + [2]*128 -> amax 2, xs = 2/448, codes 224 and 448.
    Gate channel block 0: xs*(1*128*224 + 2*128*448) = 640; block 1:
    xs*(4*128*224 + 8*128*448) = 2560; up: xs*(128*224 + 128*448) = 384.
    h = bf16(g * sigmoid(g) * u) = 245760 and 983040 (exact in bf16).
    y_j = 3*128*245760 + 1*128*983040 = 220200960 for every j (k = 1, w = 1)."""
    x = codecs.bf16_encode(np.array([[1.0] * 128 + [2.0] * 128]))
    res = forward(x, np.zeros((1, 1), np.float32), 1, closed_form_expert())
    h = codecs.bf16_decode(res["h"])
    assert (h[0, :128] == 245760.0).all() and (h[0, 128:] == 983040.0).all()
    assert (res["out_exact"] == 220200960.0).all()


def test_closed_form():
    check_closed_form()


def test_reduces_to_per_channel():
    """Scales constant over the K blocks of each channel block: the same
    outputs as per-channel fp8 with scale[n] = c[n // 128] (pinned apart)."""
    r = np.random.default_rng(3)
    E, H, I, T, k = 3, 256, 384, 12, 2
    inp = moe_synth.custom_inputs(T, H, I, E, k, fmt="fp8", seed=4)
    x = inp["x"].view(torch.int16).numpy().view(np.uint16)
    logits = inp["logits"].numpy()
    w = {n: inp["routed"][n].numpy() for n in ("w1", "w3", "w2")}
    c1, c3 = (r.uniform(0.5, 2.0, (E, I // 128)).astype(np.float32) for _ in range(2))
    c2 = r.uniform(0.5, 2.0, (E, H // 128)).astype(np.float32)
    blk = ExpertWeights("fp8_block", w["w1"], w["w3"], w["w2"],
                        np.repeat(c1[:, :, None], H // 128, axis=2), np.repeat(c3[:, :, None], H // 128, axis=2),
                        np.repeat(c2[:, :, None], I // 128, axis=2))
    chan = ExpertWeights("fp8", w["w1"], w["w3"], w["w2"], np.repeat(c1, 128, axis=1),
                         np.repeat(c3, 128, axis=1), np.repeat(c2, 128, axis=1))
    a = oracle.forward(x, logits, k, blk)
    b = oracle.forward(x, logits, k, chan)
    assert np.allclose(a["out_exact"], b["out_exact"], rtol=1e-13, atol=1e-13 * np.abs(b["out_exact"]).max())
    assert (a["out"] == b["out"]).mean() > 0.999


def check_brute_force(decode=None):
    """Every element of the block-scaled gate projection against a loop over
    k of a[k] * W[n][k] * scale[n // 128][k // 128]."""
    r = np.random.default_rng(5)
    I, H = 256, 384
    w = moe_synth.expert_weights(11, "cpu", "fp8_block", 1, H, I)
    Wb = ExpertWeights("fp8_block", *(w[n].numpy() for n in ("w1", "w3", "w2", "s1", "s3", "s2")))
    W1 = (decode or Wb.decode)(0)[0]
    a = r.standard_normal(H)
    codes = codecs.e4m3_decode(w["w1"][0].numpy())
    sc = w["s1"][0].numpy().astype(np.float64)
    got = W1 @ a
    for n in range(0, I, 37):
        want = 0.0
        for kk in range(H):
            want += a[kk] * codes[n, kk] * sc[n // 128, kk // 128]
        assert got[n] == pytest.approx(want, rel=1e-12)


def test_brute_force():
    check_brute_force()


# ----------------------------------------------------------------------------
# planted mistakes
# ----------------------------------------------------------------------------


def block_scaled_transposed(W, scales, block=128):
    sc = np.asarray(scales, dtype=np.float64).T                       # K block indexes rows
    return W * np.repeat(np.repeat(sc, block, axis=0), block, axis=1)


def block_scaled_first_k_block(W, scales, block=128):
    sc = np.asarray(scales, dtype=np.float64)
    sc = np.repeat(sc[:, :1], sc.shape[1], axis=1)                    # K block ignored
    return W * np.repeat(np.repeat(sc, block, axis=0), block, axis=1)


def decode_first_k_block(e):
    w = moe_synth.expert_weights(11, "cpu", "fp8_block", 1, 384, 256)
    W = codecs.e4m3_decode(w["w1"][0].numpy())
    return (block_scaled_first_k_block(W, w["s1"][0].numpy()),)


CASES = [
    ("scale indexed [K block][channel block]", lambda mp: mp.setattr(moe, "block_scaled", block_scaled_transposed),
     check_closed_form),
    ("K block ignored", lambda mp: mp.setattr(moe, "block_scaled", block_scaled_first_k_block), check_closed_form),
    ("K block ignored (brute force)", lambda mp: None, lambda: check_brute_force(decode_first_k_block)),
]


@pytest.mark.parametrize("name,patch,check", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, patch, check):
    patch(monkeypatch)
    with pytest.raises(AssertionError):
        check()
