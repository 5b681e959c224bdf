"""GPU parity of the LatentMoE block (the Kimi K3 page, §2.4-2.5) through the
C ABI against the CPU oracle: the dense projections (moe_linear) and the whole
block (moe_latent_forward).

Bar: routing ids / counts / offsets / permutation bit-exact (they depend on
the logits only); floating-point outputs within max|err| <= 2e-2 * RMS of
the oracle's float64 result.  The projections are checked more tightly,
element by element: within the error bound of an fp32 accumulation of the K
products (K * 2^-24 * sum |a w|) plus, for a bf16 output, half a bf16 step.  The core's quantised rows are not compared byte for byte here: they
depend on the latent, which is a floating-point result of the GPU path.
"""

import numpy as np
import pytest
import torch

import moe_synth
from gpu_helpers import DEV, OUT_TOL, bits, host, say, tolerance_ratio
from oracle import codecs, latent, moe
from oracle.latent import DenseFFN, LinearWeights
from oracle.moe import ExpertWeights

pytestmark = pytest.mark.gpu


def bf16_host(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def acc_bound(a, weights):
    """Per-element bound of an fp32 accumulation of the K products:
    K * 2^-24 * sum_k |a_k w_k| (recursive summation, any order)."""
    a = np.abs(np.asarray(a, np.float64))
    return a.shape[1] * 2.0 ** -24 * (a @ np.abs(weights.decode()).T)


def check_bf16_close(gpu_bits, exact, bound):
    """Each bf16 output within the accumulation bound plus half a bf16 step of
    the exact value; and the layer bar on the whole."""
    g = codecs.bf16_decode(gpu_bits)
    tol = bound + 2.0 ** -8 * (np.abs(exact) + bound) + 1e-30
    assert (np.abs(g - exact) <= tol).all(), float((np.abs(g - exact) / tol).max())
    assert tolerance_ratio(gpu_bits, exact) <= OUT_TOL


def mx_weights(n_out, n_in, seed):
    w = moe_synth.randn((n_out, n_in), "cpu", moe_synth.seed_of(97, 1, seed), moe_synth.WEIGHT_STD)
    return moe_synth.mxfp4_rows(w)


LINEAR_CASES = [  # M, n_out, n_in, fmt, output
    (1, 128, 128, "mxfp4", "bf16"),        # one row, one K step pair
    (77, 256, 192, "mxfp4", "f32"),        # ragged rows, three K steps
    (300, 384, 512, "bf16", "bf16"),
    (130, 128, 256, "bf16", "add"),        # addend before the rounding
    (257, 640, 384, "mxfp4", "add"),
    (2048, 1024, 320, "mxfp4", "bf16"),    # 128-row tiles; 5 K steps (not a multiple of the pipeline depth)
    (1100, 2048, 448, "bf16", "add"),      # 128-row tiles, ragged last tile, 7 K steps
]


@pytest.mark.parametrize("M,n_out,n_in,fmt,mode", LINEAR_CASES)
def test_linear(lib, M, n_out, n_in, fmt, mode):
    say("linear", M, n_out, n_in, fmt, mode)
    seed = M + n_out + n_in
    a = moe_synth.randn((M, n_in), "cpu", moe_synth.seed_of(97, 2, seed)).to(torch.bfloat16)
    if fmt == "mxfp4":
        q, s = mx_weights(n_out, n_in, seed)
        ow = LinearWeights("mxfp4", q.numpy(), s.numpy())
        gw = lib.Linear(q.to(DEV), s.to(DEV))
    else:
        w = (moe_synth.randn((n_out, n_in), "cpu", moe_synth.seed_of(97, 3, seed)) * 0.05).to(torch.bfloat16)
        ow = LinearWeights("bf16", bf16_host(w))
        gw = lib.Linear(w.to(DEV))
    addend = None
    if mode == "add":
        addend = moe_synth.randn((M, n_out), "cpu", moe_synth.seed_of(97, 4, seed))
    out = lib.moe_linear(a.to(DEV), gw, addend=None if addend is None else addend.to(DEV),
                         out_dtype=torch.float32 if mode == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    A = codecs.bf16_decode(bf16_host(a))
    exact = latent.linear(A, ow)
    bound = acc_bound(A, ow)
    if addend is not None:
        exact = exact + addend.numpy().astype(np.float64)
        bound = bound + 2.0 ** -24 * np.abs(exact)          # the fp32 add of the addend
    if mode == "f32":
        err = np.abs(host(out).astype(np.float64) - exact)
        say("  max|err|/rms", err.max() / np.sqrt(np.mean(exact * exact)))
        assert (err <= bound + 2.0 ** -24 * np.abs(exact) + 1e-30).all()
    else:
        check_bf16_close(bf16_host(out), exact, bound)


def test_linear_full_size_down_projection(lib):
    """The block's down-projection at full size (512 x 7168 -> 3584, MXFP4),
    every output row against the oracle on 16 sampled rows."""
    blk = moe_synth.latent_block_inputs(**{k: v for k, v in moe_synth.LATENT_BLOCK.items()}, device=DEV)
    c = blk["cfg"]
    say("linear full size down-projection", c)
    out = lib.moe_linear(blk["x"], lib.Linear(blk["down"]["w"], blk["down"]["s"]))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(c["T"], 16, replace=False))
    ow = LinearWeights("mxfp4", host(blk["down"]["w"]), host(blk["down"]["s"]))
    A = codecs.bf16_decode(bits(blk["x"][torch.as_tensor(rows, device=DEV)]))
    check_bf16_close(bits(out[torch.as_tensor(rows, device=DEV)]), latent.linear(A, ow), acc_bound(A, ow))


# ----------------------------------------------------------------------------
# the block
# ----------------------------------------------------------------------------


def oracle_block(blk, activation="silu"):
    down, up = (LinearWeights("mxfp4", host(blk[n]["w"]), host(blk[n]["s"])) for n in ("down", "up"))
    routed = ExpertWeights("mxfp4", *(host(blk["routed"][n]) for n in ("w1", "w3", "w2", "s1", "s3", "s2")))
    sh = None
    if blk["shared"] is not None:
        sh = DenseFFN(*(bits(blk["shared"][n]) for n in ("w1", "w3", "w2")), activation=activation)
    return down, up, routed, sh


def run_block(lib, blk, score="softmax", activation="silu", capture=True):
    c = blk["cfg"]
    T, L, E, k = c["T"], c["L"], c["E"], c["k"]
    lw = lib.LatentWeights(blk["down"], blk["up"], blk["shared"], activation=activation)
    routed = lib.Weights(blk["routed"], "mxfp4")
    dbg = None
    if capture:
        z = lambda shape, dt: torch.empty(shape, dtype=dt, device=DEV)  # noqa: E731
        dbg = dict(topk_ids=z((T, k), torch.int32), topk_w=z((T, k), torch.float32),
                   expert_counts=z((E,), torch.int32), expert_offsets=z((E + 1,), torch.int32),
                   pair_to_row=z((T, k), torch.int32), row_to_pair=z((T * k,), torch.int32),
                   latent=z((T, L), torch.bfloat16), core_out=z((T, L), torch.bfloat16))
    res = lib.moe_latent_forward(blk["x"], blk["logits"], k, lw, routed, blk["gamma"], blk["eps"],
                                 debug=dbg, score=score)
    torch.cuda.synchronize()
    return (res[0] if capture else res), dbg


BLOCK_CASES = {
    # name: (T, Hm, L, I, E, k, Is, score, shared activation)
    "small_shared": (40, 256, 128, 128, 8, 2, 256, "softmax", "silu"),
    "no_shared": (33, 384, 128, 256, 6, 3, 0, "softmax", "silu"),
    "sigmoid_situ_shared": (70, 256, 256, 128, 16, 4, 128, "sigmoid", "situ"),
    "one_token": (1, 256, 128, 128, 8, 2, 128, "softmax", "silu"),
    "ragged_rows": (131, 512, 256, 128, 8, 2, 384, "softmax", "silu"),
    # enough rows and channels for 128-row tiles in the up-projection and both
    # shared GEMMs (64-row tiles in the down-projection)
    "wide_shared": (1100, 2048, 128, 128, 8, 2, 2048, "softmax", "silu"),
}


@pytest.mark.parametrize("case", list(BLOCK_CASES))
def test_latent_forward(lib, case):
    T, Hm, L, I, E, k, Is, score, act = BLOCK_CASES[case]
    say("latent block", case, BLOCK_CASES[case])
    blk = moe_synth.latent_block_inputs(T, Hm, L, I, E, k, Is, cfg=40 + len(case), device=DEV)
    if blk["shared"] is not None:
        # gate weights x 8 (exact in bf16): gates of a few units, where SiTU
        # and SiLU part, and a shared output about as large as the
        # up-projection's, so that both are held to the bar
        blk["shared"]["w1"] = (blk["shared"]["w1"].float() * 8.0).to(torch.bfloat16)
    out, dbg = run_block(lib, blk, score, act)
    down, up, routed, sh = oracle_block(blk, act)
    ref = latent.latent_forward(bits(blk["x"]), host(blk["logits"]), k, down, routed, up, sh,
                                host(blk["gamma"]), blk["eps"], score)
    core = ref["core"]
    assert (host(dbg["topk_ids"]) == core["topk_ids"]).all()
    assert (host(dbg["expert_counts"]) == core["counts"]).all()
    assert (host(dbg["expert_offsets"]) == core["offsets"]).all()
    assert (host(dbg["pair_to_row"]) == core["pair_to_row"]).all()
    assert (host(dbg["row_to_pair"]) == core["row_to_pair"]).all()
    X = codecs.bf16_decode(bits(blk["x"]))
    check_bf16_close(bits(dbg["latent"]), latent.linear(X, down), acc_bound(X, down))
    r_core = tolerance_ratio(bits(dbg["core_out"]), core["out_exact"])
    r_out = tolerance_ratio(bits(out), ref["out_exact"])
    say("  core max|err|/rms", r_core, " block max|err|/rms", r_out)
    assert r_core <= OUT_TOL and r_out <= OUT_TOL


def test_latent_forward_full_size(lib):
    """The whole block at full size (512 tokens, hidden 7168, latent 3584, 896
    MXFP4 experts top-16, bf16 shared experts 7168 -> 6144 -> 7168): all
    routing metadata, the latent of every token (the down-projection, whose
    K is split over two workgroups per tile at this size), and the outputs
    of 3 sampled tokens."""
    blk = moe_synth.latent_block_inputs(**moe_synth.LATENT_BLOCK, device=DEV)
    c = blk["cfg"]
    T, E, k = c["T"], c["E"], c["k"]
    say("latent block full size", c)
    out, dbg = run_block(lib, blk)
    ids, w = moe.route(host(blk["logits"]), k)
    counts, offsets = moe.expert_counts_offsets(ids, E)
    p2r, r2p, _, _ = moe.permute_rows(ids, offsets, np.zeros((T, 1), np.uint8), np.zeros(T, np.float32))
    assert (host(dbg["topk_ids"]) == ids).all()
    assert (host(dbg["expert_counts"]) == counts).all()
    assert (host(dbg["pair_to_row"]) == p2r).all()
    assert (host(dbg["row_to_pair"]) == r2p).all()
    down = LinearWeights("mxfp4", host(blk["down"]["w"]), host(blk["down"]["s"]))
    X = codecs.bf16_decode(bits(blk["x"]))
    check_bf16_close(bits(dbg["latent"]), latent.linear(X, down), acc_bound(X, down))
    tokens = np.sort(np.random.default_rng(c["cfg"]).choice(T, 3, replace=False))
    up = LinearWeights("mxfp4", host(blk["up"]["w"]), host(blk["up"]["s"]))
    from gpu_helpers import DeviceStack
    routed = ExpertWeights("mxfp4", *(DeviceStack(blk["routed"][n]) for n in ("w1", "w3", "w2", "s1", "s3", "s2")))
    sh = DenseFFN(*(bits(blk["shared"][n]) for n in ("w1", "w3", "w2")))
    ref = latent.latent_forward_sampled(bits(blk["x"]), None, k, down, routed, up, tokens, sh,
                                        host(blk["gamma"]), blk["eps"], routing=(ids, w))
    r = tolerance_ratio(bits(out[torch.as_tensor(tokens, device=DEV)]), ref)
    say("  max|err|/rms", r, "over", len(tokens), "tokens")
    assert r <= OUT_TOL
