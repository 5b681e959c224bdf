"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Bar: routing ids, per-expert counts/offsets, the permutation and the
quantised token bytes/scales bit-exact; router weights within 1e-6 relative;
layer outputs within max|err| <= 2e-2 * RMS(oracle).  Small cases are checked
everywhere; the full-size workloads (the pages' prefill and decode shares,
the LatentMoE decode and the skewed full layer) are checked on all metadata
and on the outputs of sampled tokens.
"""

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from oracle import moe
from gpu_helpers import (DEV, OUT_TOL, assert_weights_close, bits, check_metadata, edge_tokens, host,
                         oracle_weights, run_forward, say, to_device, tolerance_ratio)

pytestmark = pytest.mark.gpu


def bf16_np(t):
    return t.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------

ROUTE_CASES = {
    "tiny": lambda: moe_synth.make_inputs("tiny", weights=False)["logits"],
    "integer_ties": lambda: torch.randint(-3, 3, (300, 16), generator=torch.Generator().manual_seed(1)).float(),
    "signed_zeros": lambda: torch.tensor([[-1.0, 0.0, -0.0, 0.0, -2.0, -0.0, 5.0, 5.0]] * 4),
    "all_equal": lambda: torch.zeros((33, 64)),
    "E1024_k32": lambda: torch.randn((100, 1024), generator=torch.Generator().manual_seed(2)),
    "latent_E896_k16": lambda: moe_synth.make_inputs("latent", weights=False)["logits"],
    "skewed_full": lambda: moe_synth.make_inputs("skewed", weights=False)["logits"],
    "E1": lambda: torch.randn((5, 1)),
}
ROUTE_K = {"tiny": 2, "integer_ties": 4, "signed_zeros": 3, "all_equal": 8, "E1024_k32": 32,
           "latent_E896_k16": 16, "skewed_full": 8, "E1": 1}


@pytest.mark.parametrize("case", list(ROUTE_CASES))
def test_route(lib, case):
    logits = ROUTE_CASES[case]().float().contiguous()
    k = ROUTE_K[case]
    say("route", case, tuple(logits.shape), k)
    ids, w = lib.moe_route(logits.to(DEV), k)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route(logits.numpy(), k)
    assert (host(ids) == ref_ids).all()
    assert_weights_close(host(w), ref_w)


ROUTE_SIGMOID = ["tiny", "integer_ties", "signed_zeros", "all_equal", "E1024_k32", "latent_E896_k16", "E1"]


@pytest.mark.parametrize("case", ROUTE_SIGMOID)
def test_route_sigmoid(lib, case):
    """Sigmoid scores: the same selection as the softmax, weights the
    renormalised sigmoids of the selected logits."""
    logits = ROUTE_CASES[case]().float().contiguous()
    k = ROUTE_K[case]
    say("route sigmoid", case, tuple(logits.shape), k)
    ids, w = lib.moe_route(logits.to(DEV), k, score="sigmoid")
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route(logits.numpy(), k, "sigmoid")
    assert (host(ids) == ref_ids).all()
    assert_weights_close(host(w), ref_w)


# ----------------------------------------------------------------------------
# permutation and quantisation (moe_permute)
# ----------------------------------------------------------------------------

PERMUTE_CASES = [  # T, H, E, k, hot expert
    (64, 256, 8, 2, None),
    (333, 384, 7, 3, None),
    (100, 128, 5, 1, 3),          # every token on expert 3: the other experts are empty
    (2000, 256, 16, 4, 0),
    (512, 3584, 896, 16, None),
    (2048, 8192, 8, 2, None),
    (1, 128, 1024, 32, None),
    (5000, 128, 64, 4, None),     # 20000 pairs: the grid-wide counting / ranking kernels
    (300, 128, 64, 4, None),      # the most experts the single-workgroup kernel takes
    (300, 128, 65, 4, None),      # one more: the grid-wide kernels
    (2300, 128, 256, 8, None),    # 18 chunks over 4 ranges of 5, 5, 5 and 3 chunks per expert
    (20000, 128, 1, 1, None),     # one expert, 20 chunks: one chunk per scanning thread
]


@pytest.mark.parametrize("T,H,E,k,hot", PERMUTE_CASES)
def test_permute(lib, T, H, E, k, hot):
    say("permute", T, H, E, k, hot)
    x = moe_synth.randn((T, H), "cpu", moe_synth.seed_of(91, 1, T)).to(torch.bfloat16)
    if T > 1:
        x[1] = 0.0                                    # a zero row: scale 1, signed-zero codes
        x[0, :7] = torch.tensor([448.0, -448.0, 1e-3, -1e-30, 3.0, -0.0, 0.0])
    ids = moe_synth.random_topk_ids(T, E, k, seed=T + E, hot=hot)
    res = lib.moe_permute(x.to(DEV), ids.to(DEV), E, token_order=True)
    torch.cuda.synchronize()
    xq, xs = oracle.quantize_tokens(bf16_np(x))
    counts, offsets = oracle.expert_counts_offsets(ids.numpy(), E)
    p2r, r2p, xq_rows, xs_rows = oracle.permute_rows(ids.numpy(), offsets, xq, xs)
    assert (host(res["counts"]) == counts).all()
    assert (host(res["offsets"]) == offsets).all()
    assert (host(res["pair_to_row"]) == p2r).all()
    assert (host(res["row_to_pair"]) == r2p).all()
    assert (host(res["xq_rows"]) == xq_rows).all()
    assert (host(res["xs_rows"]).view(np.uint32) == xs_rows.view(np.uint32)).all()
    assert (host(res["xq_tok"]) == xq).all()
    assert (host(res["xs_tok"]).view(np.uint32) == xs.view(np.uint32)).all()


def test_permute_skewed_full_size(lib):
    """The skewed full layer (16384 tokens, top-8 of 256): all metadata
    bit-exact; quantised bytes of 256 sampled rows."""
    inp = moe_synth.make_inputs("skewed", device=DEV, weights=False)
    c = inp["cfg"]
    T, H, E, k = c["T"], c["H"], c["E"], c["k"]
    say("permute skewed full", T, H, E, k, "alpha", c["alpha"])
    ids, _ = lib.moe_route(inp["logits"], k)
    res = lib.moe_permute(inp["x"], ids, E)
    torch.cuda.synchronize()
    ref_ids, _ = oracle.route(host(inp["logits"]), k)
    assert (host(ids) == ref_ids).all()
    counts, offsets = oracle.expert_counts_offsets(ref_ids, E)
    dummy = np.zeros((T, 1), np.uint8)
    p2r, r2p, _, _ = oracle.permute_rows(ref_ids, offsets, dummy, np.zeros(T, np.float32))
    assert (host(res["counts"]) == counts).all()
    assert counts.max() / counts.mean() == pytest.approx(5.0, abs=0.11)
    assert (host(res["offsets"]) == offsets).all()
    assert (host(res["pair_to_row"]) == p2r).all()
    assert (host(res["row_to_pair"]) == r2p).all()
    rows = np.random.default_rng(5).choice(T * k, 256, replace=False)
    toks = r2p[rows] // k
    xq, xs = oracle.quantize_tokens(bits(inp["x"][torch.as_tensor(toks, device=DEV)]))
    assert (host(res["xq_rows"][torch.as_tensor(rows, device=DEV)]) == xq).all()
    assert (host(res["xs_rows"])[rows].view(np.uint32) == xs.view(np.uint32)).all()


# ----------------------------------------------------------------------------
# whole layer, small shapes: every output element
# ----------------------------------------------------------------------------

FULL_CASES = {
    # name: (T, H, I, E, k, fmt, shared, norm)
    "tiny_config": None,
    "ragged_small_variant": (45, 384, 256, 6, 3, "fp8", False, False),
    "shared_small_variant": (40, 256, 256, 4, 2, "fp8", True, False),
    "large_variant": (300, 256, 256, 4, 2, "fp8", False, False),
    "large_variant_shared": (333, 512, 384, 3, 2, "fp8", True, False),
    "large256_ragged_shared": (1000, 256, 256, 4, 2, "fp8", True, False),
    "mxfp4_rmsnorm": (48, 256, 128, 8, 2, "mxfp4", False, True),
    "mxfp4_k_equals_E": (20, 384, 256, 4, 4, "mxfp4", False, False),
    "dense_E1_k1": (70, 256, 128, 1, 1, "fp8", False, False),
    "one_token": (1, 128, 128, 16, 4, "fp8", True, False),
    # 18000 pairs: routing and metadata by the grid-wide kernels
    "many_tokens": (9000, 128, 128, 16, 2, "fp8", False, False),
    # single-wave routing + metadata: its largest batch (4 token chunks, 32
    # experts, 8 slots) and a second chunk holding one token
    "meta_wave_T256_E32_k8": (256, 128, 128, 32, 8, "fp8", True, False),
    "meta_wave_T65": (65, 128, 128, 5, 2, "fp8", False, False),
    # decode-sized batches whose groups average >= 64 rows: the 128-row
    # gate-up kernel reading token rows through row_to_pair
    "gathered_large128_shared": (200, 256, 256, 4, 2, "fp8", True, False),
    "gathered_large128": (256, 512, 256, 2, 2, "fp8", False, False),
    # either side of the path choices: one-launch routing with the small
    # kernels gathering token rows up to 256 tokens, past that reading an
    # expert-ordered copy (as the large kernels always do); up to 4096
    # tokens one-launch routing, past that the grid-wide router
    "path_T257_small": (257, 256, 128, 16, 2, "fp8", False, False),
    "path_T4096_large": (4096, 256, 128, 8, 1, "fp8", False, False),
    "path_T4097_large": (4097, 256, 128, 8, 1, "fp8", False, False),
    # wide tokens: the fused quantisation's 8- and 16-piece-per-thread forms
    # (an odd token count leaves the last token pair half empty)
    "wide_H16384_odd_T": (7, 16384, 128, 4, 2, "fp8", True, False),
    "wide_H32768": (5, 32768, 128, 4, 2, "fp8", False, False),
    # per-block fp8 weights (one scale per 128 x 128 tile), with a per-channel
    # fp8 shared expert beside them in one launch; from 64 rows per group on
    # average both GEMMs take the large kernels (the gate-up GEMM 128-row
    # tiles with the block exponent in the MFMA and the mantissa carried by
    # the accumulators, the down GEMM 128- or 256-row tiles with the block
    # scale applied as the codes are widened)
    "block_fp8_small": (45, 384, 256, 6, 3, "fp8_block", False, False),
    "block_fp8_shared": (300, 256, 384, 4, 2, "fp8_block", True, False),
    "block_fp8_large128_down": (300, 256, 256, 4, 2, "fp8_block", False, False),
    # 48-63 rows per group: the medium gate-up kernel, with the shared expert
    # in a large-kernel gate-up launch of its own
    "block_fp8_medium_shared_split": (80, 256, 256, 4, 2, "fp8_block", True, False),
    "block_fp8_large256_down_ragged_shared": (1000, 256, 512, 4, 2, "fp8_block", True, False),
}


# (case, pack): fp8 weights K-blocked (the default) or left row-major
FULL_RUNS = [(case, True) for case in FULL_CASES] + [
    ("ragged_small_variant", False), ("large_variant_shared", False), ("one_token", False),
    ("mxfp4_rmsnorm", False), ("mxfp4_k_equals_E", False), ("block_fp8_shared", False),
    ("gathered_large128_shared", False)]


@pytest.mark.parametrize("case,pack", FULL_RUNS)
def test_forward_full(lib, case, pack):
    spec = FULL_CASES[case]
    if spec is None:
        inp = moe_synth.make_inputs("tiny")
    else:
        T, H, I, E, k, fmt, shared, norm = spec
        inp = moe_synth.custom_inputs(T, H, I, E, k, fmt=fmt, seed=len(case), shared=shared, norm=norm)
    c = inp["cfg"]
    say("forward full", case, "packed" if pack else "row-major",
        {key: c[key] for key in ("T", "H", "I", "E", "k", "fmt", "shared", "norm")})
    out, dbg, variant = run_forward(to_device(inp), pack=pack)
    say("  variant", variant)
    if case.startswith("gathered_large128"):
        assert "large128" in variant
    if case == "block_fp8_shared" or case.startswith("block_fp8_large"):
        assert variant == ("large128/fp8/down:large256" if "large256" in case else "large128/fp8")
    if case == "block_fp8_medium_shared_split":
        assert variant.startswith("medium64") and "shared:large128" in variant
    ref = oracle.forward(bf16_np(inp["x"]), inp["logits"].numpy(), c["k"],
                         oracle_weights(inp["routed"], c["fmt"]),
                         oracle_weights(inp["shared"], "fp8"),
                         None if inp["gamma"] is None else inp["gamma"].numpy(), inp["eps"])
    check_metadata(dbg, ref, c["T"], c["k"], c["E"], c["shared"])
    assert (host(dbg["xq_rows"]) == ref["xq_rows"]).all()
    assert (host(dbg["xs_rows"]).view(np.uint32) == ref["xs_rows"].view(np.uint32)).all()
    ratio = tolerance_ratio(bits(out), ref["out_exact"])
    say("  max|err|/rms", ratio)
    assert ratio <= OUT_TOL


# Router and activation variants (sigmoid scores; SiTU gate activation):
# name: (T, H, I, E, k, fmt, shared, norm, score, routed act, shared act, beta)
VARIANT_CASES = {
    # routing fused into the metadata kernel; small GEMM variant
    "sigmoid_situ_small": (45, 384, 256, 6, 3, "fp8", False, False, "sigmoid", "situ", "silu", 4.0),
    # routed SiTU next to a SiLU shared expert in one grouped launch
    "sigmoid_situ_large_shared": (333, 512, 384, 3, 2, "fp8", True, False, "sigmoid", "situ", "silu", 4.0),
    # 256-row tiles, both groups SiTU, another beta
    "situ_large256_shared": (1000, 256, 256, 4, 2, "fp8", True, False, "softmax", "situ", "situ", 2.5),
    # shared SiTU, routed SiLU
    "sigmoid_shared_situ": (300, 256, 256, 4, 2, "fp8", True, False, "sigmoid", "silu", "situ", 4.0),
    "sigmoid_situ_mxfp4_rmsnorm": (48, 256, 128, 8, 2, "mxfp4", False, True, "sigmoid", "situ", "silu", 4.0),
    # router kernel, then the metadata kernel (more than 32 experts)
    "sigmoid_situ_E64": (200, 128, 128, 64, 6, "fp8", False, False, "sigmoid", "situ", "silu", 4.0),
    # router kernel and the grid-wide metadata kernels (18000 pairs)
    "sigmoid_situ_many_tokens": (9000, 128, 128, 16, 2, "fp8", False, False, "sigmoid", "situ", "silu", 4.0),
}


@pytest.mark.parametrize("case", list(VARIANT_CASES))
def test_forward_variants(lib, case):
    T, H, I, E, k, fmt, shared, norm, score, act_r, act_s, beta = VARIANT_CASES[case]
    inp = moe_synth.custom_inputs(T, H, I, E, k, fmt=fmt, seed=len(case) + 100, shared=shared, norm=norm)
    if act_r == "situ" or act_s == "situ":
        inp["x"] = (inp["x"].float() * 4.0).to(torch.bfloat16)   # gates well past beta
    say("forward variant", case, VARIANT_CASES[case])
    out, dbg, variant = run_forward(to_device(inp), score=score, act=(act_r, act_s), beta=beta)
    say("  variant", variant)
    ref = oracle.forward(bf16_np(inp["x"]), inp["logits"].numpy(), k,
                         oracle_weights(inp["routed"], fmt, activation=act_r, beta=beta),
                         oracle_weights(inp["shared"], "fp8", activation=act_s, beta=beta),
                         None if inp["gamma"] is None else inp["gamma"].numpy(), inp["eps"], score=score)
    check_metadata(dbg, ref, T, k, E, shared)
    assert (host(dbg["xq_rows"]) == ref["xq_rows"]).all()
    ratio = tolerance_ratio(bits(out), ref["out_exact"])
    say("  max|err|/rms", ratio)
    assert ratio <= OUT_TOL


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("E,k", [(8, 2), (32, 5), (33, 3)])
def test_forward_route_ties(lib, E, k, score):
    """Integer logits with many ties and signed zeros through moe_forward: at
    most 32 experts are routed inside the metadata kernel, more by the router
    kernel; both must break ties towards the lower expert id."""
    T = 200
    inp = moe_synth.custom_inputs(T, 128, 128, E, k, seed=E + k)
    g = torch.Generator().manual_seed(E * k)
    logits = torch.randint(-2, 3, (T, E), generator=g).float()
    logits[::7] = 0.0
    logits[1::7, ::2] = -0.0
    inp["logits"] = logits
    say("forward route ties", E, k, score)
    out, dbg, _ = run_forward(to_device(inp), score=score)
    ref = oracle.forward(bf16_np(inp["x"]), logits.numpy(), k, oracle_weights(inp["routed"], "fp8"), score=score)
    check_metadata(dbg, ref, T, k, E, False)
    assert tolerance_ratio(bits(out), ref["out_exact"]) <= OUT_TOL


@pytest.mark.parametrize("T", [64, 300])
def test_forward_nan_logits_route_valid_experts(lib, T):
    """NaN logits (no infinities) rank below every number, equal ones by
    expert index, as in the oracle's sort; the ids, counts and permutation
    stay exact whichever router runs (single-wave at T=64, grid-wide at
    T=300).  Other outputs of such rows are not defined and not checked."""
    E, k = 8, 2
    inp = moe_synth.custom_inputs(T, 128, 128, E, k, seed=T)
    logits = inp["logits"].clone()
    logits[::5] = float("nan")                 # whole rows
    logits[1::5, 0:E:3] = float("nan")         # some experts of a row
    inp["logits"] = logits
    say("forward nan logits", T)
    _, dbg, _ = run_forward(to_device(inp))
    ids, _ = moe.route(logits.numpy(), k)
    counts, offsets = moe.expert_counts_offsets(ids, E)
    p2r, r2p, _, _ = moe.permute_rows(ids, offsets, np.zeros((T, 1), np.uint8), np.zeros(T, np.float32))
    assert (host(dbg["topk_ids"]) == ids).all()
    assert (host(dbg["expert_counts"]) == counts).all()
    assert (host(dbg["pair_to_row"]) == p2r).all()
    assert (host(dbg["row_to_pair"]) == r2p).all()


def test_forward_zero_tokens(lib):
    inp = to_device(moe_synth.custom_inputs(0, 256, 128, 4, 2))
    out, _, _ = run_forward(inp, capture=False)
    assert out.shape == (0, 256)


@pytest.mark.parametrize("T", [64, 300])
def test_forward_dispatch_events(lib, T):
    """The layer events stamped by the first (fused routing + quantisation kernel at T=64,
    router at T=300) and last dispatch bracket the GEMMs' own events, and the
    output is the same as without events."""
    inp = to_device(moe_synth.custom_inputs(T, 256, 256, 4, 2, seed=5, shared=True))
    ref, _, _ = run_forward(inp, capture=False)
    routed = lib.Weights(inp["routed"], "fp8")
    shared = lib.Weights(inp["shared"], "fp8")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    say("forward dispatch events", T)
    out = lib.moe_forward(inp["x"], inp["logits"], 2, routed, shared, gemm1_events=evs[0:2],
                          gemm2_events=evs[2:4], layer_events=evs[4:6])
    torch.cuda.synchronize()
    layer = evs[4].elapsed_time(evs[5])
    g1, g2 = evs[0].elapsed_time(evs[1]), evs[2].elapsed_time(evs[3])
    say("  layer ms", layer, "gemm1", g1, "gemm2", g2)
    assert 0 < g1 and 0 < g2 and g1 + g2 <= layer
    assert evs[4].elapsed_time(evs[0]) >= 0 and evs[3].elapsed_time(evs[5]) >= 0
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_forward_deterministic(lib):
    inp = to_device(moe_synth.custom_inputs(300, 256, 256, 4, 2, seed=3, shared=True))
    a, _, _ = run_forward(inp, capture=False)
    b, _, _ = run_forward(inp, capture=False)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ----------------------------------------------------------------------------
# whole layer, the full-size workloads: all metadata, sampled outputs
# ----------------------------------------------------------------------------

# The many-expert workloads (latent, skewed) with the default router and
# activation are checked on tokens that reach every expert in
# test_gpu_coverage.py.
SAMPLED = {"prefill": 24, "decode": 64, "latent": 3}


FULL_SIZE_RUNS = [("prefill", "softmax", "silu"), ("decode", "softmax", "silu"),
                  ("latent", "sigmoid", "situ"),      # the LatentMoE layer with its own router and activation
                  ("prefill", "sigmoid", "situ")]


@pytest.mark.parametrize("name,score,act", FULL_SIZE_RUNS)
def test_forward_full_size(lib, name, score, act):
    inp = moe_synth.make_inputs(name, device=DEV)
    c = inp["cfg"]
    T, E, k = c["T"], c["E"], c["k"]
    say("forward full size", name, score, act, c)
    out, dbg, variant = run_forward(inp, score=score, act=(act, act))
    say("  variant", variant)
    ids, w = oracle.route(host(inp["logits"]), k, score)
    counts, offsets = oracle.expert_counts_offsets(ids, E)
    p2r, r2p, _, _ = oracle.permute_rows(ids, offsets, np.zeros((T, 1), np.uint8), np.zeros(T, np.float32))
    ref = dict(topk_ids=ids, topk_w=w, counts=counts, offsets=offsets, pair_to_row=p2r, row_to_pair=r2p)
    check_metadata(dbg, ref, T, k, E, c["shared"])
    rng = np.random.default_rng(c["cfg"])
    n = SAMPLED[name]
    tokens = np.arange(T) if n >= T else np.sort(rng.choice(T, n, replace=False))
    # plus the tokens of the hottest expert's last (ragged) row tile and of the last row
    tile = int(variant.split("/")[0].lstrip("smalrge"))
    edge, _ = edge_tokens(counts, offsets, r2p, k, tile)
    tokens = np.unique(np.concatenate([tokens, np.asarray(edge, dtype=np.int64)]))
    tok_d = torch.as_tensor(tokens, device=DEV)
    # quantised bytes of the sampled tokens' rows
    xq, xs = oracle.quantize_tokens(bits(inp["x"][tok_d]))
    rows = p2r[tokens]
    for j in range(k):
        r_d = torch.as_tensor(rows[:, j], device=DEV)
        assert (host(dbg["xq_rows"][r_d]) == xq).all()
        assert (host(dbg["xs_rows"][r_d]).view(np.uint32) == xs.view(np.uint32)).all()
    ref_out = oracle.moe.forward_sampled(
        bits(inp["x"]), None, k, oracle_weights(inp["routed"], c["fmt"], lazy=True, activation=act), tokens,
        shared=oracle_weights(inp["shared"], "fp8", lazy=True, activation=act),
        norm_gamma=None if inp["gamma"] is None else host(inp["gamma"]), norm_eps=inp["eps"],
        routing=(ids, w))
    ratio = tolerance_ratio(bits(out[tok_d]), ref_out)
    say("  max|err|/rms", ratio, "over", len(tokens), "tokens")
    assert ratio <= OUT_TOL


@pytest.mark.parametrize("T,pack", [(300, True), (1000, False)])
def test_forward_block_fp8_special_scales(lib, T, pack):
    """Per-block fp8 on the large kernels (T tokens, H 512, I 384, 4 experts
    top-2 + a per-channel shared expert; the gate-up GEMM's 128-row tiles,
    the down GEMM's 128- or 256-row ones) with the block scales the kernels'
    split of a scale into its power of two (the MFMA's e8m0 scale) and its
    mantissa (carried by rescaling the accumulators, or applied as the down
    GEMM's weights are widened) treats specially: exact powers of two
    (mantissa 1), all-zero blocks (scale and codes 0), zero scales over
    non-zero codes and subnormal scales (e8m0 0), between blocks of ordinary
    scales, so that neighbouring K blocks' exponents jump.  Every output
    element against the oracle.  (Spreading the scales themselves over
    powers of two far apart makes each output hang on a few large terms, and
    the bf16 rounding of h then exceeds the output bar on any path: 2^+-20
    gave 0.027-0.032 x RMS on the register-fed kernels, which sum each block
    exactly.)"""
    H, I, E, k = 512, 384, 4, 2
    inp = moe_synth.custom_inputs(T, H, I, E, k, fmt="fp8_block", seed=21, shared=True)
    r = inp["routed"]
    g = torch.Generator().manual_seed(21 + T)
    for wn, sn in (("w1", "s1"), ("w3", "s3"), ("w2", "s2")):
        sc, w = r[sn], r[wn]                     # float32 [E][N/128][K/128], uint8 [E][N][K]
        pick = torch.rand(sc.shape, generator=g)
        p2 = pick < 0.1
        sc[p2] = torch.pow(2.0, torch.round(torch.log2(sc[p2])))
        sc[(pick >= 0.1) & (pick < 0.15)] = 1e-40     # subnormal
        sc[(pick >= 0.15) & (pick < 0.2)] = 0.0       # zero scale over non-zero codes
        zero = pick >= 0.9                           # all-zero blocks
        sc[zero] = 0.0
        for e, nb, kb in zero.nonzero().tolist():
            w[e, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128] = 0
    say("forward block fp8 special scales", T, "packed" if pack else "row-major")
    out, dbg, variant = run_forward(to_device(inp), pack=pack)
    say("  variant", variant)
    assert variant.startswith("large128") and ("down:large256" in variant) == (T >= 1000)
    ref = oracle.forward(bf16_np(inp["x"]), inp["logits"].numpy(), k, oracle_weights(inp["routed"], "fp8_block"),
                         oracle_weights(inp["shared"], "fp8"), None, inp["eps"])
    check_metadata(dbg, ref, T, k, E, True)
    out_b = bits(out)
    assert np.isfinite(oracle.codecs.bf16_decode(out_b)).all()
    ratio = tolerance_ratio(out_b, ref["out_exact"])
    say("  max|err|/rms", ratio)
    assert ratio <= OUT_TOL


def test_forward_block_fp8_decode_full_size(lib):
    """The decode share (64 tokens, H 8192, I 2048, 8 experts top-2) with
    per-block fp8 weights: all routing metadata and 16 sampled outputs."""
    inp = moe_synth.custom_inputs(64, 8192, 2048, 8, 2, fmt="fp8_block", seed=12, device=DEV)
    c = inp["cfg"]
    T, E, k = c["T"], c["E"], c["k"]
    say("forward block fp8 decode full size", c)
    out, dbg, variant = run_forward(inp)
    say("  variant", variant)
    ids, w = oracle.route(host(inp["logits"]), k)
    counts, offsets = oracle.expert_counts_offsets(ids, E)
    assert (host(dbg["topk_ids"]) == ids).all() and (host(dbg["expert_counts"]) == counts).all()
    tokens = np.arange(0, T, 4)
    ref_out = oracle.moe.forward_sampled(bits(inp["x"]), None, k, oracle_weights(inp["routed"], "fp8_block", lazy=True),
                                         tokens, routing=(ids, w))
    ratio = tolerance_ratio(bits(out[torch.as_tensor(tokens, device=DEV)]), ref_out)
    say("  max|err|/rms", ratio)
    assert ratio <= OUT_TOL


def test_forward_block_fp8_prefill_full_size(lib):
    """The prefill share (2048 tokens, H 8192, I 2048, 8 experts top-2, a
    per-channel fp8 shared expert) with per-block fp8 routed weights, which
    takes the 128-row large variant in the gate-up GEMM and the 256-row one
    in the down GEMM: all routing metadata, and the outputs of tokens that
    reach every expert, the first and last rows of the hottest expert's last
    (ragged) 128-row and 256-row tiles, the least-loaded expert's last row and
    the last routed row."""
    from gpu_helpers import cover_tokens
    inp = moe_synth.custom_inputs(2048, 8192, 2048, 8, 2, fmt="fp8_block", seed=13, device=DEV, shared=True)
    c = inp["cfg"]
    T, E, k = c["T"], c["E"], c["k"]
    say("forward block fp8 prefill full size", c)
    out, dbg, variant = run_forward(inp)
    say("  variant", variant)
    assert variant.startswith("large128") and "down:large256" in variant
    ids, w = oracle.route(host(inp["logits"]), k)
    counts, offsets = oracle.expert_counts_offsets(ids, E)
    p2r, r2p, _, _ = oracle.permute_rows(ids, offsets, np.zeros((T, 1), np.uint8), np.zeros(T, np.float32))
    check_metadata(dbg, dict(topk_ids=ids, topk_w=w, counts=counts, offsets=offsets, pair_to_row=p2r,
                             row_to_pair=r2p), T, k, E, shared=True)
    edge = edge_tokens(counts, offsets, r2p, k, 128)[0] + edge_tokens(counts, offsets, r2p, k, 256)[0]
    tokens = np.array(sorted(set(cover_tokens(ids, E, must=edge)) | {0, T - 1}))
    ref_out = oracle.moe.forward_sampled(bits(inp["x"]), None, k, oracle_weights(inp["routed"], "fp8_block", lazy=True),
                                         tokens, shared=oracle_weights(inp["shared"], "fp8", lazy=True),
                                         routing=(ids, w))
    ratio = tolerance_ratio(bits(out[torch.as_tensor(tokens, device=DEV)]), ref_out)
    say("  max|err|/rms", ratio, "over", len(tokens), "tokens")
    assert ratio <= OUT_TOL


# ----------------------------------------------------------------------------
# moe_expert_ffn and moe_combine on their own
# ----------------------------------------------------------------------------


def synthetic_rows(counts, H, seed):
    """Expert-grouped rows: random e4m3 codes of moderate magnitude, scales."""
    n = int(sum(counts))
    g = torch.Generator().manual_seed(seed)
    vals = torch.randn((n, H), generator=g) * 64.0
    q = vals.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    s = (torch.rand((n,), generator=g) * 0.01 + 1e-3).float()
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return q, s, offsets


@pytest.mark.parametrize("counts,fmt,pack,act", [
    ([5, 0, 17, 1, 40, 0, 3, 32], "fp8", True, "silu"),    # small variant: ragged, empty experts
    ([5, 0, 17, 1, 40, 0, 3, 32], "fp8", False, "silu"),
    ([300, 0, 129, 64, 1], "fp8", True, "silu"),            # large variant
    ([300, 0, 129, 64, 1], "fp8", False, "silu"),
    # 256-row tiles; the last tile of each group leaves 0..4 valid 32-row
    # fragments per wave row (rows mod 256 = 188, 34, 1, 33, 232, 88, 97)
    ([700, 0, 290, 513, 33, 1000, 600, 97], "fp8", True, "silu"),
    ([9, 33, 0, 2, 16, 1, 0, 20], "mxfp4", False, "silu"),
    ([9, 33, 0, 2, 16, 1, 0, 20], "mxfp4", True, "silu"),
    ([5, 0, 17, 1, 40, 0, 3, 32], "fp8_block", True, "silu"),
    ([300, 0, 129, 64, 1], "fp8_block", False, "situ"),
    # SiTU in each GEMM1 variant
    ([5, 0, 17, 1, 40, 0, 3, 32], "fp8", True, "situ"),
    ([300, 0, 129, 64, 1], "fp8", True, "situ"),
    ([700, 0, 290, 513, 33, 1000, 600, 97], "fp8", True, "situ"),
    ([9, 33, 0, 2, 16, 1, 0, 20], "mxfp4", False, "situ"),
])
def test_expert_ffn(lib, counts, fmt, pack, act):
    E, H, I = len(counts), 256, 256
    say("expert_ffn", counts, fmt, "packed" if pack else "row-major", act)
    q, s, offsets = synthetic_rows(counts, H, seed=sum(counts))
    W = moe_synth.expert_weights(77, "cpu", fmt, E, H, I)
    y = lib.moe_expert_ffn(q.to(DEV), s.to(DEV), torch.as_tensor(offsets, device=DEV),
                           lib.Weights(to_device(W), fmt, pack=pack, activation=act))
    torch.cuda.synchronize()
    y_ref = oracle.expert_ffn(q.numpy(), s.numpy(), offsets, oracle_weights(W, fmt, activation=act))[0]
    ratio = tolerance_ratio(host(y), y_ref)
    say("  max|err|/rms", ratio)
    assert ratio <= OUT_TOL


# (3, 2176, ...): 272 chunks of 8 channels, so the sliced form (no RMSNorm)
# ends with a slice of 16 chunks
@pytest.mark.parametrize("T,H,k,shared,norm", [(50, 256, 2, False, False), (17, 384, 4, True, True),
                                               (8, 8192, 8, True, False), (3, 2176, 3, True, False),
                                               (5, 2176, 2, False, True)])
def test_combine(lib, T, H, k, shared, norm):
    say("combine", T, H, k, shared, norm)
    g = torch.Generator().manual_seed(T * k)
    R = T * k
    y = torch.randn((R, H), generator=g)
    p2r = torch.randperm(R, generator=g).to(torch.int32).reshape(T, k)
    w = torch.rand((T, k), generator=g)
    w = (w / w.sum(dim=1, keepdim=True)).float()
    ysh = torch.randn((T, H), generator=g) if shared else None
    gamma = (torch.rand(H, generator=g) + 0.5).float() if norm else None
    out = lib.moe_combine(y.to(DEV), p2r.to(DEV), w.to(DEV), None if ysh is None else ysh.to(DEV),
                          None if gamma is None else gamma.to(DEV), 1e-6)
    torch.cuda.synchronize()
    args = (y.numpy().astype(np.float64), p2r.numpy(), w.numpy().astype(np.float64),
            None if ysh is None else ysh.numpy().astype(np.float64),
            None if gamma is None else gamma.numpy(), 1e-6)
    assert tolerance_ratio(bits(out), oracle.combine(*args, rounded=False)) <= OUT_TOL
    # fp32 accumulation of the same inputs, one rounding each: at most one bf16 ulp apart
    d = np.abs(bits(out).astype(np.int32) - oracle.combine(*args).astype(np.int32))
    assert d.max() <= 1 and (d == 0).mean() > 0.99


def test_combine_zero_weights(lib):
    y = torch.randn((40, 256)).to(DEV)
    p2r = torch.arange(40, dtype=torch.int32).reshape(20, 2).to(DEV)
    out = lib.moe_combine(y, p2r, torch.zeros((20, 2), device=DEV))
    torch.cuda.synchronize()
    assert (out.float() == 0).all()


# ----------------------------------------------------------------------------
# weight layout
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("E,H,I", [(3, 256, 128), (2, 384, 640)])
def test_pack_weights(lib, E, H, I):
    """moe_pack_weights moves codes only: dst[e][c][n][0:C] == src[e][n][c*C:(c+1)*C],
    C = 64 for W1/W3 and 32 for W2, bit for bit."""
    say("pack_weights", E, H, I)
    W = to_device(moe_synth.expert_weights(5, "cpu", "fp8", E, H, I))
    w = lib.Weights(W, "fp8", pack=True)
    torch.cuda.synchronize()
    assert w.layout == lib.MOE_LAYOUT_K_BLOCKED
    assert set(w.packed) == {"w1", "w3", "w2"}          # per-channel scales stay as they are
    for name, C in (("w1", 64), ("w3", 64), ("w2", 32)):
        src = host(W[name])
        N, K = src.shape[1], src.shape[2]
        want = src.reshape(E, N, K // C, C).transpose(0, 2, 1, 3).reshape(-1)
        got = host(w.packed[name]).reshape(-1)
        assert (got == want).all(), name



@pytest.mark.parametrize("E,H,I", [(3, 256, 128), (2, 384, 640)])
def test_pack_weights_mxfp4(lib, E, H, I):
    """MXFP4: codes in 64-byte chunks and e8m0 scales in 4-byte chunks, both
    dst[e][c][n][0:C] == src[e][n][c*C:(c+1)*C], bit for bit."""
    say("pack_weights mxfp4", E, H, I)
    W = to_device(moe_synth.expert_weights(6, "cpu", "mxfp4", E, H, I))
    w = lib.Weights(W, "mxfp4", pack=True)
    torch.cuda.synchronize()
    assert w.layout == lib.MOE_LAYOUT_K_BLOCKED
    for name, C in (("w1", 64), ("w3", 64), ("w2", 64), ("s1", 4), ("s3", 4), ("s2", 4)):
        src = host(W[name])
        N, K = src.shape[1], src.shape[2]
        want = src.reshape(E, N, K // C, C).transpose(0, 2, 1, 3).reshape(-1)
        assert (host(w.packed[name]).reshape(-1) == want).all(), name