"""Per-token fp8 quantisation at the e4m3 rounding midpoints, on the GPU.

The Ling-2.6-1T page, §5 "activation quantisation": each token is scaled by
s = amax / 448 and its elements x / s are encoded as fp8 e4m3 before the
scatter.  The quantised bytes must match the oracle bit for bit, and the
places where an encoder can go wrong are the rounding midpoints between
neighbouring e4m3 values (ties go to the even code), the binary32 values one
ulp either side of them, the subnormal grid below 2^-6 and its edge, and the
saturation at +-448.

The rows below are crafted so that the quotients x / s (IEEE binary32
division, as the method defines them) land on each of those points: for a
row whose largest element is a, s = f32(a / 448); every bf16 x <= a is tried
and kept when f32(x / s) is a midpoint or one binary32 ulp from one.  The
e4m3 grid used for the crafting is written here from the OCP E4M3FN
definition (bias 7, three mantissa bits, subnormal step 2^-9, largest 448);
the expected bytes come from the oracle only.

The enumeration is exhaustive (a over one binade gives every quotient a
bf16 row can produce, since scaling a row by a power of two leaves its
quotients unchanged).  It finds every midpoint below 448 as an exact
quotient, and one binary32 ulp either side of a midpoint for 16 of them.
No quotient lies two to eight ulps from a midpoint.  Bf16 activations under
the amax / 448 rule thus reach the midpoints only in these few ways, and the
rows below contain all of them, at six row scales.
"""

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_helpers import DEV, bits, host, run_forward, say, to_device

H = 256


def e4m3_positive_values():
    sub = [k * 2.0 ** -9 for k in range(1, 8)]
    normal = [(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8) if not (e == 15 and m == 7)]
    return np.array(sub + normal)


def midpoints():
    """Midpoints between consecutive non-negative e4m3 values, and 464 (the
    midpoint between 448 and the next value e4m3 would have)."""
    v = np.concatenate([[0.0], e4m3_positive_values()])
    return np.concatenate([(v[:-1] + v[1:]) / 2, [464.0]])


def _bf16_positive(lo, hi):
    """All positive bf16 values in [lo, hi] as float32."""
    b = np.arange(1, 0x7F80, dtype=np.uint32) << np.uint32(16)
    f = b.view(np.float32)
    return f[(f >= lo) & (f <= hi)]


def near_midpoint_elements():
    """Every (a, x) with a a bf16 value in [1, 2) and x a positive bf16 value
    <= a whose quotient q = f32(x / f32(a / 448)) is a midpoint or within one
    binary32 ulp of one.  Scaling a row by 2^j scales s by 2^j exactly and
    leaves every quotient as it is (while all stay normal), so rows with a
    in [1, 2) produce every quotient any row can.  Returns a list of
    (a, x, midpoint, ulp offset)."""
    mids = midpoints().astype(np.float32)
    mb = mids.view(np.int32)
    out = []
    for a in _bf16_positive(1.0, 1.9999):
        a32 = np.float32(a)
        s = np.float32(a32 / np.float32(448.0))                  # binary32 division
        xs = _bf16_positive(float(s) * 2.0 ** -11, float(a32))
        q = (xs / s).astype(np.float32)                          # binary32 division
        qb = q.view(np.int32)
        j = np.clip(np.searchsorted(mb, qb), 1, len(mb) - 1)
        near = np.where(np.abs(qb - mb[j - 1]) <= np.abs(qb - mb[j]), j - 1, j)
        d = qb - mb[near]
        keep = np.abs(d) <= 1
        out += [(float(a32), float(x), float(m), int(dd)) for x, m, dd in zip(xs[keep], mids[near[keep]], d[keep])]
    return out


# row scales 2^j: every element stays a normal bf16 and s a normal binary32
ROW_SCALES = (-96, -40, 0, 9, 40, 96)


def crafted_rows():
    """bf16 rows [N][H] (as float32 values): for each row maximum a of
    ``near_midpoint_elements``, its elements x with alternating signs, at
    every scale 2^j of ROW_SCALES; rows whose maximum's own quotient sits a
    little above 448 (saturation); and a row (s = 1) with elements at the
    subnormal edge (2^-6, 7.5 * 2^-9) and on the subnormal grid's midpoints.
    Returns (rows, hits): hits[(midpoint, ulp offset)] counts the elements
    placed there (at scale 1)."""
    by_a, hits = {}, {}
    for a, x, m, d in near_midpoint_elements():
        by_a.setdefault(a, []).append(x)
        hits[(m, d)] = hits.get((m, d), 0) + 1
    base = []
    for a, xs in sorted(by_a.items()):
        vals = [-x if i % 2 else x for i, x in enumerate(xs)]
        for i in range(0, len(vals), H - 1):
            part = [a] + vals[i:i + H - 1]
            base.append(part + [0.0] * (H - len(part)))
    rows = [np.float32(2.0 ** j) * np.array(r, dtype=np.float32) for j in ROW_SCALES for r in base]
    rng = np.random.default_rng(0)
    for a in rng.choice(_bf16_positive(2.0 ** -60, 2.0 ** 60), 64, replace=False):
        rows.append(np.array([a, -a] + [0.0] * (H - 2), dtype=np.float32))
    edge = [448.0, 2.0 ** -6, -(2.0 ** -6), 7.5 * 2.0 ** -9, -7.5 * 2.0 ** -9] + \
           [(k + 0.5) * 2.0 ** -9 * (-1) ** k for k in range(7)] + [2.0 ** -10, 2.0 ** -11]
    rows.append(np.array(edge + [0.0] * (H - len(edge)), dtype=np.float32))
    rows = np.stack(rows)
    rows = rows[rng.permutation(len(rows))]
    return rows, hits


def test_crafted_rows_reach_every_midpoint():
    """Host check of the crafting (no GPU): the rows are bf16 values; every
    midpoint below 448 is some quotient exactly, and the quotients one ulp
    from a midpoint that bf16 rows can produce are all present."""
    rows, hits = crafted_rows()
    assert (rows.view(np.uint32) & 0xFFFF == 0).all()
    mids = midpoints()
    exact = {m for (m, d) in hits if d == 0}
    assert exact == set(float(m) for m in mids[mids < 448]), sorted(set(mids) - exact)
    assert len({m for (m, d) in hits if d == -1}) >= 16 and len({m for (m, d) in hits if d == 1}) >= 16
    # the scaled rows give the same quotients: recompute one row's at every scale
    a, x, m, d = near_midpoint_elements()[0]
    for j in ROW_SCALES:
        f = np.float32(2.0 ** j)
        q = np.float32(np.float32(x) * f) / np.float32(np.float32(a) * f / np.float32(448.0))
        assert np.float32(q).view(np.int32) - np.float32(m).view(np.int32) == d


def _bf16(rows):
    return torch.from_numpy(rows.copy()).to(torch.bfloat16)


@pytest.mark.gpu
def test_quant_midpoints_permute(lib):
    """moe_permute's quantisation (one workgroup per token) on the crafted rows."""
    rows, _ = crafted_rows()
    x = _bf16(rows)
    T = x.shape[0]
    ids = moe_synth.random_topk_ids(T, 4, 2, seed=T)
    say("quant midpoints permute", T, H)
    res = lib.moe_permute(x.to(DEV), ids.to(DEV), 4, token_order=True)
    torch.cuda.synchronize()
    xq, xs = oracle.quantize_tokens(bits(x))
    assert (host(res["xq_tok"]) == xq).all()
    assert (host(res["xs_tok"]).view(np.uint32) == xs.view(np.uint32)).all()


@pytest.mark.gpu
def test_quant_midpoints_forward(lib):
    """moe_forward's one-launch routing + quantisation kernel (at most 32
    experts) on the crafted rows: the expert-ordered bytes it captures."""
    rows, _ = crafted_rows()
    x = _bf16(rows)
    T = x.shape[0]
    inp = moe_synth.custom_inputs(T, H, 128, 4, 2, seed=3)
    inp["x"] = x
    say("quant midpoints forward", T, H)
    _, dbg, _ = run_forward(to_device(inp))
    # the oracle's quantisation and permutation (the FFN is not needed here)
    ids, _ = oracle.route(inp["logits"].numpy(), 2)
    _, offsets = oracle.expert_counts_offsets(ids, 4)
    xq, xs = oracle.quantize_tokens(bits(x))
    _, _, xq_rows, xs_rows = oracle.permute_rows(ids, offsets, xq, xs)
    assert (host(dbg["xq_rows"]) == xq_rows).all()
    assert (host(dbg["xs_rows"]).view(np.uint32) == xs_rows.view(np.uint32)).all()
