"""Full-size output parity that reaches every expert.

The two many-expert workloads run once each through moe_forward at full
size: the skewed whole layer (16384 tokens, 256 experts, top-8, Zipf-biased
router logits, the pages' 16,384-token prefill of the 1T model on one
device) and the LatentMoE expert core (512 tokens of latent 3584, 896 MXFP4
experts 3584 -> 3072 -> 3584, top-16, RMSNorm; Kimi K3 page, §2.4).  All
routing metadata is compared in full.  Outputs are compared for a set of
tokens chosen so that every expert that receives a row appears among their
pairs, plus the tokens of the rows where the tiling is ragged or the row
index is large: the first and last rows of the hottest expert's last row
tile, the least-loaded expert's last row and the last routed row.  The
chosen tokens are checked in chunks (one test each); the oracle computes
each expert's rows once, when a chunk first needs that expert.
"""

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_helpers import (DEV, OUT_TOL, SampledOracle, bits, check_metadata, cover_tokens, edge_tokens, host,
                         oracle_weights, run_forward, say, tolerance_ratio)

pytestmark = pytest.mark.gpu

CHUNKS = {"skewed": 2, "latent": 4}


class Run:
    """One full-size forward on the GPU and the host copies the checks use."""

    def __init__(self, name):
        inp = moe_synth.make_inputs(name, device=DEV)
        c = self.cfg = inp["cfg"]
        T, E, k = c["T"], c["E"], c["k"]
        say("coverage run", name, c)
        out, dbg, self.variant = run_forward(inp)
        say("  variant", self.variant)
        self.tile = int(self.variant.split("/")[0].lstrip("smalrge"))
        ids, w = oracle.route(host(inp["logits"]), k)
        counts, offsets = oracle.expert_counts_offsets(ids, E)
        p2r, r2p, _, _ = oracle.permute_rows(ids, offsets, np.zeros((T, 1), np.uint8), np.zeros(T, np.float32))
        self.ref = dict(topk_ids=ids, topk_w=w, counts=counts, offsets=offsets, pair_to_row=p2r, row_to_pair=r2p)
        self.dbg = dbg
        self.edge, self.edge_rows = edge_tokens(counts, offsets, r2p, k, self.tile)
        self.tokens = cover_tokens(ids, E, must=self.edge)
        say("  tokens", len(self.tokens), "edge rows", self.edge_rows)
        self.out = bits(out)
        x = bits(inp["x"])
        tok_d = torch.as_tensor(self.tokens, device=DEV)
        # quantised bytes of every chosen token's rows
        xq, xs = oracle.quantize_tokens(x[self.tokens])
        self.rows_q_ok = True
        for j in range(k):
            r_d = torch.as_tensor(p2r[self.tokens, j], device=DEV)
            self.rows_q_ok &= bool((host(dbg["xq_rows"][r_d]) == xq).all())
            self.rows_q_ok &= bool((host(dbg["xs_rows"][r_d]).view(np.uint32) == xs.view(np.uint32)).all())
        del tok_d
        self.oracle = SampledOracle(x, ids, w, self.tokens, oracle_weights(inp["routed"], c["fmt"], lazy=True),
                                    None if inp["gamma"] is None else host(inp["gamma"]), inp["eps"])
        self.inp = inp


_RUNS = {}


def get_run(name):
    if name not in _RUNS:
        _RUNS.clear()                      # one workload's device tensors at a time
        torch.cuda.empty_cache()
        _RUNS[name] = Run(name)
    return _RUNS[name]


# each workload's metadata check, then its output chunks, so that one run serves them all
PARTS = [(n, part) for n, m in CHUNKS.items() for part in ["metadata"] + list(range(m))]


@pytest.mark.parametrize("name,part", PARTS)
def test_full_size(lib, name, part):
    """part "metadata": all routing metadata bit-exact, the skew of the
    skewed workload, every routed-to expert reached by the chosen tokens and
    the quantised bytes of their rows.  part i: the outputs of chunk i of the
    chosen tokens within max|err| <= 2e-2 * RMS(oracle)."""
    r = get_run(name)
    c = r.cfg
    if part == "metadata":
        check_metadata(r.dbg, r.ref, c["T"], c["k"], c["E"], c["shared"])
        counts = r.ref["counts"]
        if name == "skewed":
            assert counts.max() / counts.mean() == pytest.approx(5.0, abs=0.11)
            assert max(r.edge_rows) > 65536
        reached = np.unique(r.ref["topk_ids"][r.tokens])
        assert set(reached.tolist()) == set(np.flatnonzero(counts).tolist())
        assert r.rows_q_ok
        return
    n = CHUNKS[name]
    idx = np.arange(part, len(r.tokens), n)
    toks = np.asarray(r.tokens)[idx]
    say("coverage outputs", name, "chunk", part, "of", n, ":", len(toks), "tokens,",
        len(np.unique(r.ref["topk_ids"][toks])), "experts")
    ref = r.oracle.output(idx)
    ratio = tolerance_ratio(r.out[toks], ref)
    say("  max|err|/rms", ratio)
    assert ratio <= OUT_TOL


def test_full_size_release(lib):
    """Frees the cached full-size runs (their device tensors)."""
    _RUNS.clear()
    torch.cuda.empty_cache()
