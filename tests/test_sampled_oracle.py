"""Host logic of the full-size parity tests: the token cover, the edge rows,
and the threaded per-expert assembly of the oracle's output, which must give
what ``oracle.moe.forward_sampled`` gives for the same tokens."""

import numpy as np
import torch

import moe_synth
import oracle
from gpu_helpers import SampledOracle, cover_tokens, edge_tokens, oracle_weights


def test_cover_tokens_reaches_every_routed_expert():
    rng = np.random.default_rng(3)
    T, E, k = 300, 40, 3
    ids = np.stack([rng.choice(E - 2, k, replace=False) for _ in range(T)])   # experts E-2, E-1 unused
    chosen = cover_tokens(ids, E, must=[7, 7, 299])
    assert chosen[:2] == [7, 299]
    assert set(np.unique(ids[chosen]).tolist()) == set(range(E - 2))
    assert len(chosen) <= T and len(set(chosen)) == len(chosen)


def test_edge_tokens_rows():
    # expert 1 is the hottest (10 rows at 3..12, tile 4: last tile starts at row 11)
    ids = np.array([[0, 1], [1, 2], [1, 0], [1, 2], [1, 2], [2, 1], [1, 0], [1, 2], [2, 1], [1, 2]], np.int32)
    counts, offsets = oracle.expert_counts_offsets(ids, 3)
    _, r2p, _, _ = oracle.permute_rows(ids, offsets, np.zeros((10, 1), np.uint8), np.zeros(10, np.float32))
    toks, rows = edge_tokens(counts, offsets, r2p, 2, 4)
    assert list(counts) == [3, 10, 7]
    assert rows == [3 + 8, 12, 2, 19]
    assert toks == [int(r2p[r]) // 2 for r in rows]


def test_sampled_oracle_matches_forward_sampled():
    inp = moe_synth.custom_inputs(60, 256, 128, 6, 2, seed=4, norm=True)
    xb = inp["x"].view(torch.int16).numpy().view(np.uint16)
    logits = inp["logits"].numpy()
    ids, w = oracle.route(logits, 2)
    W = oracle_weights(inp["routed"], "fp8")
    tokens = [5, 17, 0, 59, 33, 40]
    gamma = inp["gamma"].numpy()
    so = SampledOracle(xb, ids, w, tokens, W, gamma, inp["eps"], threads=3)
    got_a = so.output(np.array([0, 2, 4]))
    got_b = so.output(np.array([1, 3, 5]))
    ref = oracle.moe.forward_sampled(xb, None, 2, W, np.asarray(tokens), norm_gamma=gamma, norm_eps=inp["eps"],
                                     routing=(ids, w))
    np.testing.assert_allclose(got_a, ref[[0, 2, 4]], rtol=1e-12, atol=0)
    np.testing.assert_allclose(got_b, ref[[1, 3, 5]], rtol=1e-12, atol=0)
