"""Shared helpers of the GPU parity tests (the HIP library vs the CPU oracle).

Inputs come from ``moe_synth`` only; the oracle receives host copies of
them and never anything the HIP path produced.
"""

import sys

import numpy as np
import torch

import moe_synth
import oracle
from oracle.moe import ExpertWeights

DEV = "cuda"


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t):
    """bf16 tensor -> uint16 NumPy bits on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    return t.detach().cpu().numpy()


class DeviceStack:
    """Indexable view of a stacked device tensor that copies one expert at a time."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, e):
        return self.t[e].cpu().numpy()


def oracle_weights(d, fmt, lazy=False, activation="silu", beta=4.0):
    if d is None:
        return None
    wrap = DeviceStack if lazy else host
    return ExpertWeights(fmt, *(wrap(d[k]) for k in ("w1", "w3", "w2", "s1", "s3", "s2")),
                         activation=activation, beta=beta)


def tolerance_ratio(gpu, oracle_exact):
    """max|gpu - oracle| / RMS(oracle).

    ``gpu``: bf16 bits (uint16) or float values; ``oracle_exact``: the
    oracle's float64 output before any final bf16 rounding (the layer stores
    its output as bf16, so the GPU side carries that one rounding).
    """
    g = oracle.codecs.bf16_decode(gpu) if np.asarray(gpu).dtype == np.uint16 else np.asarray(gpu, np.float64)
    r = np.asarray(oracle_exact, dtype=np.float64)
    rms = float(np.sqrt(np.mean(r * r)))
    err = float(np.max(np.abs(g - r))) if r.size else 0.0
    return err / rms if rms > 0 else err


# Output acceptance: max|err| <= 2e-2 * RMS(oracle output), fp32 accumulation.
OUT_TOL = 2e-2
# Router weights: relative 1e-6.
W_RTOL = 1e-6


def assert_weights_close(w_gpu, w_oracle):
    w_gpu = np.asarray(w_gpu, dtype=np.float64)
    err = np.abs(w_gpu - w_oracle) / np.abs(w_oracle)
    assert err.max() <= W_RTOL, err.max()


def run_forward(inp, capture=True, pack=True, score="softmax", act=("silu", "silu"), beta=4.0):
    """moe_forward on device inputs; returns (out, captured dict, variant).
    pack=False keeps fp8 weights row-major instead of K-blocked; ``act``:
    activation of the routed and of the shared experts."""
    import mixture_experts_ffn_softmax_amd as moe

    c = inp["cfg"]
    T, E, k, H = c["T"], c["E"], c["k"], c["H"]
    routed = moe.Weights(inp["routed"], c["fmt"], pack=pack, activation=act[0], beta=beta)
    shared = (moe.Weights(inp["shared"], "fp8", pack=pack, activation=act[1], beta=beta)
              if inp["shared"] is not None else None)
    dbg = None
    if capture:
        z = lambda shape, dt: torch.empty(shape, dtype=dt, device=DEV)  # noqa: E731
        dbg = dict(topk_ids=z((T, k), torch.int32), topk_w=z((T, k), torch.float32),
                   expert_counts=z((E,), torch.int32),
                   expert_offsets=z((E + (2 if shared else 1),), torch.int32),
                   pair_to_row=z((T, k), torch.int32), row_to_pair=z((T * k,), torch.int32),
                   xq_rows=z((T * k, H), torch.uint8), xs_rows=z((T * k,), torch.float32))
    res = moe.moe_forward(inp["x"], inp["logits"], k, routed, shared, inp["gamma"], inp["eps"], debug=dbg,
                          score=score)
    out, variant = res if capture else (res, None)
    torch.cuda.synchronize()
    return out, dbg, variant


def to_device(inp):
    def mv(v):
        if isinstance(v, torch.Tensor):
            return v.to(DEV)
        if isinstance(v, dict):
            return {k: mv(t) for k, t in v.items()}
        return v
    return {k: mv(v) for k, v in inp.items()}


def check_metadata(dbg, ref, T, k, E, shared):
    """Bit-exact routing ids, counts, offsets, permutation; weights rel 1e-6."""
    assert (host(dbg["topk_ids"]) == ref["topk_ids"]).all()
    assert_weights_close(host(dbg["topk_w"]), ref["topk_w"])
    assert (host(dbg["expert_counts"]) == ref["counts"]).all()
    off = host(dbg["expert_offsets"])
    assert (off[:E + 1] == ref["offsets"]).all()
    if shared:
        assert off[E + 1] == T * k + T
    assert (host(dbg["pair_to_row"]) == ref["pair_to_row"]).all()
    assert (host(dbg["row_to_pair"]) == ref["row_to_pair"]).all()


__all__ = ["moe_synth"]


# ----------------------------------------------------------------------------
# full-size workloads: sampled tokens that reach every expert
# ----------------------------------------------------------------------------


def cover_tokens(ids, n_experts, must=()):
    """Tokens, starting with ``must``, chosen greedily (most experts not yet
    reached first) until every expert that any token routes to appears among
    the chosen tokens' pairs.  Returns them in the order chosen."""
    ids = np.asarray(ids)
    T = ids.shape[0]
    onehot = np.zeros((T, n_experts), dtype=bool)
    onehot[np.arange(T)[:, None], ids] = True
    present = onehot.any(axis=0)
    chosen, covered = [], np.zeros(n_experts, dtype=bool)
    for t in must:
        if t not in chosen:
            chosen.append(int(t))
            covered |= onehot[t]
    while (present & ~covered).any():
        t = int(np.argmax((onehot & ~covered).sum(axis=1)))
        chosen.append(t)
        covered |= onehot[t]
    return chosen


def edge_tokens(counts, offsets, row_to_pair, k, tile):
    """Tokens whose rows sit where tiling is ragged or indices are large: the
    first and last rows of the hottest expert's last row tile (``tile`` rows
    per tile), the last row of the least-loaded non-empty expert, and the
    last routed row overall."""
    counts = np.asarray(counts)
    hot = int(np.argmax(counts))
    first_of_last = int(offsets[hot]) + ((int(counts[hot]) - 1) // tile) * tile
    nz = np.flatnonzero(counts)
    cold = int(nz[np.argmin(counts[nz])])
    rows = [first_of_last, int(offsets[hot + 1]) - 1, int(offsets[cold + 1]) - 1, int(offsets[-1]) - 1]
    return [int(row_to_pair[r]) // k for r in rows], rows


class OneExpert:
    """Expert e of a stacked weight tensor as a one-expert stack."""

    def __init__(self, stack, e):
        self.stack, self.e = stack, e
        self.shape = (1,) + tuple(stack.shape[1:])

    def __getitem__(self, i):
        assert i == 0
        return self.stack[self.e]


class SampledOracle:
    """The oracle's layer output for a chosen set of tokens, built from the
    oracle's own steps in the order ``oracle.moe.forward_sampled`` takes them
    (quantise the chosen tokens, permute their pairs, the expert FFN of each
    expert's rows, combine).  Rows of different experts are independent, so
    each expert's FFN runs once, for all chosen tokens' rows of that expert,
    on a thread pool, when a subset of the tokens first needs it; ``output``
    then combines any subset of the chosen tokens."""

    def __init__(self, x_bits, ids, w, tokens, weights, gamma=None, eps=1e-6, threads=None):
        import os
        self.tokens = np.asarray(tokens, dtype=np.int64)
        self.weights, self.gamma, self.eps = weights, gamma, eps
        xq, xs = oracle.quantize_tokens(np.asarray(x_bits)[self.tokens])
        self.sub_ids = np.asarray(ids)[self.tokens]
        self.w = np.asarray(w)[self.tokens]
        _, self.off = oracle.expert_counts_offsets(self.sub_ids, weights.n_experts)
        self.p2r, _, self.q, self.s = oracle.permute_rows(self.sub_ids, self.off, xq, xs)
        self.y = np.zeros((len(self.tokens) * self.sub_ids.shape[1], weights.hidden))
        self.done = set()
        self.threads = threads or min(16, os.cpu_count() or 1)

    def _expert(self, e):
        r0, r1 = int(self.off[e]), int(self.off[e + 1])
        wt = self.weights
        one = ExpertWeights(wt.fmt, *(OneExpert(getattr(wt, n), e) for n in ("w1", "w3", "w2", "s1", "s3", "s2")),
                            activation=wt.activation, beta=wt.beta)
        self.y[r0:r1] = oracle.expert_ffn(self.q[r0:r1], self.s[r0:r1], np.array([0, r1 - r0]), one)[0]

    def output(self, idx):
        """float64 output (before the bf16 rounding) of chosen tokens ``idx``
        (positions in ``tokens``)."""
        import concurrent.futures
        idx = np.asarray(idx)
        need = sorted(set(int(e) for e in np.unique(self.sub_ids[idx])) - self.done)
        with concurrent.futures.ThreadPoolExecutor(self.threads) as ex:
            list(ex.map(self._expert, need))
        self.done.update(need)
        return oracle.combine(self.y, self.p2r[idx], self.w[idx], None, self.gamma, self.eps, rounded=False)
