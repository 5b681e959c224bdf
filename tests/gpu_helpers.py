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
