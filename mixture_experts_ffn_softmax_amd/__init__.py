"""Routed mixture-of-experts layer on MI355X (gfx950): Python binding.

Thin wrappers with the names of the C ABI (include/moe.h).  They marshal
torch tensors (device memory) and the current HIP stream into the library
and allocate outputs / workspaces with torch; every step of the layer runs in
the library's kernels.  There is no fallback: if libmoe.so is missing the
import of the library fails with an error.
"""

import ctypes

import torch

from . import _lib
from ._lib import (MOE_LAYOUT_K_BLOCKED, MOE_LAYOUT_ROW_MAJOR, MOE_LIN_BF16, MOE_LIN_MXFP4, MOE_N_STAGES,
                   MOE_W_FP8, MOE_W_MXFP4, STAGE_NAMES, MoeDebug, MoeError, MoeLatent, MoeLinear, MoeWeights,
                   check)

__all__ = ["Weights", "Linear", "LatentWeights", "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_forward", "moe_forward_noalloc", "forward_workspace_size", "moe_linear", "moe_latent_forward",
           "latent_forward_workspace_size", "MoeError", "lib"]


def lib():
    return _lib.load()


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t, name, dtype, ndim=None, optional=False):
    """Checks that tensor ``t`` is a contiguous device tensor of ``dtype``
    (and ``ndim`` dimensions): the library reads raw pointers, so a wrong
    dtype or a strided view would be misread rather than converted."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Weights:
    """A group of experts: keeps the tensors alive and holds the moe_weights_t.

    ``d`` has w1, w3, w2, s1, s3, s2 as produced by ``moe_synth`` (uint8 codes;
    float32 per-channel scales for fp8, uint8 e8m0 block scales for mxfp4).
    The weights are repacked once into the K-blocked layout (moe_pack_weights;
    for MXFP4 the block scales too) unless ``pack`` is False; ``self.tensors``
    keeps the row-major originals.
    ``activation``: "silu" or "situ" (with ``beta``).
    """

    def __init__(self, d, fmt, pack=True, stream=None, activation="silu", beta=4.0):
        self.tensors = {k: v.contiguous() for k, v in d.items()}
        t = self.tensors
        self.fmt = {"fp8": MOE_W_FP8, "mxfp4": MOE_W_MXFP4, "fp8_block": _lib.MOE_W_FP8_BLOCK}[fmt]
        scale_dtype = torch.uint8 if fmt == "mxfp4" else torch.float32
        for key in ("w1", "w3", "w2"):
            _need(t.get(key), key, torch.uint8, 3)
        for key in ("s1", "s3", "s2"):
            _need(t.get(key), key, scale_dtype, 3 if fmt != "fp8" else 2)
        E, I = t["w1"].shape[0], t["w1"].shape[1]
        H = t["w2"].shape[1]
        self.n_experts, self.hidden, self.inter = E, H, I
        ptrs = [t[k].data_ptr() for k in ("w1", "w3", "w2", "s1", "s3", "s2")]
        act = _lib.MOE_ACT_SITU if activation == "situ" else _lib.MOE_ACT_SILU
        self.activation, self.beta = activation, beta
        self.c = MoeWeights(self.fmt, E, H, I, MOE_LAYOUT_ROW_MAJOR, act, beta, 0, *ptrs)
        self.packed = None
        if pack:
            moved = ("w1", "w3", "w2") + (("s1", "s3", "s2") if self.fmt == MOE_W_MXFP4 else ())
            self.packed = {k: torch.empty_like(t[k]) for k in moved}
            dst_ptrs = [(self.packed[k] if k in self.packed else t[k]).data_ptr()
                        for k in ("w1", "w3", "w2", "s1", "s3", "s2")]
            dst = MoeWeights(self.fmt, E, H, I, MOE_LAYOUT_K_BLOCKED, act, beta, 0, *dst_ptrs)
            check(lib().moe_pack_weights(ctypes.byref(self.c), ctypes.byref(dst), _stream(stream)))
            self.c = dst

    @property
    def layout(self):
        return self.c.layout

    def ref(self):
        return ctypes.byref(self.c)


# dtypes of the intermediates a debug capture may receive
_DEBUG_DTYPES = dict(topk_ids=torch.int32, topk_w=torch.float32, expert_counts=torch.int32,
                     expert_offsets=torch.int32, pair_to_row=torch.int32, row_to_pair=torch.int32,
                     xq_rows=torch.uint8, xs_rows=torch.float32, latent=torch.bfloat16,
                     core_out=torch.bfloat16)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def _score(score):
    return {"softmax": _lib.MOE_SCORE_SOFTMAX, "sigmoid": _lib.MOE_SCORE_SIGMOID}[score]


def moe_route(logits, top_k, topk_ids=None, topk_w=None, score="softmax", stream=None):
    _need(logits, "logits", torch.float32, 2)
    _need(topk_ids, "topk_ids", torch.int32, 2, optional=True)
    _need(topk_w, "topk_w", torch.float32, 2, optional=True)
    T, E = logits.shape
    dev = logits.device
    topk_ids = _empty((T, top_k), torch.int32, dev) if topk_ids is None else topk_ids
    topk_w = _empty((T, top_k), torch.float32, dev) if topk_w is None else topk_w
    check(lib().moe_route(_p(logits), T, E, top_k, _score(score), _p(topk_ids), _p(topk_w),
                          _stream(stream)))
    return topk_ids, topk_w


def moe_permute(x, topk_ids, n_experts, token_order=False, stream=None):
    """Returns dict(counts, offsets, pair_to_row, row_to_pair, xq_rows, xs_rows[, xq_tok, xs_tok])."""
    _need(x, "x", torch.bfloat16, 2)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    T, H = x.shape
    k = topk_ids.shape[1]
    dev = x.device
    R = T * k
    out = dict(counts=_empty((n_experts,), torch.int32, dev),
               offsets=_empty((n_experts + 1,), torch.int32, dev),
               pair_to_row=_empty((T, k), torch.int32, dev),
               row_to_pair=_empty((R,), torch.int32, dev),
               xq_rows=_empty((R, H), torch.uint8, dev),
               xs_rows=_empty((R,), torch.float32, dev))
    if token_order:
        out["xq_tok"] = _empty((T, H), torch.uint8, dev)
        out["xs_tok"] = _empty((T,), torch.float32, dev)
    nbytes = lib().moe_permute_workspace_size(T, k, n_experts)
    ws = _empty((nbytes,), torch.uint8, dev)
    check(lib().moe_permute(_p(x), T, H, _p(topk_ids), k, n_experts, _p(out["counts"]),
                            _p(out["offsets"]), _p(out["pair_to_row"]), _p(out["row_to_pair"]),
                            _p(out["xq_rows"]), _p(out["xs_rows"]), _p(out.get("xq_tok")),
                            _p(out.get("xs_tok")), _p(ws), nbytes, _stream(stream)))
    return out


def moe_expert_ffn(xq_rows, xs_rows, expert_offsets, weights, stream=None):
    _need(xq_rows, "xq_rows", torch.uint8, 2)
    _need(xs_rows, "xs_rows", torch.float32, 1)
    _need(expert_offsets, "expert_offsets", torch.int32, 1)
    n_rows = xq_rows.shape[0]
    dev = xq_rows.device
    y = _empty((n_rows, weights.hidden), torch.float32, dev)
    nbytes = lib().moe_expert_ffn_workspace_size(n_rows, weights.ref())
    ws = _empty((max(nbytes, 1),), torch.uint8, dev)
    check(lib().moe_expert_ffn(_p(xq_rows), _p(xs_rows), n_rows, _p(expert_offsets), weights.ref(),
                               _p(y), _p(ws), nbytes, _stream(stream)))
    return y


def moe_combine(y_rows, pair_to_row, topk_w, y_shared=None, norm_gamma=None, norm_eps=1e-6,
                stream=None):
    _need(y_rows, "y_rows", torch.float32, 2)
    _need(pair_to_row, "pair_to_row", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    _need(y_shared, "y_shared", torch.float32, 2, optional=True)
    _need(norm_gamma, "norm_gamma", torch.float32, 1, optional=True)
    T, k = pair_to_row.shape
    H = y_rows.shape[1]
    out = _empty((T, H), torch.bfloat16, y_rows.device)
    check(lib().moe_combine(_p(y_rows), _p(pair_to_row), _p(topk_w), T, H, k, _p(y_shared),
                            _p(norm_gamma), float(norm_eps), _p(out), _stream(stream)))
    return out


def forward_workspace_size(T, top_k, routed, use_shared):
    return lib().moe_forward_workspace_size(T, top_k, routed.ref(), int(bool(use_shared)))


def moe_forward(x, logits, top_k, routed, shared=None, norm_gamma=None, norm_eps=1e-6, out=None,
                ws=None, debug=None, events=None, gemm1_events=None, gemm2_events=None,
                layer_events=None, score="softmax", stream=None):
    """The whole layer.  ``debug``: dict of device tensors to capture
    (keys topk_ids, topk_w, expert_counts, expert_offsets, pair_to_row,
    row_to_pair, xq_rows, xs_rows).  ``events``: list of MOE_N_STAGES + 1
    torch.cuda.Event (or None) recorded at the stage boundaries.
    ``gemm1_events`` / ``gemm2_events``: (start, stop) torch.cuda.Event stamped
    by the gate-up / down GEMM's dispatch; ``layer_events``: (start, stop)
    stamped by the layer's first and last dispatch.  Returns ``out`` (and the
    chosen kernel variant string when debug is given)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(logits, "logits", torch.float32, 2)
    _need(norm_gamma, "norm_gamma", torch.float32, 1, optional=True)
    _need(out, "out", torch.bfloat16, 2, optional=True)
    _need(ws, "ws", torch.uint8, 1, optional=True)
    T, H = x.shape
    dev = x.device
    out = _empty((T, H), torch.bfloat16, dev) if out is None else out
    nbytes = forward_workspace_size(T, top_k, routed, shared is not None)
    if ws is None:
        ws = _empty((nbytes,), torch.uint8, dev)
    dbg = None
    if debug is not None or any(v is not None for v in (events, gemm1_events, gemm2_events, layer_events)):
        dbg = MoeDebug()
        for key, t in (debug or {}).items():
            _need(t, f"debug[{key}]", _DEBUG_DTYPES[key])
            setattr(dbg, key, t.data_ptr())
        for i, ev in enumerate(events or []):
            if ev is not None:
                dbg.events[i] = ev.cuda_event
        for i, ev in enumerate(gemm1_events or []):
            dbg.gemm1_events[i] = ev.cuda_event
        for i, ev in enumerate(gemm2_events or []):
            dbg.gemm2_events[i] = ev.cuda_event
        for i, ev in enumerate(layer_events or []):
            dbg.layer_events[i] = ev.cuda_event
    check(lib().moe_forward(_p(x), _p(logits), T, top_k, _score(score), routed.ref(), int(shared is not None),
                            shared.ref() if shared is not None else None, _p(norm_gamma),
                            float(norm_eps), _p(out), ctypes.byref(dbg) if dbg is not None else None,
                            _p(ws), _nbytes(ws), _stream(stream)))
    if debug is not None:
        return out, dbg.variant.decode()
    return out


def moe_forward_noalloc(x, logits, top_k, routed, shared=None, norm_gamma=None, norm_eps=1e-6, out=None,
                        debug=None, score="softmax", stream=None):
    """moe_forward with the library's per-device scratch as its workspace:
    the call allocates nothing on the device (``out`` may be passed in for a
    call that allocates nothing at all).  Calls that need more than
    MOE_NOALLOC_SCRATCH_BYTES of workspace raise MoeError (MOE_ERR_WORKSPACE).
    ``debug`` as for moe_forward.  Returns ``out`` (and the variant string
    when debug is given)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(logits, "logits", torch.float32, 2)
    _need(norm_gamma, "norm_gamma", torch.float32, 1, optional=True)
    _need(out, "out", torch.bfloat16, 2, optional=True)
    T, H = x.shape
    out = _empty((T, H), torch.bfloat16, x.device) if out is None else out
    dbg = None
    if debug is not None:
        dbg = MoeDebug()
        for key, t in debug.items():
            _need(t, f"debug[{key}]", _DEBUG_DTYPES[key])
            setattr(dbg, key, t.data_ptr())
    check(lib().moe_forward_noalloc(_p(x), _p(logits), T, top_k, _score(score), routed.ref(),
                                    int(shared is not None), shared.ref() if shared is not None else None,
                                    _p(norm_gamma), float(norm_eps), _p(out),
                                    ctypes.byref(dbg) if dbg is not None else None, _stream(stream)))
    if debug is not None:
        return out, dbg.variant.decode()
    return out


# ----------------------------------------------------------------------------
# LatentMoE block
# ----------------------------------------------------------------------------


class Linear:
    """One dense projection W [n_out][n_in]: ``w`` uint8 MXFP4 codes [n_out][n_in/2]
    with ``s`` uint8 e8m0 [n_out][n_in/32], or ``w`` bf16 [n_out][n_in] (s None)."""

    def __init__(self, w, s=None):
        self.w = w.contiguous()
        self.s = None if s is None else s.contiguous()
        mx = self.s is not None
        n_in = self.w.shape[1] * (2 if mx else 1)
        self.c = MoeLinear(MOE_LIN_MXFP4 if mx else MOE_LIN_BF16, self.w.shape[0], n_in, 0,
                           self.w.data_ptr(), self.s.data_ptr() if mx else None)

    def ref(self):
        return ctypes.byref(self.c)


class LatentWeights:
    """The block's weights around the routed experts: ``down`` / ``up`` dicts
    {w, s} (MXFP4), ``shared`` dict {w1, w3, w2} of bf16 tensors or None."""

    def __init__(self, down, up, shared=None, activation="silu", beta=4.0):
        self.down, self.up = Linear(down["w"], down["s"]), Linear(up["w"], up["s"])
        self.shared = None if shared is None else {k: v.contiguous() for k, v in shared.items()}
        sh = self.shared
        act = _lib.MOE_ACT_SITU if activation == "situ" else _lib.MOE_ACT_SILU
        self.hidden, self.latent = self.down.c.n_in, self.down.c.n_out
        self.c = MoeLatent(self.down.c, self.up.c, 0 if sh is None else sh["w1"].shape[0], act, beta, 0,
                           *((None, None, None) if sh is None else (sh[k].data_ptr() for k in ("w1", "w3", "w2"))))

    def ref(self):
        return ctypes.byref(self.c)


def moe_linear(a, weights, addend=None, out_dtype=torch.bfloat16, out=None, stream=None):
    """out = a W^T (+ addend before the bf16 rounding)."""
    _need(a, "a", torch.bfloat16, 2)
    _need(addend, "addend", torch.float32, 2, optional=True)
    if out is not None and out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    if out is not None:
        _need(out, "out", out.dtype, 2)
    M = a.shape[0]
    if out is None:
        out = _empty((M, weights.c.n_out), out_dtype, a.device)
    bf = out.dtype == torch.bfloat16
    check(lib().moe_linear(_p(a), M, weights.ref(), _p(addend), _p(out) if bf else None,
                           None if bf else _p(out), _stream(stream)))
    return out


def latent_forward_workspace_size(T, top_k, latent, routed):
    return lib().moe_latent_forward_workspace_size(T, top_k, routed.ref(), latent.ref())


def moe_latent_forward(x, logits, top_k, latent, routed, norm_gamma=None, norm_eps=1e-6, out=None, ws=None,
                       debug=None, layer_events=None, gemm1_events=None, gemm2_events=None, score="softmax",
                       stream=None):
    """The LatentMoE block.  ``debug``: dict of device tensors as for
    moe_forward plus ``latent`` and ``core_out`` (bf16 [T][L]);
    ``layer_events`` bracket the block, ``gemm1_events`` / ``gemm2_events``
    the routed core's GEMMs.  Returns ``out`` (and the core's kernel variant
    string when debug is given)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(logits, "logits", torch.float32, 2)
    _need(norm_gamma, "norm_gamma", torch.float32, 1, optional=True)
    _need(out, "out", torch.bfloat16, 2, optional=True)
    _need(ws, "ws", torch.uint8, 1, optional=True)
    T = x.shape[0]
    out = _empty((T, latent.hidden), torch.bfloat16, x.device) if out is None else out
    nbytes = latent_forward_workspace_size(T, top_k, latent, routed)
    if ws is None:
        ws = _empty((max(nbytes, 1),), torch.uint8, x.device)
    dbg = None
    if debug is not None or any(v is not None for v in (layer_events, gemm1_events, gemm2_events)):
        dbg = MoeDebug()
        for key, t in (debug or {}).items():
            _need(t, f"debug[{key}]", _DEBUG_DTYPES[key])
            setattr(dbg, key, t.data_ptr())
        for name, evs in (("layer_events", layer_events), ("gemm1_events", gemm1_events),
                          ("gemm2_events", gemm2_events)):
            for i, ev in enumerate(evs or []):
                getattr(dbg, name)[i] = ev.cuda_event
    check(lib().moe_latent_forward(_p(x), _p(logits), T, top_k, _score(score), latent.ref(), routed.ref(),
                                   _p(norm_gamma), float(norm_eps), _p(out),
                                   ctypes.byref(dbg) if dbg is not None else None, _p(ws), _nbytes(ws),
                                   _stream(stream)))
    if debug is not None:
        return out, dbg.variant.decode()
    return out
