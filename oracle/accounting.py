"""Algorithmic work of the layer: FLOPs and bytes, as the cost model counts them.

TEST INFRASTRUCTURE ONLY (see the package docstring).

*Ling-2.6-1T on TPU*, §1 "MoE kernel cost model" counts the FFN work as two
gate/up matrices of 2*M*H*I flops each (FFN1) plus one down matrix of
2*M*I*H (FFN2), i.e. 6*M*H*I per routed row, with the shared expert adding
the same per token it runs on; and the expert-weight HBM read as
3*H*I bytes per fp8 expert.  *Kimi K3 on TPU*, §2.4 counts a LatentMoE expert
as 3*3584*3072 parameters and §2.5 gives MXFP4 as 4.25 bits per element
(4-bit codes plus one 8-bit scale per 32 elements).

Bytes here are the method's own traffic: the weights and scales of experts
that receive at least one row, plus the layer's inputs and output.
Intermediates are implementation traffic and are not counted.
"""

import numpy as np


def ffn_flops(rows, hidden, inter):
    """FFN1 + FFN2 flops for ``rows`` rows through one expert shape."""
    ffn1 = 2 * (2 * rows * hidden * inter)
    ffn2 = 2 * rows * inter * hidden
    return ffn1 + ffn2


def layer_flops(T, top_k, hidden, inter, shared_tokens=0, shared_inter=None):
    """Routed rows T*k through the routed FFN plus the shared expert's tokens."""
    shared_inter = inter if shared_inter is None else shared_inter
    return ffn_flops(T * top_k, hidden, inter) + ffn_flops(shared_tokens, hidden, shared_inter)


def expert_weight_bytes(hidden, inter, fmt):
    """(code bytes, scale bytes) of one expert's W1, W3, W2."""
    elems = 3 * hidden * inter
    if fmt == "fp8":
        return elems, 4 * (2 * inter + hidden)      # fp32 scale per output channel
    if fmt == "mxfp4":
        return elems // 2, elems // 32               # 4-bit codes, one byte per 32
    raise ValueError(fmt)


def mx_bits_per_element(elem_bits=4, scale_bits=8, group=32):
    return elem_bits + scale_bits / group


def layer_bytes(T, n_experts_touched, hidden, inter, fmt, n_experts_total,
                shared=False, shared_inter=None, top_k=1):
    """Algorithmic bytes: touched experts' weights and scales, x (bf16),
    router logits (fp32) and out (bf16); the shared expert's weights if used."""
    code, scale = expert_weight_bytes(hidden, inter, fmt)
    total = n_experts_touched * (code + scale)
    if shared:
        c2, s2 = expert_weight_bytes(hidden, inter if shared_inter is None else shared_inter, "fp8")
        total += c2 + s2
    total += T * hidden * 2 + T * n_experts_total * 4 + T * hidden * 2
    return total


def touched_experts(topk_ids, n_experts):
    """Number of experts that receive at least one routed row."""
    return int(np.unique(np.asarray(topk_ids).ravel()).size)
