"""Seeded synthetic inputs for the routed MoE layer.

This module only draws inputs.  It holds none of the layer's arithmetic: the
router, the activation quantisation, the permutation, the FFN and the combine
live in the GPU library and, independently, in the CPU oracle.  Both receive
the same tensors from here.

Workloads (shapes from the pages' per-device shares, see the design notes):

=====  ======  =====  =====  ====  ===  ======  ================================
name   T       H      I      E     k    format  extras
=====  ======  =====  =====  ====  ===  ======  ================================
tiny   64      256    128    8     2    fp8     --
prefill 2048   8192   2048   8     2    fp8     shared expert 8192->2048->8192
decode 64      8192   2048   8     2    fp8     --
latent 512     3584   3072   896   16   mxfp4   RMSNorm (gamma = 1, eps = 1e-6)
skewed 16384   8192   2048   256   8    fp8     Zipf-biased logits, hottest ~5x
=====  ======  =====  =====  ====  ===  ======  ================================

``latent_block_inputs`` draws the whole LatentMoE block (hidden 7168, the
``latent`` core over 3584, MXFP4 down/up projections, bf16 shared experts
7168 -> 6144 -> 7168) with the same recipe (projection weights quantised per
32-element block to MXFP4, shared weights rounded to bf16).

Recipe: activations ~ N(0,1) rounded to bf16; router logits ~ N(0,1) in fp32
(plus, for ``skewed``, a per-expert bias -alpha*1.1*ln(rank) over a seeded
rank permutation, alpha bisected so the hottest expert gets 4.9-5.1x the mean
row count); weights ~ 0.02*N(0,1) in fp32, quantised per output row to fp8
e4m3 with scale amax/448 (torch's float8_e4m3fn cast), per 128 x 128 tile to
fp8 with one fp32 scale amax/448 per tile ("fp8_block"), or per 32-element
block to MXFP4 (e2m1 codes, e8m0 scale 2^(floor(log2 amax) - 2)).

Every tensor comes from its own torch.Generator seeded by
(2026, workload, tensor, expert), so any expert can be regenerated alone.
torch's CPU and GPU generators differ; a run draws on one device and hands
host copies of the same tensors to the oracle.
"""

import torch

CONFIGS = {
    "tiny":    dict(cfg=1, T=64,    H=256,  I=128,  E=8,   k=2,  fmt="fp8",   shared=False, norm=False, skew=False),
    "prefill": dict(cfg=2, T=2048,  H=8192, I=2048, E=8,   k=2,  fmt="fp8",   shared=True,  norm=False, skew=False),
    "decode":  dict(cfg=3, T=64,    H=8192, I=2048, E=8,   k=2,  fmt="fp8",   shared=False, norm=False, skew=False),
    "latent":  dict(cfg=4, T=512,   H=3584, I=3072, E=896, k=16, fmt="mxfp4", shared=False, norm=True,  skew=False),
    "skewed":  dict(cfg=5, T=16384, H=8192, I=2048, E=256, k=8,  fmt="fp8",   shared=False, norm=False, skew=True),
    # the prefill and decode shares with per-block fp8 routed weights
    "prefill_block": dict(cfg=7, T=2048, H=8192, I=2048, E=8, k=2, fmt="fp8_block", shared=True, norm=False,
                          skew=False),
    "decode_block":  dict(cfg=8, T=64,   H=8192, I=2048, E=8, k=2, fmt="fp8_block", shared=False, norm=False,
                          skew=False),
}

T_LOGITS, T_X, T_W1, T_W3, T_W2, T_SW1, T_SW3, T_SW2, T_RANK, T_DOWN, T_UP = range(11)
NORM_EPS = 1e-6
WEIGHT_STD = 0.02


def seed_of(cfg, tensor, expert=0, base=2026):
    return ((base * 100 + cfg) * 100 + tensor) * 100000 + expert


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, device, seed, std=1.0):
    t = torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    return t * std if std != 1.0 else t


# ----------------------------------------------------------------------------
# weight quantisers (input preparation only)
# ----------------------------------------------------------------------------


def fp8_rows(w):
    """float32 [N][K] -> (e4m3 codes uint8 [N][K], per-row scale float32 [N])."""
    amax = w.abs().amax(dim=1)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (w / s[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.contiguous(), s.contiguous()


def fp8_blocks(w, block=128):
    """float32 [N][K] -> (e4m3 codes uint8 [N][K], one scale float32 per
    block x block tile [N/block][K/block], amax/448 of the tile)."""
    N, K = w.shape
    t = w.reshape(N // block, block, K // block, block)
    amax = t.abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (t / s[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(N, K).contiguous(), s.contiguous()


_E2M1_MIDS_DOWN = (0.25, 1.25, 2.5, 5.0)   # a tie here goes to the lower (even) code
_E2M1_MIDS_UP = (0.75, 1.75, 3.5)          # a tie here goes to the upper (even) code


def _mxfp4_codes(w, group=32):
    """float32 [..., K] -> (e2m1 codes int32 [..., K], e8m0 biased exponents
    int32 [..., K/group]): scale 2^(floor(log2 amax) - 2) per block, codes by
    round to nearest, ties to even."""
    wb = w.reshape(*w.shape[:-1], w.shape[-1] // group, group)
    amax = wb.abs().amax(dim=-1)
    e = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2
    e = torch.where(amax > 0, e, torch.full_like(e, -127.0)).clamp(-127, 127)
    v = wb / torch.pow(2.0, e)[..., None]
    mag = v.abs().clamp(max=6.0)
    code = torch.zeros(mag.shape, dtype=torch.int32, device=w.device)
    for m in _E2M1_MIDS_DOWN:
        code += (mag > m).int()
    for m in _E2M1_MIDS_UP:
        code += (mag >= m).int()
    code = code | (((v < 0) & (code > 0)).int() << 3)
    return code.reshape(w.shape), (e + 127).int()


def _words(vals, bits):
    """int32 [..., n] of `bits`-bit fields (n * bits a multiple of 32) ->
    int32 words [..., n * bits / 32], field i of a word at bit i * bits, so
    that the words viewed as bytes list the fields in order (little endian)."""
    per = 32 // bits
    v = vals.reshape(*vals.shape[:-1], -1, per).long()
    w = (v << (torch.arange(per, device=vals.device, dtype=torch.int64) * bits)).sum(dim=-1)
    return torch.where(w >= 2 ** 31, w - 2 ** 32, w).int()


def _mxfp4_words(w, group=32):
    """float32 [..., K], K % 128 == 0 -> (codes as int32 words [..., K/8],
    e8m0 scales as int32 words [..., K/128]); viewed as bytes they are the
    packed codes [..., K/2] (element 2i in the low nibble of byte i) and the
    scales [..., K/32].  Built from whole 32-bit words: no byte-wise device
    kernels (a byte-wise conversion or copy per tensor, for every expert,
    was most of the generator's launches)."""
    code, e = _mxfp4_codes(w, group)
    return _words(code, 4), _words(e, 8)


def _mxfp4_rows_bytes(w, group=32):
    """The same encoding built byte by byte (any K % group == 0)."""
    N, K = w.shape
    code, e = _mxfp4_codes(w, group)
    code = code.to(torch.uint8)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    return packed, e.to(torch.uint8).contiguous()


def mxfp4_rows(w, group=32):
    """float32 [N][K] -> (packed uint8 [N][K/2], e8m0 uint8 [N][K/group])."""
    if w.shape[1] % 128 == 0 and group == 32:
        cw, sw = _mxfp4_words(w, group)
        return cw.view(torch.uint8), sw.view(torch.uint8)
    return _mxfp4_rows_bytes(w, group)


# experts quantised together by expert_weights (MXFP4): bounds the float32
# temporaries to a few GB at the LatentMoE shape
_MX_CHUNK = 16


def _mxfp4_experts(cfg, device, tid, n_experts, shape):
    """MXFP4 weights of n_experts experts of `shape` [N][K] (K % 128 == 0):
    each expert drawn from its own generator, quantised a chunk of experts at
    a time, stacked as int32 words and viewed as bytes at the end."""
    N, K = shape
    codes = torch.empty((n_experts, N, K // 8), dtype=torch.int32, device=device)
    scales = torch.empty((n_experts, N, K // 128), dtype=torch.int32, device=device)
    buf = torch.empty((min(_MX_CHUNK, max(n_experts, 1)), N, K), dtype=torch.float32, device=device)
    for e0 in range(0, n_experts, _MX_CHUNK):
        c = min(_MX_CHUNK, n_experts - e0)
        for i in range(c):
            torch.randn(shape, generator=_gen(device, seed_of(cfg, tid, e0 + i)), device=device, out=buf[i])
        w = buf[:c] * WEIGHT_STD
        codes[e0:e0 + c], scales[e0:e0 + c] = _mxfp4_words(w)
    return codes.view(torch.uint8), scales.view(torch.uint8)


def expert_weights(cfg, device, fmt, n_experts, hidden, inter, tensors=(T_W1, T_W3, T_W2)):
    """Stacked weights {w1,w3,w2,s1,s3,s2} of n_experts experts on ``device``."""
    out = {}
    shapes = {tensors[0]: (inter, hidden), tensors[1]: (inter, hidden), tensors[2]: (hidden, inter)}
    for name, tid in zip(("1", "3", "2"), tensors):
        if fmt == "mxfp4" and shapes[tid][1] % 128 == 0:
            out["w" + name], out["s" + name] = _mxfp4_experts(cfg, device, tid, n_experts, shapes[tid])
            continue
        codes, scales = [], []
        for e in range(n_experts):
            w = randn(shapes[tid], device, seed_of(cfg, tid, e), WEIGHT_STD)
            q, s = fp8_rows(w) if fmt == "fp8" else fp8_blocks(w) if fmt == "fp8_block" else mxfp4_rows(w)
            codes.append(q)
            scales.append(s)
        out["w" + name] = torch.stack(codes).contiguous()
        out["s" + name] = torch.stack(scales).contiguous()
    return out


# ----------------------------------------------------------------------------
# activations and logits
# ----------------------------------------------------------------------------


def _hottest_over_mean(logits, k):
    ids = torch.topk(logits, k, dim=1).indices.reshape(-1)
    counts = torch.bincount(ids, minlength=logits.shape[1]).double()
    return (counts.max() / counts.mean()).item()


def skew_bias(cfg, T, E, k, base_logits, device, target=5.0):
    """Per-expert bias -alpha*1.1*ln(rank) with alpha bisected to the target skew."""
    perm = torch.randperm(E, generator=_gen("cpu", seed_of(cfg, T_RANK)))
    rank = torch.empty(E, dtype=torch.float64)
    rank[perm] = torch.arange(1, E + 1, dtype=torch.float64)
    shape = (-1.1 * torch.log(rank)).to(torch.float32).to(device)
    lo, hi = 0.0, 2.0
    alpha = 1.0
    for _ in range(40):
        alpha = 0.5 * (lo + hi)
        r = _hottest_over_mean(base_logits + alpha * shape[None, :], k)
        if abs(r - target) <= 0.1:
            break
        if r < target:
            lo = alpha
        else:
            hi = alpha
    return alpha * shape, alpha


def make_inputs(name, device="cpu", weights=True):
    """All inputs of one workload as torch tensors on ``device``.

    Returns a dict: cfg (the CONFIGS entry plus alpha), x (bfloat16 [T][H]),
    logits (float32 [T][E]), routed (dict w1,w3,w2,s1,s3,s2), shared (dict or
    None), gamma (float32 [H] or None), eps.
    """
    c = dict(CONFIGS[name])
    T, H, I, E, k = c["T"], c["H"], c["I"], c["E"], c["k"]
    x = randn((T, H), device, seed_of(c["cfg"], T_X)).to(torch.bfloat16)
    logits = randn((T, E), device, seed_of(c["cfg"], T_LOGITS))
    c["alpha"] = None
    if c["skew"]:
        bias, alpha = skew_bias(c["cfg"], T, E, k, logits, device)
        logits = (logits + bias[None, :]).contiguous()
        c["alpha"] = alpha
    routed = expert_weights(c["cfg"], device, c["fmt"], E, H, I) if weights else None
    shared = None
    if c["shared"] and weights:
        shared = expert_weights(c["cfg"], device, "fp8", 1, H, I, (T_SW1, T_SW3, T_SW2))
    gamma = torch.ones(H, dtype=torch.float32, device=device) if c["norm"] else None
    return dict(cfg=c, x=x, logits=logits, routed=routed, shared=shared, gamma=gamma, eps=NORM_EPS)


def custom_inputs(T, H, I, E, k, fmt="fp8", seed=7, device="cpu", shared=False, norm=False,
                  logits=None):
    """Inputs of an arbitrary shape with the same recipe (for edge-case tests)."""
    cfg = 90 + (seed % 10)
    x = randn((T, H), device, seed_of(cfg, T_X, seed)).to(torch.bfloat16)
    if logits is None:
        logits = randn((T, E), device, seed_of(cfg, T_LOGITS, seed))
    routed = expert_weights(cfg * 1000 + seed, device, fmt, E, H, I)
    sh = expert_weights(cfg * 1000 + seed, device, "fp8", 1, H, I, (T_SW1, T_SW3, T_SW2)) if shared else None
    gamma = torch.ones(H, dtype=torch.float32, device=device) if norm else None
    c = dict(cfg=cfg, T=T, H=H, I=I, E=E, k=k, fmt=fmt, shared=shared, norm=norm, skew=False, alpha=None)
    return dict(cfg=c, x=x, logits=logits, routed=routed, shared=sh, gamma=gamma, eps=NORM_EPS)


# The LatentMoE block (the routed core of ``latent`` plus its projections and
# shared experts): hidden 7168 -> latent 3584 -> 896 experts top-16 -> RMSNorm
# -> 7168, shared experts 7168 -> 6144 -> 7168 on the hidden stream.
LATENT_BLOCK = dict(cfg=6, T=512, Hm=7168, L=3584, I=3072, E=896, k=16, Is=6144)


def latent_block_inputs(T, Hm, L, I, E, k, Is, cfg=6, device="cpu", weights=True):
    """Inputs of the LatentMoE block, same recipe: x bf16 [T][Hm], logits
    float32 [T][E]; down {w, s} MXFP4 [L][Hm/2] + [L][Hm/32]; up {w, s} MXFP4
    [Hm][L/2] + [Hm][L/32]; routed MXFP4 experts over L; shared bf16
    {w1, w3} [Is][Hm], {w2} [Hm][Is] (Is = 0: none); gamma ones [L]."""
    x = randn((T, Hm), device, seed_of(cfg, T_X)).to(torch.bfloat16)
    logits = randn((T, E), device, seed_of(cfg, T_LOGITS))
    c = dict(cfg=cfg, T=T, Hm=Hm, L=L, I=I, E=E, k=k, Is=Is, fmt="mxfp4")
    out = dict(cfg=c, x=x, logits=logits, down=None, up=None, routed=None, shared=None,
               gamma=torch.ones(L, dtype=torch.float32, device=device), eps=NORM_EPS)
    if not weights:
        return out
    for name, tid, shape in (("down", T_DOWN, (L, Hm)), ("up", T_UP, (Hm, L))):
        w, sc = mxfp4_rows(randn(shape, device, seed_of(cfg, tid), WEIGHT_STD))
        out[name] = dict(w=w, s=sc)
    out["routed"] = expert_weights(cfg, device, "mxfp4", E, L, I)
    if Is > 0:
        out["shared"] = {n: randn(shape, device, seed_of(cfg, tid), WEIGHT_STD).to(torch.bfloat16).contiguous()
                         for n, tid, shape in (("w1", T_SW1, (Is, Hm)), ("w3", T_SW3, (Is, Hm)),
                                               ("w2", T_SW2, (Hm, Is)))}
    return out


def random_topk_ids(T, E, k, seed, device="cpu", hot=None):
    """Seeded routing choices: k distinct experts per token, in a random slot
    order; with ``hot`` = e, every token's first slot is expert e (so other
    experts may get no rows)."""
    g = _gen("cpu", seed_of(95, T_RANK, seed))
    ids = torch.argsort(torch.rand((T, E), generator=g), dim=1)[:, :k].to(torch.int32)
    if hot is not None and T > 0:
        # swap `hot` into slot 0; the k experts stay distinct
        first = ids[:, 0].clone()
        ids[:, 0] = hot
        pos = ids[:, 1:] == hot
        ids[:, 1:] = torch.where(pos, first[:, None].expand_as(ids[:, 1:]), ids[:, 1:])
    return ids.contiguous().to(device)


def to_numpy(inputs):
    """Host NumPy copies for the oracle: x as uint16 bf16 bits, the rest as is."""
    import numpy as np

    def cpu(t):
        return None if t is None else t.detach().cpu()

    out = dict(cfg=inputs["cfg"], eps=inputs["eps"])
    out["x"] = cpu(inputs["x"]).view(torch.int16).numpy().view(np.uint16)
    out["logits"] = cpu(inputs["logits"]).numpy()
    for key in ("routed", "shared"):
        d = inputs[key]
        out[key] = None if d is None else {n: cpu(t).numpy() for n, t in d.items()}
    out["gamma"] = None if inputs["gamma"] is None else cpu(inputs["gamma"]).numpy()
    return out


def weight_bytes_per_expert(H, I, fmt):
    """Code bytes (and MXFP4's block scales) of one expert's W1, W3, W2."""
    return 3 * H * I if fmt in ("fp8", "fp8_block") else 3 * H * I // 2 + 3 * H * I // 32


def ceil_div(a, b):
    return -(-a // b)


