"""The oracle's FLOP / byte accounting against the figures the pages print."""

import math
import os

import pytest

from oracle import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cost_model.txt")


def load_golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            key, value, unit = line.split()[:3]
            vals[key] = (float(value), float(unit))
    return vals


def recomputed():
    """Each printed figure, recomputed from the shapes the pages state."""
    H, I = 8192, 2048
    rows = 16384 * 8 // 32
    per_expert = rows // 8
    ffn1 = 8 * 2 * (2 * per_expert * H * I)
    routed = 8 * acc.ffn_flops(per_expert, H, I)
    shared = acc.ffn_flops(rows, H, I)
    expert_mb = acc.expert_weight_bytes(H, I, "fp8")[0] / 1e6
    local_mb = 8 * expert_mb
    lat = acc.expert_weight_bytes(3584, 3072, "fp8")[0]      # one byte per element = parameter count
    return dict(
        rows_per_device=rows,
        ffn1_gflop=ffn1 / 1e9,
        ffn2_gflop=(routed - ffn1) / 1e9,
        routed_gflop=routed / 1e9,
        shared_gflop=shared / 1e9,
        total_gflop=(routed + shared) / 1e9,
        compute_bound_ms=(routed + shared) / 1e9 / 2307.0,
        scatter_elems=rows * H,
        scatter_bf16_mb=rows * H * 2 / 1e6,
        scatter_fp8_mb=rows * H / 1e6,
        expert_fp8_mb=expert_mb,
        local_experts_mb=local_mb,
        hbm_once_ms=local_mb / 3.69e6 * 1e3,
        hbm_bts160_ms=math.ceil(per_expert / 160) * local_mb / 3.69e6 * 1e3,
        latent_expert_mparams=lat / 1e6,
        latent_layer_bparams=896 * lat / 1e9,
        mxfp4_bits=acc.mx_bits_per_element(),
    )


def test_cost_model_matches_pages():
    gold = load_golden()
    mine = recomputed()
    assert set(gold) == set(mine)
    # The pages print rounded (sometimes truncated) figures: agree to within
    # one unit of the last printed digit.
    for key, (value, unit) in gold.items():
        assert abs(mine[key] - value) <= unit, (key, mine[key], value)


def test_layer_flops_consistent():
    # Routed rows T*k plus shared tokens, 6*H*I each.
    assert acc.layer_flops(2048, 2, 8192, 2048, shared_tokens=2048) == 6 * 8192 * 2048 * (4096 + 2048)
    assert acc.layer_flops(64, 2, 256, 128) == 6 * 256 * 128 * 128


def test_mxfp4_bytes():
    code, scale = acc.expert_weight_bytes(3584, 3072, "mxfp4")
    # 4.25 bits per element
    assert (code + scale) * 8 == pytest.approx(3 * 3584 * 3072 * 4.25)
