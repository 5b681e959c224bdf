"""The seeded input generators (host logic, no GPU): the MXFP4 weight encoder
built from whole 32-bit words gives the same bytes as the same encoding built
byte by byte, and the chunked per-expert generation gives every expert the
weights its own generator draws alone.

These are input-preparation checks only; the encoding the layer uses is
pinned in the oracle's codec tests.
"""

import torch

import moe_synth as ms


def test_mxfp4_words_equal_bytes():
    g = torch.Generator().manual_seed(1)
    for K in (128, 256, 384, 1024):
        w = torch.randn((37, K), generator=g) * 0.02
        w[3] = 0.0                                    # all-zero blocks: scale code 0
        w[5, :32] = -0.0
        # every e2m1 rounding midpoint, both signs, and the saturation at 6
        mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
        w[7, :64] = torch.cat([mids, -mids] * 4) * 2.0 ** -3
        w[8, :8] = torch.tensor([6.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0])
        w[9, :32] = 1e30                              # large blocks: exponent clamped at 127
        a = ms.mxfp4_rows(w)
        b = ms._mxfp4_rows_bytes(w)
        assert a[0].dtype == torch.uint8 and a[1].dtype == torch.uint8
        assert a[0].shape == (37, K // 2) and a[1].shape == (37, K // 32)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), K


def test_mxfp4_experts_match_single_expert_draws():
    E, H, I = 20, 256, 384                            # more experts than one quantisation chunk
    W = ms.expert_weights(4, "cpu", "mxfp4", E, H, I)
    for n, tid, shape in (("1", ms.T_W1, (I, H)), ("3", ms.T_W3, (I, H)), ("2", ms.T_W2, (H, I))):
        assert W["w" + n].shape == (E, shape[0], shape[1] // 2)
        assert W["s" + n].shape == (E, shape[0], shape[1] // 32)
        for e in (0, 7, 15, 16, 19):
            q, s = ms._mxfp4_rows_bytes(ms.randn(shape, "cpu", ms.seed_of(4, tid, e), ms.WEIGHT_STD))
            assert torch.equal(W["w" + n][e], q) and torch.equal(W["s" + n][e], s), (n, e)
