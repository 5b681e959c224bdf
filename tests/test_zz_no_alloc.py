"""moe_forward_noalloc on the GPU: the entry point whose workspace is the
library's per-device scratch array, against moe_forward with a caller
workspace on the same inputs -- two calls in a row, the second smaller, each
bit for bit (the same kernels run on the same data), and a call beyond the
scratch rejected with nothing written."""

import numpy as np
import pytest
import torch

import moe_synth
from gpu_helpers import DEV, bits, host, say, to_device

pytestmark = pytest.mark.gpu


def capture(T, E, k, H, shared):
    z = lambda shape, dt: torch.empty(shape, dtype=dt, device=DEV)  # noqa: E731
    return dict(topk_ids=z((T, k), torch.int32), topk_w=z((T, k), torch.float32),
                expert_counts=z((E,), torch.int32), expert_offsets=z((E + (2 if shared else 1),), torch.int32),
                pair_to_row=z((T, k), torch.int32), row_to_pair=z((T * k,), torch.int32),
                xq_rows=z((T * k, H), torch.uint8), xs_rows=z((T * k,), torch.float32))


def run_both(lib, inp):
    c = inp["cfg"]
    T, E, k, H = c["T"], c["E"], c["k"], c["H"]
    routed = lib.Weights(inp["routed"], c["fmt"])
    shared = lib.Weights(inp["shared"], "fp8") if inp["shared"] is not None else None
    d_ref, d_na = capture(T, E, k, H, shared is not None), capture(T, E, k, H, shared is not None)
    ref, v_ref = lib.moe_forward(inp["x"], inp["logits"], k, routed, shared, inp["gamma"], inp["eps"], debug=d_ref)
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    got, v_na = lib.moe_forward_noalloc(inp["x"], inp["logits"], k, routed, shared, inp["gamma"], inp["eps"],
                                        out=out, debug=d_na)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return ref, got, d_ref, d_na, v_ref, v_na, free0, free1


@pytest.mark.parametrize("T", [300, 37])
def test_noalloc_matches_forward(lib, T):
    """T = 300 then T = 37 (a smaller call reusing the scratch the first left
    behind): outputs and every captured intermediate equal moe_forward's."""
    inp = to_device(moe_synth.custom_inputs(T, 1024, 512, 8, 2, seed=T, shared=True))
    say("noalloc vs forward", T)
    ref, got, d_ref, d_na, v_ref, v_na, free0, free1 = run_both(lib, inp)
    say("  variants", v_ref, v_na, "device free bytes before/after", free0, free1)
    assert v_ref == v_na
    assert np.array_equal(bits(got), bits(ref))
    for key in d_ref:
        assert np.array_equal(host(d_na[key]), host(d_ref[key])), key
    if T == 37:
        # the scratch is already resolved: the call allocated nothing
        assert free1 == free0


def test_noalloc_rejects_beyond_scratch(lib):
    T, H, I = 2048, 8192, 2048
    inp = moe_synth.custom_inputs(T, H, I, 8, 2, seed=4, shared=True, device=DEV)
    routed, shared = lib.Weights(inp["routed"], "fp8"), lib.Weights(inp["shared"], "fp8")
    need = lib.forward_workspace_size(T, 2, routed, True)
    assert need > lib._lib.MOE_NOALLOC_SCRATCH_BYTES
    out = torch.full((T, H), 7.0, dtype=torch.bfloat16, device=DEV)
    say("noalloc beyond scratch", T, H, I, need)
    with pytest.raises(lib.MoeError) as err:
        lib.moe_forward_noalloc(inp["x"], inp["logits"], 2, routed, shared, out=out)
    assert err.value.status == lib._lib.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all()
