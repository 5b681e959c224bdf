"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before anything is enqueued
(no GPU is touched: every call here fails validation).
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

from mixture_experts_ffn_softmax_amd import _lib
from mixture_experts_ffn_softmax_amd._lib import (MOE_ERR_ALIGN, MOE_ERR_NULL, MOE_ERR_SHAPE,
                                                  MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_OK,
                                                  MoeDebug, MoeLatent, MoeLinear, MoeWeights)

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")

A = 0x10000          # fake, 16-byte aligned "device" addresses: never dereferenced here
MIS = 0x10008        # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libmoe.so not built (run __graft_entry__.build())")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.moe_version()
    for s in range(7):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(99) == b"unknown status"


def test_struct_layouts(tmp_path):
    """The ctypes mirrors match the C header: sizes and field offsets as a C
    compiler lays the structs out (gcc on the header itself)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "moe.h"\n'
        'int main(void) { printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(moe_weights_t),'
        ' offsetof(moe_weights_t, w1), offsetof(moe_weights_t, s2), sizeof(moe_debug_t),'
        ' offsetof(moe_debug_t, events), offsetof(moe_debug_t, variant),'
        ' offsetof(moe_debug_t, gemm1_events), offsetof(moe_debug_t, gemm2_events),'
        ' offsetof(moe_weights_t, act_beta), offsetof(moe_debug_t, layer_events),'
        ' offsetof(moe_debug_t, core_out), sizeof(moe_linear_t), offsetof(moe_linear_t, s),'
        ' sizeof(moe_latent_t), offsetof(moe_latent_t, sw2)); return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got == [ctypes.sizeof(MoeWeights), MoeWeights.w1.offset, MoeWeights.s2.offset,
                   ctypes.sizeof(MoeDebug), MoeDebug.events.offset, MoeDebug.variant.offset,
                   MoeDebug.gemm1_events.offset, MoeDebug.gemm2_events.offset, MoeWeights.act_beta.offset,
                   MoeDebug.layer_events.offset, MoeDebug.core_out.offset, ctypes.sizeof(MoeLinear),
                   MoeLinear.s.offset, ctypes.sizeof(MoeLatent), MoeLatent.sw2.offset]


def fp8_weights(E=8, H=256, I=128, fmt=0, layout=0, **over):
    w = MoeWeights(fmt, E, H, I, layout, 0, 4.0, 0, A, A, A, A, A, A)
    for k, v in over.items():
        setattr(w, k, v)
    return w


def test_route_validation(lib):
    r = lib.moe_route
    assert r(A, -1, 8, 2, 0, A, A, None) == MOE_ERR_SHAPE
    assert r(A, 4, 0, 1, 0, A, A, None) == MOE_ERR_SHAPE
    assert r(A, 4, 1025, 1, 0, A, A, None) == MOE_ERR_SHAPE
    assert r(A, 4, 8, 9, 0, A, A, None) == MOE_ERR_SHAPE          # k > E
    assert r(A, 4, 64, 33, 0, A, A, None) == MOE_ERR_SHAPE         # k > 32
    assert r(A, 1 << 30, 8, 2, 0, A, A, None) == MOE_ERR_SHAPE     # T*k overflows
    assert r(None, 4, 8, 2, 0, A, A, None) == MOE_ERR_NULL
    assert b"logits" in lib.moe_last_error()
    assert r(A, 4, 8, 2, 0, MIS, A, None) == MOE_ERR_ALIGN
    assert r(A, 4, 8, 2, 2, A, A, None) == MOE_ERR_UNSUPPORTED  # unknown score function
    assert r(A, 0, 8, 2, 0, None, None, None) == MOE_OK            # T = 0: nothing to do
    assert lib.moe_last_error() == b""


def test_permute_validation(lib):
    p = lib.moe_permute
    ws = lib.moe_permute_workspace_size(16, 2, 8)
    assert ws > 0
    args = [A, 16, 256, A, 2, 8, A, A, A, A, A, A, None, None, A, ws, None]

    def call(**kw):
        a = list(args)
        names = ["x", "T", "H", "ids", "k", "E", "counts", "offsets", "p2r", "r2p", "xq", "xs",
                 "xq_tok", "xs_tok", "ws", "ws_bytes", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return p(*a)

    assert call(H=200) == MOE_ERR_SHAPE
    assert call(H=0) == MOE_ERR_SHAPE
    assert call(x=None) == MOE_ERR_NULL
    assert call(xq=MIS) == MOE_ERR_ALIGN
    assert call(xq_tok=A) == MOE_ERR_NULL                       # xq_tok without xs_tok
    assert call(ws_bytes=ws - 1) == MOE_ERR_WORKSPACE
    assert call(ws=None) == MOE_ERR_WORKSPACE


def test_expert_ffn_validation(lib):
    f = lib.moe_expert_ffn
    w = fp8_weights()
    ws = lib.moe_expert_ffn_workspace_size(64, ctypes.byref(w))
    assert ws >= 64 * 128 * 2          # bf16 h
    assert f(A, A, 64, A, None, A, A, ws, None) == MOE_ERR_NULL
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(fmt=7)), A, A, ws, None) == MOE_ERR_UNSUPPORTED
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(H=100)), A, A, ws, None) == MOE_ERR_SHAPE
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(I=0)), A, A, ws, None) == MOE_ERR_SHAPE
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(E=0)), A, A, ws, None) == MOE_ERR_SHAPE
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(w2=None)), A, A, ws, None) == MOE_ERR_NULL
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(s3=MIS)), A, A, ws, None) == MOE_ERR_ALIGN
    assert f(A, A, -1, A, ctypes.byref(w), A, A, ws, None) == MOE_ERR_SHAPE
    assert f(A, A, 64, A, ctypes.byref(w), A, A, ws - 1, None) == MOE_ERR_WORKSPACE
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(layout=2)), A, A, ws, None) == MOE_ERR_UNSUPPORTED
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(reserved=1)), A, A, ws, None) == MOE_ERR_SHAPE
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(activation=2)), A, A, ws, None) == MOE_ERR_UNSUPPORTED
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(activation=1, act_beta=0.0)), A, A, ws, None) == MOE_ERR_SHAPE
    assert f(A, A, 64, A, ctypes.byref(fp8_weights(activation=1, act_beta=float("inf"))), A, A, ws, None) == MOE_ERR_SHAPE
    assert f(None, None, 0, None, ctypes.byref(w), None, None, 0, None) == MOE_OK


def test_combine_validation(lib):
    c = lib.moe_combine
    assert c(A, A, A, 4, 256, 0, None, None, 1e-6, A, None) == MOE_ERR_SHAPE
    assert c(A, A, A, 4, 255, 2, None, None, 1e-6, A, None) == MOE_ERR_SHAPE
    assert c(A, A, A, 4, 256, 2, None, A, -1.0, A, None) == MOE_ERR_SHAPE
    assert c(A, A, A, 4, 256, 2, MIS, None, 1e-6, A, None) == MOE_ERR_ALIGN
    assert c(A, None, A, 4, 256, 2, None, None, 1e-6, A, None) == MOE_ERR_NULL
    assert c(None, None, None, 0, 256, 2, None, None, 1e-6, None, None) == MOE_OK


def test_forward_validation(lib):
    fw = lib.moe_forward
    w = fp8_weights()
    ws = lib.moe_forward_workspace_size(16, 2, ctypes.byref(w), 0)
    sh = fp8_weights(E=1)
    ws_sh = lib.moe_forward_workspace_size(16, 2, ctypes.byref(w), 1)
    assert ws_sh > ws

    def call(T=16, k=2, routed=w, use_shared=0, shared=None, out=A, dbg=None, wsb=ws, x=A, score=0):
        return fw(x, A, T, k, score, ctypes.byref(routed), use_shared,
                  ctypes.byref(shared) if shared is not None else None, None, 1e-6, out,
                  ctypes.byref(dbg) if dbg is not None else None, A, wsb, None)

    assert call(k=9) == MOE_ERR_SHAPE
    assert call(use_shared=1) == MOE_ERR_NULL
    assert call(use_shared=1, shared=fp8_weights(E=2)) == MOE_ERR_SHAPE
    assert call(use_shared=1, shared=fp8_weights(E=1, I=256)) == MOE_ERR_UNSUPPORTED
    assert call(use_shared=1, shared=fp8_weights(E=1, fmt=1)) == MOE_ERR_UNSUPPORTED
    assert call(use_shared=1, shared=sh, wsb=ws) == MOE_ERR_WORKSPACE
    assert call(out=None) == MOE_ERR_NULL
    assert call(x=MIS) == MOE_ERR_ALIGN
    d = MoeDebug()
    d.xq_rows = MIS
    assert call(dbg=d) == MOE_ERR_ALIGN
    assert call(routed=fp8_weights(E=1024), use_shared=1, shared=sh, wsb=1 << 40) == MOE_ERR_UNSUPPORTED
    assert call(score=5) == MOE_ERR_UNSUPPORTED
    assert call(T=0) == MOE_OK


def test_workspace_sizes_grow(lib):
    w = fp8_weights(E=8, H=8192, I=2048)
    a = lib.moe_forward_workspace_size(64, 2, ctypes.byref(w), 0)
    b = lib.moe_forward_workspace_size(2048, 2, ctypes.byref(w), 0)
    # h (bf16) and y (fp32) per row, plus the quantised tokens kept in token
    # order (up to 32 experts and 4096 tokens, routed in the quantising launch)
    assert b > a and b >= 4096 * (2 * 2048 + 4 * 8192) + 2048 * 8192
    # beyond 32 experts the quantised rows are scattered to expert order
    w64 = fp8_weights(E=64, H=8192, I=2048)
    assert lib.moe_forward_workspace_size(2048, 2, ctypes.byref(w64), 0) >= 4096 * (2 * 2048 + 5 * 8192)
    assert lib.moe_forward_workspace_size(-1, 2, ctypes.byref(w), 0) == 0


def test_pack_weights_validation(lib):
    pk = lib.moe_pack_weights
    E, H, I = 4, 256, 128
    n = E * H * I
    src = fp8_weights(E, H, I, w1=0x100000, w3=0x100000 + n, w2=0x100000 + 2 * n)
    base = 0x4000000
    dst = fp8_weights(E, H, I, layout=1, w1=base, w3=base + n, w2=base + 2 * n)
    call = lambda a, b: pk(ctypes.byref(a), ctypes.byref(b), None)
    assert pk(None, ctypes.byref(dst), None) == MOE_ERR_NULL
    assert call(fp8_weights(E, H, I, fmt=1), dst) == MOE_ERR_SHAPE          # formats differ
    # MXFP4: the scales are written too, so they must not overlap src's
    n4, s4 = n // 2, n // 32
    msrc = fp8_weights(E, H, I, fmt=1, w1=0x100000, w3=0x100000 + n4, w2=0x100000 + 2 * n4,
                       s1=0x200000, s3=0x200000 + s4, s2=0x200000 + 2 * s4)
    mdst = dict(fmt=1, layout=1, w1=base, w3=base + n4, w2=base + 2 * n4)
    assert call(msrc, fp8_weights(E, H, I, s1=0x200000 + s4 // 2, s3=base + 3 * n4, s2=base + 4 * n4,
                                  **mdst)) == MOE_ERR_SHAPE
    assert call(msrc, fp8_weights(E, H, I, s1=base + 3 * n4, s3=base + 3 * n4 + s4 // 2, s2=base + 4 * n4,
                                  **mdst)) == MOE_ERR_SHAPE
    assert call(dst, dst) == MOE_ERR_SHAPE                      # src not row-major
    assert call(src, src) == MOE_ERR_SHAPE                      # dst not K-blocked
    assert call(src, fp8_weights(E, H, 256, layout=1, w1=base, w3=base + 2 * n, w2=base + 4 * n)) == MOE_ERR_SHAPE
    assert call(src, fp8_weights(E, H, I, layout=1, w1=0x100000 + n // 2, w3=base, w2=base + n)) == MOE_ERR_SHAPE
    assert call(src, fp8_weights(E, H, I, layout=1, w1=base, w3=base + n // 2, w2=base + 2 * n)) == MOE_ERR_SHAPE
    assert call(src, fp8_weights(E, H, I, layout=1, w1=base + 8)) == MOE_ERR_ALIGN


def linear_w(fmt=0, n_out=256, n_in=128, w=A, s=A, reserved=0):
    return MoeLinear(fmt, n_out, n_in, reserved, w, s if fmt == 0 else None)


def test_linear_validation(lib):
    f = lib.moe_linear
    w = linear_w()
    assert f(A, 8, None, None, A, None, None) == MOE_ERR_NULL
    assert f(A, 8, ctypes.byref(linear_w(fmt=2)), None, A, None, None) == MOE_ERR_UNSUPPORTED
    assert f(A, 8, ctypes.byref(linear_w(n_out=200)), None, A, None, None) == MOE_ERR_SHAPE
    assert f(A, 8, ctypes.byref(linear_w(n_in=96)), None, A, None, None) == MOE_ERR_SHAPE
    assert f(A, 8, ctypes.byref(linear_w(s=None)), None, A, None, None) == MOE_ERR_NULL      # MXFP4 scales
    bf = MoeLinear(1, 256, 128, 0, A, A)
    assert f(A, 8, ctypes.byref(bf), None, A, None, None) == MOE_ERR_SHAPE                 # bf16 with scales
    assert f(A, 8, ctypes.byref(linear_w(reserved=1)), None, A, None, None) == MOE_ERR_SHAPE
    assert f(A, 8, ctypes.byref(linear_w(w=MIS)), None, A, None, None) == MOE_ERR_ALIGN
    assert f(A, 8, ctypes.byref(w), None, A, A, None) == MOE_ERR_SHAPE                     # two outputs
    assert f(A, 8, ctypes.byref(w), None, None, None, None) == MOE_ERR_SHAPE               # no output
    assert f(A, 8, ctypes.byref(w), A, None, A, None) == MOE_ERR_SHAPE                     # addend with f32 out
    assert f(A, -1, ctypes.byref(w), None, A, None, None) == MOE_ERR_SHAPE
    assert f(None, 8, ctypes.byref(w), None, A, None, None) == MOE_ERR_NULL
    assert f(A, 8, ctypes.byref(w), None, MIS, None, None) == MOE_ERR_ALIGN
    assert f(None, 0, ctypes.byref(w), None, A, None, None) == MOE_OK


def latent_w(Hm=512, L=256, Is=384, **over):
    lw = MoeLatent(linear_w(0, L, Hm), linear_w(0, Hm, L), Is, 0, 4.0, 0, A, A, A)
    for k, v in over.items():
        setattr(lw, k, v)
    return lw


def test_latent_forward_validation(lib):
    fw = lib.moe_latent_forward
    routed = fp8_weights(E=8, H=256, I=128, fmt=1)
    lw = latent_w()
    ws = lib.moe_latent_forward_workspace_size(16, 2, ctypes.byref(routed), ctypes.byref(lw))
    core = lib.moe_forward_workspace_size(16, 2, ctypes.byref(routed), 0)
    assert ws > core + 16 * (2 * 256 * 2 + 512 * 4 + 384 * 2)

    def call(T=16, k=2, latent=lw, r=routed, wsb=ws, score=0, out=A, dbg=None, eps=1e-6, gamma=None):
        return fw(A, A, T, k, score, ctypes.byref(latent) if latent is not None else None, ctypes.byref(r),
                  gamma, eps, out, ctypes.byref(dbg) if dbg is not None else None, A, wsb, None)

    assert call(latent=None) == MOE_ERR_NULL
    assert call(latent=latent_w(L=384)) == MOE_ERR_SHAPE                    # routed hidden != latent
    bad_up = latent_w()
    bad_up.up = linear_w(0, 512, 384)
    assert call(latent=bad_up) == MOE_ERR_SHAPE                              # up does not invert down
    assert call(latent=latent_w(Is=100)) == MOE_ERR_SHAPE
    assert call(latent=latent_w(shared_activation=3)) == MOE_ERR_UNSUPPORTED
    assert call(latent=latent_w(shared_activation=1, shared_beta=0.0)) == MOE_ERR_SHAPE
    assert call(latent=latent_w(sw2=None)) == MOE_ERR_NULL
    no_shared = latent_w(Is=0, sw1=None, sw3=None, sw2=None)
    ws0 = lib.moe_latent_forward_workspace_size(16, 2, ctypes.byref(routed), ctypes.byref(no_shared))
    assert core < ws0 < ws                                                   # no shared buffers
    assert call(latent=no_shared, wsb=ws0 - 1) == MOE_ERR_WORKSPACE
    assert call(latent=latent_w(reserved=2)) == MOE_ERR_SHAPE
    assert call(k=9) == MOE_ERR_SHAPE
    assert call(score=3) == MOE_ERR_UNSUPPORTED
    assert call(eps=-1.0, gamma=A) == MOE_ERR_SHAPE
    assert call(wsb=ws - 1) == MOE_ERR_WORKSPACE
    assert call(out=None) == MOE_ERR_NULL
    d = MoeDebug()
    d.latent = MIS
    assert call(dbg=d) == MOE_ERR_ALIGN
    assert call(T=0) == MOE_OK


def test_forward_noalloc_validation(lib):
    """The no-alloc entry point checks its arguments as moe_forward does, and
    rejects a call whose workspace would exceed its scratch, all before any
    device call."""
    fn = lib.moe_forward_noalloc
    w = fp8_weights()
    sh = fp8_weights(E=1)

    def call(T=16, k=2, routed=w, use_shared=0, shared=None, out=A, x=A, score=0):
        return fn(x, A, T, k, score, ctypes.byref(routed), use_shared,
                  ctypes.byref(shared) if shared is not None else None, None, 1e-6, out, None, None)

    assert call(k=9) == MOE_ERR_SHAPE
    assert call(use_shared=1) == MOE_ERR_NULL
    assert call(out=None) == MOE_ERR_NULL
    assert call(x=MIS) == MOE_ERR_ALIGN
    assert call(score=5) == MOE_ERR_UNSUPPORTED
    assert call(T=0) == MOE_OK
    big = fp8_weights(E=8, H=8192, I=2048)
    need = lib.moe_forward_workspace_size(4096, 2, ctypes.byref(big), 1)
    assert need > _lib.MOE_NOALLOC_SCRATCH_BYTES
    assert call(T=4096, routed=big, use_shared=1, shared=fp8_weights(E=1, H=8192, I=2048)) == MOE_ERR_WORKSPACE
    assert b"scratch" in lib.moe_last_error()
