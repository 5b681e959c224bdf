"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory (tensor.data_ptr()) and the stream
handle (torch.cuda.current_stream().cuda_stream); nothing here computes.
Loading fails loudly if the library has not been built.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE = range(7)
MOE_W_FP8, MOE_W_MXFP4, MOE_W_FP8_BLOCK = 0, 1, 2
MOE_LAYOUT_ROW_MAJOR, MOE_LAYOUT_K_BLOCKED = 0, 1
(MOE_STAGE_ROUTE, MOE_STAGE_PERMUTE, MOE_STAGE_GEMM1, MOE_STAGE_GEMM2, MOE_STAGE_COMBINE,
 MOE_N_STAGES) = range(6)
STAGE_NAMES = ["route", "permute", "gemm1", "gemm2", "combine"]
MOE_ACT_SILU, MOE_ACT_SITU = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_LIN_MXFP4, MOE_LIN_BF16 = 0, 1
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20   # the scratch moe_forward_noalloc holds per device

# Every function include/moe.h declares.
EXPORTS = [
    "moe_route", "moe_permute_workspace_size", "moe_permute", "moe_expert_ffn_workspace_size",
    "moe_expert_ffn", "moe_combine", "moe_forward_workspace_size", "moe_forward", "moe_forward_noalloc",
    "moe_pack_weights", "moe_linear", "moe_latent_forward_workspace_size", "moe_latent_forward",
    "moe_status_string", "moe_last_error", "moe_version",
]


class MoeWeights(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32), ("layout", ctypes.c_int32), ("activation", ctypes.c_int32),
        ("act_beta", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p),
        ("s1", ctypes.c_void_p), ("s3", ctypes.c_void_p), ("s2", ctypes.c_void_p),
    ]


class MoeDebug(ctypes.Structure):
    _fields_ = [
        ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
        ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
        ("pair_to_row", ctypes.c_void_p), ("row_to_pair", ctypes.c_void_p),
        ("xq_rows", ctypes.c_void_p), ("xs_rows", ctypes.c_void_p),
        ("events", ctypes.c_void_p * (MOE_N_STAGES + 1)),
        ("variant", ctypes.c_char * 96),
        ("gemm1_events", ctypes.c_void_p * 2),
        ("gemm2_events", ctypes.c_void_p * 2),
        ("layer_events", ctypes.c_void_p * 2),
        ("latent", ctypes.c_void_p), ("core_out", ctypes.c_void_p),
    ]


class MoeLinear(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32), ("n_out", ctypes.c_int32), ("n_in", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("w", ctypes.c_void_p), ("s", ctypes.c_void_p),
    ]


class MoeLatent(ctypes.Structure):
    _fields_ = [
        ("down", MoeLinear), ("up", MoeLinear),
        ("shared_inter", ctypes.c_int32), ("shared_activation", ctypes.c_int32),
        ("shared_beta", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("sw1", ctypes.c_void_p), ("sw3", ctypes.c_void_p), ("sw2", ctypes.c_void_p),
    ]


_VP, _I32, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_WP, _DP = ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeDebug)
_LP, _LTP = ctypes.POINTER(MoeLinear), ctypes.POINTER(MoeLatent)

SIGNATURES = {
    "moe_route": (_I32, [_VP, _I32, _I32, _I32, _I32, _VP, _VP, _VP]),
    "moe_permute_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "moe_permute": (_I32, [_VP, _I32, _I32, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                           _VP, _SZ, _VP]),
    "moe_expert_ffn_workspace_size": (_SZ, [_I32, _WP]),
    "moe_expert_ffn": (_I32, [_VP, _VP, _I32, _VP, _WP, _VP, _VP, _SZ, _VP]),
    "moe_combine": (_I32, [_VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP, _F32, _VP, _VP]),
    "moe_forward_workspace_size": (_SZ, [_I32, _I32, _WP, _I32]),
    "moe_forward": (_I32, [_VP, _VP, _I32, _I32, _I32, _WP, _I32, _WP, _VP, _F32, _VP, _DP, _VP, _SZ, _VP]),
    "moe_forward_noalloc": (_I32, [_VP, _VP, _I32, _I32, _I32, _WP, _I32, _WP, _VP, _F32, _VP, _DP, _VP]),
    "moe_pack_weights": (_I32, [_WP, _WP, _VP]),
    "moe_linear": (_I32, [_VP, _I32, _LP, _VP, _VP, _VP, _VP]),
    "moe_latent_forward_workspace_size": (_SZ, [_I32, _I32, _WP, _LTP]),
    "moe_latent_forward": (_I32, [_VP, _VP, _I32, _I32, _I32, _LTP, _WP, _VP, _F32, _VP, _DP, _VP, _SZ, _VP]),
    "moe_status_string": (ctypes.c_char_p, [_I32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_char_p, []),
}

_lib = None


def load(path=LIB_PATH):
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python mixture_experts_ffn_softmax_amd/build.py` (hipcc, gfx950)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class MoeError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"status {status} ({load().moe_status_string(status).decode()}): {detail}")


def check(status):
    if status != MOE_OK:
        raise MoeError(status, load().moe_last_error().decode())
    return status
