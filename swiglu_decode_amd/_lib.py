"""ctypes loader for libswiglu_decode.so (argument marshalling only)."""

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libswiglu_decode.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "swiglu_decode.h")

FMT_BLOCK128 = 1
FMT_MX32 = 2
MAX_M = 128

STATUS = {0: "SGD_OK", -1: "SGD_EINVAL", -2: "SGD_EALIGN", -3: "SGD_EDIM",
          -4: "SGD_EWORKSPACE", -5: "SGD_EFMT", -6: "SGD_EHIP", -7: "SGD_ETIMEOUT"}
SGD_ETIMEOUT = -7


class SgdWeight(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


class SgdError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_f = ctypes.c_float
_wp = ctypes.POINTER(SgdWeight)

SIGNATURES = {
    "sgd_status_str": (ctypes.c_char_p, [_i]),
    "sgd_abi_version": (_i, []),
    "sgd_packed_codes_bytes": (_sz, [_i, _i, _i]),
    "sgd_packed_scales_bytes": (_sz, [_i, _i, _i]),
    "sgd_quantize_pack_weight": (_i, [_i, _vp, _i, _i, _vp, _vp, _vp]),
    "sgd_unpack_weight": (_i, [_wp, _vp, _vp, _vp]),
    "sgd_quantize_act": (_i, [_i, _vp, _i, _i, _vp, _vp, _vp]),
    "sgd_gemm_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "sgd_mlp_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "sgd_workspace_clear": (_i, [_vp, _sz, _vp]),
    "sgd_scaled_gemm": (_i, [_vp, _i, _wp, _vp, _vp, _sz, _vp]),
    "sgd_fused_swiglu_mlp": (_i, [_vp, _i, _wp, _wp, _wp, _vp, _vp, _sz, _vp]),
    "sgd_fused_swiglu_mlp_noalloc": (_i, [_vp, _i, _wp, _wp, _wp, _vp, _vp]),
    "sgd_fused_swiglu_block": (_i, [_vp, _i, _wp, _wp, _wp, _f, _vp, _vp, _sz, _vp]),
    "sgd_gemm_large_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "sgd_scaled_gemm_large": (_i, [_vp, _i, _wp, _vp, _vp, _sz, _vp]),
    "sgd_mlp_prefill_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "sgd_swiglu_mlp_prefill": (_i, [_vp, _i, _wp, _wp, _vp, _vp, _sz, _vp]),
    "sgd_kv_cache_bytes": (_sz, [_i, _i]),
    "sgd_kv_cache_write": (_i, [_i, _vp, _vp, _i, _i, _i, _vp, _i, _vp]),
    "sgd_paged_attention_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "sgd_paged_decode_attention": (_i, [_vp, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _f, _vp, _vp, _sz, _vp]),
    "sgd_scaled_gemm_f32": (_i, [_vp, _i, _wp, _vp, _vp, _sz, _vp]),
    "sgd_act_scales_bytes": (_sz, [_i, _i, _i]),
    "sgd_swiglu_quantize": (_i, [_i, _vp, _i, _i, _vp, _vp, _vp]),
    "sgd_scaled_gemm_q": (_i, [_vp, _vp, _i, _wp, _vp, _vp, _sz, _vp]),
    "sgd_bf16_to_f32": (_i, [_vp, _i, _i, _vp, _vp]),
    "sgd_rmsnorm_bf16": (_i, [_vp, _i, _i, _f, _vp, _vp]),
    "sgd_residual_add": (_i, [_vp, _vp, _i, _i, _vp]),
    "sgd_residual_rmsnorm_bf16": (_i, [_vp, _vp, _i, _i, _f, _vp, _vp]),
    "sgd_head_logits": (_i, [_vp, _i, _i, _vp, _i, _vp, _vp]),
    "sgd_argmax_rows": (_i, [_vp, _i, _i, _vp, _vp]),
    "sgd_read_stream": (_i, [_vp, _sz, _vp, _vp]),
    "sgd_set_wait_budget_us": (ctypes.c_uint32, [ctypes.c_uint32]),
    "sgd_set_keep_intermediates": (ctypes.c_int, [ctypes.c_int]),
    "sgd_workspace_status": (_i, [_vp, _vp]),
    "sgd_mlp_workspace_layout": (_i, [_i, _i, _i, _i, ctypes.POINTER(_sz)]),
}

_LIB = None


def header_symbols():
    """Names of the functions declared in include/swiglu_decode.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgd_[a-z0-9_]+)\s*\(", text)))


def load():
    """Load the built library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m swiglu_decode_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(fn_name, status):
    if status != 0:
        msg = load().sgd_status_str(status).decode()
        raise SgdError(fn_name, status, msg)
