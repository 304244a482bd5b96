"""ctypes binding of libmoe_latent.so (argument marshalling only).

Every compute step runs in the HIP library; this module only turns torch
tensors into device pointers and a stream handle.  If the library has not been
built, loading raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libmoe_latent.so")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE, MOE_EHIP, MOE_EINTERNAL = 0, -1, -2, -3, -4, -5
MOE_OPND_BF16X2, MOE_OPND_BF16, MOE_OPND_MX8X3, MOE_OPND_MX6X3 = 0, 1, 2, 3
MOE_OP_GATEUP_SITU, MOE_OP_DOWN, MOE_OP_GATEUP_SITU_BF16X2 = 0, 1, 2
MOE_DT_F32, MOE_DT_BF16, MOE_DT_BF16X2 = 0, 1, 2
MOE_ROUTE_NOALLOC_SCRATCH_BYTES = 8 << 20
(MOE_FN_ROUTE, MOE_FN_PERMUTE, MOE_FN_GROUPED_GEMM, MOE_FN_COMBINE_NORM_UP, MOE_FN_SHARED_FFN,
 MOE_FN_REAP_SALIENCY, MOE_FN_COMBINE_NORM_UP_REAP, MOE_FN_GROUPED_GEMM_TWO_BANK) = range(8)
MOE_WF_MXFP4, MOE_WF_AFFINE2 = 0, 1

EXPORTS = ("moe_abi_version", "moe_strerror", "moe_workspace_bytes", "moe_route", "moe_permute",
           "mxfp4_grouped_gemm", "moe_combine_norm_up", "shared_expert_ffn", "moe_reap_saliency",
           "moe_combine_norm_up_reap", "moe_route_capped", "moe_route_noalloc",
           "moe_grouped_gemm_two_bank")


class MoeShape(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("latent", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_shared", ctypes.c_int32),
        ("shared_inter", ctypes.c_int32), ("beta", ctypes.c_float), ("beta_lin", ctypes.c_float),
        ("rms_eps", ctypes.c_float), ("operand_mode", ctypes.c_int32),
    ]


class MoeExpertBank(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("packed", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("packed3", ctypes.c_void_p), ("scale3", ctypes.c_void_p), ("bias3", ctypes.c_void_p),
    ]


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {code} ({msg})")
        self.code = code


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library not built: {p} (run `python -m mxfp4_latent_moe_amd.build`)")
    lib = ctypes.CDLL(p)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sp = ctypes.POINTER(MoeShape)
    lib.moe_abi_version.restype = i32
    lib.moe_abi_version.argtypes = []
    lib.moe_strerror.restype = ctypes.c_char_p
    lib.moe_strerror.argtypes = [i32]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_workspace_bytes.argtypes = [sp, i32, i32]
    lib.moe_route.restype = i32
    lib.moe_route.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_permute.restype = i32
    lib.moe_permute.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mxfp4_grouped_gemm.restype = i32
    lib.mxfp4_grouped_gemm.argtypes = [sp, i32, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_combine_norm_up.restype = i32
    lib.moe_combine_norm_up.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.shared_expert_ffn.restype = i32
    lib.shared_expert_ffn.argtypes = [sp, i32, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.moe_reap_saliency.restype = i32
    lib.moe_reap_saliency.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    bp = ctypes.POINTER(MoeExpertBank)
    lib.moe_grouped_gemm_two_bank.restype = i32
    lib.moe_grouped_gemm_two_bank.argtypes = [sp, i32, i32, vp, vp, vp, i32, i32, bp, bp, vp, vp, vp, sz, vp]
    lib.moe_route_noalloc.restype = i32
    lib.moe_route_noalloc.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_route_capped.restype = i32
    lib.moe_route_capped.argtypes = [sp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_combine_norm_up_reap.restype = i32
    lib.moe_combine_norm_up_reap.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, sz, vp]
    if path is None:
        _lib = lib
    return lib


def check(fn: str, code: int) -> None:
    if code != MOE_OK:
        raise MoeError(fn, code, load().moe_strerror(code).decode())


def make_shape(hidden, latent, n_experts, top_k, inter, n_shared, shared_inter,
               beta=4.0, beta_lin=25.0, rms_eps=1e-6, operand_mode=MOE_OPND_BF16X2) -> MoeShape:
    return MoeShape(hidden, latent, n_experts, top_k, inter, n_shared, shared_inter,
                    beta, beta_lin, rms_eps, operand_mode)
