"""Loads libflint_moe.so (the HIP library) through ctypes.

torch is imported first on purpose: the library's HIP runtime dependency
(libamdhip64.so.7) then resolves to the copy torch already loaded, so streams
and device pointers from torch are valid inside the library.  There is no
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (load order, see above)

HERE = os.path.dirname(os.path.abspath(__file__))
# FLINT_SANITIZE_DIR=<dir> loads the build in <dir> whose host code carries
# AddressSanitizer and UndefinedBehaviorSanitizer (made by
# tests/sanitize_host.py, which also preloads their runtime); its device code
# is the same as the default build's.
LIBRARY = os.path.join(os.environ.get("FLINT_SANITIZE_DIR") or HERE, "libflint_moe.so")

_lib = None


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("up", ctypes.c_void_p), ("down", ctypes.c_void_p), ("shared_gate", ctypes.c_void_p),
                ("shared_up", ctypes.c_void_p), ("shared_down", ctypes.c_void_p)]


class WeightsMx4(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p)] + [
        (f"{name}_{part}", ctypes.c_void_p)
        for name in ("gate", "up", "down", "shared_gate", "shared_up", "shared_down") for part in ("q", "s")]


class DenseDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("dtype", ctypes.c_int32)]


EXPORTS = ("flint_status_string", "flint_moe_workspace_bytes", "flint_moe_route", "flint_moe_dispatch",
           "flint_moe_forward", "flint_moe_forward_profiled", "flint_moe_forward_mx4",
           "flint_dense_workspace_bytes", "flint_dense_mlp", "flint_rmsnorm", "flint_moe_forward_static",
           "flint_moe_forward_fused", "flint_moe_forward_rmsnorm")


def load():
    """The loaded library (raises RuntimeError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(
            f"{LIBRARY} is missing: build it with `python -m routed_expert_ffn_flint_amd.build` "
            "(the Flint MoE layer has no CPU or PyTorch fallback)")
    lib = ctypes.CDLL(LIBRARY)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(Dims)
    lib.flint_status_string.argtypes = [I32]
    lib.flint_status_string.restype = ctypes.c_char_p
    lib.flint_moe_workspace_bytes.argtypes = [D, I32]
    lib.flint_moe_workspace_bytes.restype = SZ
    lib.flint_moe_route.argtypes = [D, I32, P, P, P, P, P, P, SZ, P]
    lib.flint_moe_route.restype = I32
    lib.flint_moe_dispatch.argtypes = [D, I32, P, P, P, P, P, P, SZ, P]
    lib.flint_moe_dispatch.restype = I32
    lib.flint_moe_forward.argtypes = [D, I32, P, ctypes.POINTER(Weights), P, I32, P, P, P, SZ, P]
    lib.flint_moe_forward.restype = I32
    lib.flint_moe_forward_profiled.argtypes = [D, I32, P, ctypes.POINTER(Weights), P, I32, P, P, P, SZ, P, P]
    lib.flint_moe_forward_profiled.restype = I32
    lib.flint_moe_forward_mx4.argtypes = [D, I32, P, ctypes.POINTER(WeightsMx4), P, I32, P, P, P, SZ, P, P]
    lib.flint_moe_forward_mx4.restype = I32
    DD = ctypes.POINTER(DenseDims)
    lib.flint_dense_workspace_bytes.argtypes = [DD, I32]
    lib.flint_dense_workspace_bytes.restype = SZ
    lib.flint_dense_mlp.argtypes = [DD, I32, P, P, P, P, P, I32, P, SZ, P, P]
    lib.flint_dense_mlp.restype = I32
    lib.flint_rmsnorm.argtypes = [I32, I32, P, P, ctypes.c_float, P]
    lib.flint_rmsnorm.restype = I32
    lib.flint_moe_forward_static.argtypes = [D, I32, P, ctypes.POINTER(Weights), P, I32, P, P, P]
    lib.flint_moe_forward_static.restype = I32
    lib.flint_moe_forward_fused.argtypes = [D, I32, P, ctypes.POINTER(Weights), P, I32, P, P, P, SZ, P, P]
    lib.flint_moe_forward_fused.restype = I32
    lib.flint_moe_forward_rmsnorm.argtypes = [D, I32, P, ctypes.POINTER(Weights), P, I32, P, ctypes.c_float, P, P,
                                              P, SZ, P, P]
    lib.flint_moe_forward_rmsnorm.restype = I32
    _lib = lib
    return lib
