"""ctypes wrapper around the C oracle (``flint_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of
the benchmark use this module to check the GPU path.  The product package never
imports it.  Arrays are numpy; every floating-point input is a float32 array that
holds the exact values of the layer's storage type (bf16 values widen exactly).

What each function computes is documented in ``flint_oracle.c`` next to the C
code, with the passages of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "flint_oracle.c")
# FLINT_SANITIZE_DIR=<dir> selects a build in <dir> with AddressSanitizer and
# UndefinedBehaviorSanitizer (clang, whose shared runtime the process must
# preload: tests/sanitize_host.py runs the CPU suite that way).
SANITIZE_DIR = os.environ.get("FLINT_SANITIZE_DIR")
SANITIZE = bool(SANITIZE_DIR)
LIBRARY = os.path.join(SANITIZE_DIR, "liboracle.so") if SANITIZE else os.path.join(_HERE, "liboracle.so")
CLANG = "/opt/rocm/llvm/bin/clang"


def compile_source(src: str, out: str) -> str:
    """Compile an oracle source file with gcc (-O2, IEEE double, no fast-math,
    OpenMP over tokens) into a shared library at ``out``; under FLINT_SANITIZE_DIR
    with clang and the address and undefined-behaviour sanitizers instead
    (undefined behaviour is fatal, as a memory error is)."""
    tmp = f"{out}.tmp{os.getpid()}"  # per process: parallel test workers may build at once
    if SANITIZE:
        cmd = [CLANG, "-O1", "-g", "-fPIC", "-shared", "-fopenmp=libgomp", "-fno-fast-math", "-ffp-contract=off",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
               "-std=c11", "-Wall", "-o", tmp, src, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-std=c11", "-Wall", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``flint_oracle.c`` into ``liboracle.so`` next to it."""
    if force or not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        compile_source(SOURCE, LIBRARY)
    return LIBRARY


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("n_experts", ctypes.c_int), ("top_k", ctypes.c_int),
                ("inter", ctypes.c_int), ("shared_inter", ctypes.c_int), ("h_is_bf16", ctypes.c_int)]


def dims(hidden, n_experts, top_k, inter, shared_inter, bf16: bool) -> Dims:
    return Dims(hidden, n_experts, top_k, inter, shared_inter, 1 if bf16 else 0)


def _f32(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _i32(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: oracle rejected its arguments (code {rc})")


class Oracle:
    """The oracle's functions bound to one compiled library: the default build of
    ``flint_oracle.c``, or another build of an oracle source (the pin tests also
    load deliberately broken copies to show that the pins catch mistakes)."""

    def __init__(self, path: str | None = None):
        if path is None:
            if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
                build(force=True)
            path = LIBRARY
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        D = ctypes.POINTER(Dims)
        lib.oracle_route.argtypes = [D, ctypes.c_int, P, P, P, P, P, P]
        lib.oracle_scores.argtypes = [D, ctypes.c_int, P, P, P, P]
        lib.oracle_dispatch.argtypes = [D, ctypes.c_int, P, P, P, P, P]
        lib.oracle_forward.argtypes = [D, ctypes.c_int] + [P] * 14
        lib.oracle_rmsnorm.argtypes = [ctypes.c_int, ctypes.c_int, P, ctypes.c_double, P]
        lib.oracle_round_bf16.argtypes = [P, P, ctypes.c_int64]
        lib.oracle_param_counts.argtypes = [D, P]
        lib.oracle_mx4_dequant.argtypes = [ctypes.c_int64, ctypes.c_int, P, P, P]
        lib.oracle_mx4_untile.argtypes = [ctypes.c_int64, ctypes.c_int, P, P, P, P]
        lib.oracle_dense_mlp.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P, P]
        for f in ("oracle_route", "oracle_scores", "oracle_dispatch", "oracle_forward",
                  "oracle_rmsnorm", "oracle_mx4_dequant", "oracle_mx4_untile", "oracle_dense_mlp"):
            getattr(lib, f).restype = ctypes.c_int
        lib.oracle_round_bf16.restype = None
        lib.oracle_param_counts.restype = None
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        self.lib = lib
        self.path = path

    def route(self, d: Dims, x, w_router, bias=None):
        """Returns (topk_idx [T,K] int32 ascending, topk_w [T,K] float32, near_tie [T] bool)."""
        x = _f32(x)
        T = x.shape[0]
        idx = np.zeros((T, d.top_k), np.int32)
        w = np.zeros((T, d.top_k), np.float32)
        tie = np.zeros((T,), np.uint8)
        wr, b = _f32(w_router), _f32(bias)
        _check(self.lib.oracle_route(ctypes.byref(d), T, _p(x), _p(wr), _p(b), _p(idx), _p(w),
                                     _p(tie)), "oracle_route")
        return idx, w, tie.astype(bool)

    def scores(self, d: Dims, x, w_router, bias=None):
        """Float32 sigmoid scores [T, E]."""
        x = _f32(x)
        T = x.shape[0]
        s = np.zeros((T, d.n_experts), np.float32)
        wr, b = _f32(w_router), _f32(bias)
        _check(self.lib.oracle_scores(ctypes.byref(d), T, _p(x), _p(wr), _p(b), _p(s)),
               "oracle_scores")
        return s

    def dispatch(self, d: Dims, topk_idx):
        """Returns (counts [E], offsets [E+1], sorted_token [T*K], slot_of [T*K]) int32."""
        idx = _i32(topk_idx).reshape(-1, d.top_k)
        T = idx.shape[0]
        n = T * d.top_k
        counts = np.zeros((d.n_experts,), np.int32)
        offsets = np.zeros((d.n_experts + 1,), np.int32)
        st = np.zeros((max(n, 1),), np.int32)
        so = np.zeros((max(n, 1),), np.int32)
        _check(self.lib.oracle_dispatch(ctypes.byref(d), T, _p(idx), _p(counts), _p(offsets),
                                        _p(st), _p(so)), "oracle_dispatch")
        return counts, offsets, st[:n], so[:n]

    def forward(self, d: Dims, x, w, force_idx=None):
        """The whole layer.  ``w`` is a dict with router, bias (or None), gate, up,
        down, shared_gate, shared_up, shared_down (arrays of exact values).
        Returns (out [T,H] float32, topk_idx, topk_w, near_tie)."""
        x = _f32(x)
        T = x.shape[0]
        out = np.zeros((T, d.hidden), np.float32)
        idx = np.zeros((T, d.top_k), np.int32)
        tw = np.zeros((T, d.top_k), np.float32)
        tie = np.zeros((T,), np.uint8)
        arrs = [_f32(w["router"]), _f32(w.get("bias")), _f32(w["gate"]), _f32(w["up"]),
                _f32(w["down"])]
        if d.shared_inter > 0:
            arrs += [_f32(w["shared_gate"]), _f32(w["shared_up"]), _f32(w["shared_down"])]
        else:
            arrs += [None, None, None]
        fi = _i32(force_idx)
        rc = self.lib.oracle_forward(ctypes.byref(d), T, _p(x), *[_p(a) for a in arrs], _p(fi),
                                     _p(out), _p(idx), _p(tw), _p(tie))
        _check(rc, "oracle_forward")
        return out, idx, tw, tie.astype(bool)

    def rmsnorm(self, x, eps=1e-6):
        """y / sqrt(mean(y^2) + eps) per row, rounded to bf16 (returned as float32 values)."""
        x = _f32(x)
        T, H = x.shape
        out = np.zeros_like(x)
        _check(self.lib.oracle_rmsnorm(T, H, _p(x), eps, _p(out)), "oracle_rmsnorm")
        return out

    def round_bf16(self, a):
        a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
        out = np.zeros_like(a)
        self.lib.oracle_round_bf16(_p(a), _p(out), a.size)
        return out

    def mx4_dequant(self, codes, scales):
        """Block-scaled 4-bit weights (MXFP4, see flint_oracle.c) to float32:
        codes uint8 [..., n/2], scales uint8 [..., n/32] -> [..., n]."""
        codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
        scales = np.ascontiguousarray(np.asarray(scales, dtype=np.uint8))
        n = codes.shape[-1] * 2
        if scales.shape[:-1] != codes.shape[:-1] or scales.shape[-1] * 32 != n:
            raise ValueError("mx4_dequant: codes [..., n/2] and scales [..., n/32] disagree")
        rows = int(np.prod(codes.shape[:-1], dtype=np.int64))
        out = np.zeros(codes.shape[:-1] + (n,), np.float32)
        _check(self.lib.oracle_mx4_dequant(rows, n, _p(codes), _p(scales), _p(out)), "oracle_mx4_dequant")
        return out

    def dense_mlp(self, x, w_gate, w_up, w_down, h_bf16=True):
        """A dense gated MLP layer (see flint_oracle.c): x [T, H], gate/up [I, H],
        down [H, I] -> float32 [T, H]; h rounded to bf16 (h_bf16) or float32."""
        x = _f32(x)
        wg, wu, wd = _f32(w_gate), _f32(w_up), _f32(w_down)
        T, H = x.shape
        I = wg.shape[0]
        if wg.shape != (I, H) or wu.shape != (I, H) or wd.shape != (H, I):
            raise ValueError("dense_mlp: gate/up [I, H] and down [H, I]")
        out = np.zeros((T, H), np.float32)
        _check(self.lib.oracle_dense_mlp(T, H, I, 1 if h_bf16 else 0, _p(x), _p(wg), _p(wu), _p(wd), _p(out)),
               "oracle_dense_mlp")
        return out

    def mx4_untile(self, codes, scales):
        """The tiled byte order of the library's MXFP4 arrays back to row-major.
        A tile is 16 rows x one 32-element block: codes [..., R/16, n/32, 16, 16]
        hold, per tile, row r's 16 bytes; scales [..., R/16, n/32, 16] row r's
        scale byte.  Returns codes [..., R, n/2] and scales [..., R, n/32]."""
        codes = np.asarray(codes, dtype=np.uint8)
        scales = np.asarray(scales, dtype=np.uint8)
        if codes.shape[-2:] != (16, 16) or scales.shape[-1] != 16 or codes.shape[:-1] != scales.shape:
            raise ValueError("mx4_untile: codes [..., R/16, n/32, 16, 16] and scales [..., R/16, n/32, 16]")
        lead, rb, nb = codes.shape[:-4], codes.shape[-4], codes.shape[-3]
        rows = int(np.prod(lead, dtype=np.int64)) * rb * 16
        codes = np.ascontiguousarray(codes)
        scales = np.ascontiguousarray(scales)
        c = np.zeros(lead + (rb * 16, nb * 16), np.uint8)
        s = np.zeros(lead + (rb * 16, nb), np.uint8)
        _check(self.lib.oracle_mx4_untile(rows, nb * 32, _p(codes), _p(scales), _p(c), _p(s)), "oracle_mx4_untile")
        return c, s

    def mx4_dequant_tiled(self, codes, scales):
        """mx4_dequant of arrays in the library's tiled order (see mx4_untile)."""
        return self.mx4_dequant(*self.mx4_untile(codes, scales))

    def mx4_weights(self, w):
        """A layer's weights with the expert matrices in MXFP4, tiled order (keys
        <name>_q and <name>_s for gate, up, down and, when present, the shared
        expert's) -> the float32 weights dict that forward() takes (router and
        bias as given)."""
        out = {"router": w["router"], "bias": w.get("bias")}
        for name in ("gate", "up", "down", "shared_gate", "shared_up", "shared_down"):
            if w.get(name + "_q") is not None:
                out[name] = self.mx4_dequant_tiled(w[name + "_q"], w[name + "_s"])
        return out

    def threads(self) -> int:
        """Threads the oracle's OpenMP loops use."""
        return int(self.lib.oracle_threads())

    def set_threads(self, n: int) -> None:
        """Threads for the oracle's OpenMP loops from now on."""
        self.lib.oracle_set_threads(int(n))

    def param_counts(self, d: Dims):
        """(router, routed total, one expert, shared expert, active expert params per token)."""
        out = np.zeros((5,), np.int64)
        self.lib.oracle_param_counts(ctypes.byref(d), _p(out))
        return tuple(int(v) for v in out)


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def route(d, x, w_router, bias=None):
    return default().route(d, x, w_router, bias)


def scores(d, x, w_router, bias=None):
    return default().scores(d, x, w_router, bias)


def dispatch(d, topk_idx):
    return default().dispatch(d, topk_idx)


def forward(d, x, w, force_idx=None):
    return default().forward(d, x, w, force_idx)


def rmsnorm(x, eps=1e-6):
    return default().rmsnorm(x, eps)


def round_bf16(a):
    return default().round_bf16(a)


def param_counts(d):
    return default().param_counts(d)


def mx4_dequant(codes, scales):
    return default().mx4_dequant(codes, scales)


def mx4_untile(codes, scales):
    return default().mx4_untile(codes, scales)


def dense_mlp(x, w_gate, w_up, w_down, h_bf16=True):
    return default().dense_mlp(x, w_gate, w_up, w_down, h_bf16)


def mx4_dequant_tiled(codes, scales):
    return default().mx4_dequant_tiled(codes, scales)


def mx4_weights(w):
    return default().mx4_weights(w)
