"""The C-ABI library without a GPU: it loads, exports every declared symbol,
sizes its workspace, and refuses bad arguments on the host before any launch.

Only paths that return before the first kernel launch are exercised here; the
pointers passed are never dereferenced (validation looks at them as integers).
"""
import ctypes
import os
import re

import pytest

from routed_expert_ffn_flint_amd import _lib, api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flint_moe.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced
FAKE_WS = 0x100000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIBRARY):
        from routed_expert_ffn_flint_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(flint_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and nothing C++-mangled is needed to use it: the exported names are plain
    out = os.popen(f"nm -D --defined-only {_lib.LIBRARY}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, re.M), name


def flint_dims(**kw):
    base = dict(hidden=2048, n_experts=256, top_k=6, inter=512, shared_inter=1024, dtype=api.BF16)
    base.update(kw)
    return api.make_dims(**base)


def test_status_strings(lib):
    for code in range(5):
        assert api.flint_status_string(code)
    assert "unknown" in api.flint_status_string(99)


def test_workspace_bytes(lib):
    d = flint_dims()
    small = api.flint_moe_workspace_bytes(d, 32)
    big = api.flint_moe_workspace_bytes(d, 16384)
    assert 0 < small < big
    # holds at least the float32 expert outputs of every (token, expert) pair
    assert big >= 16384 * 6 * 2048 * 4
    assert api.flint_moe_workspace_bytes(d, 0) > 0
    assert api.flint_moe_workspace_bytes(d, -1) == 0
    assert api.flint_moe_workspace_bytes(flint_dims(top_k=9), 32) == 0
    assert api.flint_moe_workspace_bytes(flint_dims(hidden=2000), 32) == 0


def _forward(lib, d, T, ws_bytes=None, x=FAKE, out=FAKE, out_dtype=api.F32, w=None, ws=FAKE_WS):
    if w is None:
        w = _lib.Weights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    if ws_bytes is None:
        ws_bytes = api.flint_moe_workspace_bytes(d, T) if T >= 0 else 0
    return lib.flint_moe_forward(ctypes.byref(d), T, x, ctypes.byref(w), out, out_dtype, None, None, ws,
                                 ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=9), api.UNSUPPORTED),
    (dict(n_experts=257, top_k=6), api.UNSUPPORTED),
    (dict(top_k=0), api.INVALID_ARG),
    (dict(n_experts=4, top_k=6), api.INVALID_ARG),
    (dict(hidden=2000), api.UNSUPPORTED),
    (dict(inter=500), api.UNSUPPORTED),
    (dict(shared_inter=1000), api.UNSUPPORTED),
    (dict(shared_inter=-64), api.INVALID_ARG),
    (dict(dtype=7), api.UNSUPPORTED),
    (dict(hidden=16384), api.UNSUPPORTED),
])
def test_forward_refuses_unsupported_shapes(lib, kw, status):
    d = flint_dims(**kw)
    assert _forward(lib, d, 32, ws_bytes=1 << 30) == status


def test_forward_argument_errors(lib):
    d = flint_dims()
    assert _forward(lib, d, -1) == api.INVALID_ARG
    assert _forward(lib, d, 0) == api.OK  # no-op, nothing launched
    assert _forward(lib, d, 32, x=None) == api.INVALID_ARG
    assert _forward(lib, d, 32, out=None) == api.INVALID_ARG
    assert _forward(lib, d, 32, x=FAKE + 2) == api.UNSUPPORTED  # misaligned
    assert _forward(lib, d, 32, out_dtype=5) == api.UNSUPPORTED
    need = api.flint_moe_workspace_bytes(d, 32)
    assert _forward(lib, d, 32, ws_bytes=need - 1) == api.WORKSPACE_TOO_SMALL
    assert _forward(lib, d, 32, ws=None) == api.INVALID_ARG
    assert _forward(lib, d, 32, ws=FAKE_WS + 16) == api.UNSUPPORTED  # workspace must be 256-byte aligned
    no_shared = _lib.Weights(FAKE, None, FAKE, FAKE, FAKE, None, None, None)
    assert _forward(lib, d, 32, w=no_shared) == api.INVALID_ARG
    no_gate = _lib.Weights(FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert _forward(lib, d, 32, w=no_gate) == api.INVALID_ARG
    assert _forward(lib, d, 1 << 30) == api.UNSUPPORTED  # T*K overflows int32


def test_route_and_dispatch_argument_errors(lib):
    d = flint_dims()
    need = api.flint_moe_workspace_bytes(d, 32)
    r = lib.flint_moe_route
    assert r(ctypes.byref(d), -1, FAKE, FAKE, None, FAKE, FAKE, FAKE_WS, need, None) == api.INVALID_ARG
    assert r(ctypes.byref(d), 0, None, None, None, None, None, None, 0, None) == api.OK
    assert r(ctypes.byref(d), 32, None, FAKE, None, FAKE, FAKE, FAKE_WS, need, None) == api.INVALID_ARG
    assert r(ctypes.byref(d), 32, FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE_WS, need, None) == api.UNSUPPORTED
    assert r(ctypes.byref(d), 32, FAKE, FAKE, None, FAKE, FAKE, FAKE_WS, need - 1, None) == api.WORKSPACE_TOO_SMALL
    dd = lib.flint_moe_dispatch
    assert dd(ctypes.byref(d), 32, FAKE, None, FAKE, FAKE, FAKE, FAKE_WS, need, None) == api.INVALID_ARG
    assert dd(ctypes.byref(d), 32, None, FAKE, FAKE, FAKE, FAKE, FAKE_WS, need, None) == api.INVALID_ARG
    assert dd(ctypes.byref(d), -3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE_WS, need, None) == api.INVALID_ARG
    bad = flint_dims(top_k=9)
    assert dd(ctypes.byref(bad), 32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE_WS, need, None) == api.UNSUPPORTED


def test_rmsnorm_argument_errors(lib):
    f = lib.flint_rmsnorm
    assert f(-1, 2048, FAKE, FAKE, 1e-6, None) == api.INVALID_ARG
    assert f(4, 100, FAKE, FAKE, 1e-6, None) == api.UNSUPPORTED
    assert f(0, 2048, None, None, 1e-6, None) == api.OK
    assert f(4, 2048, None, FAKE, 1e-6, None) == api.INVALID_ARG
    assert f(4, 2048, FAKE, FAKE, -1.0, None) == api.INVALID_ARG


def test_binding_raises_on_refusal(lib):
    with pytest.raises(api.FlintError) as ei:
        api.workspace(flint_dims(top_k=9), 32, device="cpu")
    assert ei.value.status == api.UNSUPPORTED


def _forward_mx4(lib, d, T, ws_bytes=None, w=None, ws=FAKE_WS, x=FAKE):
    if w is None:
        fields = {f"{n}_{p}": FAKE for n in ("gate", "up", "down", "shared_gate", "shared_up", "shared_down")
                  for p in ("q", "s")}
        w = _lib.WeightsMx4(router=FAKE, router_bias=None, **fields)
    if ws_bytes is None:
        ws_bytes = api.flint_moe_workspace_bytes(d, T) if T >= 0 else 0
    return lib.flint_moe_forward_mx4(ctypes.byref(d), T, x, ctypes.byref(w), FAKE, api.F32, None, None, ws,
                                     ws_bytes, None, None)


def test_forward_mx4_refusals(lib):
    d = flint_dims()
    assert _forward_mx4(lib, d, 0) == api.OK  # no-op
    assert _forward_mx4(lib, flint_dims(dtype=api.F32), 32) == api.UNSUPPORTED  # bf16 activations only
    assert _forward_mx4(lib, d, 513) == api.UNSUPPORTED  # small batches only
    assert _forward_mx4(lib, flint_dims(hidden=1536), 32) == api.UNSUPPORTED  # H % 1024
    assert _forward_mx4(lib, flint_dims(inter=128), 32) == api.UNSUPPORTED  # I % 256
    assert _forward_mx4(lib, flint_dims(shared_inter=640), 32) == api.UNSUPPORTED  # Is % 256
    assert _forward_mx4(lib, d, 32, x=None) == api.INVALID_ARG
    assert _forward_mx4(lib, d, 32, ws_bytes=api.flint_moe_workspace_bytes(d, 32) - 1) == \
        api.WORKSPACE_TOO_SMALL
    fields = {f"{n}_{p}": FAKE for n in ("gate", "up", "down", "shared_gate", "shared_up", "shared_down")
              for p in ("q", "s")}
    fields["down_s"] = None
    assert _forward_mx4(lib, d, 32, w=_lib.WeightsMx4(router=FAKE, router_bias=None, **fields)) == \
        api.INVALID_ARG
    fields["down_s"] = FAKE
    fields["gate_q"] = FAKE + 8
    assert _forward_mx4(lib, d, 32, w=_lib.WeightsMx4(router=FAKE, router_bias=None, **fields)) == \
        api.UNSUPPORTED  # code arrays 16-byte aligned
    # no shared expert: its pointers may be NULL
    ns = flint_dims(shared_inter=0)
    fields = {f"{n}_{p}": FAKE for n in ("gate", "up", "down") for p in ("q", "s")}
    w = _lib.WeightsMx4(router=FAKE, router_bias=None, **fields)
    assert _forward_mx4(lib, ns, 0, w=w) == api.OK


def _dense(lib, dd, T, ws_bytes=None, x=FAKE, out_dtype=api.F32, ws=FAKE_WS):
    if ws_bytes is None:
        ws_bytes = lib.flint_dense_workspace_bytes(ctypes.byref(dd), T) if T >= 0 else 0
    return lib.flint_dense_mlp(ctypes.byref(dd), T, x, FAKE, FAKE, FAKE, FAKE, out_dtype, ws, ws_bytes, None, None)


def test_dense_mlp_refusals(lib):
    dd = _lib.DenseDims(hidden=2048, inter=6144, dtype=api.BF16)
    n32 = lib.flint_dense_workspace_bytes(ctypes.byref(dd), 32)
    # h [T][I] bf16 and y [T][H] float32 at least
    assert n32 >= 32 * 6144 * 2 + 32 * 2048 * 4
    assert lib.flint_dense_workspace_bytes(ctypes.byref(dd), 64) > n32
    assert _dense(lib, dd, 0) == api.OK  # no-op
    assert _dense(lib, dd, -1) == api.INVALID_ARG
    assert _dense(lib, _lib.DenseDims(hidden=2048, inter=6144, dtype=7), 32) == api.UNSUPPORTED
    assert _dense(lib, _lib.DenseDims(hidden=2000, inter=6144, dtype=api.BF16), 32) == api.UNSUPPORTED
    assert _dense(lib, _lib.DenseDims(hidden=2048, inter=6100, dtype=api.BF16), 32) == api.UNSUPPORTED
    assert _dense(lib, _lib.DenseDims(hidden=2048, inter=16448, dtype=api.BF16), 32) == api.UNSUPPORTED
    assert _dense(lib, _lib.DenseDims(hidden=0, inter=6144, dtype=api.BF16), 32) == api.INVALID_ARG
    assert _dense(lib, dd, 32, x=None) == api.INVALID_ARG
    assert _dense(lib, dd, 32, x=FAKE + 4) == api.UNSUPPORTED  # 16-byte alignment
    assert _dense(lib, dd, 32, out_dtype=5) == api.UNSUPPORTED
    assert _dense(lib, dd, 32, ws_bytes=n32 - 1) == api.WORKSPACE_TOO_SMALL
    assert _dense(lib, dd, 32, ws=FAKE_WS + 16) == api.UNSUPPORTED  # 256-byte aligned workspace
    assert _dense(lib, dd, 32, ws=None) == api.INVALID_ARG


def _forward_static(lib, d, T, x=FAKE, w=None, out=FAKE, out_dtype=api.F32):
    w = w or _lib.Weights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    return lib.flint_moe_forward_static(ctypes.byref(d), T, x, ctypes.byref(w), out, out_dtype, None, None, None)


def test_forward_static_refusals(lib):
    """The allocation-free entry point refuses on the host, before it looks up
    its device scratch: the same argument errors as flint_moe_forward, and any
    shape whose workspace would exceed the static scratch."""
    d = flint_dims()
    assert _forward_static(lib, d, -1) == api.INVALID_ARG
    assert _forward_static(lib, d, 0) == api.OK
    assert _forward_static(lib, d, 32, x=None) == api.INVALID_ARG
    assert _forward_static(lib, d, 32, x=FAKE + 2) == api.UNSUPPORTED
    assert _forward_static(lib, flint_dims(top_k=9), 32) == api.UNSUPPORTED
    no_gate = _lib.Weights(FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert _forward_static(lib, d, 32, w=no_gate) == api.INVALID_ARG
    limit = 48 << 20  # FLINT_STATIC_SCRATCH_BYTES
    assert re.search(r"FLINT_STATIC_SCRATCH_BYTES \(\(size_t\)48 << 20\)", open(HEADER).read())
    T_max = max(T for T in range(1, 2048) if api.flint_moe_workspace_bytes(d, T) <= limit)
    assert T_max >= 512  # the decode batches and the 256-token stack fit
    # the largest batch the header states for the Flint layer
    stated = re.search(r"the Flint layer up to T = (\d+) tokens", open(HEADER).read())
    assert stated and int(stated.group(1)) == T_max
    assert _forward_static(lib, d, T_max + 1) == api.WORKSPACE_TOO_SMALL
    assert _forward_static(lib, d, 100_000) == api.WORKSPACE_TOO_SMALL


def test_forward_fused_refusals(lib):
    """The fused decode entry point takes bf16 batches of 1..64 tokens with H and
    I multiples of 256 and Is a multiple of I (at most 8 of them); it refuses
    anything else on the host, after the checks flint_moe_forward makes."""
    def call(d, T):
        w = _lib.Weights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
        return lib.flint_moe_forward_fused(ctypes.byref(d), T, FAKE, ctypes.byref(w), FAKE, api.F32, None, None,
                                           FAKE_WS, 1 << 30, None, None)
    assert call(flint_dims(), -1) == api.INVALID_ARG
    assert call(flint_dims(), 0) == api.OK
    assert call(flint_dims(), 65) == api.UNSUPPORTED
    assert call(flint_dims(dtype=api.F32), 32) == api.UNSUPPORTED
    assert call(flint_dims(hidden=128), 32) == api.UNSUPPORTED
    assert call(flint_dims(inter=192, shared_inter=0), 32) == api.UNSUPPORTED
    assert call(flint_dims(shared_inter=768), 32) == api.UNSUPPORTED  # not a multiple of I = 512


def test_forward_rmsnorm_refusals(lib):
    """flint_moe_forward_rmsnorm makes flint_moe_forward's checks, then its own:
    a norm output that is given, 16-byte aligned and clear of out, and eps >= 0."""
    d = flint_dims()
    need = api.flint_moe_workspace_bytes(d, 32)
    w = _lib.Weights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    norm_ok = 0x200000  # clear of out (32 x 2048 float32 from FAKE) and of the workspace

    def call(T, norm=norm_ok, eps=1e-6, ws_bytes=need, out=FAKE):
        return lib.flint_moe_forward_rmsnorm(ctypes.byref(d), T, FAKE, ctypes.byref(w), out, api.F32, norm, eps,
                                             None, None, FAKE_WS, ws_bytes, None, None)
    assert call(-1) == api.INVALID_ARG
    assert call(0, norm=None) == api.OK  # no-op, nothing launched
    assert call(32, out=None) == api.INVALID_ARG
    assert call(32, norm=None) == api.INVALID_ARG
    assert call(32, norm=norm_ok + 8) == api.UNSUPPORTED  # misaligned
    assert call(32, eps=-1.0) == api.INVALID_ARG
    assert call(32, eps=float("nan")) == api.INVALID_ARG
    assert call(32, ws_bytes=need - 1) == api.WORKSPACE_TOO_SMALL
    assert call(32, norm=FAKE + 0x10000) == api.INVALID_ARG  # inside out
    assert call(32, norm=FAKE - 0x10000 + 16) == api.INVALID_ARG  # runs into out
