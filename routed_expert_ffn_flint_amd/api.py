"""Python binding of the Flint MoE C ABI (argument marshalling only).

Function names match the C entry points in include/flint_moe.h.  Tensors are
torch tensors on the GPU; the binding checks their device, dtype, shape and
contiguity, passes their data pointers and the current (or given) stream, and
raises FlintError on any status other than FLINT_OK.  Every computation runs in
the library's HIP kernels.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import DenseDims, Dims, Weights, WeightsMx4, load

OK, INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, DEVICE_ERROR = 0, 1, 2, 3, 4
F32, BF16 = 0, 1


class FlintError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {flint_status_string(status)} (status {status})")


def flint_status_string(status: int) -> str:
    return load().flint_status_string(int(status)).decode()


def make_dims(hidden, n_experts, top_k, inter, shared_inter, dtype) -> Dims:
    if isinstance(dtype, torch.dtype):
        dtype = BF16 if dtype == torch.bfloat16 else F32 if dtype == torch.float32 else -1
    return Dims(hidden, n_experts, top_k, inter, shared_inter, dtype)


def dims_of(wl) -> Dims:
    """Dims of an inputs.Workload."""
    return make_dims(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, BF16 if wl.bf16 else F32)


def dense_dims_of(wl) -> DenseDims:
    """DenseDims of a dense workload (inputs.Workload with dense=True)."""
    return DenseDims(hidden=wl.hidden, inter=wl.inter, dtype=BF16 if wl.bf16 else F32)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check_tensor(name, t, dtype=None, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _elem(d: Dims):
    return torch.bfloat16 if d.dtype == BF16 else torch.float32


def flint_moe_workspace_bytes(d: Dims, T: int) -> int:
    return int(load().flint_moe_workspace_bytes(ctypes.byref(d), int(T)))


def workspace(d: Dims, T: int, device="cuda") -> torch.Tensor:
    """A workspace tensor of the size the library asks for (torch allocates it)."""
    n = flint_moe_workspace_bytes(d, T)
    if n == 0 and T > 0:
        raise FlintError(UNSUPPORTED, "flint_moe_workspace_bytes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def flint_moe_route(d: Dims, x, router, router_bias, topk_idx, topk_w, ws, stream=None):
    T = x.shape[0]
    _check_tensor("x", x, _elem(d), (T, d.hidden))
    _check_tensor("router", router, _elem(d), (d.n_experts, d.hidden))
    _check_tensor("router_bias", router_bias, torch.float32, (d.n_experts,))
    _check_tensor("topk_idx", topk_idx, torch.int32, (T, d.top_k))
    _check_tensor("topk_w", topk_w, torch.float32, (T, d.top_k))
    _check_tensor("ws", ws, torch.uint8)
    st = load().flint_moe_route(ctypes.byref(d), T, _ptr(x), _ptr(router), _ptr(router_bias), _ptr(topk_idx),
                                _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream))
    if st != OK:
        raise FlintError(st, "flint_moe_route")


def flint_moe_dispatch(d: Dims, topk_idx, counts, offsets, sorted_token, slot_of, ws, stream=None):
    T = topk_idx.shape[0]
    _check_tensor("topk_idx", topk_idx, torch.int32, (T, d.top_k))
    _check_tensor("expert_counts", counts, torch.int32, (d.n_experts,))
    _check_tensor("expert_offsets", offsets, torch.int32, (d.n_experts + 1,))
    _check_tensor("sorted_token", sorted_token, torch.int32, (T * d.top_k,))
    _check_tensor("slot_of", slot_of, torch.int32, (T * d.top_k,))
    _check_tensor("ws", ws, torch.uint8)
    st = load().flint_moe_dispatch(ctypes.byref(d), T, _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                                   _ptr(sorted_token), _ptr(slot_of), _ptr(ws), ws.numel(), _stream(stream))
    if st != OK:
        raise FlintError(st, "flint_moe_dispatch")


def weights_struct(d: Dims, w: dict) -> Weights:
    el = _elem(d)
    E, H, I, Is = d.n_experts, d.hidden, d.inter, d.shared_inter
    _check_tensor("router", w["router"], el, (E, H))
    _check_tensor("router_bias", w.get("bias"), torch.float32, (E,))
    _check_tensor("gate", w["gate"], el, (E, I, H))
    _check_tensor("up", w["up"], el, (E, I, H))
    _check_tensor("down", w["down"], el, (E, H, I))
    if Is > 0:
        _check_tensor("shared_gate", w["shared_gate"], el, (Is, H))
        _check_tensor("shared_up", w["shared_up"], el, (Is, H))
        _check_tensor("shared_down", w["shared_down"], el, (H, Is))
    g = (lambda k: _ptr(w.get(k)) if Is > 0 else None)
    return Weights(_ptr(w["router"]), _ptr(w.get("bias")), _ptr(w["gate"]), _ptr(w["up"]), _ptr(w["down"]),
                   g("shared_gate"), g("shared_up"), g("shared_down"))


def flint_moe_forward(d: Dims, x, weights, out, topk_idx_out=None, topk_w_out=None, ws=None, stream=None,
                      events=None):
    """weights: a dict of tensors (see inputs.make_layer) or a prepared Weights struct.
    events: None, or 10 hipEvent_t handles (ints / c_void_p) -- then the call goes
    to flint_moe_forward_profiled, which stamps a start and a stop event around
    each of the five stages."""
    T = x.shape[0]
    _check_tensor("x", x, _elem(d), (T, d.hidden))
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _check_tensor("out", out, None, (T, d.hidden))
    _check_tensor("topk_idx_out", topk_idx_out, torch.int32, (T, d.top_k))
    _check_tensor("topk_w_out", topk_w_out, torch.float32, (T, d.top_k))
    _check_tensor("ws", ws, torch.uint8)
    ws_struct = weights if isinstance(weights, Weights) else weights_struct(d, weights)
    out_dt = BF16 if out.dtype == torch.bfloat16 else F32
    args = (ctypes.byref(d), T, _ptr(x), ctypes.byref(ws_struct), _ptr(out), out_dt, _ptr(topk_idx_out),
            _ptr(topk_w_out), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    if events is None:
        st = load().flint_moe_forward(*args)
    else:
        if len(events) != 10:
            raise ValueError("events: 10 hipEvent_t handles (start/stop of 5 stages)")
        arr = (ctypes.c_void_p * 10)(*[e.value if isinstance(e, ctypes.c_void_p) else e for e in events])
        st = load().flint_moe_forward_profiled(*args, arr)
    if st != OK:
        raise FlintError(st, "flint_moe_forward" if events is None else "flint_moe_forward_profiled")


def flint_moe_forward_fused(d: Dims, x, weights, out, topk_idx_out=None, topk_w_out=None, ws=None, stream=None,
                            events=None):
    """The layer through the persistent fused decode kernel (bf16, up to 64
    tokens; see include/flint_moe.h); arguments as flint_moe_forward, events
    None or 10 hipEvent_t handles."""
    T = x.shape[0]
    _check_tensor("x", x, _elem(d), (T, d.hidden))
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _check_tensor("out", out, None, (T, d.hidden))
    _check_tensor("topk_idx_out", topk_idx_out, torch.int32, (T, d.top_k))
    _check_tensor("topk_w_out", topk_w_out, torch.float32, (T, d.top_k))
    _check_tensor("ws", ws, torch.uint8)
    ws_struct = weights if isinstance(weights, Weights) else weights_struct(d, weights)
    out_dt = BF16 if out.dtype == torch.bfloat16 else F32
    arr = None
    if events is not None:
        if len(events) != 10:
            raise ValueError("events: 10 hipEvent_t handles (start/stop of 5 stages)")
        arr = (ctypes.c_void_p * 10)(*[e.value if isinstance(e, ctypes.c_void_p) else e for e in events])
    st = load().flint_moe_forward_fused(ctypes.byref(d), T, _ptr(x), ctypes.byref(ws_struct), _ptr(out), out_dt,
                                        _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws),
                                        0 if ws is None else ws.numel(), _stream(stream), arr)
    if st != OK:
        raise FlintError(st, "flint_moe_forward_fused")


def flint_moe_forward_static(d: Dims, x, weights, out, topk_idx_out=None, topk_w_out=None, stream=None):
    """flint_moe_forward without a workspace argument: the library's own static
    device scratch (FLINT_STATIC_SCRATCH_BYTES per GPU) serves as the workspace,
    and the call allocates nothing.  Calls that overlap on one GPU race."""
    T = x.shape[0]
    _check_tensor("x", x, _elem(d), (T, d.hidden))
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _check_tensor("out", out, None, (T, d.hidden))
    _check_tensor("topk_idx_out", topk_idx_out, torch.int32, (T, d.top_k))
    _check_tensor("topk_w_out", topk_w_out, torch.float32, (T, d.top_k))
    ws_struct = weights if isinstance(weights, Weights) else weights_struct(d, weights)
    out_dt = BF16 if out.dtype == torch.bfloat16 else F32
    st = load().flint_moe_forward_static(ctypes.byref(d), T, _ptr(x), ctypes.byref(ws_struct), _ptr(out), out_dt,
                                         _ptr(topk_idx_out), _ptr(topk_w_out), _stream(stream))
    if st != OK:
        raise FlintError(st, "flint_moe_forward_static")


def weights_mx4_struct(d: Dims, w: dict) -> WeightsMx4:
    """MXFP4 expert weights in the tiled order of flint_moe_forward_mx4 (keys
    <name>_q codes [..., rows/16, cols/32, 16, 16] and <name>_s scales [...,
    rows/16, cols/32, 16], uint8; see inputs.mx4_quantize and inputs.mx4_tile)
    plus the bf16 router and optional bias."""
    E, H, I, Is = d.n_experts, d.hidden, d.inter, d.shared_inter
    _check_tensor("router", w["router"], torch.bfloat16, (E, H))
    _check_tensor("router_bias", w.get("bias"), torch.float32, (E,))
    shapes = {"gate": (E, I, H), "up": (E, I, H), "down": (E, H, I)}
    if Is > 0:
        shapes.update({"shared_gate": (Is, H), "shared_up": (Is, H), "shared_down": (H, Is)})
    ptrs = {}
    for name, shp in shapes.items():
        tiles = shp[:-2] + (shp[-2] // 16, shp[-1] // 32, 16)
        _check_tensor(name + "_q", w[name + "_q"], torch.uint8, tiles + (16,))
        _check_tensor(name + "_s", w[name + "_s"], torch.uint8, tiles)
        ptrs[name + "_q"], ptrs[name + "_s"] = _ptr(w[name + "_q"]), _ptr(w[name + "_s"])
    return WeightsMx4(router=_ptr(w["router"]), router_bias=_ptr(w.get("bias")), **ptrs)


def flint_moe_forward_mx4(d: Dims, x, weights, out, topk_idx_out=None, topk_w_out=None, ws=None, stream=None,
                          events=None):
    """flint_moe_forward with MXFP4 expert weights: ``weights`` is a dict (see
    weights_mx4_struct) or a prepared WeightsMx4; events as in flint_moe_forward."""
    T = x.shape[0]
    _check_tensor("x", x, torch.bfloat16, (T, d.hidden))
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _check_tensor("out", out, None, (T, d.hidden))
    _check_tensor("topk_idx_out", topk_idx_out, torch.int32, (T, d.top_k))
    _check_tensor("topk_w_out", topk_w_out, torch.float32, (T, d.top_k))
    _check_tensor("ws", ws, torch.uint8)
    ws_struct = weights if isinstance(weights, WeightsMx4) else weights_mx4_struct(d, weights)
    out_dt = BF16 if out.dtype == torch.bfloat16 else F32
    arr = None
    if events is not None:
        if len(events) != 10:
            raise ValueError("events: 10 hipEvent_t handles (start/stop of 5 stages)")
        arr = (ctypes.c_void_p * 10)(*[e.value if isinstance(e, ctypes.c_void_p) else e for e in events])
    st = load().flint_moe_forward_mx4(ctypes.byref(d), T, _ptr(x), ctypes.byref(ws_struct), _ptr(out), out_dt,
                                      _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(stream), arr)
    if st != OK:
        raise FlintError(st, "flint_moe_forward_mx4")


def flint_dense_workspace_bytes(dd: DenseDims, T: int) -> int:
    return int(load().flint_dense_workspace_bytes(ctypes.byref(dd), int(T)))


def dense_workspace(dd: DenseDims, T: int, device="cuda") -> torch.Tensor:
    n = flint_dense_workspace_bytes(dd, T)
    if n == 0 and T > 0:
        raise FlintError(UNSUPPORTED, "flint_dense_workspace_bytes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def flint_dense_mlp(dd: DenseDims, x, gate, up, down, out, ws, stream=None, events=None):
    """The dense gated MLP layer: x [T, H], gate/up [I, H], down [H, I] in
    dd.dtype; out [T, H] float32 or bfloat16; events: None or 6 hipEvent_t
    handles (start/stop of gate/up, down, output)."""
    T = x.shape[0]
    el = torch.bfloat16 if dd.dtype == BF16 else torch.float32
    _check_tensor("x", x, el, (T, dd.hidden))
    _check_tensor("gate", gate, el, (dd.inter, dd.hidden))
    _check_tensor("up", up, el, (dd.inter, dd.hidden))
    _check_tensor("down", down, el, (dd.hidden, dd.inter))
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _check_tensor("out", out, None, (T, dd.hidden))
    _check_tensor("ws", ws, torch.uint8)
    arr = None
    if events is not None:
        if len(events) != 6:
            raise ValueError("events: 6 hipEvent_t handles (start/stop of 3 stages)")
        arr = (ctypes.c_void_p * 6)(*[e.value if isinstance(e, ctypes.c_void_p) else e for e in events])
    st = load().flint_dense_mlp(ctypes.byref(dd), T, _ptr(x), _ptr(gate), _ptr(up), _ptr(down), _ptr(out),
                                BF16 if out.dtype == torch.bfloat16 else F32, _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream), arr)
    if st != OK:
        raise FlintError(st, "flint_dense_mlp")


def dense_mlp(x, gate, up, down, out_dtype=torch.float32, ws=None, stream=None):
    """Allocates the output (and workspace) and runs flint_dense_mlp."""
    T, H = x.shape
    dd = DenseDims(hidden=H, inter=gate.shape[0], dtype=BF16 if x.dtype == torch.bfloat16 else F32)
    out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    if ws is None:
        ws = dense_workspace(dd, T, x.device)
    flint_dense_mlp(dd, x, gate, up, down, out, ws, stream)
    return out


def flint_moe_forward_rmsnorm(d: Dims, x, weights, out, norm_out, eps=1e-6, topk_idx_out=None, topk_w_out=None,
                              ws=None, stream=None, events=None):
    """The layer (as flint_moe_forward) and, in its combine, RMSNorm of its
    float32 output into norm_out ([T][H] bfloat16; it may be x itself, not out);
    events as in flint_moe_forward."""
    T = x.shape[0]
    _check_tensor("x", x, _elem(d), (T, d.hidden))
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _check_tensor("out", out, None, (T, d.hidden))
    _check_tensor("norm_out", norm_out, torch.bfloat16, (T, d.hidden))
    _check_tensor("topk_idx_out", topk_idx_out, torch.int32, (T, d.top_k))
    _check_tensor("topk_w_out", topk_w_out, torch.float32, (T, d.top_k))
    _check_tensor("ws", ws, torch.uint8)
    ws_struct = weights if isinstance(weights, Weights) else weights_struct(d, weights)
    out_dt = BF16 if out.dtype == torch.bfloat16 else F32
    arr = None
    if events is not None:
        if len(events) != 10:
            raise ValueError("events: 10 hipEvent_t handles (start/stop of 5 stages)")
        arr = (ctypes.c_void_p * 10)(*[e.value if isinstance(e, ctypes.c_void_p) else e for e in events])
    st = load().flint_moe_forward_rmsnorm(ctypes.byref(d), T, _ptr(x), ctypes.byref(ws_struct), _ptr(out), out_dt,
                                          _ptr(norm_out), float(eps), _ptr(topk_idx_out), _ptr(topk_w_out),
                                          _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream), arr)
    if st != OK:
        raise FlintError(st, "flint_moe_forward_rmsnorm")


def flint_rmsnorm(inp, out, eps=1e-6, stream=None):
    T, H = inp.shape
    _check_tensor("in", inp, torch.float32, (T, H))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    st = load().flint_rmsnorm(T, H, _ptr(inp), _ptr(out), float(eps), _stream(stream))
    if st != OK:
        raise FlintError(st, "flint_rmsnorm")


# ---- convenience: allocate outputs with torch, then call the entry points ----

def forward(d: Dims, x, weights, out_dtype=torch.float32, ws=None, stream=None, return_routing=False,
            fused=False):
    """The layer; MXFP4 weight dicts (keys ending in _q/_s) go to flint_moe_forward_mx4,
    fused=True to flint_moe_forward_fused."""
    T = x.shape[0]
    out = torch.empty((T, d.hidden), dtype=out_dtype, device=x.device)
    idx = torch.empty((T, d.top_k), dtype=torch.int32, device=x.device) if return_routing else None
    tw = torch.empty((T, d.top_k), dtype=torch.float32, device=x.device) if return_routing else None
    if ws is None:
        ws = workspace(d, T, x.device)
    if isinstance(weights, WeightsMx4) or (isinstance(weights, dict) and "gate_q" in weights):
        flint_moe_forward_mx4(d, x, weights, out, idx, tw, ws, stream)
    elif fused:
        flint_moe_forward_fused(d, x, weights, out, idx, tw, ws, stream)
    else:
        flint_moe_forward(d, x, weights, out, idx, tw, ws, stream)
    return (out, idx, tw) if return_routing else out


def forward_rmsnorm(d: Dims, x, weights, eps=1e-6, out_dtype=torch.float32, ws=None, stream=None):
    """The layer and the RMSNorm of its float32 output (flint_moe_forward_rmsnorm):
    returns (out, norm_out)."""
    T = x.shape[0]
    out = torch.empty((T, d.hidden), dtype=out_dtype, device=x.device)
    norm = torch.empty((T, d.hidden), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = workspace(d, T, x.device)
    flint_moe_forward_rmsnorm(d, x, weights, out, norm, eps, ws=ws, stream=stream)
    return out, norm


def route(d: Dims, x, router, bias=None, ws=None, stream=None):
    T = x.shape[0]
    idx = torch.empty((T, d.top_k), dtype=torch.int32, device=x.device)
    tw = torch.empty((T, d.top_k), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(d, T, x.device)
    flint_moe_route(d, x, router, bias, idx, tw, ws, stream)
    return idx, tw


def dispatch(d: Dims, topk_idx, ws=None, stream=None):
    T = topk_idx.shape[0]
    dev = topk_idx.device
    counts = torch.empty((d.n_experts,), dtype=torch.int32, device=dev)
    offsets = torch.empty((d.n_experts + 1,), dtype=torch.int32, device=dev)
    st = torch.empty((T * d.top_k,), dtype=torch.int32, device=dev)
    so = torch.empty((T * d.top_k,), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(d, T, dev)
    flint_moe_dispatch(d, topk_idx, counts, offsets, st, so, ws, stream)
    return counts, offsets, st, so


def rmsnorm(inp, eps=1e-6, stream=None):
    out = torch.empty(inp.shape, dtype=torch.bfloat16, device=inp.device)
    flint_rmsnorm(inp, out, eps, stream)
    return out
