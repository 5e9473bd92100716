"""Dense-mixture brute force, used only to pin the oracle on tiny shapes.

A second, independent formulation of the same layer, written with numpy in
float64 and shaped differently from the oracle on purpose: every expert is run
on every token, and the routing enters only as a dense gate vector that is zero
outside the selected set,

    out[t] = sum_e  gate[t, e] * expert_e(x_t)  +  shared(x_t),
    gate[t, e] = s_e / sum_{j in S_t} s_j  if e in S_t else 0,

so there is no dispatch, no permutation and no per-token expert list.  Selection
uses numpy's lexicographic sort on (-score, expert id).  The bf16 rounding of the
intermediate uses numpy's frexp/rint on float64 values.
"""
from __future__ import annotations

import numpy as np


def bf16_round(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    m, ex = np.frexp(a)                      # a = m * 2**ex, 0.5 <= |m| < 1
    ulp_exp = np.maximum(ex - 8, -133)
    return np.where(a == 0, a, np.ldexp(np.rint(np.ldexp(a, -ulp_exp)), ulp_exp))


def _silu(g):
    return g / (1.0 + np.exp(-g))


def routing(x, router, bias, top_k):
    """Float32 scores, the selected sets (ascending) and the dense gate matrix."""
    x = np.asarray(x, np.float64)
    z = (x @ np.asarray(router, np.float64).T)
    if bias is not None:
        z = z + np.asarray(bias, np.float64)[None, :]
    z = z.astype(np.float32)
    s = (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)
    T, E = s.shape
    sets = np.zeros((T, top_k), np.int64)
    gate = np.zeros((T, E), np.float64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -s[t].astype(np.float64)))
        chosen = np.sort(order[:top_k])
        sets[t] = chosen
        tot = np.sum(s[t, chosen].astype(np.float64))
        gate[t, chosen] = (s[t, chosen].astype(np.float64) / tot).astype(np.float32)
    return s, sets, gate


def expert_all_tokens(x, wg, wu, wd, h_bf16: bool):
    x = np.asarray(x, np.float64)
    g = x @ np.asarray(wg, np.float64).T            # [T, width]
    u = x @ np.asarray(wu, np.float64).T
    h = _silu(g) * u
    h = bf16_round(h) if h_bf16 else h.astype(np.float32).astype(np.float64)
    return h @ np.asarray(wd, np.float64).T         # [T, H]


def layer(x, w: dict, top_k: int, h_bf16: bool):
    """Returns (out float32 [T,H], sets [T,K], gate [T,E])."""
    s, sets, gate = routing(x, w["router"], w.get("bias"), top_k)
    E = np.asarray(w["router"]).shape[0]
    x64 = np.asarray(x, np.float64)
    acc = np.zeros((x64.shape[0], x64.shape[1]), np.float64)
    for e in range(E):
        y = expert_all_tokens(x64, w["gate"][e], w["up"][e], w["down"][e], h_bf16)
        acc += gate[:, e:e + 1] * y
    if w.get("shared_gate") is not None:
        acc += expert_all_tokens(x64, w["shared_gate"], w["shared_up"], w["shared_down"], h_bf16)
    return acc.astype(np.float32), sets, gate
