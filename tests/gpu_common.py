"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same inputs, and compare under the stated bars.

Bars (the layer's own tolerances):
  - routing indices and the dispatch permutation: bit-exact, except tokens whose
    K-th and (K+1)-th oracle scores are closer than 1e-5 (either set is correct
    there); those are counted, and their outputs are checked against the oracle
    recomputed with the GPU's set;
  - routing weights: |gpu - oracle| <= 2e-6 (float32 scores from different
    accumulation orders of the same dot product);
  - layer outputs (bf16 inputs, fp32 accumulation): max |gpu - oracle| <= 1e-2 *
    rms(oracle output).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as orc
from routed_expert_ffn_flint_amd import api, inputs

OUT_TOL = 1e-2       # max |delta| / rms(oracle)
WEIGHT_TOL = 2e-6
TIE_GAP = 1e-5       # the near-tie threshold on the oracle's K-th / (K+1)-th scores


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X; none is visible"
    from routed_expert_ffn_flint_amd import _lib
    _lib.load()  # raises if the HIP library is missing: there is no fallback


def oracle_dims(wl):
    return orc.dims(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, wl.bf16)


def host_weights(w: dict, experts=None) -> dict:
    """Exact float32 host copies.  With ``experts`` given, only those experts'
    gate/up/down are copied (the rest stay zero pages): enough for an oracle run
    whose tokens select only those experts."""
    out = {"router": inputs.to_numpy_f32(w["router"]), "bias": inputs.to_numpy_f32(w.get("bias"))}
    for k in ("shared_gate", "shared_up", "shared_down"):
        out[k] = inputs.to_numpy_f32(w.get(k))
    for k in ("gate", "up", "down"):
        if experts is None:
            out[k] = inputs.to_numpy_f32(w[k])
        else:
            full = np.zeros(tuple(w[k].shape), np.float32)
            ex = torch.as_tensor(np.asarray(sorted(experts)), device=w[k].device, dtype=torch.long)
            if len(ex):
                full[ex.cpu().numpy()] = w[k].index_select(0, ex).float().cpu().numpy()
            out[k] = full
    return out


def host_weights_mx4(w: dict, experts=None) -> dict:
    """MXFP4 weights (tiled codes and scales on the device) decoded by the oracle
    into float32 host arrays; with ``experts`` given, only those experts'
    matrices (the rest stay zero), as in host_weights."""
    out = {"router": inputs.to_numpy_f32(w["router"]), "bias": inputs.to_numpy_f32(w.get("bias"))}
    for k in ("shared_gate", "shared_up", "shared_down"):
        if w.get(k + "_q") is not None:
            out[k] = orc.mx4_dequant_tiled(w[k + "_q"].cpu().numpy(), w[k + "_s"].cpu().numpy())
    for k in ("gate", "up", "down"):
        q, sc = w[k + "_q"], w[k + "_s"]
        E, RB, KB = q.shape[:3]
        shape = (E, RB * 16, KB * 32)
        if experts is None:
            out[k] = orc.mx4_dequant_tiled(q.cpu().numpy(), sc.cpu().numpy())
        else:
            full = np.zeros(shape, np.float32)
            ex = torch.as_tensor(np.asarray(sorted(experts)), device=q.device, dtype=torch.long)
            if len(ex):
                full[ex.cpu().numpy()] = orc.mx4_dequant_tiled(q.index_select(0, ex).cpu().numpy(),
                                                                sc.index_select(0, ex).cpu().numpy())
            out[k] = full
    return out


def parity_mx4(wl, w_dev, x_dev, out_dtype=torch.float32):
    """Every token of an MXFP4 layer against the oracle run on the decoded weights."""
    out, idx, tw = gpu_layer(wl, w_dev, x_dev, out_dtype)
    d = oracle_dims(wl)
    xh = inputs.to_numpy_f32(x_dev)
    router = inputs.to_numpy_f32(w_dev["router"])
    bias = inputs.to_numpy_f32(w_dev.get("bias"))
    o_idx, o_w, tie = orc.route(d, xh, router, bias)
    gi, gw = idx.cpu().numpy(), tw.cpu().numpy()
    nties = check_routing(gi, gw, o_idx, o_w, tie, wl.name, scores_fn(d, xh, router, bias))
    wh = host_weights_mx4(w_dev, set(gi.ravel().tolist()))
    ref, _, _, _ = orc.forward(d, xh, wh, force_idx=gi)
    rel = check_output(out.float().cpu().numpy(), ref, wl.name)
    return {"near_ties": nties, "rel_err": rel, "idx": gi, "out": out}


def check_routing(gpu_idx, gpu_w, ora_idx, ora_w, near_tie, where="", scores_of=None):
    """Returns the number of near-tie tokens whose sets differ.

    Tokens whose GPU set equals the oracle's: weights within WEIGHT_TOL.  A
    token whose set differs must be a near tie (oracle K-th and (K+1)-th scores
    closer than TIE_GAP), and the GPU's set must itself be a correct answer,
    decided on the oracle's float32 scores (``scores_of(rows)`` returns them,
    [len(rows), E]): every selected score at least every unselected one minus
    TIE_GAP; the experts in one set and not the other all within TIE_GAP of the
    oracle's K-th score; and the GPU's weights equal to the scores renormalised
    over the GPU's own set (1/K each if they sum to 0)."""
    gpu_idx = np.asarray(gpu_idx)
    ora_idx = np.asarray(ora_idx)
    gpu_w = np.asarray(gpu_w)
    K = gpu_idx.shape[1]
    differ = np.any(gpu_idx != ora_idx, axis=1)
    bad = differ & ~np.asarray(near_tie)
    assert not bad.any(), (f"{where}: {int(bad.sum())} tokens route differently without a near tie, "
                           f"first {np.nonzero(bad)[0][:5].tolist()}")
    # every GPU row: K distinct ascending experts
    assert np.all(np.diff(gpu_idx, axis=1) > 0), f"{where}: rows not strictly ascending"
    same = ~differ
    if same.any():
        dw = np.abs(gpu_w[same] - np.asarray(ora_w)[same])
        assert dw.max() <= WEIGHT_TOL, f"{where}: routing weight off by {dw.max():.3g}"
    np.testing.assert_allclose(np.asarray(gpu_w, np.float64).sum(1), 1.0, atol=2e-6)
    rows = np.nonzero(differ)[0]
    if len(rows):
        assert scores_of is not None, f"{where}: tokens differ; their oracle scores are needed to check them"
        sc = np.asarray(scores_of(rows), np.float64)
        E = sc.shape[1]
        for j, t in enumerate(rows):
            s = sc[j]
            sel = gpu_idx[t]
            assert sel.min() >= 0 and sel.max() < E, f"{where}: token {t}: expert id out of range"
            mask = np.zeros(E, bool)
            mask[sel] = True
            s_k = np.sort(s)[::-1][K - 1]
            if K < E:
                assert s[mask].min() >= s[~mask].max() - TIE_GAP, (
                    f"{where}: token {t}: GPU set {sel.tolist()} is not a top-{K} set "
                    f"(selected min {s[mask].min():.9g} < unselected max {s[~mask].max():.9g} - {TIE_GAP})")
            swapped = np.setxor1d(sel, ora_idx[t])
            assert np.all(np.abs(s[swapped] - s_k) < TIE_GAP), (
                f"{where}: token {t}: experts {swapped.tolist()} differ from the oracle's set but are not "
                f"within {TIE_GAP} of the K-th score")
            tot = s[sel].sum()
            ref_w = s[sel] / tot if tot > 0 else np.full(K, 1.0 / K)
            dw = np.max(np.abs(gpu_w[t] - ref_w))
            assert dw <= WEIGHT_TOL, f"{where}: token {t}: weights off by {dw:.3g} on the GPU's own set"
    return int(differ.sum())


def scores_fn(d, xh, router, bias):
    """scores_of(rows) for check_routing: the oracle's float32 scores of those tokens."""
    return lambda rows: orc.scores(d, np.asarray(xh)[np.asarray(rows)], router, bias)


def check_output(gpu_out, ora_out, where=""):
    g = np.asarray(gpu_out, np.float64)
    o = np.asarray(ora_out, np.float64)
    assert np.all(np.isfinite(g)), f"{where}: non-finite GPU output"
    rms = float(np.sqrt(np.mean(o * o)))
    err = float(np.max(np.abs(g - o))) if g.size else 0.0
    assert err <= OUT_TOL * rms, f"{where}: max|delta| = {err:.4g} = {err / rms:.3g} rms (bar {OUT_TOL})"
    return err / rms if rms > 0 else 0.0


def gpu_layer(wl, w, x, out_dtype=torch.float32):
    d = api.dims_of(wl)
    out, idx, tw = api.forward(d, x, w, out_dtype=out_dtype, return_routing=True)
    torch.cuda.synchronize()
    return out, idx, tw


def parity_full(wl, w_dev, x_dev, out_dtype=torch.float32):
    """Whole-batch parity against the oracle on every token.  Returns stats."""
    out, idx, tw = gpu_layer(wl, w_dev, x_dev, out_dtype)
    d = oracle_dims(wl)
    wh = host_weights(w_dev)
    xh = inputs.to_numpy_f32(x_dev)
    o_idx, o_w, tie = orc.route(d, xh, wh["router"], wh["bias"])
    gi, gw = idx.cpu().numpy(), tw.cpu().numpy()
    nties = check_routing(gi, gw, o_idx, o_w, tie, wl.name, scores_fn(d, xh, wh["router"], wh["bias"]))
    ref, _, _, _ = orc.forward(d, xh, wh, force_idx=gi)
    if out_dtype == torch.bfloat16:
        # compare against the oracle rounded the same way, with one bf16 ulp of slack
        refb = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
        g = out.float().cpu().numpy()
        ulp = np.abs(refb) * 2.0 ** -7 + 1e-30
        assert np.all(np.abs(g - refb) <= ulp), f"{wl.name}: bf16 output off by more than one ulp"
        rel = float(np.max(np.abs(g - ref)) / np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    else:
        rel = check_output(out.cpu().numpy(), ref, wl.name)
    return {"near_ties": nties, "rel_err": rel, "idx": gi}


def parity_sampled(wl, w_dev, x_dev, sample, out_dtype=torch.float32):
    """Full-size parity: routing of every token (exact, near ties exempt) and the
    outputs of the sampled tokens, each recomputed by the oracle one by one."""
    out, idx, tw = gpu_layer(wl, w_dev, x_dev, out_dtype)
    d = oracle_dims(wl)
    xh = inputs.to_numpy_f32(x_dev)
    router = inputs.to_numpy_f32(w_dev["router"])
    bias = inputs.to_numpy_f32(w_dev.get("bias"))
    o_idx, o_w, tie = orc.route(d, xh, router, bias)
    gi, gw = idx.cpu().numpy(), tw.cpu().numpy()
    nties = check_routing(gi, gw, o_idx, o_w, tie, wl.name, scores_fn(d, xh, router, bias))
    sample = np.asarray(sorted(set(int(t) for t in sample)))
    experts = set(gi[sample].ravel().tolist())
    wh = host_weights(w_dev, experts)
    ref, _, _, _ = orc.forward(d, xh[sample], wh, force_idx=gi[sample])
    rel = check_output(out.float().cpu().numpy()[sample], ref, wl.name + " (sampled)")
    return {"near_ties": nties, "rel_err": rel, "idx": gi, "w": gw, "out": out}
