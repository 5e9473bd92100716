"""GPU parity: the HIP path, called through the C ABI, against the oracle.

Small cases run the oracle on every token, with shapes chosen to span several
tiles and leave ragged tails (T not a multiple of the 16/32/128-row tiles or the
256-token dispatch tile; expert counts that are not multiples of 16).  The
named workloads run at full size: routing of every token is checked, the
dispatch permutation is checked bit for bit, and the outputs of every token
(prefill4096, skew16384, seven whole layers of stack47) or of sampled tokens
(the rest) are recomputed by the oracle.  Batches whose intermediate arrays
pass 2^31 elements check the 64-bit offsets.  Calls captured in HIP graphs and
replayed, and calls on two streams at once, must equal eager calls bit for
bit.  Router logits pushed far outside their usual range check the sigmoid's
saturated, subnormal and underflowing scores.  Bars are in gpu_common.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gpu_common as G
import oracle_pins
from oracle import oracle as orc
from routed_expert_ffn_flint_amd import api, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()
    yield
    torch.cuda.synchronize()


def _layer(wl, device="cuda"):
    # small layers are drawn on the CPU generator and copied, large ones drawn on the GPU
    if wl.n_experts * wl.inter * wl.hidden <= (1 << 24):
        w = inputs.make_layer(wl, 0, "cpu")
        w = {k: (v.to(device) if v is not None else None) for k, v in w.items()}
        x = inputs.make_tokens(wl, device="cpu").to(device)
    else:
        w = inputs.make_layer(wl, 0, device)
        x = inputs.make_tokens(wl, device=device)
    return w, x


SMALL = [
    # name,       T,  H,   E,  K, I,   Is,  bf16,  bias
    ("t1",        1,  128, 16, 2, 64,  64,  True,  False),
    ("t5_noshr",  5,  64,  8,  3, 64,  0,   True,  False),
    ("t17_e20",   17, 192, 20, 3, 128, 64,  True,  True),
    ("t33",       33, 256, 32, 6, 64,  128, True,  False),
    ("t24_s4",    24, 256, 16, 2, 64,  256, True,  False),   # shared down split 4 ways
    ("t40_kE",    40, 128, 8,  8, 64,  64,  True,  False),
    ("t24_e256_k8", 24, 2048, 256, 8, 512, 1024, True, True),  # the most experts and the largest K
    ("t64_k1",    64, 128, 16, 1, 128, 64,  True,  True),
    ("t100_f32",  100, 128, 24, 4, 64, 128, False, True),
    # the largest batch whose top-k and dispatch run as one launch, and the next
    ("t128_flint", 128, 2048, 256, 6, 512, 1024, True, False),
    ("t129",      129, 256, 64, 6, 128, 128, True, True),
    ("t300",      300, 256, 64, 6, 128, 128, True, False),   # two dispatch tiles, 16-row tiles
    ("t600_f32",  600, 128, 16, 2, 64, 64,  False, False),
    ("t1100",     1100, 256, 32, 4, 64, 128, True, True),    # tiled expert kernels, large router
    ("t700_mid",  700, 256, 128, 4, 128, 128, True, False),  # 64-row gate/up and down tiles
    ("t480_dmid", 480, 256, 128, 4, 128, 128, True, True),   # 16-row gate/up tiles, 64-row down tiles
    ("t600_midg", 600, 256, 64, 4, 128, 256, True, True),    # 64-row gate/up tiles, 128-row down tiles
    ("t640_midn", 640, 256, 64, 4, 192, 64, True, False),    # 64-row gate/up tiles of 128 columns (widths not whole 256-column tiles)
    ("t1024_flint", 1024, 2048, 256, 6, 512, 1024, True, False),  # the Flint shape on 64-row gate/up and down tiles
    ("t2100_big", 2100, 256, 16, 4, 128, 128, True, True),   # 256-row tiles, router split over H
    ("t5000_ns",  5000, 128, 8,  2, 128, 0,   True, False),  # 256-row tiles, no shared expert
    # the fused decode kernel (bf16, T <= 64, H and I multiples of 256, Is a multiple of I)
    ("fz_t7",       7,   512, 24, 3, 256, 512, True, True),
    ("fz_t1_k1",    1,   256, 8,  1, 256, 256, True, False),
    ("fz_t64_k8",   64,  1024, 64, 8, 256, 0,  True, False),   # no shared expert, every queue busy
    ("fz_t40_e200", 40,  768, 200, 6, 512, 1024, True, True),  # E not a multiple of 16, H = 3 x 256
    ("fz_t19_s4",   19,  512, 32, 4, 256, 1024, True, False),  # four shared slices
    ("fz_t2_e256",  2,   2048, 256, 6, 512, 1024, True, False),  # most queues hold one unit or none
    # float32 layers on the weight-streaming kernels (H, I, Is multiples of 256)
    ("t40_f32_st",  40,  256, 16, 2, 256, 512, False, False),
    ("t200_f32_st", 200, 512, 32, 6, 256, 256, False, True),
    ("t512_f32_st", 512, 256, 16, 4, 256, 256, False, False),  # the largest float32 streaming batch
]


FUSED = [c for c in SMALL if c[0].startswith("fz_")] + [
    # name,      T,  H,    E,   K, I,   Is,   bf16, bias
    ("fz_flint1",  1,  2048, 256, 6, 512, 1024, True, False),
    ("fz_flint8",  8,  2048, 256, 6, 512, 1024, True, True),
    ("fz_flint32", 32, 2048, 256, 6, 512, 1024, True, False),
    ("fz_flint64", 64, 2048, 256, 6, 512, 1024, True, False),  # the largest fused batch
]


@pytest.mark.parametrize("case", FUSED, ids=[c[0] for c in FUSED])
def test_fused_entry_point_equals_forward(case):
    """flint_moe_forward_fused (top-k through down in one persistent kernel)
    gives flint_moe_forward's bits (routing and outputs), and those are the
    oracle's on every token."""
    name, T, H, E, K, I, Is, bf16, bias = case
    wl = inputs.custom(name, T, H, E, K, I, Is, bf16, seed=6, zipf=bias)
    w, x = _layer(wl)
    d = api.dims_of(wl)
    ref = api.forward(d, x, w, return_routing=True)
    got = api.forward(d, x, w, return_routing=True, fused=True)
    torch.cuda.synchronize()
    for r, g, what in zip(ref, got, ("out", "topk_idx", "topk_w")):
        assert torch.equal(r.view(torch.uint8), g.view(torch.uint8)), f"{name}: fused {what} differs"
    st = G.parity_full(wl, w, x)
    print(f"{name}: fused == forward, rel_err={st['rel_err']:.3g} near_ties={st['near_ties']}")


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_forward_small_every_token(case):
    name, T, H, E, K, I, Is, bf16, bias = case
    wl = inputs.custom(name, T, H, E, K, I, Is, bf16, seed=3, zipf=bias)
    w, x = _layer(wl)
    st = G.parity_full(wl, w, x)
    print(f"{name}: rel_err={st['rel_err']:.3g} near_ties={st['near_ties']}")


def test_forward_bf16_output():
    wl = inputs.custom("bf16out", 48, 256, 16, 4, 64, 64, True, seed=4)
    w, x = _layer(wl)
    G.parity_full(wl, w, x, out_dtype=torch.bfloat16)


def test_toy_workload():
    wl = inputs.WORKLOADS["toy"]
    w, x = _layer(wl)
    st = G.parity_full(wl, w, x)
    assert st["rel_err"] < 1e-4  # fp32 throughout: far inside the bar
    print(f"toy: rel_err={st['rel_err']:.3g}")


def test_decode32_every_token():
    wl = inputs.WORKLOADS["decode32"]
    w, x = _layer(wl)
    st = G.parity_full(wl, w, x)
    print(f"decode32: rel_err={st['rel_err']:.3g} near_ties={st['near_ties']} "
          f"distinct experts={len(np.unique(st['idx']))}")


@pytest.mark.parametrize("T", [1, 5, 16, 17, 33, 159, 160, 256, 257, 512, 513])
def test_flint_layer_small_batches(T):
    """Flint-shaped layer (H=2048, 256 experts top-6, 512/1024 wide) at batch
    sizes around the kernels' boundaries (weight streaming up to 159 tokens,
    16-row tiles from 160 to 512, the large tiles from 513; up to 16 tokens
    top-k and dispatch share one work-group, up to 256 the dispatch is one
    work-group): routing and outputs of every token."""
    wl = inputs.Workload(f"flint_T{T}", T, 2048, 256, 6, 512, 1024, True, 5)
    w, x = _layer(wl)
    st = G.parity_sampled(wl, w, x, list(range(T)))
    _check_dispatch_of(wl, st["idx"])
    print(f"flint T={T}: rel_err={st['rel_err']:.3g} near_ties={st['near_ties']}")


def _check_dispatch_of(wl, gi):
    d = api.dims_of(wl)
    idx_dev = torch.from_numpy(gi).to("cuda")
    counts, offsets, st_, so = [t.cpu().numpy() for t in api.dispatch(d, idx_dev)]
    torch.cuda.synchronize()
    oc, oo, ost, oso = orc.dispatch(G.oracle_dims(wl), gi)
    np.testing.assert_array_equal(counts, oc)
    np.testing.assert_array_equal(offsets, oo)
    np.testing.assert_array_equal(st_, ost)
    np.testing.assert_array_equal(so, oso)
    return counts


@pytest.mark.parametrize("T", [5, 600])
def test_largest_supported_shape(T):
    """The largest widths the library takes (H = 8192, I = Is = 4096, K = 8; 32
    experts to bound the memory): T = 5 on the streaming kernels (every
    token), T = 600 on the tiled kernels (routing of every token, outputs of
    sampled ones)."""
    wl = inputs.Workload(f"max_T{T}", T, 8192, 32, 8, 4096, 4096, True, 9)
    w, x = _layer(wl)
    # (T = 600: 40 tokens spread over the batch and its two ends; the oracle
    # spends ~2 GFLOP in double on each token of this shape)
    sample = list(range(T)) if T <= 8 else sorted(set(np.linspace(0, T - 1, 40).astype(int).tolist()) | {1, T - 2})
    st = G.parity_sampled(wl, w, x, sample)
    print(f"max_T{T}: rel_err={st['rel_err']:.3g} near_ties={st['near_ties']}")


@pytest.mark.parametrize("name", ["prefill4096", "skew16384"])
def test_full_size_layer_every_token(name):
    """The prefill and skewed workloads at full size: routing, dispatch and the
    output of every token against the oracle (every row tile and n-tile of the
    tiled kernels, the hot experts' many row tiles included)."""
    wl = inputs.WORKLOADS[name]
    w, x = _layer(wl)
    st = G.parity_full(wl, w, x)
    counts = _check_dispatch_of(wl, st["idx"])
    mean = counts.mean()
    print(f"{name}: every token, rel_err={st['rel_err']:.3g} near_ties={st['near_ties']} max/mean load "
          f"{counts.max() / mean:.1f} min {counts.min()} experts>10x mean {(counts > 10 * mean).sum()}")
    if wl.zipf_bias:
        assert counts.max() > 10 * mean  # the skewed workload really is skewed


def test_routed_outputs_past_2_31_elements():
    """A Flint-shape batch whose routed outputs [T*K, H] span more than 2^31
    float32 elements (T = 180000: 1.08 M slots of 2048).  The dispatch
    permutation is checked bit for bit; the routing and outputs of sampled
    tokens are recomputed by the oracle.  The sample includes tokens whose
    slots lie past element 2^31, where a 32-bit offset would wrap."""
    T = 180_000
    wl = dataclasses.replace(inputs.WORKLOADS["prefill4096"], name="flint_T180000", T=T)
    K, H = wl.top_k, wl.hidden
    assert T * K * H > 2**31
    w, x = _layer(wl)
    out, idx, tw = G.gpu_layer(wl, w, x)
    gi, gw = idx.cpu().numpy(), tw.cpu().numpy()
    _check_dispatch_of(wl, gi)
    _, _, _, slot_of = orc.dispatch(G.oracle_dims(wl), gi)
    far = np.nonzero((slot_of.reshape(T, K).astype(np.int64) * H >= 2**31).any(1))[0]
    assert len(far) > 0
    rng = np.random.default_rng(2)
    sample = sorted(set(far[:: max(1, len(far) // 24)][:24].tolist())
                    | set(rng.choice(T, 16, replace=False).tolist()) | {0, T - 1})
    rows = torch.as_tensor(sample, device=x.device)
    xh = inputs.to_numpy_f32(x.index_select(0, rows))
    d = G.oracle_dims(wl)
    o_idx, o_w, tie = orc.route(d, xh, inputs.to_numpy_f32(w["router"]), inputs.to_numpy_f32(w.get("bias")))
    nties = G.check_routing(gi[sample], gw[sample], o_idx, o_w, tie, wl.name,
                            G.scores_fn(d, xh, inputs.to_numpy_f32(w["router"]), inputs.to_numpy_f32(w.get("bias"))))
    wh = G.host_weights(w, set(gi[sample].ravel().tolist()))
    ref, _, _, _ = orc.forward(d, xh, wh, force_idx=gi[sample])
    rel = G.check_output(out.index_select(0, rows).float().cpu().numpy(), ref, wl.name + " (sampled)")
    print(f"flint_T180000: {len(far)} tokens with slots past 2^31 elements, rel_err={rel:.3g} near_ties={nties}")


STACK_FULL_LAYERS = (0, 8, 16, 24, 32, 40, 46)


def test_stack47_layer_by_layer():
    """47 distinct layers resident in HBM, RMSNorm between layers.  Each layer is
    checked against the oracle fed the GPU's own input to that layer (a flipped
    near tie would otherwise cascade): every token of layers 0, 8, ..., 40 and
    46, sampled tokens of the others; each RMSNorm is checked on every token."""
    wl = inputs.WORKLOADS["stack47"]
    d = api.dims_of(wl)
    layers = [inputs.make_layer(wl, l, "cuda") for l in range(wl.layers)]
    x = inputs.make_tokens(wl, device="cuda")
    ws = api.workspace(d, wl.T)
    rng = np.random.default_rng(7)
    eps = float(np.float32(1e-6))
    worst = 0.0
    ties = 0
    for l, w in enumerate(layers):
        sample = rng.choice(wl.T, 8, replace=False)
        one = inputs.Workload(f"stack47/L{l}", wl.T, wl.hidden, wl.n_experts, wl.top_k, wl.inter,
                              wl.shared_inter, True, wl.seed)
        if l in STACK_FULL_LAYERS:
            st = G.parity_full(one, w, x)
            out, _, _ = G.gpu_layer(one, w, x)  # (deterministic: the same bits parity_full checked)
            st["out"] = out
        else:
            st = G.parity_sampled(one, w, x, sample)
        worst = max(worst, st["rel_err"])
        ties += st["near_ties"]
        if l % 8 == 0:
            print(f"stack47 layer {l}: rel_err={st['rel_err']:.3g}", flush=True)
        if l + 1 < wl.layers:
            y = st["out"]
            x = api.rmsnorm(y, eps)
            torch.cuda.synchronize()
            ref = orc.rmsnorm(y.cpu().numpy(), eps)
            np.testing.assert_array_equal(x.float().cpu().numpy(), ref)
    del ws
    print(f"stack47: worst rel_err={worst:.3g} near_ties={ties}")


@pytest.mark.parametrize("case", [(1, 16, 2), (100, 16, 6), (256, 256, 6), (257, 64, 8), (1000, 256, 6),
                                  (5000, 256, 1), (3000, 20, 3)])
def test_dispatch_random_assignments(case):
    T, E, K = case
    rng = np.random.default_rng(T + E + K)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)  # rows unsorted
    wl = inputs.custom("disp", T, 64, E, K, 64, 0, True)
    counts = _check_dispatch_of(wl, idx)
    oracle_pins.check_dispatch_invariants(idx, E, counts, *[t for t in orc.dispatch(G.oracle_dims(wl), idx)[1:]])


@pytest.mark.parametrize("T", [8, 32])  # the forward call's top-k + dispatch: one work-group / two kernels
def test_route_entry_point_matches_forward_routing(T):
    wl = inputs.WORKLOADS["decode32"] if T == 32 else inputs.Workload("flint_T8", T, 2048, 256, 6, 512, 1024,
                                                                       True, 0)
    w, x = _layer(wl)
    d = api.dims_of(wl)
    idx, tw = api.route(d, x, w["router"], w.get("bias"))
    _, idx2, tw2 = G.gpu_layer(wl, w, x)
    assert torch.equal(idx, idx2) and torch.equal(tw, tw2)


# one wave per token (T <= 4096), 16-lane groups above; T = 12 through the
# forward call, whose top-k shares a work-group with the dispatch (T <= 16)
@pytest.mark.parametrize("T,via", [(12, "forward"), (37, "route"), (1500, "route"), (4100, "route")])
def test_route_exact_ties_go_to_the_lower_index(T, via):
    """Router rows in groups of four identical rows, group g scaled by (1 + g):
    the four experts of a group get equal float32 scores on both sides, so with
    K = 6 the boundary falls inside a group for every token and the selection
    must take that group's lowest ids.  Distinct groups are far apart except for
    tokens with x . r0 near 0, which are left out (counted)."""
    H, E, K = 256, 64, 6
    g = torch.Generator().manual_seed(11)
    r0 = torch.randn(H, generator=g) * 0.05
    router = ((1.0 + (torch.arange(E) // 4).float())[:, None] * r0[None, :]).to(torch.bfloat16)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    wl = inputs.custom("ties", T, H, E, K, 64, 0, True)
    if via == "route":
        idx, tw = api.route(api.dims_of(wl), x.cuda(), router.cuda(), None)
    else:
        w = {k: (v.cuda() if v is not None else None) for k, v in inputs.make_layer(wl, 0, "cpu").items()}
        w["router"] = router.cuda()
        _, idx, tw = api.forward(api.dims_of(wl), x.cuda(), w, return_routing=True)
    dd = G.oracle_dims(wl)
    xh, rh = inputs.to_numpy_f32(x), inputs.to_numpy_f32(router)
    o_idx, o_w, _ = orc.route(dd, xh, rh, None)
    sc = orc.scores(dd, xh, rh, None)
    checked = boundary_ties = 0
    for t in range(T):
        vals = np.unique(sc[t])[::-1]  # distinct scores, descending
        if np.min(vals[:-1] - vals[1:]) < 1e-5:
            continue  # distinct groups too close to call
        srt = np.sort(sc[t])[::-1]
        boundary_ties += int(srt[K - 1] == srt[K])
        checked += 1
        assert idx[t].tolist() == o_idx[t].tolist(), (t, idx[t].tolist(), o_idx[t].tolist())
        np.testing.assert_allclose(tw[t].cpu().numpy(), o_w[t], rtol=0, atol=G.WEIGHT_TOL)
    print(f"ties T={T}: {checked} tokens checked, {boundary_ties} with a tie at the boundary")
    assert checked >= T // 2 and boundary_ties == checked


def _extreme_router(regime, E, H):
    """bf16 router rows c_e * (1, ..., 1) whose products with the tokens below
    give logits H * s_t * c_e exactly in float32 on both sides:
    saturated  z in [20, 120]: every score rounds to 1.0 (all equal)
    subnormal  z in about [-95.2, -88.6]: scores are float32 subnormals, in
               groups of equal c_e (logit steps of 0.5 between groups)
    zero       z <= -110: every score underflows to 0"""
    e = torch.arange(E, dtype=torch.float64)
    if regime == "saturated":
        hc = 20.0 + 40.0 * e / E
    elif regime == "subnormal":
        hc = -(88.6 + 4.4 * ((e * 37) % E) / E)  # shuffled, so the best ids are not the lowest
    else:
        hc = -(110.0 + 20.0 * e / E)
    c = (hc / H).to(torch.bfloat16)
    return c[:, None].expand(E, H).contiguous()


def _extreme_tokens(regime, T, H):
    # s_t in [1, 2) for the saturated and zero regimes, within 2.4% of 1 for
    # the subnormal one (keeps z inside the subnormal range)
    k = torch.arange(T, dtype=torch.float64)
    s = 1.0 + ((k % 128) / 128.0 if regime != "subnormal" else (k % 4) / 128.0)
    return s.to(torch.bfloat16)[:, None].expand(T, H).contiguous()


@pytest.mark.parametrize("regime", ["saturated", "subnormal", "zero"])
@pytest.mark.parametrize("T,via", [(12, "forward"), (37, "route"), (1500, "route"), (4100, "route")])
def test_route_extreme_logits(T, via, regime):
    """Logits far outside the N(0, 0.02) range, through every top-k kernel:
    saturated scores (all 1.0: the lowest K ids, weights 1/K), subnormal scores
    (e^z / (1 + e^z) stays nonzero below z = -88.7, where 1 / (1 + e^-z)
    would give 0), and scores that underflow to 0 (weights 1/K, not 0/0).
    Selection must equal the oracle's exactly (distinct logits differ by at
    least 0.5 here), weights within the float32 precision of the scores, and
    the layer output (forward) finite and within the bar."""
    H, E, K = 256, 64, 6
    router = _extreme_router(regime, E, H)
    x = _extreme_tokens(regime, T, H)
    wl = inputs.custom(f"extreme_{regime}", T, H, E, K, 64, 64, True, seed=2)
    if via == "route":
        idx, tw = api.route(api.dims_of(wl), x.cuda(), router.cuda(), None)
    else:
        w = {k: (v.cuda() if v is not None else None) for k, v in inputs.make_layer(wl, 0, "cpu").items()}
        w["router"] = router.cuda()
        out, idx, tw = api.forward(api.dims_of(wl), x.cuda(), w, return_routing=True)
    torch.cuda.synchronize()
    gi, gw = idx.cpu().numpy(), tw.cpu().numpy()
    dd = G.oracle_dims(wl)
    xh, rh = inputs.to_numpy_f32(x), inputs.to_numpy_f32(router)
    o_idx, o_w, _ = orc.route(dd, xh, rh, None)
    sc = orc.scores(dd, xh, rh, None)
    np.testing.assert_array_equal(gi, o_idx)
    assert np.all(np.isfinite(gw))
    sel_sum = np.take_along_axis(sc.astype(np.float64), o_idx, 1).sum(1)
    if regime == "saturated":
        assert np.all(sc == 1.0)
        np.testing.assert_array_equal(gi, np.tile(np.arange(K), (T, 1)))
        np.testing.assert_array_equal(gw, np.full((T, K), np.float32(1.0 / K)))
    elif regime == "zero":
        assert np.all(sc == 0.0)
        np.testing.assert_array_equal(gi, np.tile(np.arange(K), (T, 1)))
        np.testing.assert_array_equal(gw, np.full((T, K), np.float32(1.0 / K)))
    else:
        assert np.all(sel_sum > 0) and np.all(sc < np.finfo(np.float32).tiny)
        # each score is a multiple of 2^-149; one step of difference per score
        # moves a weight by at most about 2^-149 / sum
        tol = 3.0 * 2.0 ** -149 / sel_sum[:, None] + G.WEIGHT_TOL
        assert np.all(np.abs(gw - o_w) <= tol), float(np.max(np.abs(gw - o_w) - tol))
    if via == "forward":
        ref, _, _, _ = orc.forward(dd, xh, G.host_weights(w), force_idx=gi)
        G.check_output(out.cpu().numpy(), ref, f"extreme_{regime}")


@pytest.mark.parametrize("which", ["routed", "shared", "both"])
@pytest.mark.parametrize("scale_log2", [20, 40])
def test_tiled_outputs_beyond_fp16_range(scale_log2, which):
    """On the tiled kernels the routed and the shared expert's outputs travel
    to the combine as fp16 with a power-of-two exponent per row and 64
    columns.  Down weights of half the experts (routed), of the shared expert,
    or both, multiplied by 2^20 or 2^40 (exact in bf16), put those outputs far
    past fp16's largest value (65504) while the others stay small: the result
    must be finite and within the bar on every token."""
    wl = inputs.custom(f"y16_big_{scale_log2}_{which}", 600, 256, 16, 4, 128, 128, True, seed=23)
    w, x = _layer(wl)
    if which in ("routed", "both"):
        w["down"][::2].mul_(2.0 ** scale_log2)
    if which in ("shared", "both"):
        w["shared_down"].mul_(2.0 ** scale_log2)
    st = G.parity_full(wl, w, x)
    print(f"y16 {which} x2^{scale_log2}: rel_err={st['rel_err']:.3g}")


@pytest.mark.parametrize("name", ["decode32", "prefill4096"])
def test_deterministic(name):
    wl = inputs.WORKLOADS[name]
    w, x = _layer(wl)
    a, ia, wa = G.gpu_layer(wl, w, x)
    b, ib, wb = G.gpu_layer(wl, w, x)
    assert torch.equal(ia, ib) and torch.equal(wa, wb)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("T", [32, 600])
def test_buffer_placement_does_not_change_results(T):
    """The workspace's intermediate arrays are placed at a phase against the
    output buffer: output and workspace at other offsets (the output 16-byte
    aligned only) must give the same bits."""
    wl = inputs.Workload(f"place_T{T}", T, 2048, 256, 6, 512, 1024, True, 7)
    w, x = _layer(wl)
    d = api.dims_of(wl)
    need = api.flint_moe_workspace_bytes(d, T)
    ref = torch.empty((T, d.hidden), dtype=torch.float32, device="cuda")
    api.flint_moe_forward(d, x, w, ref, ws=torch.empty(need, dtype=torch.uint8, device="cuda"))
    big = torch.empty(T * d.hidden * 4 + 8192, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(need + 8192, dtype=torch.uint8, device="cuda")
    for out_off, ws_off in ((16, 0), (272, 256), (1040, 3840), (4080, 1024)):
        out = big[out_off:out_off + T * d.hidden * 4].view(torch.float32).view(T, d.hidden)
        api.flint_moe_forward(d, x, w, out, ws=wsb[ws_off:ws_off + need])
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), (out_off, ws_off)


def test_empty_batch_is_a_noop():
    wl = inputs.WORKLOADS["decode32"]
    d = api.dims_of(wl)
    w, _ = _layer(wl)
    x = torch.empty((0, wl.hidden), dtype=torch.bfloat16, device="cuda")
    out = api.forward(d, x, w)
    torch.cuda.synchronize()
    assert out.shape == (0, wl.hidden)
    counts, offsets, _, _ = api.dispatch(d, torch.empty((0, wl.top_k), dtype=torch.int32, device="cuda"))
    assert int(counts.abs().sum()) == 0 and int(offsets.abs().sum()) == 0


@pytest.mark.parametrize("shape", [
    ("fr1", 1, 2048, 256, 6, 512, 1024, True),     # streaming kernels
    ("fr32", 32, 2048, 256, 6, 512, 1024, True),   # streaming kernels
    ("fr200", 200, 2048, 256, 6, 512, 1024, True),  # 16-row tiles
    ("fr600", 600, 2048, 256, 6, 512, 1024, True),  # large tiles (fp16 routed outputs)
    ("fr64_f32", 64, 256, 16, 2, 256, 512, False),  # float32 layer
], ids=lambda s: s[0])
def test_forward_rmsnorm_equals_forward_then_rmsnorm(shape):
    """flint_moe_forward_rmsnorm gives flint_moe_forward's output and, as its
    norm, flint_rmsnorm of the float32 output, bit for bit, on every kernel path;
    with a bf16 out too, and with the norm written over x."""
    name, T, H, E, K, I, Is, bf16 = shape
    wl = inputs.custom(name, T, H, E, K, I, Is, bf16, seed=9)
    w, x = _layer(wl)
    d = api.dims_of(wl)
    eps = 1e-6
    ref = api.forward(d, x, w)
    ref_norm = api.rmsnorm(ref, eps)
    out, norm = api.forward_rmsnorm(d, x, w, eps)
    ref16 = api.forward(d, x, w, out_dtype=torch.bfloat16)
    out16, norm16 = api.forward_rmsnorm(d, x, w, eps, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8)), f"{name}: layer output differs"
    assert torch.equal(norm.view(torch.uint8), ref_norm.view(torch.uint8)), f"{name}: norm differs"
    assert torch.equal(out16.view(torch.uint8), ref16.view(torch.uint8)), f"{name}: bf16 layer output differs"
    assert torch.equal(norm16.view(torch.uint8), ref_norm.view(torch.uint8)), f"{name}: norm (bf16 out) differs"
    if bf16:  # the next layer's input written over this layer's
        xx = x.clone()
        out2 = torch.empty_like(ref)
        api.flint_moe_forward_rmsnorm(d, xx, w, out2, xx, eps, ws=api.workspace(d, T, x.device))
        torch.cuda.synchronize()
        assert torch.equal(xx.view(torch.uint8), ref_norm.view(torch.uint8)), f"{name}: norm over x differs"
        assert torch.equal(out2.view(torch.uint8), ref.view(torch.uint8)), f"{name}: output with the norm over x"


def test_rmsnorm_matches_oracle():
    y = torch.randn((300, 2048), generator=torch.Generator().manual_seed(5)) * 3
    eps = float(np.float32(1e-6))
    got = api.rmsnorm(y.to("cuda"), eps).float().cpu().numpy()
    np.testing.assert_array_equal(got, orc.rmsnorm(y.numpy(), eps))


PROFILED = ["decode32", "prefill4096"]


@pytest.mark.parametrize("name", PROFILED)
def test_profiled_forward_same_bits_and_ordered_stages(name):
    """flint_moe_forward_profiled runs the same kernels as flint_moe_forward (same
    bits out) and stamps five disjoint, ordered stage intervals that fit inside
    the call's own span on the stream."""
    import ctypes
    wl = inputs.WORKLOADS[name]
    w, x = _layer(wl)
    d = api.dims_of(wl)
    a, ia, wa = G.gpu_layer(wl, w, x)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(12):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e)
    T = wl.T
    out = torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, wl.top_k), dtype=torch.float32, device="cuda")
    ws = api.workspace(d, T)
    stream = torch.cuda.current_stream()
    assert hip.hipEventRecord(evs[10], ctypes.c_void_p(stream.cuda_stream)) == 0
    api.flint_moe_forward(d, x, w, out, idx, tw, ws, stream, events=evs[:10])
    assert hip.hipEventRecord(evs[11], ctypes.c_void_p(stream.cuda_stream)) == 0
    torch.cuda.synchronize()
    assert torch.equal(ia, idx) and torch.equal(wa, tw)
    assert torch.equal(a.view(torch.int32), out.view(torch.int32))

    def ms(i, j):
        v = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(v), evs[i], evs[j]) == 0
        return v.value

    stages = [ms(2 * s, 2 * s + 1) for s in range(5)]
    assert all(t > 0 for t in stages), stages
    # each stage starts after the previous one stopped
    for s in range(4):
        assert ms(2 * s + 1, 2 * s + 2) >= 0
    total = ms(10, 11)
    assert sum(stages) <= total * 1.001 + 1e-3, (stages, total)
    print(f"{name}: stages_us={[round(t * 1e3, 1) for t in stages]} span_us={total * 1e3:.1f}")
    for e in evs:
        hip.hipEventDestroy(e)


# ---- MXFP4 expert weights (flint_moe_forward_mx4) ------------------------

MX4_CASES = [
    # name,        T,  H,    E,  K, I,   Is,  bias
    ("mx4_t33",    33, 1024, 16, 4, 512, 512, True),
    ("mx4_t7_ns",  7,  1024, 8,  2, 512, 0,   False),
    ("mx4_t200",   200, 2048, 32, 6, 512, 1024, True),
    ("mx4_t9_i256", 9,  1024, 8,  2, 256, 256,  False),  # the smallest supported widths
    ("mx4_t300",   300, 1024, 32, 6, 512, 512,  True),   # wide gate/up and down items
]


@pytest.mark.parametrize("case", MX4_CASES, ids=[c[0] for c in MX4_CASES])
def test_mx4_small_every_token(case):
    name, T, H, E, K, I, Is, bias = case
    wl = inputs.custom(name, T, H, E, K, I, Is, True, seed=5, zipf=bias, mx4=True)
    w, x = _layer(wl)
    st = G.parity_mx4(wl, w, x)
    print(f"{name}: rel_err={st['rel_err']:.3g} near_ties={st['near_ties']}")


def test_mx4_decode32_every_token_and_deterministic():
    wl = inputs.WORKLOADS["decode32_mx4"]
    w = inputs.make_layer(wl, 0, "cuda")
    x = inputs.make_tokens(wl, device="cuda")
    st = G.parity_mx4(wl, w, x)
    again, _, _ = G.gpu_layer(wl, w, x)
    assert torch.equal(st["out"].view(torch.int32), again.view(torch.int32))
    print(f"decode32_mx4: rel_err={st['rel_err']:.3g} near_ties={st['near_ties']}")


def test_mx4_largest_batch_every_token():
    """The largest batch the MXFP4 entry point takes (T = 512), Flint shape."""
    wl = inputs.custom("mx4_t512", 512, 2048, 256, 6, 512, 1024, True, seed=7, mx4=True)
    w, x = _layer(wl)
    st = G.parity_mx4(wl, w, x)
    print(f"mx4_t512: rel_err={st['rel_err']:.3g} near_ties={st['near_ties']}")


def test_mx4_largest_widths():
    """MXFP4 at the largest widths it takes (H = 8192, I = Is = 4096, K = 8; 32
    experts to bound the memory), T = 5, every token."""
    wl = inputs.custom("mx4_max", 5, 8192, 32, 8, 4096, 4096, True, seed=8, mx4=True)
    w, x = _layer(wl)
    st = G.parity_mx4(wl, w, x)
    print(f"mx4_max: rel_err={st['rel_err']:.3g} near_ties={st['near_ties']}")


# ---- dense MLP layer (flint_dense_mlp) ---------------------------------------

DENSE_CASES = [
    # name,         T,    H,    I,    bf16
    ("d_t1",        1,    128,  192,  True),    # 32-row tiled configurations, down split 3 ways
    ("d_t33",       33,   256,  320,  True),    # two 32-row tiles, the second ragged; down split 5 ways
    ("d_t7_f32",    7,    128,  64,   False),
    ("d_t128",      128,  256,  512,  True),    # the largest dense batch on the 32-row tiles
    ("d_t129",      129,  256,  512,  True),    # the smallest on the large-batch tiles, down split 8 ways
    ("d_t600",      600,  256,  512,  True),    # large-batch (tiled) kernels, down split 8 ways
    ("d_t1000",     1000, 256,  6144, True),    # 256 x 256 gate/up tiles, ragged last tile
    ("d_t700_f32",  700,  128,  128,  False),   # float32 large-batch kernels
    ("d_flint32",   32,   2048, 6144, True),    # the dense layer's width, decode batch (down split 8 ways)
    ("d_flint100",  100,  2048, 6144, True),    # four 32-row tiles, the last ragged; the 4-stage gate/up ring
    ("d_t20_w1536", 20,   1024, 1536, True),    # down split 8 ways, 192 of the width each
    ("d_t40_f32",   40,   256,  512,  False),   # float32 on the streaming kernels
    ("d_t300_f32",  300,  256,  768,  False),   # float32 on the streaming kernels, down split
]


def _dense(wl, device="cuda"):
    if wl.inter * wl.hidden <= (1 << 22):
        w = {k: v.to(device) for k, v in inputs.make_dense(wl, 0, "cpu").items()}
        x = inputs.make_tokens(wl, device="cpu").to(device)
    else:
        w = inputs.make_dense(wl, 0, device)
        x = inputs.make_tokens(wl, device=device)
    return w, x


def _dense_check(wl, w, x, rows=None, out_dtype=torch.float32):
    out = api.dense_mlp(x, w["gate"], w["up"], w["down"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = np.arange(wl.T) if rows is None else rows
    ref = orc.dense_mlp(inputs.to_numpy_f32(x)[rows], inputs.to_numpy_f32(w["gate"]),
                        inputs.to_numpy_f32(w["up"]), inputs.to_numpy_f32(w["down"]), h_bf16=wl.bf16)
    got = out.float().cpu().numpy()[rows]
    if out_dtype == torch.bfloat16:
        ref = inputs.to_numpy_f32(torch.from_numpy(ref).to(torch.bfloat16))
    rel = G.check_output(got, ref, wl.name)
    return out, rel


@pytest.mark.parametrize("case", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_dense_every_token(case):
    name, T, H, I, bf16 = case
    wl = inputs.custom(name, T, H, 0, 0, I, 0, bf16, seed=13, dense=True)
    w, x = _dense(wl)
    out, rel = _dense_check(wl, w, x)
    print(f"{name}: rel_err={rel:.3g}")
    again = api.dense_mlp(x, w["gate"], w["up"], w["down"])
    assert torch.equal(out.view(torch.int32), again.view(torch.int32))  # deterministic


@pytest.mark.parametrize("shape", [(45, 256, 704), (24, 1024, 1536)])  # one combine input; eight partial sums
def test_dense_bf16_output(shape):
    T, H, I = shape
    wl = inputs.custom("d_bf16out", T, H, 0, 0, I, 0, True, seed=2, dense=True)
    w, x = _dense(wl)
    _dense_check(wl, w, x, out_dtype=torch.bfloat16)


@pytest.mark.parametrize("T", [5, 200])
def test_dense_largest_widths(T):
    """The dense layer at the largest widths it takes (H = 8192, width 16384):
    T = 5 on the 32-row tiles (every token), T = 200 on the large-batch tiles
    (sampled tokens)."""
    wl = inputs.custom(f"d_max_T{T}", T, 8192, 0, 0, 16384, 0, True, seed=17, dense=True)
    w, x = _dense(wl)
    rows = None if T <= 8 else np.array([0, 1, T // 2, T - 1])
    _, rel = _dense_check(wl, w, x, rows=rows)
    print(f"d_max_T{T}: rel_err={rel:.3g}")


def test_dense_hidden_past_2_31_elements():
    """A dense batch whose intermediate [T, width] passes 2^31 elements
    (T = 140000, width 16384): rows from 131072 on sit past element 2^31,
    where a 32-bit offset would wrap; sampled rows on both sides."""
    T, H, I = 140_000, 2048, 16384
    assert T * I > 2**31
    wl = inputs.custom("d_T140000", T, H, 0, 0, I, 0, True, seed=19, dense=True)
    w, x = _dense(wl)
    rows = np.array([0, 1, 70_000, 131_071, 131_072, 131_073, 135_001, T - 2, T - 1])
    _, rel = _dense_check(wl, w, x, rows=rows)
    print(f"d_T140000: rel_err={rel:.3g}")


def test_dense4096_sampled():
    wl = inputs.WORKLOADS["dense4096"]
    w, x = _dense(wl)
    rows = np.unique(np.concatenate([np.arange(0, wl.T, 97), [wl.T - 1]]))
    _, rel = _dense_check(wl, w, x, rows=rows)
    print(f"dense4096: rel_err={rel:.3g} on {len(rows)} tokens")


def test_mx4_scale_extremes_and_nan_blocks():
    """MXFP4 scales away from the quantiser's range: every block's scale byte
    redrawn in 127 +- 12, some blocks at 0 (2^-127, subnormal weights), and one
    block of one routed expert at 255 (NaN): the GPU must agree with the oracle
    wherever the oracle is finite, and be NaN exactly where it is NaN."""
    wl = inputs.custom("mx4_scales", 40, 1024, 8, 2, 512, 512, True, seed=21, mx4=True)
    w, x = _layer(wl)
    g = torch.Generator().manual_seed(4)
    for k in ("gate", "up", "down", "shared_gate", "shared_up", "shared_down"):
        s = w[k + "_s"]
        new = torch.randint(115, 140, tuple(s.shape), generator=g, dtype=torch.int32).to(torch.uint8)
        new.view(-1)[::97] = 0
        s.copy_(new.to(s.device))
    d = api.dims_of(wl)
    idx, _ = api.route(d, x, w["router"], w.get("bias"))
    hot = int(idx[0, 0])  # an expert token 0 uses
    w["up_s"][hot, 0, 0, 3] = 255  # up row 3 of that expert, first block
    out, gi, tw = G.gpu_layer(wl, w, x)
    dd = G.oracle_dims(wl)
    wh = G.host_weights_mx4(w)
    ref, _, _, _ = orc.forward(dd, inputs.to_numpy_f32(x), wh, force_idx=gi.cpu().numpy())
    got = out.float().cpu().numpy()
    nan_ref = np.isnan(ref)
    assert nan_ref[0].all()  # token 0 routes through the NaN block
    np.testing.assert_array_equal(np.isnan(got), nan_ref)
    fin = ~nan_ref.any(axis=1)
    assert fin.sum() >= 5
    G.check_output(got[fin], ref[fin], "mx4_scales")


GRAPH_CASES = [
    # workload,       T
    ("decode32",      8),     # one-work-group top-k + dispatch, streaming experts
    ("decode32",      32),    # the decode batch: top-k + dispatch in one launch of many work-groups
    ("decode32",      200),   # one-work-group dispatch, 16-row tiles
    ("prefill4096",   600),   # three-kernel dispatch, tiled experts
    ("decode32_mx4",  32),    # MXFP4 expert weights
    ("dense32",       32),    # dense layer, 32-row tiles, split down product
    ("dense4096",     600),   # dense layer, tiled, split down product
    ("stack47",       256),   # flint_moe_forward_rmsnorm: the norm in the combine
    ("stack47",       64),    # the same on the streaming kernels
]


@pytest.mark.parametrize("case", GRAPH_CASES, ids=[f"{c[0]}_T{c[1]}" for c in GRAPH_CASES])
def test_graph_replays_match_eager(case):
    """One call captured in a HIP graph and replayed three times.  Before each
    replay an eager call on other tokens runs with the same workspace, and the
    outputs are overwritten, so each replay starts from a dirty workspace.
    Every replay must equal the eager result bit for bit, routing included."""
    name, T = case
    wl = dataclasses.replace(inputs.WORKLOADS[name], name=f"{name}_T{T}", T=T)
    x = inputs.make_tokens(wl, device="cuda")
    x2 = inputs.make_tokens(wl, device="cuda", stream=1)
    if wl.dense:
        w = inputs.make_dense(wl, 0, "cuda")
        dd = api.dense_dims_of(wl)
        ws = api.dense_workspace(dd, T)
        ref = api.dense_mlp(x, w["gate"], w["up"], w["down"], ws=ws)
        outs = [torch.empty_like(ref)]
        refs = [ref]

        def call():
            api.flint_dense_mlp(dd, x, w["gate"], w["up"], w["down"], outs[0], ws)

        def dirty():
            api.dense_mlp(x2, w["gate"], w["up"], w["down"], ws=ws)
    else:
        w = inputs.make_layer(wl, 0, "cuda")
        d = api.dims_of(wl)
        ws = api.workspace(d, T)
        refs = list(api.forward(d, x, w, ws=ws, return_routing=True))
        outs = [torch.empty_like(r) for r in refs]
        if wl.mx4:
            wst = api.weights_mx4_struct(d, w)
            entry = api.flint_moe_forward_mx4
        else:
            wst = api.weights_struct(d, w)
            entry = api.flint_moe_forward
        stacked = wl.layers > 1
        if stacked:  # the layer with the norm of its output (the next layer's input)
            refs.append(api.rmsnorm(refs[0]))
            outs.append(torch.empty_like(refs[3]))

        def call():
            if stacked:
                api.flint_moe_forward_rmsnorm(d, x, wst, outs[0], outs[3], 1e-6, outs[1], outs[2], ws)
            else:
                entry(d, x, wst, outs[0], outs[1], outs[2], ws)

        def dirty():
            api.forward(d, x2, w, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    for r in range(3):
        dirty()
        for o in outs:
            o.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o.view(torch.uint8), ref.view(torch.uint8)), f"{name} T={T}: replay {r} differs"


def test_fused_graph_replays_and_concurrent_calls():
    """The fused entry point captured in a HIP graph and replayed (a dirty
    workspace before each replay) equals its eager result bit for bit; and two
    fused calls running at once on two streams (their persistent grids then
    share the GPU, so not every work-group is resident at first) both finish
    with their eager results."""
    wl = dataclasses.replace(inputs.WORKLOADS["decode32"], name="fused_graph")
    w = inputs.make_layer(wl, 0, "cuda")
    d = api.dims_of(wl)
    wst = api.weights_struct(d, w)
    xs = [inputs.make_tokens(wl, device="cuda", stream=i) for i in range(2)]
    wss = [api.workspace(d, wl.T) for _ in range(2)]
    refs = [api.forward(d, xs[i], w, ws=wss[i], return_routing=True, fused=True) for i in range(2)]
    torch.cuda.synchronize()
    outs = [torch.empty_like(r) for r in refs[0]]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            api.flint_moe_forward_fused(d, xs[0], wst, *outs, ws=wss[0], stream=s)
    torch.cuda.synchronize()
    for r in range(3):
        api.forward(d, xs[1], w, ws=wss[0], fused=True)  # dirties the workspace
        for o in outs:
            o.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs[0]):
            assert torch.equal(o.view(torch.uint8), ref.view(torch.uint8)), f"replay {r} differs"
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs2 = [[torch.full_like(r, -1) for r in refs[i]] for i in range(2)]
    for st_ in streams:
        st_.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for i in (0, 1):
            api.flint_moe_forward_fused(d, xs[i], wst, *outs2[i], ws=wss[i], stream=streams[i])
    torch.cuda.synchronize()
    for i in (0, 1):
        for o, ref in zip(outs2[i], refs[i]):
            assert torch.equal(o.view(torch.uint8), ref.view(torch.uint8)), f"stream {i} differs"


@pytest.mark.parametrize("T", [32, 600])
def test_concurrent_streams_with_own_workspaces(T):
    """Calls on two streams at once, each with its own workspace and inputs,
    launches interleaved: each result equals its eager one bit for bit (the
    library keeps no device state between calls)."""
    wl = dataclasses.replace(inputs.WORKLOADS["prefill4096"], name=f"conc_T{T}", T=T)
    w = inputs.make_layer(wl, 0, "cuda")
    d = api.dims_of(wl)
    xs = [inputs.make_tokens(wl, device="cuda", stream=i) for i in range(2)]
    wss = [api.workspace(d, T) for _ in range(2)]
    refs = [api.forward(d, xs[i], w, ws=wss[i], return_routing=True) for i in range(2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [[torch.full_like(r, -1) for r in refs[i]] for i in range(2)]
    wst = api.weights_struct(d, w)
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(2):
        for i in (0, 1):
            api.flint_moe_forward(d, xs[i], wst, *outs[i], wss[i], stream=streams[i])
    torch.cuda.synchronize()
    for i in (0, 1):
        for o, ref in zip(outs[i], refs[i]):
            assert torch.equal(o.view(torch.uint8), ref.view(torch.uint8)), f"T={T} stream {i} differs"
