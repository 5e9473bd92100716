"""Pins for the CPU oracle: checks against facts fixed by the pages and by
mathematics, not against the oracle itself.

Each ``pin_*`` function takes an ``Oracle`` and raises AssertionError when the
oracle disagrees.  ``test_oracle_pins.py`` runs them on the oracle, and runs
them again on deliberately broken copies of the oracle's source to show that
each plausible mistake is caught by at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import brute_mixture as brute
from oracle.oracle import dims

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _random_layer(rng, H, E, I, Is, bf16, bias=False, std=0.3):
    """Small random layer (values made exact in bf16 when bf16=True)."""
    def draw(*shape):
        a = (rng.standard_normal(shape) * std).astype(np.float32)
        if bf16:
            a = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
        return a
    w = {"router": draw(E, H), "gate": draw(E, I, H), "up": draw(E, I, H), "down": draw(E, H, I),
         "bias": (rng.standard_normal(E) * 0.5).astype(np.float32) if bias else None}
    if Is > 0:
        w["shared_gate"] = draw(Is, H)
        w["shared_up"] = draw(Is, H)
        w["shared_down"] = draw(H, Is)
    return w


def _random_x(rng, T, H, bf16):
    a = rng.standard_normal((T, H)).astype(np.float32)
    if bf16:
        a = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    return a


# --------------------------------------------------------------------------
# P1: the pages' own parameter count selects the gated three-matrix expert.

def pin_param_counts(orc):
    g = json.load(open(os.path.join(GOLDEN, "flint_param_counts.json")))
    s = g["shape"]
    d = dims(s["hidden"], s["n_experts"], s["top_k"], s["expert_inter"], s["shared_inter"], True)
    router, routed, one, shared, active = orc.param_counts(d)
    L = s["moe_layers"]
    assert round(routed * L / 1e9, 1) == g["printed"]["routed_experts_total_billions"], routed * L
    assert round(active * L / 1e9, 1) == g["printed"]["six_experts_plus_shared_per_token_billions"], active * L
    assert router == s["n_experts"] * s["hidden"]
    # A two-matrix expert (no gate) would not match the printed figures.
    assert round(routed * 2 / 3 * L / 1e9, 1) != g["printed"]["routed_experts_total_billions"]


# --------------------------------------------------------------------------
# bf16 rounding: the format's definition on chosen values, and torch's
# float32 -> bfloat16 conversion (round to nearest even) on random values.

def pin_bf16_rounding(orc):
    u = 2.0 ** -7  # one bf16 ulp at 1.0
    cases = {
        1.0: 1.0,
        1.0 + u: 1.0 + u,                 # representable
        1.0 + u / 2: 1.0,                 # tie, round to even (1.0)
        1.0 + 3 * u / 2: 1.0 + 2 * u,     # tie, round to even (1 + 2u)
        1.0 + u / 2 + 2.0 ** -30: 1.0 + u,  # just above the tie
        -(1.0 + 3 * u / 2): -(1.0 + 2 * u),
        1.5 * 2.0 ** -133: 2.0 ** -132,   # subnormal grid (spacing 2^-133), tie to even
        2.5 * 2.0 ** -133: 2.0 ** -132,
        0.25 * 2.0 ** -133: 0.0,
        0.0: 0.0,
        65536.0 + 255.0: 65536.0,         # ulp at 2^16 is 512
        65536.0 + 256.0: 65536.0,         # tie, even
        65536.0 + 257.0: 65536.0 + 512.0,
    }
    got = orc.round_bf16(np.array(list(cases.keys())))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    r = _rng(11).standard_normal(20000).astype(np.float32) * np.float32(3.0)
    ref = torch.from_numpy(r).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(orc.round_bf16(r.astype(np.float64)), ref)


# --------------------------------------------------------------------------
# Routing closed forms.  With one hidden unit and x = [1], the logits are the
# router weights.  float32(ln 3), 0, float32(-ln 3), float32(ln 7) give sigmoid
# scores that round to exactly 3/4, 1/2, 1/4 and 7/8 in float32 (the float32
# error of the logit moves the score by less than 1e-8, under half a float32
# ulp of these values).

_LN3 = math.log(3.0)
_LN7 = math.log(7.0)


def _hand_router():
    return np.array([[_LN3], [0.0], [-_LN3], [_LN7]], np.float32)


def pin_routing_hand_top2(orc):
    d = dims(1, 4, 2, 1, 0, False)
    idx, w, tie = orc.route(d, np.ones((1, 1), np.float32), _hand_router())
    # top-2 of {3/4, 1/2, 1/4, 7/8} = experts 3 and 0; weights (3/4)/(13/8), (7/8)/(13/8).
    np.testing.assert_array_equal(idx, [[0, 3]])
    np.testing.assert_array_equal(w, np.array([[6 / 13, 7 / 13]], np.float32))
    assert not tie[0]
    # A softmax over the selected logits would give 3/10 and 7/10 instead.
    assert abs(float(w[0, 0]) - 0.3) > 0.1


def pin_routing_hand_all(orc):
    d = dims(1, 4, 4, 1, 0, False)
    idx, w, tie = orc.route(d, np.ones((1, 1), np.float32), _hand_router())
    # K = E: every expert, weights s_e / (19/8).
    np.testing.assert_array_equal(idx, [[0, 1, 2, 3]])
    np.testing.assert_array_equal(w, np.array([[6 / 19, 4 / 19, 2 / 19, 7 / 19]], np.float32))
    assert not tie[0]


def pin_routing_equal_logits(orc):
    # Zero router: every score is exactly 1/2; the lowest K indices win; w = 1/K.
    for E, K in ((16, 2), (256, 6), (8, 8)):
        d = dims(32, E, K, 1, 0, False)
        x = _random_x(_rng(E), 5, 32, False)
        idx, w, tie = orc.route(d, x, np.zeros((E, 32), np.float32))
        np.testing.assert_array_equal(idx, np.tile(np.arange(K), (5, 1)))
        np.testing.assert_array_equal(w, np.full((5, K), np.float32(1.0 / K)))
        assert tie.all() == (K < E)


def pin_routing_tie_break(orc):
    # Experts 1 and 2 have identical router rows: only one fits, the lower index wins.
    wr = np.array([[2.0], [1.0], [1.0], [-1.0]], np.float32)
    d = dims(1, 4, 2, 1, 0, False)
    idx, _, tie = orc.route(d, np.ones((1, 1), np.float32), wr)
    np.testing.assert_array_equal(idx, [[0, 1]])
    assert tie[0]  # 2nd and 3rd scores are equal: gap 0 < 1e-5


def pin_routing_limits(orc):
    # z << 0: sigmoid(z) ~ exp(z), so the weights approach a softmax over the
    # selected logits: logits -30 and -30 + ln 2 give weights 1/3 and 2/3.
    d = dims(1, 3, 2, 1, 0, False)
    wr = np.array([[-30.0], [-30.0 + math.log(2.0)], [-40.0]], np.float32)
    _, w, _ = orc.route(d, np.ones((1, 1), np.float32), wr)
    np.testing.assert_allclose(w[0], [1 / 3, 2 / 3], rtol=2e-6)
    # z >> 0: every selected score is 1 in float32, so w = 1/K.
    wr = np.array([[30.0], [25.0], [-1.0]], np.float32)
    _, w, _ = orc.route(d, np.ones((1, 1), np.float32), wr)
    np.testing.assert_array_equal(w[0], np.float32([0.5, 0.5]))


def pin_near_tie_threshold(orc):
    # The near-tie flag marks tokens whose K-th and (K+1)-th float32 scores
    # differ by less than 1e-5.  With x = [1] the logits are the router weights;
    # near 0, sigmoid(-d) = 1/2 - d/4 + O(d^3), so logits 0 and -4g put a gap of
    # g between the two scores (float32 spacing there is 3e-8, far below the
    # 1e-7 margins used).  K = 2 of 4 experts; the boundary is between the
    # expert with logit 0 and the one with logit -4g.
    d = dims(1, 4, 2, 1, 0, False)
    for gap, flagged in ((0.9e-5, True), (1.1e-5, False), (0.5e-5, True), (2e-5, False)):
        wr = np.array([[3.0], [0.0], [-4.0 * gap], [-3.0]], np.float32)
        idx, _, tie = orc.route(d, np.ones((1, 1), np.float32), wr)
        np.testing.assert_array_equal(idx, [[0, 1]])
        assert bool(tie[0]) == flagged, (gap, bool(tie[0]))
    # Only the boundary gap counts: a gap of 4e-6 between the first and second
    # scores, 1.1e-5 at the boundary -> not flagged.
    wr = np.array([[1.6e-5], [0.0], [-4.4e-5], [-3.0]], np.float32)
    _, _, tie = orc.route(d, np.ones((1, 1), np.float32), wr)
    assert not tie[0]
    # K = E: no (K+1)-th score, never flagged, even with equal scores.
    _, _, tie = orc.route(dims(1, 2, 2, 1, 0, False), np.ones((1, 1), np.float32),
                          np.zeros((2, 1), np.float32))
    assert not tie[0]


def pin_routing_subnormal_scores(orc):
    # Below z = -87.3 the sigmoid, e^z / (1 + e^z) ~ e^z, is a float32 subnormal
    # (spacing 2^-149 = 1.4e-45); it stays nonzero down to z ~ -103.3.  Logits
    # -95 and -95 + ln 2 give scores 5.5e-42 and twice that (about 3900 and
    # 7800 subnormal steps), so the weights are 1/3 and 2/3 to within 1e-3
    # (the softmax limit of the sigmoid weights); logit -110 underflows to 0.
    d = dims(1, 3, 2, 1, 0, False)
    wr = np.array([[-95.0], [-95.0 + math.log(2.0)], [-110.0]], np.float32)
    idx, w, _ = orc.route(d, np.ones((1, 1), np.float32), wr)
    np.testing.assert_array_equal(idx, [[0, 1]])
    np.testing.assert_allclose(w[0], [1 / 3, 2 / 3], atol=1e-3)
    s = orc.scores(d, np.ones((1, 1), np.float32), wr)[0]
    assert 0.0 < s[0] < np.finfo(np.float32).tiny and s[2] == 0.0
    np.testing.assert_allclose(s[1] / s[0], 2.0, rtol=1e-3)


def pin_routing_zero_scores(orc):
    # Every logit below -103.3: every float32 score is 0, so all are equal: the
    # lowest K ids are selected and, the normalisation being 0/0, each gets 1/K.
    d = dims(1, 5, 3, 1, 0, False)
    wr = np.array([[-120.0], [-104.5], [-300.0], [-150.0], [-110.0]], np.float32)
    idx, w, tie = orc.route(d, np.ones((1, 1), np.float32), wr)
    np.testing.assert_array_equal(idx, [[0, 1, 2]])
    np.testing.assert_array_equal(w, np.full((1, 3), np.float32(1 / 3)))
    assert tie[0]
    np.testing.assert_array_equal(orc.scores(d, np.ones((1, 1), np.float32), wr), np.zeros((1, 5), np.float32))


def pin_routing_bias(orc):
    # The bias enters the logit: a large bias on expert 2 makes it selected.
    d = dims(1, 4, 1, 1, 0, False)
    idx, w, _ = orc.route(d, np.ones((1, 1), np.float32), _hand_router(),
                          np.array([0, 0, 10.0, 0], np.float32))
    np.testing.assert_array_equal(idx, [[2]])
    np.testing.assert_array_equal(w, [[1.0]])


def pin_routing_library(orc):
    # Scores against torch (float64 matmul and sigmoid), selection against a
    # stable sort: the K first of (score descending, index ascending).
    rng = _rng(3)
    for (T, H, E, K, bias) in ((40, 48, 16, 2, False), (30, 64, 64, 6, True)):
        x = _random_x(rng, T, H, True)
        wr = (rng.standard_normal((E, H)) * 0.2).astype(np.float32)
        b = (rng.standard_normal(E)).astype(np.float32) if bias else None
        d = dims(H, E, K, 1, 0, True)
        idx, w, _ = orc.route(d, x, wr, b)
        z = torch.from_numpy(x).double() @ torch.from_numpy(wr).double().T
        if b is not None:
            z = z + torch.from_numpy(b).double()
        s = torch.sigmoid(z.float().double()).float()
        np.testing.assert_array_equal(orc.scores(d, x, wr, b), s.numpy())
        order = torch.sort(-s.double(), dim=1, stable=True).indices[:, :K]
        ref_idx = torch.sort(order, dim=1).values
        np.testing.assert_array_equal(idx, ref_idx.numpy())
        sel = torch.gather(s.double(), 1, ref_idx)
        np.testing.assert_array_equal(w, (sel / sel.sum(1, keepdim=True)).float().numpy())


# --------------------------------------------------------------------------
# Expert closed form: E = K = 1, H = 2, I = 1.  x = [1, 0], gate row [ln 3, 0],
# up row [2, 0]: g = ln 3 (float32), u = 2, silu(g) = g * sigmoid(g) = (3/4) ln 3,
# h = (3/2) ln 3.  down = [[1], [-1/2]] gives out = [(3/2) ln 3, -(3/4) ln 3].
# A shared expert with gate row [0, ln 3], up row [0, 4], down [[1/4], [1]] on
# x = [1, 1] adds h_s = 3 ln 3 times (1/4, 1).

def pin_expert_closed_form(orc):
    g32 = float(np.float32(_LN3))
    sig = 1.0 / (1.0 + math.exp(-g32))
    w = {"router": np.zeros((1, 2), np.float32),
         "gate": np.array([[[_LN3, 0.0]]], np.float32), "up": np.array([[[2.0, 0.0]]], np.float32),
         "down": np.array([[[1.0], [-0.5]]], np.float32), "bias": None}
    d = dims(2, 1, 1, 1, 0, False)
    out, idx, tw, _ = orc.forward(d, np.array([[1.0, 0.0]], np.float32), w)
    np.testing.assert_array_equal(idx, [[0]])
    np.testing.assert_array_equal(tw, [[1.0]])
    np.testing.assert_allclose(out[0], [1.5 * _LN3, -0.75 * _LN3], rtol=1e-6)
    h = float(np.float32(2.0 * g32 * sig))
    np.testing.assert_array_equal(out[0], np.float32([h, -0.5 * h]))
    # with a shared expert
    w.update({"shared_gate": np.array([[0.0, _LN3]], np.float32),
              "shared_up": np.array([[0.0, 4.0]], np.float32),
              "shared_down": np.array([[0.25], [1.0]], np.float32)})
    d = dims(2, 1, 1, 1, 1, False)
    out, _, _, _ = orc.forward(d, np.array([[1.0, 1.0]], np.float32), w)
    hs = 3.0 * _LN3
    np.testing.assert_allclose(out[0], [1.5 * _LN3 + 0.25 * hs, -0.75 * _LN3 + hs], rtol=1e-6)


def pin_bf16_intermediate(orc):
    # With bf16 h, the same closed form rounds h = (3/2) ln 3 = 1.6479... to the
    # nearest bf16 value, 1.6484375 (211/128), before the down projection.
    w = {"router": np.zeros((1, 2), np.float32),
         "gate": np.array([[[_LN3, 0.0]]], np.float32), "up": np.array([[[2.0, 0.0]]], np.float32),
         "down": np.array([[[1.0], [-0.5]]], np.float32), "bias": None}
    d = dims(2, 1, 1, 1, 0, True)
    out, _, _, _ = orc.forward(d, np.array([[1.0, 0.0]], np.float32), w)
    np.testing.assert_array_equal(out[0], np.float32([211 / 128, -211 / 256]))


# --------------------------------------------------------------------------
# Dense-mixture brute force on tiny, deliberately non-square shapes.

def pin_dense_mixture(orc):
    rng = _rng(5)
    for (T, H, E, K, I, Is, bf16, bias) in ((9, 24, 5, 3, 7, 9, True, False),
                                             (12, 16, 6, 2, 5, 0, False, True),
                                             (7, 20, 4, 4, 3, 6, True, True),
                                             (10, 12, 3, 1, 4, 5, False, False)):
        w = _random_layer(rng, H, E, I, Is, bf16, bias)
        x = _random_x(rng, T, H, bf16)
        d = dims(H, E, K, I, Is, bf16)
        out, idx, tw, _ = orc.forward(d, x, w)
        ref, sets, gate = brute.layer(x, w, K, bf16)
        np.testing.assert_array_equal(idx, sets)
        np.testing.assert_array_equal(tw, np.take_along_axis(gate, sets, 1).astype(np.float32))
        scale = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
        assert np.max(np.abs(out - ref)) <= 1e-6 * scale, np.max(np.abs(out - ref)) / scale


def pin_shared_split(orc):
    # The shared expert is linear in its intermediate channels after the gate:
    # width-2m output = width-m output (first half) + width-m output (second half).
    rng = _rng(8)
    H, E, K, I, Is = 32, 4, 2, 8, 12
    w = _random_layer(rng, H, E, I, Is, True)
    x = _random_x(rng, 6, H, True)
    full, _, _, _ = orc.forward(dims(H, E, K, I, Is, True), x, w)
    routed, _, _, _ = orc.forward(dims(H, E, K, I, 0, True), x, w)
    halves = []
    for sl in (slice(0, Is // 2), slice(Is // 2, Is)):
        wh = dict(w, shared_gate=w["shared_gate"][sl], shared_up=w["shared_up"][sl],
                  shared_down=np.ascontiguousarray(w["shared_down"][:, sl]))
        o, _, _, _ = orc.forward(dims(H, E, K, I, Is // 2, True), x, wh)
        halves.append(o.astype(np.float64) - routed)
    scale = float(np.sqrt(np.mean(full.astype(np.float64) ** 2)))
    assert np.max(np.abs(full - routed - halves[0] - halves[1])) <= 1e-5 * scale


def pin_token_permutation(orc):
    rng = _rng(9)
    H, E, K, I, Is = 16, 6, 2, 4, 4
    w = _random_layer(rng, H, E, I, Is, True, bias=True)
    x = _random_x(rng, 11, H, True)
    d = dims(H, E, K, I, Is, True)
    out, idx, _, _ = orc.forward(d, x, w)
    perm = rng.permutation(11)
    out_p, idx_p, _, _ = orc.forward(d, x[perm], w)
    np.testing.assert_array_equal(out_p, out[perm])
    np.testing.assert_array_equal(idx_p, idx[perm])


# --------------------------------------------------------------------------
# Dispatch: a hand-worked case, invariants, and a library stable sort.

def pin_dispatch_hand(orc):
    g = json.load(open(os.path.join(GOLDEN, "dispatch_hand.json")))
    d = dims(8, g["n_experts"], g["top_k"], 8, 0, True)
    counts, offsets, st, so = orc.dispatch(d, np.array(g["topk_idx"], np.int32))
    np.testing.assert_array_equal(counts, g["counts"])
    np.testing.assert_array_equal(offsets, g["offsets"])
    np.testing.assert_array_equal(st, g["sorted_token"])
    np.testing.assert_array_equal(so, g["slot_of"])


def check_dispatch_invariants(topk_idx, E, counts, offsets, sorted_token, slot_of):
    """Invariants of a correct dispatch (also used on GPU results)."""
    topk_idx = np.asarray(topk_idx)
    T, K = topk_idx.shape
    assert counts.sum() == T * K
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(counts, np.bincount(topk_idx.ravel(), minlength=E))
    assert sorted(slot_of.tolist()) == list(range(T * K))
    for t in range(T):
        for k in range(K):
            s = slot_of[t * K + k]
            e = topk_idx[t, k]
            assert sorted_token[s] == t
            assert offsets[e] <= s < offsets[e + 1]
    for e in range(E):
        seg = sorted_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


def pin_dispatch_invariants(orc):
    rng = _rng(13)
    for (T, E, K) in ((50, 16, 2), (37, 64, 6), (1, 8, 8), (0, 4, 2)):
        idx = np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]) \
            if T else np.zeros((0, K), np.int32)
        d = dims(8, E, K, 8, 0, True)
        counts, offsets, st, so = orc.dispatch(d, idx)
        check_dispatch_invariants(idx, E, counts, offsets, st, so)
        # library: a stable argsort of the flattened expert ids is the same grouping
        flat = idx.reshape(-1)
        order = np.argsort(flat, kind="stable")
        np.testing.assert_array_equal(st, order // K)
        inv = np.empty_like(order)
        inv[order] = np.arange(order.size)
        np.testing.assert_array_equal(so, inv)


# --------------------------------------------------------------------------
# RMSNorm between stacked layers, against torch's rms_norm in float64 then
# torch's bf16 rounding.

def pin_rmsnorm(orc):
    x = np.array([[3.0, 4.0], [1.0, 1.0]], np.float32)
    got = orc.rmsnorm(x, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (2,), eps=1e-6)
    np.testing.assert_array_equal(got, ref.to(torch.bfloat16).float().numpy())
    # Random rows: the float64 library result rounded once to bf16 (numpy's
    # frexp/rint rounding, itself checked against torch in test_oracle_pins).
    x = (_rng(4).standard_normal((7, 96)) * 5).astype(np.float32)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (96,), eps=1e-6)
    np.testing.assert_array_equal(orc.rmsnorm(x, 1e-6), brute.bf16_round(ref.numpy()).astype(np.float32))


# --------------------------------------------------------------------------
# Block-scaled 4-bit weights (OCP Microscaling MXFP4, the format the oracle
# defines for the low-bit workloads): values fixed by the format's definition.

# FP4 E2M1 code -> value, as the OCP MX v1.0 specification tabulates it
# (codes 0-7 positive, 8-15 the same magnitudes negated).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _mx4_row(codes16, scale):
    """One 32-element block (codes16: 32 codes, low-indexed in the low nibble)."""
    c = np.asarray(codes16, np.uint8)
    packed = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)[None, :]
    return packed, np.array([[scale]], np.uint8)


def pin_mx4_element_table(orc):
    codes = list(range(16)) * 2
    q, s = _mx4_row(codes, 127)  # scale 2^0
    got = orc.mx4_dequant(q, s)[0]
    want = np.array(E2M1_TABLE * 2, np.float32)
    np.testing.assert_array_equal(got, want)
    assert all(np.signbit(got[8:16]))  # codes 8-15 carry the sign, including -0


def pin_mx4_scale(orc):
    # E8M0 byte b means 2^(b-127); 255 is NaN.  Code 2 is 1.0, code 7 is 6.0.
    # The decoded value is a float32 product: 6 * 2^127 (b = 254) is past the
    # largest float32 and so decodes to +inf.
    f32_max = float(np.finfo(np.float32).max)
    for b in (0, 1, 100, 127, 200, 254):
        q, s = _mx4_row([2, 7] * 16, b)
        got = orc.mx4_dequant(q, s)[0]
        assert got[0] == np.float32(math.ldexp(1.0, b - 127)), (b, got[0])
        six = 6.0 * math.ldexp(1.0, b - 127)
        assert got[1] == (np.float32(six) if six <= f32_max else np.float32(np.inf)), (b, got[1])
    assert np.isposinf(orc.mx4_dequant(*_mx4_row([7] * 32, 254))[0][0])
    q, s = _mx4_row([2] * 32, 255)
    assert np.all(np.isnan(orc.mx4_dequant(q, s)))


def pin_mx4_layout(orc):
    # Two rows of two blocks each; element 2i in the low nibble of byte i.
    # Row 0: block 0 scale 2^-3, block 1 scale 2^2; row 1: 2^0 and 2^-1.
    # Element j of each block takes code (j + row) % 16.
    scales = np.array([[124, 129], [127, 126]], np.uint8)
    codes = np.zeros((2, 64), np.uint8)
    want = np.zeros((2, 64), np.float32)
    for r in range(2):
        for j in range(64):
            c = (j % 32 + r) % 16
            codes[r, j] = c
            want[r, j] = E2M1_TABLE[c] * 2.0 ** (int(scales[r, j // 32]) - 127)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    np.testing.assert_array_equal(orc.mx4_dequant(packed, scales), want)
    assert packed[0, 0] == 0x10  # hand check of the packing: elements 0 (code 0) and 1 (code 1)


def pin_mx4_tiled_layout(orc):
    # A 32 x 64 matrix is 2 x 2 tiles (16 rows x 32 elements each), stored tile
    # (0,0), (0,1), (1,0), (1,1); a tile holds 16 rows of 16 code bytes, then the
    # next tile.  Hand-placed markers and where the definition puts them:
    #   code byte 0    tile 0, row 0,  byte 0   -> row 0,  byte 0
    #   code byte 255  tile 0, row 15, byte 15  -> row 15, byte 15
    #   code byte 256  tile 1, row 0,  byte 0   -> row 0,  byte 16
    #   code byte 512  tile 2, row 0,  byte 0   -> row 16, byte 0
    #   code byte 786  tile 3, row 1,  byte 2   -> row 17, byte 18 (elements 36, 37)
    #   scale byte 17  tile 1, row 1            -> scales[1][1]
    #   scale byte 40  tile 2, row 8            -> scales[24][0]
    codes_t = np.zeros(2 * 2 * 16 * 16, np.uint8)
    scales_t = np.zeros(2 * 2 * 16, np.uint8)
    marks = {0: (0, 0), 255: (15, 15), 256: (0, 16), 512: (16, 0), 786: (17, 18)}
    for i, flat in enumerate(marks):
        codes_t[flat] = 1 + i
    scales_t[17], scales_t[40] = 200, 201
    c, s = orc.mx4_untile(codes_t.reshape(2, 2, 16, 16), scales_t.reshape(2, 2, 16))
    assert c.shape == (32, 32) and s.shape == (32, 2)
    for i, (flat, (r, b)) in enumerate(marks.items()):
        assert c[r, b] == 1 + i, (flat, r, b)
    assert np.count_nonzero(c) == len(marks)
    assert s[1, 1] == 200 and s[24, 0] == 201 and np.count_nonzero(s) == 2
    # stacked matrices: the second one's first tile is row 32's first bytes
    codes2 = np.zeros((2, 2, 2, 16, 16), np.uint8)
    codes2[1, 0, 0, 0, 0] = 9
    c2, _ = orc.mx4_untile(codes2, np.zeros((2, 2, 2, 16), np.uint8))
    assert c2.shape == (2, 32, 32) and c2[1, 0, 0] == 9 and np.count_nonzero(c2) == 1


DENSE_INTER = 6144  # dense MLP width: not printed; the page's ~75M for two layers fits it


def pin_dense_param_count(orc):
    # two dense layers of the gated three-matrix form at hidden 2048, width 6144:
    # the page's "about 75M" (a two-matrix form would give ~50M)
    g = json.load(open(os.path.join(GOLDEN, "flint_param_counts.json")))
    H, L = g["shape"]["hidden"], g["shape"]["dense_layers"]
    printed = g["printed"]["two_dense_layers_millions"]
    assert round(L * 3 * H * DENSE_INTER / 1e6) == printed
    assert round(L * 2 * H * DENSE_INTER / 1e6) != printed
    # a gated dense layer of this width runs: one token, weights of the right sizes
    rng = np.random.default_rng(0)
    H2, I2 = 64, 96
    x = rng.standard_normal((1, H2)).astype(np.float32)
    out = orc.dense_mlp(x, rng.standard_normal((I2, H2)).astype(np.float32) * 0.1,
                        rng.standard_normal((I2, H2)).astype(np.float32) * 0.1,
                        rng.standard_normal((H2, I2)).astype(np.float32) * 0.1)
    assert out.shape == (1, H2) and np.all(np.isfinite(out))


def pin_dense_closed_form(orc):
    # H = 2, I = 1, x = (1, 0): g = ln 3, u = 2, silu(g) = (3/4) ln 3, h = (3/2) ln 3,
    # down (1, -1/2) -> out = ((3/2) ln 3, -(3/4) ln 3); bf16 h is 211/128.
    x = np.array([[1.0, 0.0]], np.float32)
    wg = np.array([[_LN3, 0.0]], np.float32)
    wu = np.array([[2.0, 0.0]], np.float32)
    wd = np.array([[1.0], [-0.5]], np.float32)
    out = orc.dense_mlp(x, wg, wu, wd, h_bf16=False)
    np.testing.assert_allclose(out[0], [1.5 * _LN3, -0.75 * _LN3], rtol=1e-6)
    out = orc.dense_mlp(x, wg, wu, wd, h_bf16=True)
    np.testing.assert_array_equal(out[0], np.float32([211 / 128, -211 / 256]))
    # tokens are independent: a batch gives each row's single-token result
    rng = np.random.default_rng(5)
    xs = rng.standard_normal((3, 2)).astype(np.float32)
    batch = orc.dense_mlp(xs, wg, wu, wd)
    for t in range(3):
        np.testing.assert_array_equal(batch[t], orc.dense_mlp(xs[t:t + 1], wg, wu, wd)[0])


def pin_dense_is_the_shared_expert_alone(orc):
    # a MoE layer whose routed experts are all zero is its shared expert alone,
    # i.e. a dense MLP with the shared expert's weights
    rng = np.random.default_rng(9)
    T, H, E, K, I, Is = 5, 32, 4, 2, 16, 48
    w = {"router": rng.standard_normal((E, H)).astype(np.float32), "bias": None,
         "gate": np.zeros((E, I, H), np.float32), "up": np.zeros((E, I, H), np.float32),
         "down": np.zeros((E, H, I), np.float32),
         "shared_gate": rng.standard_normal((Is, H)).astype(np.float32) * 0.2,
         "shared_up": rng.standard_normal((Is, H)).astype(np.float32) * 0.2,
         "shared_down": rng.standard_normal((H, Is)).astype(np.float32) * 0.2}
    x = rng.standard_normal((T, H)).astype(np.float32)
    layer, _, _, _ = orc.forward(dims(H, E, K, I, Is, True), x, w)
    dense = orc.dense_mlp(x, w["shared_gate"], w["shared_up"], w["shared_down"], h_bf16=True)
    np.testing.assert_array_equal(layer, dense)


ALL_PINS = [pin_param_counts, pin_bf16_rounding, pin_routing_hand_top2, pin_routing_hand_all,
            pin_routing_equal_logits, pin_routing_tie_break, pin_near_tie_threshold,
            pin_routing_subnormal_scores, pin_routing_zero_scores, pin_routing_limits, pin_routing_bias,
            pin_routing_library, pin_expert_closed_form, pin_bf16_intermediate, pin_dense_mixture,
            pin_shared_split, pin_token_permutation, pin_dispatch_hand, pin_dispatch_invariants,
            pin_rmsnorm, pin_mx4_element_table, pin_mx4_scale, pin_mx4_layout, pin_mx4_tiled_layout,
            pin_dense_param_count, pin_dense_closed_form, pin_dense_is_the_shared_expert_alone]
