"""The routing comparison the GPU parity tests use (gpu_common.check_routing),
checked on the CPU with hand-made scores: it must accept a different set only
where the oracle flags a near tie AND the other set is itself a top-K set of
the oracle's scores with weights renormalised over it, and reject the rest."""
import numpy as np
import pytest

import gpu_common as G

# One token, E = 6, K = 2.  Oracle scores: experts 3 and 1 on top, expert 5
# 0.6e-5 below expert 1 (a near tie), experts 0, 2, 4 far below.
SC = np.array([[0.20, 0.700000, 0.10, 0.90, 0.05, 0.699994]], np.float32)
ORA_IDX = np.array([[1, 3]])
ORA_W = (SC[0, [1, 3]] / SC[0, [1, 3]].sum()).astype(np.float32)[None]
TIE = np.array([True])


def scores_of(rows):
    return SC[np.asarray(rows)]


def _w(sel):
    s = SC[0, sel].astype(np.float64)
    return (s / s.sum()).astype(np.float32)[None]


def test_same_set_passes():
    assert G.check_routing(ORA_IDX, ORA_W, ORA_IDX, ORA_W, TIE, "same", scores_of) == 0


def test_valid_near_tie_swap_passes():
    sel = np.array([[3, 5]])
    assert G.check_routing(sel, _w([3, 5]), ORA_IDX, ORA_W, TIE, "swap", scores_of) == 1


def test_invalid_set_on_a_near_tie_token_is_rejected():
    # expert 0 is far below the K-th score: not a correct answer even though the
    # token is a near tie
    sel = np.array([[0, 3]])
    with pytest.raises(AssertionError, match="not a top-2 set|not within"):
        G.check_routing(sel, _w([0, 3]), ORA_IDX, ORA_W, TIE, "bad", scores_of)


def test_swap_of_the_top_expert_is_rejected():
    # experts 1 and 5 (dropping the clear winner 3): selected min 0.699994 is below
    # the unselected 0.9
    sel = np.array([[1, 5]])
    with pytest.raises(AssertionError):
        G.check_routing(sel, _w([1, 5]), ORA_IDX, ORA_W, TIE, "top", scores_of)


def test_wrong_weights_on_the_other_set_are_rejected():
    sel = np.array([[3, 5]])
    with pytest.raises(AssertionError, match="weights off"):
        G.check_routing(sel, ORA_W[:, ::-1].copy(), ORA_IDX, ORA_W, TIE, "weights", scores_of)


def test_differing_set_without_near_tie_is_rejected():
    sel = np.array([[3, 5]])
    with pytest.raises(AssertionError, match="without a near tie"):
        G.check_routing(sel, _w([3, 5]), ORA_IDX, ORA_W, np.array([False]), "notie", scores_of)


def test_differing_set_needs_the_scores():
    sel = np.array([[3, 5]])
    with pytest.raises(AssertionError, match="scores are needed"):
        G.check_routing(sel, _w([3, 5]), ORA_IDX, ORA_W, TIE, "noscores", None)


def test_all_zero_scores_take_equal_weights():
    sc = np.zeros((1, 4), np.float32)
    idx = np.array([[0, 1]])
    w = np.full((1, 2), 0.5, np.float32)
    # the oracle's own set: lowest ids; a GPU set {0, 2} is equally valid (all equal)
    assert G.check_routing(np.array([[0, 2]]), w, idx, w, np.array([True]), "zeros", lambda r: sc[r]) == 1
