"""The routing acceptance rule itself (CPU only).

tests/paritylib.check_routing decides whether a GPU routing is acceptable
against the oracle's float64 selection scores.  Every planted wrong routing
below must be rejected, and the oracle's own routing plus a legitimate
near-tie swap must be accepted.
"""
import numpy as np
import pytest

import oracle
import paritylib as P

SCALE = 2.5


def _routing(sel_rows, k):
    """An oracle.Routing for hand-written selection scores (zero bias, so the
    sigmoid scores equal the selection scores)."""
    sel = np.asarray(sel_rows, dtype=np.float64)
    T, E = sel.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -sel), axis=1)
    idx = order[:, :k]
    ranked = np.take_along_axis(sel, order, axis=1)
    margin = ranked[:, k - 1] - ranked[:, k] if k < E else np.full(T, np.inf)
    chosen = np.take_along_axis(sel, idx, axis=1)
    w = SCALE * chosen / chosen.sum(axis=1, keepdims=True)
    return oracle.Routing(idx=idx, w=w, s=sel.copy(), sel=sel, margin=margin)


def _weights(ref, idx):
    s = np.take_along_axis(ref.s, np.asarray(idx), axis=1)
    return SCALE * s / s.sum(axis=1, keepdims=True)


# Token 0: a near tie between experts 3, 4 and 5 (margin 5e-5 <= 1e-4) with a
# clear winner, expert 0.  Token 1: a clear token (margin 0.1).
SEL = [[0.9, 0.8, 0.7, 0.60005, 0.60000, 0.59995],
       [0.1, 0.9, 0.3, 0.8, 0.7, 0.6]]
K = 4


def test_oracle_routing_is_accepted():
    ref = _routing(SEL, K)
    assert ref.margin[0] <= P.MARGIN < ref.margin[1]
    rc = P.check_routing(ref.idx, ref.w, ref, SCALE)
    assert rc.near_ties == 1 and rc.differing_sets == 0


def test_near_tie_swap_within_margin_is_accepted():
    ref = _routing(SEL, K)
    idx = ref.idx.copy()
    idx[0] = [0, 1, 2, 4]  # expert 4 (0.60000) for expert 3 (0.60005): within MARGIN
    rc = P.check_routing(idx, _weights(ref, idx), ref, SCALE)
    assert rc.differing_sets == 1
    np.testing.assert_array_equal(rc.effective_idx[0], [0, 1, 2, 4])


def test_near_tie_order_swap_within_margin_is_accepted():
    ref = _routing([[0.9, 0.8, 0.70004, 0.70000, 0.5, 0.1]], 3)
    idx = np.array([[0, 1, 3]])  # 0.70000 ahead of nothing it trails by > MARGIN
    P.check_routing(idx, _weights(ref, idx), ref, SCALE)
    idx = np.array([[0, 3, 1]])  # 3 (0.70000) before 1 (0.8): an inversion of 0.1
    with pytest.raises(AssertionError):
        P.check_routing(idx, _weights(ref, idx), ref, SCALE)


@pytest.mark.parametrize("case", ["drop_top_on_near_tie", "wrong_order_clear", "repeated_id",
                                  "other_set_clear", "tie_index_order"])
def test_planted_wrong_routing_is_rejected(case):
    ref = _routing(SEL, K)
    idx = ref.idx.copy()
    if case == "drop_top_on_near_tie":
        # Every chosen score is within MARGIN of the k-th, yet the clear winner
        # (0.9) is left out.
        idx[0] = [1, 2, 3, 4]
    elif case == "wrong_order_clear":
        idx[1] = [3, 1, 4, 5]  # 0.8 reported ahead of 0.9
    elif case == "repeated_id":
        idx[1] = [1, 1, 3, 4]
    elif case == "other_set_clear":
        idx[1] = [1, 3, 4, 2]  # expert 2 (0.3) for expert 5 (0.6) on a clear token
    elif case == "tie_index_order":
        ref = _routing([[0.5, 0.5, 0.5, 0.5, 0.1]], 2)  # exact ties: lower index first
        idx = np.array([[1, 0]])
    w = _weights(ref, idx) if case != "repeated_id" else ref.w
    with pytest.raises(AssertionError):
        P.check_routing(idx, w, ref, SCALE)


def test_weights_must_follow_reported_order():
    ref = _routing(SEL, K)
    w = ref.w.copy()
    w[1] = w[1][::-1]  # right set and order, weights reversed
    with pytest.raises(AssertionError):
        P.check_routing(ref.idx, w, ref, SCALE)
