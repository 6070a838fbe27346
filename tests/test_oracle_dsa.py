"""Pins of the sparse-attention oracle (indexer scores, top-k selection,
attention over selected rows): brute force, reductions to the dense MLA
forms, invariants, and planted mistakes that the pins must catch."""
import itertools

import numpy as np
import pytest

from oracle import dsa as D
from oracle import model as M

RNG = np.random.default_rng(23)


def brute_scores(q, w, K):
    """Pure-Python loops: sum over heads of weight * max(0, dot)."""
    out = []
    for s in range(K.shape[0]):
        tot = 0.0
        for j in range(q.shape[0]):
            dot = 0.0
            for i in range(q.shape[1]):
                dot += float(q[j, i]) * float(K[s, i])
            tot += float(w[j]) * (dot if dot > 0.0 else 0.0)
        out.append(tot)
    return np.array(out)


def brute_topk(scores, k):
    """Every subset of size min(k, n) ranked: the chosen set has the largest
    sorted score vector, and among equal ones the smallest positions."""
    n = len(scores)
    best = None
    for sub in itertools.combinations(range(n), min(k, n)):
        key = (sorted((scores[i] for i in sub), reverse=True), [-i for i in sub])
        if best is None or key > best[0]:
            best = (key, sub)
    return np.array(best[1], np.int64)


def pin_index_scores(fn=D.index_scores):
    for HI, dI, n in ((1, 4, 3), (3, 5, 7), (4, 8, 11)):
        q, w, K = RNG.standard_normal((HI, dI)), RNG.standard_normal(HI), RNG.standard_normal((n, dI))
        np.testing.assert_allclose(fn(q, w, K), brute_scores(q, w, K), rtol=1e-12, atol=1e-12)
    # a head whose dots are all negative contributes nothing
    K = np.abs(RNG.standard_normal((6, 4)))
    q = np.vstack([np.abs(RNG.standard_normal(4)), -np.abs(RNG.standard_normal(4))])
    w = np.array([0.5, 100.0])
    np.testing.assert_allclose(fn(q, w, K), 0.5 * (K @ q[0]), rtol=1e-12)
    # linear in the weights, positively homogeneous in the queries
    q, w, K = RNG.standard_normal((3, 6)), RNG.standard_normal(3), RNG.standard_normal((9, 6))
    np.testing.assert_allclose(fn(q, 2.5 * w, K), 2.5 * fn(q, w, K), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fn(3.0 * q, w, K), 3.0 * fn(q, w, K), rtol=1e-12, atol=1e-12)


def test_index_scores():
    pin_index_scores()


def pin_select_topk(fn=D.select_topk):
    # brute force over every subset, with and without ties
    for n, k in ((1, 1), (5, 2), (6, 3), (7, 7), (4, 9), (8, 1)):
        for trial in range(3):
            s = RNG.integers(-2, 3, n).astype(np.float64) if trial else RNG.standard_normal(n)
            np.testing.assert_array_equal(fn(s, k), brute_topk(s, k))
    # all equal: the first k positions
    np.testing.assert_array_equal(fn(np.zeros(10), 4), np.arange(4))
    # strictly increasing: the last k positions, ascending
    np.testing.assert_array_equal(fn(np.arange(10.0), 3), np.array([7, 8, 9]))
    # k >= n: every position
    np.testing.assert_array_equal(fn(RNG.standard_normal(5), 5), np.arange(5))
    # -0.0 and +0.0 are equal scores: the lower position wins
    np.testing.assert_array_equal(fn(np.array([-1.0, 0.0, -0.0, -2.0]), 2), np.array([1, 2]))
    np.testing.assert_array_equal(fn(np.array([-0.0, -1.0, 0.0]), 1), np.array([0]))
    # the router's top-k (already pinned) picks the same set
    s = RNG.standard_normal(300)
    np.testing.assert_array_equal(fn(s, 37), np.sort(M.topk_indices(s, 37)))


def test_select_topk():
    pin_select_topk()


def pin_sparse_mla(fn=D.sparse_mla):
    H, dn, dr, dc, dv, T = 3, 5, 4, 6, 7, 13
    tau = 0.31
    qn, qp = RNG.standard_normal((H, dn)), RNG.standard_normal((H, dr))
    C, R = RNG.standard_normal((T, dc)), RNG.standard_normal((T, dr))
    W_UK, W_UV = RNG.standard_normal((H, dn, dc)), RNG.standard_normal((H, dv, dc))
    q_lat = np.einsum("hnc,hn->hc", W_UK, qn)
    # every position selected: the explicit per-head keys and values of the naive form
    o_naive, _ = M.mla_naive(qn, qp, C, R, W_UK, W_UV, tau)
    o_lat = fn(q_lat, qp, C, R, np.arange(T), tau)
    np.testing.assert_allclose(np.einsum("hvc,hc->hv", W_UV, o_lat), o_naive, rtol=1e-10, atol=1e-12)
    # a subset equals the naive form over the gathered cache, whatever its order
    sel = np.array([11, 2, 7, 0, 5])
    o_sub, _ = M.mla_naive(qn, qp, C[sel], R[sel], W_UK, W_UV, tau)
    for order in (sel, sel[::-1], np.sort(sel)):
        np.testing.assert_allclose(np.einsum("hvc,hc->hv", W_UV, fn(q_lat, qp, C, R, order, tau)), o_sub,
                                   rtol=1e-10, atol=1e-12)
    # one selected position: its latent row, for every head
    np.testing.assert_allclose(fn(q_lat, qp, C, R, np.array([9]), tau), np.tile(C[9], (H, 1)), rtol=1e-14)
    # equal scores on two rows: their mean
    Z = np.zeros((2, dc)); Z[0, 0], Z[1, 1] = 1.0, 1.0
    out = fn(np.zeros((1, dc)), np.zeros((1, dr)), Z, np.zeros((2, dr)), np.array([0, 1]), tau)
    np.testing.assert_allclose(out[0, :2], [0.5, 0.5], rtol=1e-14)


def test_sparse_mla():
    pin_sparse_mla()


def test_dsa_decode_composes_the_three():
    HI, dI, T, H, dc, dr = 4, 8, 40, 2, 6, 4
    q, w, K = RNG.standard_normal((HI, dI)), RNG.random(HI), RNG.standard_normal((T, dI))
    ql, qp = RNG.standard_normal((H, dc)), RNG.standard_normal((H, dr))
    C, R = RNG.standard_normal((T, dc)), RNG.standard_normal((T, dr))
    o, sel, sc = D.dsa_decode(q, w, K, ql, qp, C, R, 9, 0.4)
    np.testing.assert_allclose(sc, brute_scores(q, w, K), rtol=1e-12, atol=1e-12)
    assert len(sel) == 9 and np.all(np.diff(sel) > 0)
    assert sc[sel].min() >= np.delete(sc, sel).max()
    np.testing.assert_allclose(o, D.sparse_mla(ql, qp, C, R, sel, 0.4), rtol=1e-14)


PLANTED = {
    "index_scores": (pin_index_scores, [
        lambda q, w, K: np.maximum(K @ q.T, 0.0) @ w * 1.0001,                       # scale slip
        lambda q, w, K: (K @ q.T) @ w,                                               # ReLU dropped
        lambda q, w, K: np.maximum((K @ q.T) @ np.ones(q.shape[0]) * w.mean(), 0.0),  # ReLU after the sum
    ]),
    "select_topk": (pin_select_topk, [
        lambda s, k: np.sort(np.argsort(-s)[:k]),                                     # unstable ties
        lambda s, k: np.sort(np.argsort(s)[:k]),                                      # smallest instead
        lambda s, k: np.argsort(-np.asarray(s), kind="stable")[:k],                   # not ascending
        lambda s, k: np.sort(np.lexsort((-np.arange(len(s)), -np.asarray(s)))[:k]),   # ties to the higher
    ]),
    "sparse_mla": (pin_sparse_mla, [
        lambda ql, qp, C, R, sel, tau: D.sparse_mla(ql, qp, C, R, np.sort(sel)[:-1] if len(sel) > 2 else sel, tau),
        lambda ql, qp, C, R, sel, tau: D.sparse_mla(ql, -qp, C, R, sel, tau),         # rotary sign
        lambda ql, qp, C, R, sel, tau: D.sparse_mla(ql, qp, C, R, sel, 1.0),           # scale dropped
    ]),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_mistakes_are_caught(name):
    pin, bad = PLANTED[name]
    for f in bad:
        with pytest.raises(AssertionError):
            pin(fn=f)
