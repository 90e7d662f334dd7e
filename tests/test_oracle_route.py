"""Pins for the oracle's routing (CPU only).

What the routing must satisfy comes from the grouping recipe of the article on
Unsloth x NVIDIA optimisations ("Optimisation 3: MoE routing grouped once"):
counts from one bincount over all T*k assignments, offsets from the counts, a
stable sort by expert id, and the same per-expert token lists as the
per-expert search loop it replaces.  Top-k is checked against a brute-force
Python sort, the weights against scipy's softmax.
"""
import numpy as np
import pytest
import scipy.special

import oracle
from synth import CONFIGS, LayerDims, make_logits

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _brute_topk(L, k):
    T, E = L.shape
    return np.array([sorted(range(E), key=lambda e: (-float(L[t, e]), e))[:k] for t in range(T)],
                    dtype=np.int32)


@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (33, 16, 5), (7, 4, 4), (5, 1, 1), (64, 32, 1)])
def test_topk_matches_brute_force_with_ties(T, E, k):
    rng = np.random.default_rng(1)
    # small integer logits force many ties; tie -> lower expert id first
    L = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    ids, w = oracle.topk_softmax(L, k)
    np.testing.assert_array_equal(ids, _brute_topk(L, k))
    # signed zeros compare equal, so they tie too
    L2 = np.where(L == 0, np.float32(-0.0), L)
    np.testing.assert_array_equal(oracle.topk_softmax(L2, k)[0], ids)


def test_topk_continuous_matches_brute_force():
    L = make_logits(CONFIGS["tiny"])
    np.testing.assert_array_equal(oracle.topk_softmax(L, 2)[0], _brute_topk(L, 2))


def test_weights_softmax_of_selected():
    L = make_logits(CONFIGS["tiny"])
    for k in (1, 2, 5, 8):
        ids, w = oracle.topk_softmax(L, k)
        assert w.dtype == np.float32
        np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-6)
        # softmax over all E, then keep the selected ones and renormalise
        full = scipy.special.softmax(L.astype(np.float64), axis=1)
        sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
        np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-6)
        assert np.all(np.diff(w, axis=1) <= 0)  # descending, like the logits
    # k = 1: the single weight is exactly one
    assert np.all(oracle.topk_softmax(L, 1)[1] == 1.0)
    # k = E: the full softmax, permuted into descending order
    ids, w = oracle.topk_softmax(L, 8)
    full = scipy.special.softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-6)


def _check_routing(ids, E):
    T, k = ids.shape
    R = oracle.route(ids, E)
    flat = ids.reshape(-1)
    # counts: one bincount; cross-check with a plain loop
    assert int(R.counts.sum()) == T * k
    for e in range(E):
        assert R.counts[e] == sum(1 for v in flat.tolist() if v == e)
    # offsets: exclusive prefix of counts, length E+1
    assert R.offsets.shape == (E + 1,) and R.offsets[0] == 0 and R.offsets[E] == T * k
    np.testing.assert_array_equal(np.diff(R.offsets), R.counts)
    # a permutation with its inverse
    assert sorted(R.sorted_pair.tolist()) == list(range(T * k))
    np.testing.assert_array_equal(R.pair_pos[R.sorted_pair], np.arange(T * k))
    naive = oracle.route_naive(ids, E)
    for e in range(E):
        seg = R.sorted_pair[R.offsets[e]:R.offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)  # stable
        tok, slot = naive[e]
        # same tokens in the same order as the per-expert search loop
        np.testing.assert_array_equal(seg // k, tok)
        np.testing.assert_array_equal(seg % k, slot)
    return R


@pytest.mark.parametrize("dims", [CONFIGS["tiny"],
                                  LayerDims(100, 64, 64, 16, 1, 4),
                                  LayerDims(9, 64, 64, 6, 6, 4),
                                  LayerDims(1, 64, 64, 5, 3, 4),
                                  LayerDims(40, 64, 64, 1, 1, 4)])
def test_route_invariants(dims):
    ids, _ = oracle.topk_softmax(make_logits(dims, seed=3), dims.k)
    _check_routing(ids, dims.E)


def test_route_all_tokens_one_expert():
    L = np.zeros((20, 6), np.float32)
    L[:, 4] = 5.0
    ids, w = oracle.topk_softmax(L, 2)
    assert np.all(ids[:, 0] == 4) and np.all(ids[:, 1] == 0)
    R = _check_routing(ids, 6)
    assert R.counts.tolist() == [20, 0, 0, 0, 20, 0]


def test_stress_recipe_skew():
    dims = LayerDims(512, 64, 64, 128, 8, 4, logits_recipe="stress")
    ids, w = oracle.topk_softmax(make_logits(dims), 8)
    R = _check_routing(ids, 128)
    c = np.sort(R.counts)[::-1]
    assert c[:4].tolist() == [512] * 4          # 4 hot experts take every token
    assert int(c[:4].sum()) * 2 == 512 * 8      # = half of all assignments
    assert int((R.counts == 0).sum()) == 16     # 16 empty experts
    assert np.all(w > 0) and np.all(w < 1)


def test_zipf_recipe_marginals():
    dims = LayerDims(20000, 64, 64, 32, 4, 4, logits_recipe="zipf")
    L = make_logits(dims)
    ids, _ = oracle.topk_softmax(L, 4)
    H = sum(i ** -1.1 for i in range(1, 33))
    p_top, p_last = 1.0 / H, 32 ** -1.1 / H
    assert abs(p_top - 0.284) < 1e-3 and abs(p_last - 0.0063) < 1e-4
    # Gumbel-top-k: the first pick is expert e with probability p_e
    first = np.bincount(ids[:, 0], minlength=32) / dims.T
    assert abs(first.max() - p_top) < 0.015


def _brute_topk_nan(L, k):
    """Full per-row sort with NaN below every number (-inf included)."""
    T, E = L.shape

    def key(t, e):
        v = float(L[t, e])
        return (0, 0.0, e) if v != v else (-1, -v, e)
    return np.array([sorted(range(E), key=lambda e: key(t, e))[:k] for t in range(T)],
                    dtype=np.int32)


def test_topk_nan_and_infinite_logits():
    rng = np.random.default_rng(11)
    L = rng.normal(size=(40, 12)).astype(np.float32)
    L[0] = np.nan                                  # a diverged router row
    L[1, :10] = np.nan                             # fewer finite logits than k
    L[2, [3, 7]] = -np.inf
    L[2, [1, 5]] = np.nan                          # NaN below -inf
    L[3, 4] = np.inf
    L[4, ::2] = np.nan
    L[5] = -np.inf
    for k in (1, 3, 4, 12):
        ids, w = oracle.topk_softmax(L, k)
        np.testing.assert_array_equal(ids, _brute_topk_nan(L, k))
        assert ids.min() >= 0 and ids.max() < 12
        R = oracle.route(ids, 12)
        assert int(R.counts.sum()) == 40 * k
        fin = np.all(np.isfinite(np.take_along_axis(L, ids.astype(np.int64), 1)), axis=1)
        assert np.all(np.isfinite(w[fin]))
        np.testing.assert_allclose(w[fin].sum(axis=1), 1.0, atol=1e-6)
    ids, _ = oracle.topk_softmax(L, 3)
    assert ids[0].tolist() == [0, 1, 2]            # all NaN: lowest ids
    assert ids[1].tolist() == [10, 11, 0]          # the two numbers, then the lowest NaN
    assert ids[2, 2] not in (1, 5)


@pytest.mark.parametrize("S", [0, 1])
def test_gather_rows_follow_the_per_expert_search(S):
    dims = LayerDims(37, 64, 64, 7, 3, 4, n_shared=S)
    ids, w = oracle.topk_softmax(make_logits(dims, seed=4), dims.k)
    R = oracle.route(ids, dims.E)
    tok, wgt = oracle.gather_rows(R, w, dims.T, dims.k, S)
    assert tok.shape == (dims.P_tot,) and wgt.shape == (dims.P_tot,)
    for e, (t_e, s_e) in enumerate(oracle.route_naive(ids, dims.E)):
        seg = slice(R.offsets[e], R.offsets[e + 1])
        np.testing.assert_array_equal(tok[seg], t_e)
        np.testing.assert_array_equal(wgt[seg], w[t_e, s_e])
    if S:
        np.testing.assert_array_equal(tok[dims.P:], np.arange(dims.T))
        assert np.all(wgt[dims.P:] == 1.0)
