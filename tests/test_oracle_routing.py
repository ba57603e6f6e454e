"""Pins for the oracle's fan-in, top-k routing and dispatch plan (CPU only).

Each check ties the oracle to something other than itself: a closed form, an
invariant the selection must satisfy, or a library routine the pages name
(softmax, stable argsort, bincount, cumsum -- "[RFC]: Async GPU Connector",
section "Data flow"; fan-in/split -- "Data on the wire", Steps 2-4).
"""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

from combine_afd_slot_amd.inputs import WORKLOADS, make_inputs, fanin4_seq_lens, FANIN4_SEQ_LENS


def _rank_key(l):
    # library stable sort: primary key larger logit, secondary lower index
    return np.lexsort((np.arange(l.shape[0]), -l.astype(np.float64)))


# ----------------------------------------------------------------- fan-in
def test_fanin_offsets_are_exclusive_scan(orc):
    seq = [7, 0, 13, 1]
    off = orc.fanin(seq)
    assert off.tolist() == [0, 7, 7, 20, 21]
    assert off[-1] == sum(seq)  # total_tokens = sum(seq_lens)


def test_fanin_capacity_rejected(orc):
    with pytest.raises(ValueError):
        orc.fanin([5, 17], token_cap=16)
    with pytest.raises(ValueError):
        orc.fanin([-1, 3])


def test_fanin4_lengths_follow_recipe():
    assert fanin4_seq_lens(0) == FANIN4_SEQ_LENS
    assert sum(FANIN4_SEQ_LENS) == 14196


# ----------------------------------------------------------------- routing
@pytest.mark.parametrize("E,K", [(8, 2), (64, 6), (256, 8), (5, 5), (3, 1)])
def test_route_invariants(orc, E, K):
    rng = np.random.default_rng(E * 31 + K)
    L = rng.standard_normal((300, E), dtype=np.float32)
    # force ties in a third of the rows
    L[::3] = np.round(L[::3] * 2) / 2
    ids, w = orc.route(L, K)
    for t in range(L.shape[0]):
        l, sel = L[t], ids[t]
        assert len(set(sel.tolist())) == K
        vals = l[sel]
        assert np.all(vals[:-1] >= vals[1:])
        for a, b in zip(sel[:-1], sel[1:]):
            assert l[a] > l[b] or (l[a] == l[b] and a < b)
        last = sel[-1]
        for e in set(range(E)) - set(sel.tolist()):
            assert l[e] < l[last] or (l[e] == l[last] and e > last)
        assert sel.tolist() == _rank_key(l)[:K].tolist()
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_route_subset_brute_force_tiny(orc):
    # every K-subset of E=8 experts: the chosen set is the one with the largest
    # logit sum, unique when logits are distinct
    inp = make_inputs(WORKLOADS["tiny"], with_weights=False)
    L = inp["L"]
    ids, _ = orc.route(L, 2)
    for t in range(L.shape[0]):
        best = max(itertools.combinations(range(8), 2), key=lambda s: sum(float(L[t, e]) for e in s))
        assert sorted(ids[t].tolist()) == sorted(best)


def test_route_all_equal_ties(orc):
    L = np.full((4, 16), 0.25, dtype=np.float32)
    ids, w = orc.route(L, 5)
    assert (ids == np.arange(5)).all()
    assert (w == 0.2).all()


def test_route_negative_zero_ties_positive_zero(orc):
    L = np.full((1, 6), -3.0, dtype=np.float32)
    L[0, 4] = 0.0
    L[0, 1] = -0.0
    ids, w = orc.route(L, 2)
    assert ids[0].tolist() == [1, 4]  # equal values: lower index first
    assert w[0, 0] == w[0, 1] == 0.5


def test_route_k_equals_e_is_softmax(orc):
    rng = np.random.default_rng(3)
    L = rng.standard_normal((50, 12), dtype=np.float32) * 3
    ids, w = orc.route(L, 12)
    ref = softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids, axis=1), rtol=1e-13, atol=1e-16)


def test_route_k1_unit_weight(orc):
    rng = np.random.default_rng(4)
    L = rng.standard_normal((40, 9), dtype=np.float32)
    ids, w = orc.route(L, 1)
    assert (ids[:, 0] == L.argmax(axis=1)).all()
    assert (w == 1.0).all()


def test_route_renormalized_matches_softmax_restricted(orc):
    rng = np.random.default_rng(5)
    L = rng.standard_normal((64, 64), dtype=np.float32)
    ids, w = orc.route(L, 6, renorm=1)
    sm = softmax(L.astype(np.float64), axis=1)
    top = np.take_along_axis(sm, ids, axis=1)
    np.testing.assert_allclose(w, top / top.sum(axis=1, keepdims=True), rtol=1e-12)
    ids0, w0 = orc.route(L, 6, renorm=0)
    assert (ids0 == ids).all()
    np.testing.assert_allclose(w0, top, rtol=1e-12)


def test_route_rejects_nonfinite(orc):
    L = np.zeros((2, 4), dtype=np.float32)
    L[1, 2] = np.nan
    with pytest.raises(ValueError):
        orc.route(L, 2)


# ----------------------------------------------------------------- dispatch
@pytest.mark.parametrize("T,E,K", [(20, 8, 2), (1000, 64, 6), (257, 256, 8), (0, 4, 2), (33, 7, 7)])
def test_dispatch_is_stable_argsort(orc, T, E, K):
    rng = np.random.default_rng(T + E + K)
    # skewed ids so that some experts are empty
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]) if T else np.zeros((0, K), np.int32)
    ids = np.where(rng.random(ids.shape) < 0.3, ids % max(1, E // 3), ids).astype(np.int32)
    # rows must still hold distinct ids for a top-k; the plan does not need it,
    # so the skew may repeat ids inside a row, which the stable order handles
    counts, eoff, perm, inv = orc.dispatch(ids, E)
    flat = ids.reshape(-1)
    assert (counts == np.bincount(flat, minlength=E)).all()
    assert eoff.tolist() == [0] + np.cumsum(counts).tolist()
    assert (perm == np.argsort(flat, kind="stable")).all()
    assert (inv[perm] == np.arange(T * K)).all()
    assert (perm[inv] == np.arange(T * K)).all()
    for e in range(E):
        grp = perm[eoff[e]:eoff[e + 1]]
        assert (flat[grp] == e).all()
        assert (np.diff(grp) > 0).all()
    assert counts.sum() == T * K
