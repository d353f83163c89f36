"""Pins for the oracle's routing (top-K + renormalised softmax) and permutation."""
import numpy as np

from oracle import reference as R


def _logits(rng, T, E, ties=True):
    l = rng.standard_normal((T, E)).astype(np.float32)
    if ties:  # plant exact ties, including at the K-th place
        l[::3, 1] = l[::3, E - 1]
        l[1::4, :4] = 0.25
    return l


def test_topk_matches_brute_force_sort():
    rng = np.random.default_rng(10)
    for T, E, K in [(50, 8, 2), (40, 64, 6), (20, 256, 8), (8, 5, 5)]:
        l = _logits(rng, T, E)
        ids, p = R.route(l, K)
        for t in range(T):
            # stable sort on (-logit, expert id)
            order = sorted(range(E), key=lambda e: (-float(l[t, e]), e))
            assert list(ids[t]) == order[:K]


def test_weights_properties():
    rng = np.random.default_rng(11)
    l = _logits(rng, 64, 32, ties=False)
    ids, p = R.route(l, 6)
    assert np.all(np.abs(p.sum(1) - 1.0) < 1e-14)
    assert np.all(np.diff(p, axis=1) <= 0)
    # exp ratios between chosen experts are fixed by the logits
    t = 7
    r = p[t, 0] / p[t, 3]
    assert abs(r / np.exp(float(l[t, ids[t, 0]]) - float(l[t, ids[t, 3]])) - 1) < 1e-13


def test_uniform_when_all_logits_equal():
    for E in (2, 8, 64):
        ids, p = R.route(np.zeros((3, E), np.float32), E)
        assert np.all(ids == np.arange(E)) and np.all(p == 1.0 / E)


def test_k1_weight_is_one():
    rng = np.random.default_rng(12)
    ids, p = R.route(_logits(rng, 10, 16), 1)
    assert np.all(p == 1.0)


def test_permutation_invariants():
    rng = np.random.default_rng(13)
    for T, E, K in [(64, 8, 2), (33, 256, 8), (1, 4, 4), (100, 16, 1)]:
        ids, _ = R.route(_logits(rng, T, E), K)
        counts, offsets, r2r, rt2row = R.permute(ids, E)
        Rn = T * K
        assert offsets[0] == 0 and offsets[E] == Rn and np.all(np.diff(offsets) == counts)
        assert np.array_equal(np.sort(r2r), np.arange(Rn))
        assert np.array_equal(rt2row[r2r], np.arange(Rn))
        flat = ids.ravel()
        assert np.array_equal(np.bincount(flat, minlength=E), counts)
        # rows are grouped by expert, tokens ascending inside a group
        assert np.all(np.diff(flat[r2r]) >= 0)
        for e in range(E):
            seg = r2r[offsets[e]:offsets[e + 1]]
            assert np.all(np.diff(seg) > 0)
        # equals a stable sort of the routes by expert
        assert np.array_equal(r2r, np.argsort(flat, kind="stable"))


def test_permutation_degenerate_one_expert():
    T, E, K = 9, 8, 1
    l = np.zeros((T, E), np.float32)
    l[:, 3] = 5.0
    ids, _ = R.route(l, K)
    counts, offsets, r2r, rt2row = R.permute(ids, E)
    assert counts[3] == T and counts.sum() == T
    assert np.array_equal(r2r, np.arange(T))
