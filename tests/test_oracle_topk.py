"""Pins for the oracle's top-k.

Checked against a brute-force characterisation on tiny rows (the unique subset
of size m in which every chosen position beats every unchosen one, ties going
to the lower position), the validity checks of pypto-lib "DeepSeek V4.1
Flash" section "Decode composition" (eligibility, uniqueness, ascending
logical positions, trailing -1, cutoff quality), and the special case k >=
visible span selecting everything.
"""
import itertools

import numpy as np
import pytest

import oracle


def _beats(s, i, j):
    # i ranks above j: larger score, or equal score and lower position; NaN last
    si, sj = s[i], s[j]
    if np.isnan(si) or np.isnan(sj):
        if np.isnan(si) and np.isnan(sj):
            return i < j
        return np.isnan(sj)
    return si > sj or (si == sj and i < j)


def _brute(s, m):
    n = len(s)
    found = []
    for S in itertools.combinations(range(n), m):
        rest = [j for j in range(n) if j not in S]
        if all(_beats(s, i, j) for i in S for j in rest):
            found.append(S)
    assert len(found) == 1
    return list(found[0])


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 10))
    k = int(rng.integers(1, 6))
    # few distinct values so ties are common; a NaN now and then
    s = rng.integers(-3, 3, n).astype(np.float64)
    if seed % 3 == 0:
        s[rng.integers(0, n)] = np.nan
    if seed % 4 == 1:
        s[rng.integers(0, n)] = -np.inf
    row = np.full((1, 12), 7.0)  # junk past the visible span must be ignored
    row[0, :n] = s
    idx, val, err = oracle.topk(row, np.array([n - 1]), 1, 1, k)
    assert err == 0
    m = min(k, n)
    exp = _brute(s, m)
    assert idx[0, :m].tolist() == exp
    assert idx[0, m:].tolist() == [-1] * (k - m)
    assert np.array_equal(val[0, :m], s[exp], equal_nan=True)
    assert np.all(val[0, m:] == -np.inf)


def test_k_covers_everything_selects_all_visible():
    rng = np.random.default_rng(11)
    s = rng.standard_normal((3, 64))
    pos = np.array([9, 63, 20])
    idx, _, _ = oracle.topk(s, pos, 2, 3, 40)
    for t, p in enumerate(pos):
        n = (p + 1) // 2
        assert idx[t, :n].tolist() == list(range(n))
        assert np.all(idx[t, n:] == -1)


def test_validity_checks_on_random_rows():
    rng = np.random.default_rng(12)
    n, k = 1000, 64
    s = rng.standard_normal((4, n))
    pos = np.array([n - 1, 500, 63, -1])
    idx, val, _ = oracle.topk(s, pos, 1, 4, k)
    for t in range(4):
        nv = max(0, pos[t] + 1)
        m = min(k, nv)
        sel = idx[t, :m]
        assert np.all(np.diff(sel) > 0)                 # unique, ascending
        assert np.all((sel >= 0) & (sel < nv))          # eligible
        assert np.all(idx[t, m:] == -1)                 # trailing -1
        if 0 < m < nv:
            rest = np.setdiff1d(np.arange(nv), sel)
            assert s[t, sel].min() >= s[t, rest].max()  # cutoff quality


def test_all_equal_scores_take_lowest_positions():
    s = np.zeros((1, 50))
    idx, _, _ = oracle.topk(s, np.array([49]), 1, 1, 7)
    assert idx[0].tolist() == list(range(7))


def test_visible_span_wider_than_row_flags():
    s = np.arange(8, dtype=np.float64)[None, :]
    idx, _, err = oracle.topk(s, np.array([100]), 1, 1, 3)
    assert err == oracle.EFLAG_POS_RANGE and idx[0].tolist() == [5, 6, 7]
