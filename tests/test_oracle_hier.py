"""Pins for the oracle's hierarchical selection (candidate blocks, then a
reindex layer's scores and top-k inside them).

pypto-lib "DeepSeek V4.1 Flash", section "Decode composition", fixes the
structure: the full layer picks blocks of eight compressed positions, and the
reindex layers select only inside that mask, in compressed-position space.
The pins reduce each function to one that is already pinned (block size 1 is
the plain top-k; a mask that holds every visible block is the plain index
scoring and top-k), check a hand-worked example, and check the selection
properties the same section lists (eligibility, uniqueness, ascending
order, trailing -1, cutoff quality).
"""
import numpy as np
import pytest

import oracle
from tests.tiny import PAGE, paged_pool


def _rand_scores(rng, T, width, ties=False):
    s = rng.standard_normal((T, width))
    if ties:
        s = np.round(s * 2) / 2   # many exact ties
    return s


@pytest.mark.parametrize("seed", range(6))
def test_block_of_one_is_plain_topk(seed):
    rng = np.random.default_rng(seed)
    T, width = 5, 97
    s = _rand_scores(rng, T, width, ties=seed % 2 == 1)
    pos = rng.integers(-1, 2 * width, size=T).astype(np.int32)
    for kb in (1, 7, 50, 200):
        got, e1 = oracle.candidate_blocks(s, pos, 2, T, 1, kb)
        want, _, e2 = oracle.topk(s, pos, 2, T, kb)
        np.testing.assert_array_equal(got, want)
        assert e1 == e2


def test_hand_worked_example():
    # 19 visible positions (p = 18, ratio 1), blocks of 4: blocks 0..4, block 4
    # holds positions 16, 17, 18 (19 is not visible).
    s = np.array([[0.1, 0.2, 0.3, 0.4,     # block 0: max 0.4
                   5.0, -1.0, -1.0, -1.0,  # block 1: max 5.0
                   0.4, 0.0, 0.0, 0.0,     # block 2: max 0.4 (ties block 0)
                   -3.0, -2.0, -4.0, -9.0,  # block 3: max -2.0
                   1.0, 0.5, 0.5, 99.0]])  # block 4: max 1.0 (99 is past the span)
    pos = np.array([18], np.int32)
    cb, err = oracle.candidate_blocks(s, pos, 1, 1, 4, 3)
    # ranking: block 1 (5.0), block 4 (1.0), block 0 (0.4, lower id), block 2, block 3
    np.testing.assert_array_equal(cb, [[0, 1, 4]])
    assert err == 0
    cb, _ = oracle.candidate_blocks(s, pos, 1, 1, 4, 4)
    np.testing.assert_array_equal(cb, [[0, 1, 2, 4]])
    cb, _ = oracle.candidate_blocks(s, pos, 1, 1, 4, 8)
    np.testing.assert_array_equal(cb, [[0, 1, 2, 3, 4, -1, -1, -1]])
    # a row with nothing visible selects nothing
    cb, _ = oracle.candidate_blocks(s, np.array([-1], np.int32), 1, 1, 4, 3)
    np.testing.assert_array_equal(cb, [[-1, -1, -1]])


@pytest.mark.parametrize("seed", range(8))
def test_selection_properties(seed):
    rng = np.random.default_rng(100 + seed)
    T, width, block = 6, 203, 8
    s = _rand_scores(rng, T, width, ties=seed % 2 == 0)
    pos = rng.integers(0, width + 20, size=T).astype(np.int32)
    kb = int(rng.integers(1, 30))
    cb, err = oracle.candidate_blocks(s, pos, 1, T, block, kb)
    for t in range(T):
        n = min(int(pos[t]) + 1, width)
        nb = -(-n // block)
        bmax = [max(s[t, j * block:min(n, (j + 1) * block)]) for j in range(nb)]
        m = min(kb, nb)
        row = cb[t]
        assert np.all(row[m:] == -1) and np.all(row[:m] >= 0) and np.all(row[:m] < nb)
        assert np.all(np.diff(row[:m]) > 0)
        chosen = set(row[:m].tolist())
        rest = [j for j in range(nb) if j not in chosen]
        if rest:
            worst_in = min((bmax[j], -j) for j in chosen)
            best_out = max((bmax[j], -j) for j in rest)
            assert worst_in > best_out   # strict in (score, -id) order
    assert err == (oracle.EFLAG_POS_RANGE if np.any(pos + 1 > width) else 0)


def test_monotone_transform_invariance():
    rng = np.random.default_rng(7)
    s = _rand_scores(rng, 4, 160, ties=True)
    pos = np.array([159, 100, 37, 8], np.int32)
    a, _ = oracle.candidate_blocks(s, pos, 1, 4, 8, 5)
    b, _ = oracle.candidate_blocks(3.0 * s + 7.0, pos, 1, 4, 8, 5)
    np.testing.assert_array_equal(a, b)


def _index_case(rng, n, T, ratio, Hi=4, Di=32):
    keys = rng.integers(-127, 128, size=(n, Di)).astype(np.int8)
    kscale = rng.uniform(0.005, 0.02, size=n).astype(np.float32)
    pages = -(-n // PAGE)
    bt = rng.permutation(pages + 2)[:pages].astype(np.int32)[None, :]
    nblk = pages + 2
    idx_kv = paged_pool([keys], bt, nblk)
    idx_scale = paged_pool([kscale], bt, nblk, fill=1.0)
    q8 = rng.integers(-127, 128, size=(T, Hi, Di)).astype(np.int8)
    qs = rng.uniform(0.001, 0.01, size=(T, Hi)).astype(np.float32)
    w = (rng.standard_normal((T, Hi)) / 2).astype(np.float32)
    pos = np.sort(rng.integers(0, n * ratio, size=T)).astype(np.int32)
    return dict(q_idx=q8, q_scale=qs, head_w=w, idx_kv=idx_kv, idx_scale=idx_scale,
                block_table=bt, query_start_loc=np.array([0, T], np.int32), positions=pos,
                num_tokens=T, ratio=ratio)


@pytest.mark.parametrize("seed", range(4))
def test_candidate_scores_are_the_full_scores_at_candidate_positions(seed):
    rng = np.random.default_rng(200 + seed)
    n, T, ratio, block = 300, 4, 2, 8
    c = _index_case(rng, n, T, ratio)
    full, e_full = oracle.index_scores(score_stride=3 * PAGE, **c)
    kb = 9
    cand = np.full((T, kb), -1, np.int32)
    for t in range(T):
        nb = -(-oracle.visible_count(int(c["positions"][t]), ratio) // block)
        pick = np.sort(rng.choice(nb, size=min(kb - 1, nb), replace=False))
        cand[t, :len(pick)] = pick
    sc, err = oracle.index_scores_in_candidates(cand_blocks=cand, block=block, **c)
    assert err == e_full == 0
    for t in range(T):
        nv = oracle.visible_count(int(c["positions"][t]), ratio)
        for i in range(kb * block):
            blk = cand[t, i // block]
            p = blk * block + i % block
            if blk >= 0 and p < nv:
                assert sc[t, i] == full[t, p]
            else:
                assert sc[t, i] == -np.inf


@pytest.mark.parametrize("seed", range(4))
def test_mask_of_every_block_is_the_plain_selection(seed):
    rng = np.random.default_rng(300 + seed)
    n, T, ratio, block, k = 250, 5, 1, 8, 17
    c = _index_case(rng, n, T, ratio)
    full, _ = oracle.index_scores(score_stride=2 * PAGE, **c)
    want_i, want_v, _ = oracle.topk(full, c["positions"], ratio, T, k)
    kb = -(-2 * PAGE // block)
    cand, _ = oracle.candidate_blocks(full, c["positions"], ratio, T, block, kb)
    sc, _ = oracle.index_scores_in_candidates(cand_blocks=cand, block=block, **c)
    got_i, got_v, _ = oracle.topk_in_candidates(sc, cand, block, c["positions"], ratio, T, k)
    np.testing.assert_array_equal(got_i, want_i)
    np.testing.assert_array_equal(got_v, want_v)


@pytest.mark.parametrize("seed", range(4))
def test_reindex_selection_inside_the_mask(seed):
    rng = np.random.default_rng(400 + seed)
    n, T, ratio, block, k = 400, 4, 1, 8, 12
    c = _index_case(rng, n, T, ratio)
    full, _ = oracle.index_scores(score_stride=4 * PAGE, **c)
    cand, _ = oracle.candidate_blocks(full, c["positions"], ratio, T, block, 5)
    # a different index query for the reindex layer
    c2 = dict(c, q_idx=rng.integers(-127, 128, size=c["q_idx"].shape).astype(np.int8))
    sc, _ = oracle.index_scores_in_candidates(cand_blocks=cand, block=block, **c2)
    got_i, got_v, _ = oracle.topk_in_candidates(sc, cand, block, c["positions"], ratio, T, k)
    full2, _ = oracle.index_scores(score_stride=4 * PAGE, **c2)
    for t in range(T):
        nv = oracle.visible_count(int(c["positions"][t]), ratio)
        allowed = {int(b) * block + o for b in cand[t] if b >= 0 for o in range(block)
                   if int(b) * block + o < nv}
        m = min(k, len(allowed))
        row = got_i[t]
        assert np.all(row[m:] == -1) and np.all(np.diff(row[:m]) > 0)
        assert set(row[:m].tolist()) <= allowed
        # the same as the plain top-k over the layer's full scores, with every
        # position outside the mask pushed below the candidates
        masked = np.full_like(full2[t], -1e300)
        masked[sorted(allowed)] = full2[t, sorted(allowed)]
        ref, _, _ = oracle.topk(masked[None, :], np.array([c["positions"][t]]), ratio, 1, m)
        np.testing.assert_array_equal(row[:m], ref[0])
        np.testing.assert_array_equal(got_v[t, :m], full2[t, row[:m]])


def test_candidate_past_the_span_is_flagged():
    rng = np.random.default_rng(9)
    c = _index_case(rng, 200, 2, 1)
    nb = -(-oracle.visible_count(int(c["positions"][0]), 1) // 8)
    cand = np.array([[0, nb, -1], [0, -1, -1]], np.int32)
    sc, err = oracle.index_scores_in_candidates(cand_blocks=cand, block=8, **c)
    assert err & oracle.EFLAG_TOPK_RANGE
    assert np.all(sc[0, 8:16] == -np.inf)
