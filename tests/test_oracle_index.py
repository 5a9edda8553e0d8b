"""Pins for the oracle's lightning-indexer scores.

Checked against: the hand-worked example in tests/golden/index_score_hand.json,
the visibility worked example of gitcode hyper-parallel issue #2 section 8.2,
a one-head special case that reduces to a plain dot product, the identity
relu(x) - relu(-x) = x (pins ReLU placement and signs), exact extreme integer
dots, invariance under a block-table shuffle, and exact rational arithmetic
on tiny random cases.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.tiny import PAGE, paged_pool, random_block_table


def _case_from_dense(keys, kscale, q8, qs, w, positions, ratio, block_table=None, num_blocks=None):
    """One request, len(positions) rows; keys [n, Di] laid into pages."""
    n = keys.shape[0]
    pages = max(1, -(-n // PAGE))
    if block_table is None:
        block_table = np.arange(pages, dtype=np.int32)[None, :][:, ::-1].copy()
        num_blocks = pages
    idx_kv = paged_pool([keys.astype(np.int8)], block_table, num_blocks)
    idx_scale = paged_pool([kscale.astype(np.float32)], block_table, num_blocks, fill=1.0)
    T = len(positions)
    qsl = np.array([0, T], np.int32)
    return dict(q_idx=np.asarray(q8, np.int8), q_scale=np.asarray(qs, np.float32),
                head_w=np.asarray(w, np.float32), idx_kv=idx_kv, idx_scale=idx_scale,
                block_table=block_table, query_start_loc=qsl,
                positions=np.asarray(positions, np.int32), num_tokens=T, ratio=ratio,
                score_stride=pages * PAGE)


def test_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "index_score_hand.json")))
    keys = np.array(g["keys"])
    for case in g["cases"]:
        a = _case_from_dense(keys, np.array(g["key_scale"]), [g["q8"]], [g["q_scale"]],
                             [g["head_w"]], [case["position"]], case["ratio"])
        s, err = oracle.index_scores(**a)
        assert err == 0
        exp = [float(v) for v in case["expected"]]
        got = s[0, :4]
        for e, v in zip(exp, got):
            if e == float("-inf"):
                assert v == -np.inf
            else:
                assert v == e  # exact: dyadic inputs
        assert np.all(s[0, 4:] == -np.inf)


def test_visibility_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "visibility.json")))
    for c in g["compressed_visibility"]["cases"]:
        n = oracle.visible_count(c["p"], c["ratio"])
        assert all(x < n for x in c["visible"])
        assert all(x >= n for x in c["not_visible"])
    for c in g["window"]["cases"]:
        assert list(oracle.window_positions(c["p"], c["window"])) == c["sees"]
    assert oracle.visible_count(-1, 1) == 0 and oracle.visible_count(-5, 2) == 0
    assert oracle.visible_count(0, 1) == 1 and oracle.visible_count(0, 2) == 0


def test_single_head_is_relu_of_dot():
    rng = np.random.default_rng(3)
    n, Di = 300, 32
    keys = rng.integers(-127, 128, (n, Di))
    q = rng.integers(-127, 128, (1, 1, Di))
    a = _case_from_dense(keys, np.ones(n), q, [[1.0]], [[1.0]], [n - 1], 1)
    s, _ = oracle.index_scores(**a)
    ref = np.maximum(keys @ q[0, 0], 0)
    assert np.array_equal(s[0, :n], ref.astype(np.float64))
    assert (ref == 0).sum() > 50  # the ReLU is exercised


def test_relu_difference_is_linear():
    rng = np.random.default_rng(4)
    n, Hi, Di = 257, 4, 32
    keys = rng.integers(-127, 128, (n, Di))
    ks = rng.uniform(0.005, 0.02, n)
    q = rng.integers(-127, 128, (1, Hi, Di))
    qs = rng.uniform(0.01, 0.1, (1, Hi))
    w = rng.standard_normal((1, Hi))
    a = _case_from_dense(keys, ks, q, qs, w, [n - 1], 1)
    sp, _ = oracle.index_scores(**a)
    a["q_idx"] = -a["q_idx"]
    sn, _ = oracle.index_scores(**a)
    # the pool stores key scales as float32; use the same stored values
    ks32 = ks.astype(np.float32).astype(np.float64)
    lin = np.einsum("h,h,c,hc->c", a["head_w"][0].astype(np.float64),
                    a["q_scale"][0].astype(np.float64), ks32,
                    (q[0] @ keys.T).astype(np.float64))
    assert np.allclose(sp[0, :n] - sn[0, :n], lin, rtol=1e-12, atol=1e-12)


def test_extreme_integer_dot_is_exact():
    Di = 128
    keys = np.stack([np.full(Di, 127), np.full(Di, -127), np.tile([127, -127], Di // 2)])
    q = np.full((1, 1, Di), 127)
    a = _case_from_dense(keys, np.ones(3), q, [[1.0]], [[1.0]], [2], 1)
    s, _ = oracle.index_scores(**a)
    assert s[0, :3].tolist() == [128 * 127 * 127, 0.0, 0.0]
    a["q_idx"] = -a["q_idx"]
    s, _ = oracle.index_scores(**a)
    assert s[0, :3].tolist() == [0.0, 128 * 127 * 127, 0.0]


def test_block_table_shuffle_invariance():
    rng = np.random.default_rng(5)
    B, pages, Hi, Di = 2, 3, 4, 32
    n = pages * PAGE
    dense = [rng.integers(-127, 128, (n, Di)).astype(np.int8) for _ in range(B)]
    dsc = [rng.uniform(0.005, 0.02, n).astype(np.float32) for _ in range(B)]
    q = rng.integers(-127, 128, (4, Hi, Di)).astype(np.int8)
    qs = rng.uniform(0.01, 0.1, (4, Hi)).astype(np.float32)
    w = rng.standard_normal((4, Hi)).astype(np.float32)
    pos = np.array([n - 1, 200, 2 * n - 1, 5], np.int32)  # ratio 2 below
    qsl = np.array([0, 2, 4], np.int32)
    outs = []
    for seed in (0, 1):
        bt, nb = random_block_table(np.random.default_rng(seed), B, pages, extra=2)
        kv = paged_pool(dense, bt, nb)
        sc = paged_pool(dsc, bt, nb, fill=1.0)
        s, err = oracle.index_scores(q, qs, w, kv, sc, bt, qsl, pos, 4, 2, n)
        assert err == 0
        outs.append(s)
    assert np.array_equal(outs[0], outs[1])
    # the request-local layout matters: row 0 of request 0 used dense[0]
    assert np.isfinite(outs[0][0, : n // 2]).all() and np.all(outs[0][0, n // 2:] == -np.inf)


def test_exact_rational_tiny():
    rng = np.random.default_rng(6)
    n, Hi, Di = 9, 3, 8
    keys = rng.integers(-127, 128, (n, Di))
    ks = rng.uniform(0.005, 0.02, n).astype(np.float32)
    q = rng.integers(-127, 128, (1, Hi, Di))
    qs = rng.uniform(0.01, 0.1, (1, Hi)).astype(np.float32)
    w = rng.standard_normal((1, Hi)).astype(np.float32)
    a = _case_from_dense(keys, ks, q, qs, w, [n - 1], 1)
    s, _ = oracle.index_scores(**a)
    for c in range(n):
        tot = Fraction(0)
        for h in range(Hi):
            d = sum(int(q[0, h, i]) * int(keys[c, i]) for i in range(Di))
            v = Fraction(float(qs[0, h])) * Fraction(float(ks[c])) * d
            tot += Fraction(float(w[0, h])) * max(v, Fraction(0))
        assert s[0, c] == pytest.approx(float(tot), rel=1e-14, abs=1e-300)


def test_contract_flags():
    rng = np.random.default_rng(7)
    Hi, Di = 2, 32
    keys = rng.integers(-127, 128, (2 * PAGE, Di))
    a = _case_from_dense(keys, np.ones(2 * PAGE), rng.integers(-5, 5, (2, Hi, Di)),
                         np.ones((2, Hi)), np.ones((2, Hi)), [2 * PAGE - 1, 2 * PAGE - 1], 1)
    # invalid block id on the second page: those positions score -inf
    a["block_table"] = a["block_table"].copy()
    a["block_table"][0, 1] = 99
    s, err = oracle.index_scores(**a)
    assert err == oracle.EFLAG_BLOCK_RANGE
    assert np.isfinite(s[:, :PAGE]).all() and np.all(s[:, PAGE:] == -np.inf)
    # a row that no request owns
    a["block_table"][0, 1] = 0
    a["query_start_loc"] = np.array([0, 1], np.int32)
    s, err = oracle.index_scores(**a)
    assert err == oracle.EFLAG_META and np.all(s[1] == -np.inf) and np.isfinite(s[0]).all()
    # visible span wider than the score row
    a["query_start_loc"] = np.array([0, 2], np.int32)
    a["score_stride"] = PAGE
    s, err = oracle.index_scores(**a)
    assert err == oracle.EFLAG_POS_RANGE and s.shape == (2, PAGE) and np.isfinite(s).all()
