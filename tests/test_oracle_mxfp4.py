"""Pins for the oracle's MXFP4 index plane (E2M1 values, one E8M0 scale per
32 elements).

* The E8M0 convention, 2^(byte - 127), against the value the pages state
  (tests/golden/e8m0_scale.json).
* The E2M1 magnitudes against the format's definition (1 sign bit, 2
  exponent bits with bias 1 and a subnormal at exponent 0, 1 mantissa bit):
  0, 0.5, 1, 1.5, 2, 3, 4, 6, and the element order inside a byte.
* The scorer reduces to the pinned INT8 scorer when every group of a row
  shares one scale (E2M1 values are halves of integers), and each group's
  scale multiplies exactly that group's part of the dot.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests.tiny import PAGE, paged_pool

E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e8m0_convention(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "e8m0_scale.json")))
    for c in g["cases"]:
        assert oracle.decode_e8m0(np.array([c["byte"]]))[0] == c["value"]
    assert np.isnan(oracle.decode_e8m0(np.array([255]))[0])


def test_e2m1_values_and_nibble_order():
    codes = np.array([[(2 * i + 1) << 4 | (2 * i) for i in range(8)]], np.uint8)
    v = oracle.decode_e2m1(codes)[0]
    want = E2M1_MAGNITUDES + [-x for x in E2M1_MAGNITUDES]
    np.testing.assert_array_equal(v, want)
    assert np.signbit(v[8])            # code 8 is -0
    # the element with the lower index sits in bits 0-3
    np.testing.assert_array_equal(oracle.decode_e2m1(np.array([[0x21]], np.uint8))[0], [0.5, 1.0])


def _mx_case(rng, n, T, Hi=8, Di=128, uniform_scales=False, ratio=1):
    kc = rng.integers(0, 256, size=(n, Di // 2), dtype=np.uint8)
    ks = rng.integers(120, 131, size=(n, Di // 32)).astype(np.uint8)
    qc = rng.integers(0, 256, size=(T, Hi, Di // 2), dtype=np.uint8)
    qs = rng.integers(120, 131, size=(T, Hi, Di // 32)).astype(np.uint8)
    if uniform_scales:
        ks[:] = ks[:, :1]
        qs[:] = qs[:, :, :1]
    pages = -(-n // PAGE)
    bt = rng.permutation(pages + 1)[:pages].astype(np.int32)[None, :]
    kv = paged_pool([kc], bt, pages + 1)
    sc = paged_pool([ks], bt, pages + 1, fill=127)
    w = (rng.standard_normal((T, Hi)) / 2).astype(np.float32)
    pos = np.sort(rng.integers(0, n * ratio, size=T)).astype(np.int32)
    return dict(q_fp4=qc, q_sc=qs, head_w=w, idx_fp4=kv, idx_sc=sc, block_table=bt,
                query_start_loc=np.array([0, T], np.int32), positions=pos, num_tokens=T,
                ratio=ratio, score_stride=pages * PAGE), (kc, ks, qc, qs)


@pytest.mark.parametrize("seed", range(4))
def test_uniform_scales_reduce_to_int8_scorer(seed):
    rng = np.random.default_rng(seed)
    c, (kc, ks, qc, qs) = _mx_case(rng, 300, 3, uniform_scales=True)
    got, e1 = oracle.index_scores_mxfp4(**c)
    # E2M1 values are halves of integers in [-6, 6]: as INT8 codes 2*v with a
    # per-row scale 0.5 * 2^(byte - 127) the INT8 scorer computes the same
    q8 = (2 * oracle.decode_e2m1(qc)).astype(np.int8)
    k8 = (2 * oracle.decode_e2m1(kc)).astype(np.int8)
    qscale = (0.5 * np.ldexp(1.0, qs[:, :, 0].astype(np.int64) - 127)).astype(np.float32)
    kscale = (0.5 * np.ldexp(1.0, ks[:, 0].astype(np.int64) - 127)).astype(np.float32)
    bt = c["block_table"]
    nb = bt.shape[1] + 1
    want, e2 = oracle.index_scores(q8, qscale, c["head_w"], paged_pool([k8], bt, nb),
                                   paged_pool([kscale], bt, nb, fill=1.0), bt,
                                   c["query_start_loc"], c["positions"], c["num_tokens"],
                                   c["ratio"], c["score_stride"])
    np.testing.assert_array_equal(got, want)
    assert e1 == e2 == 0


def test_group_scale_multiplies_its_group():
    rng = np.random.default_rng(5)
    c, (kc, ks, qc, qs) = _mx_case(rng, 40, 1, Hi=1)
    c["head_w"][:] = 1.0
    n = oracle.visible_count(int(c["positions"][0]), 1)
    base_rows = oracle.mx_rows(qc[0], qs[0])[0]
    keys = oracle.mx_rows(kc[:n], ks[:n])
    for g in range(4):
        part = base_rows[32 * g:32 * (g + 1)] @ keys[:, 32 * g:32 * (g + 1)].T
        qs2 = qs.copy()
        qs2[0, 0, g] += 1          # this group's query scale doubles
        c2 = dict(c, q_sc=qs2)
        a, _ = oracle.index_scores_mxfp4(**dict(c, head_w=c["head_w"]))
        b, _ = oracle.index_scores_mxfp4(**c2)
        full = base_rows @ keys.T
        np.testing.assert_array_equal(a[0, :n], np.maximum(full, 0.0))
        np.testing.assert_array_equal(b[0, :n], np.maximum(full + part, 0.0))


def test_flags_match_the_int8_scorer():
    rng = np.random.default_rng(8)
    c, _ = _mx_case(rng, 256, 4)
    c["positions"] = np.array([-1, 10, 900, 255], np.int32)   # nothing visible / past the table
    c["query_start_loc"] = np.array([0, 3], np.int32)          # row 3 unowned
    s, err = oracle.index_scores_mxfp4(**c)
    assert err == oracle.EFLAG_META | oracle.EFLAG_POS_RANGE
    assert np.all(np.isneginf(s[0])) and np.all(np.isneginf(s[3]))
    assert np.all(np.isfinite(s[1, :11])) and np.all(np.isneginf(s[1, 11:]))
