"""Pins for the oracle's FP8 index plane (E4M3 key and query codes, FP32 per-row
key scales and per-(row, head) query scales).

* Codes that encode integers reduce the scorer exactly to the pinned INT8
  scorer on those integers.  The integer codes are built here from the
  format's definition (sign | exponent with bias 7 | 3 mantissa bits), not
  from the oracle's decoder.
* A hand-worked row with fractional, subnormal and largest-magnitude codes,
  a key whose dot is negative (ReLU to zero) and the visibility cut.
"""
from fractions import Fraction

import numpy as np

import oracle
from tests.tiny import PAGE, paged_pool


def e4m3_code_of_int(v: int) -> int:
    """The E4M3 code of an integer |v| <= 16 from the format's definition:
    v = 2^e * (1 + m / 8) with exponent field e + 7."""
    if v == 0:
        return 0
    sign = 0x80 if v < 0 else 0
    a = abs(int(v))
    e = a.bit_length() - 1
    m = (a - (1 << e)) * 8 // (1 << e)
    assert (1 << e) * (8 + m) == 8 * a, a   # exactly representable
    return sign | ((e + 7) << 3) | m


def test_integer_codes_match_the_format():
    for v in range(-16, 17):
        assert oracle.decode_e4m3(np.array([e4m3_code_of_int(v)], np.uint8))[0] == v


def _case(rng, n, T, Hi, Di, ratio=1):
    kv = rng.integers(-16, 17, size=(n, Di))
    q = rng.integers(-16, 17, size=(T, Hi, Di))
    ks = rng.uniform(0.01, 0.1, size=n).astype(np.float32)
    qs = rng.uniform(0.01, 0.1, size=(T, Hi)).astype(np.float32)
    w = (rng.standard_normal((T, Hi)) / 2).astype(np.float32)
    pages = -(-n // PAGE)
    bt = rng.permutation(pages + 2)[:pages].astype(np.int32)[None, :]
    pos = np.sort(rng.integers(0, n * ratio, size=T)).astype(np.int32)
    enc = np.vectorize(e4m3_code_of_int)
    common = dict(head_w=w, block_table=bt, query_start_loc=np.array([0, T], np.int32),
                  positions=pos, num_tokens=T, ratio=ratio, score_stride=pages * PAGE)
    int8 = dict(q_idx=q.astype(np.int8), q_scale=qs,
                idx_kv=paged_pool([kv.astype(np.int8)], bt, pages + 2),
                idx_scale=paged_pool([ks], bt, pages + 2), **common)
    fp8 = dict(q_fp8=enc(q).astype(np.uint8), q_scale=qs,
               idx_fp8=paged_pool([enc(kv).astype(np.uint8)], bt, pages + 2),
               idx_scale=paged_pool([ks], bt, pages + 2), **common)
    return int8, fp8


def test_integer_codes_reduce_to_the_int8_scorer():
    rng = np.random.default_rng(31)
    for n, T, Hi, Di, ratio in [(300, 3, 8, 64, 1), (700, 2, 5, 128, 2), (129, 4, 1, 32, 1)]:
        int8, fp8 = _case(rng, n, T, Hi, Di, ratio)
        a, ea = oracle.index_scores(**int8)
        b, eb = oracle.index_scores_fp8(**fp8)
        assert ea == eb == 0
        np.testing.assert_array_equal(a, b)


def test_hand_worked_row():
    # codes: 0.5 = 0x30, -1.125 = 0xB9, 2^-9 (smallest subnormal) = 0x01, 448 = 0x7E,
    #        2 = 0x40, -0.5 = 0xB0, 2^-6 (smallest normal) = 0x08, 1 = 0x38, -1 = 0xB8
    q = np.array([[[0x30, 0xB9, 0x01, 0x7E]]], np.uint8)          # [T=1, Hi=1, Di=4]
    k0 = [0x40, 0xB0, 0x08, 0x38]   # dot = 1 + 0.5625 + 2^-15 + 448
    k1 = [0x40, 0xB0, 0x08, 0xB8]   # dot = 1 + 0.5625 + 2^-15 - 448 < 0
    k2 = [0x38, 0x38, 0x38, 0x38]   # not visible to the row
    bt = np.array([[1]], np.int32)
    keys = paged_pool([np.array([k0, k1, k2], np.uint8)], bt, 2)
    ks = paged_pool([np.array([2.0, 2.0, 2.0], np.float32)], bt, 2)
    s, err = oracle.index_scores_fp8(q, np.array([[0.25]], np.float32),
                                     np.array([[1.5]], np.float32), keys, ks, bt,
                                     np.array([0, 1], np.int32), np.array([1], np.int32), 1, 1,
                                     PAGE)
    assert err == 0
    dot0 = Fraction(1) + Fraction(9, 16) + Fraction(1, 2 ** 15) + 448
    assert Fraction(s[0, 0]) == Fraction(3, 2) * Fraction(1, 4) * 2 * dot0
    assert s[0, 1] == 0.0
    assert np.isneginf(s[0, 2:]).all()
