"""Pins for the oracle's RoPE-row materialisation and adjacent-pair rotation.

The row contract comes from pypto-lib "DeepSeek V4.1 Flash", section
"Serving-owned full RoPE tables"; the rotation is multiplication by e^{i theta}
of the complex number x[2i] + i x[2i+1], checked against Python's complex type.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest

import oracle
import synthetic

SENTINEL = np.uint32(0x7FC0DEAD)  # a NaN payload no computation produces


def _sentinel(shape):
    return np.full(shape, SENTINEL, dtype=np.uint32).view(np.float32)


def test_identity_and_copy_and_padding(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "rope_contract.json")))
    cos, sin = synthetic.rope_tables(64, 16, 10000.0)
    pos = np.array([5, -1, 63, -7, 3, 2], dtype=np.int32)
    rc, rs = _sentinel((6, 8)), _sentinel((6, 8))
    err = oracle.materialize_rope_rows(cos, sin, pos, 4, rc, rs)
    assert err == 0
    # bit copies for nonnegative positions
    assert np.array_equal(rc[0].view(np.uint32), cos[5].view(np.uint32))
    assert np.array_equal(rs[2].view(np.uint32), sin[63].view(np.uint32))
    # identity for negative positions: cos exactly 1, sin exactly +0 (sign bit clear)
    for t in (1, 3):
        assert np.all(rc[t] == g["identity_cos"])
        assert np.all(rs[t].view(np.uint32) == g["identity_sin_bits"])
    # rows past num_tokens untouched
    assert np.all(rc[4:].view(np.uint32) == SENTINEL)
    assert np.all(rs[4:].view(np.uint32) == SENTINEL)


def test_zero_tokens_touch_nothing():
    cos, sin = synthetic.rope_tables(8, 4, 10000.0)
    rc, rs = _sentinel((3, 2)), _sentinel((3, 2))
    assert oracle.materialize_rope_rows(cos, sin, np.array([1, 2, 3], np.int32), 0, rc, rs) == 0
    assert np.all(rc.view(np.uint32) == SENTINEL) and np.all(rs.view(np.uint32) == SENTINEL)


def test_position_past_capacity_flags_and_leaves_row():
    cos, sin = synthetic.rope_tables(8, 4, 10000.0)
    rc, rs = _sentinel((2, 2)), _sentinel((2, 2))
    err = oracle.materialize_rope_rows(cos, sin, np.array([8, 7], np.int32), 2, rc, rs)
    assert err == oracle.EFLAG_POS_RANGE
    assert np.all(rc[0].view(np.uint32) == SENTINEL)
    assert np.array_equal(rc[1], cos[7])


def test_table_fixture_is_textbook_rope():
    # the fixture tables (caller inputs) against cos/sin of p * theta^(-2i/R)
    cos, sin = synthetic.rope_tables(1 << 12, 64, 10000.0)
    for p in (0, 1, 77, 4095):
        for i in (0, 1, 13, 31):
            ang = p * 10000.0 ** (-2.0 * i / 64)
            assert cos[p, i] == np.float32(math.cos(ang))
            assert sin[p, i] == np.float32(math.sin(ang))


def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(8)
    th = rng.uniform(-4, 4, 4)
    y = oracle.rotate_adjacent_pairs(x, np.cos(th), np.sin(th))
    for i in range(4):
        z = complex(x[2 * i], x[2 * i + 1]) * cmath.exp(1j * th[i])
        assert y[2 * i] == pytest.approx(z.real, abs=1e-14)
        assert y[2 * i + 1] == pytest.approx(z.imag, abs=1e-14)


def test_rotation_quarter_turn_and_norm_and_composition():
    # quarter turn maps the real axis to the imaginary axis
    y = oracle.rotate_adjacent_pairs(np.array([1.0, 0.0]), np.array([0.0]), np.array([1.0]))
    assert y.tolist() == [0.0, 1.0]
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 16))
    a, b = rng.uniform(-3, 3, 8), rng.uniform(-3, 3, 8)
    ya = oracle.rotate_adjacent_pairs(x, np.cos(a), np.sin(a))
    # pair norms preserved
    assert np.allclose(np.hypot(ya[:, 0::2], ya[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]))
    # rotating by a then b equals rotating by a + b
    yab = oracle.rotate_adjacent_pairs(ya, np.cos(b), np.sin(b))
    assert np.allclose(yab, oracle.rotate_adjacent_pairs(x, np.cos(a + b), np.sin(a + b)))
    # identity row leaves x unchanged exactly
    assert np.array_equal(oracle.rotate_adjacent_pairs(x, np.ones(8), np.zeros(8)), x)
