"""Pins for the oracle's inverse RoPE of the attention output.

* Each rope pair is multiplied by the conjugate of its rope row's complex
  number (Python complex arithmetic, an independent route; with FP32 tables
  cos^2 + sin^2 is 1 only to FP32 precision, so this is the conjugate, not a
  division), channels outside the span and rows past num_tokens are
  unchanged, and an identity rope row changes nothing.
* Forward rotation then inverse is the identity (unit-modulus float64 rows).
* Keys at the query's own position: when every key/value row's rope span is
  rotated by the query row's angles, the inverse-rotated attention output is
  the attention-weighted mix of the unrotated rows, with the weights computed
  here by scipy from complex-rotated logits.
"""
import math

import numpy as np
from scipy.special import softmax

import oracle
from tests.tiny import PAGE, bf16_bits, bf16_value, paged_pool


def _rope(rng, T, half):
    ang = rng.uniform(-3, 3, (T, half))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def test_conjugate_rotation_by_complex_arithmetic():
    rng = np.random.default_rng(40)
    T, H, D, R, off = 3, 2, 24, 8, 12
    out = rng.standard_normal((T, H, D))
    c, s = _rope(rng, T, R // 2)
    got = oracle.inverse_rope(out, c, s, off, num_tokens=2)
    for t in range(2):
        for h in range(H):
            for i in range(R // 2):
                z = complex(out[t, h, off + 2 * i], out[t, h, off + 2 * i + 1])
                w = z * complex(float(c[t, i]), float(s[t, i])).conjugate()
                assert abs(got[t, h, off + 2 * i] - w.real) < 1e-12
                assert abs(got[t, h, off + 2 * i + 1] - w.imag) < 1e-12
    keep = np.ones(D, bool)
    keep[off:off + R] = False
    assert np.array_equal(got[:2][:, :, keep], out[:2][:, :, keep])
    assert np.array_equal(got[2], out[2])                 # past num_tokens
    ident = oracle.inverse_rope(out, np.ones_like(c), np.zeros_like(s), off, num_tokens=3)
    assert np.array_equal(ident, out)


def test_forward_then_inverse_is_identity():
    rng = np.random.default_rng(41)
    T, H, D, R = 4, 3, 16, 16
    x = rng.standard_normal((T, H, D))
    ang = rng.uniform(-3, 3, (T, R // 2))
    c, s = np.cos(ang), np.sin(ang)
    fwd = x.copy()
    for t in range(T):
        fwd[t] = oracle.rotate_adjacent_pairs(x[t], c[t], s[t])
    back = oracle.inverse_rope(fwd, c, s, 0, num_tokens=T)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-12)


def test_keys_at_the_query_position_give_unrotated_values():
    rng = np.random.default_rng(42)
    H, D, R, W, ratio, k = 4, 32, 8, 16, 2, 6
    off = D - R
    # one query row per request, so "the query's angle" is one rope row per request
    ctx = (300, 200)
    pos = np.array([c - 1 for c in ctx], np.int32)
    T = len(ctx)
    c, s = _rope(rng, T, R // 2)
    cdense, wdense, raw_c, raw_w = [], [], [], []
    for b, n in enumerate(ctx):
        cr = rng.standard_normal((3 * PAGE, D))
        wr = rng.standard_normal((3 * PAGE, D))
        # the rope span of every row of request b rotated by its query's angles,
        # then rounded to BF16 (the cache format)
        for arr in (cr, wr):
            arr[:, off:] = oracle.rotate_adjacent_pairs(arr[:, off:], c[b], s[b])
        cdense.append(bf16_bits(cr))
        wdense.append(bf16_bits(wr))
        # the unrotated rows the BF16 values stand for
        for arr, keep in ((bf16_value(cdense[-1]), raw_c), (bf16_value(wdense[-1]), raw_w)):
            u = arr.copy()
            u[:, off:] = oracle.rotate_adjacent_pairs(arr[:, off:], c[b], -s[b].astype(np.float64))
            keep.append(u)
    cbt = np.array([[0, 1, 2], [3, 4, 5]], np.int32)
    wbt = np.array([[6, 7, 8], [9, 10, 11]], np.int32)
    cmp_kv = paged_pool(cdense, cbt, 12)
    win_kv = paged_pool(wdense, wbt, 12)
    q = bf16_bits(rng.standard_normal((T, H, D)))
    sel = np.full((T, k), -1, np.int32)
    for t in range(T):
        nv = oracle.visible_count(pos[t], ratio)
        sel[t, :k] = np.sort(rng.choice(nv, k, replace=False))
    sink = rng.standard_normal(H).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    out, lse, err = oracle.sparse_attn(q, c, s, off, cmp_kv, cbt, sel, ratio, win_kv, wbt, W,
                                       sink, scale, np.array([0, 1, 2], np.int32), pos, T)
    assert err == 0
    inv = oracle.inverse_rope(out, c, s, off, T)
    for t in range(T):
        p = int(pos[t])
        rows = list(range(p - W + 1, p + 1))
        kv_rot = np.concatenate([bf16_value(wdense[t][rows]), bf16_value(cdense[t][sel[t]])])
        kv_raw = np.concatenate([raw_w[t][rows], raw_c[t][sel[t]]])
        qv = bf16_value(q[t])
        for h in range(H):
            for i in range(R // 2):
                z = complex(qv[h, off + 2 * i], qv[h, off + 2 * i + 1]) * complex(
                    float(c[t, i]), float(s[t, i]))
                qv[h, off + 2 * i], qv[h, off + 2 * i + 1] = z.real, z.imag
        logits = scale * qv @ kv_rot.T
        pr = softmax(np.concatenate([logits, sink[:, None].astype(np.float64)], axis=1), axis=1)
        np.testing.assert_allclose(inv[t], pr[:, :-1] @ kv_raw, rtol=0, atol=1e-10)
