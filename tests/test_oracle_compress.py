"""Pins for the oracle's ratio-2 compressor publication and its state ring.

* BF16 rounding from float64: values of the format worked by hand, ties to
  even.
* Pooling: equal gates average the pair; gates ln 3 apart weight it 1/4, 3/4;
  RMSNorm then gives a hand-computed row; a quarter-turn rope row maps
  (x, y) to (-y, x) and the identity row changes nothing.
* The ring: slot p % CAP of the request's block, only the last min(chunk,
  CAP) rows of a chunk written, the predecessor of a chunk's first odd token
  read from the ring before the chunk overwrites that slot.
* Chunking invariance: one request's tokens compressed in one chunk or in
  several (the ring carrying the pending token) publish the same rows and
  leave the same ring.
* Contract: a disabled request (block -1) and negative positions touch
  nothing; an out-of-pool state block or publication page and an unowned row
  are flagged.
"""
import math

import numpy as np

import oracle

PAGE = 128


def test_bf16_rounding_by_hand():
    cases = {1.0: 0x3F80, 1.0 + 2 ** -8: 0x3F80, 1.0 + 3 * 2 ** -9: 0x3F81, 3.0: 0x4040,
             -2.0: 0xC000, 1.0 + 2 ** -7 + 2 ** -8: 0x3F82, 0.5 - 2 ** -12: 0x3F00}
    for v, bits in cases.items():
        assert int(oracle.f64_to_bf16(np.array([v]))[0]) == bits, v


def _call(kv, g, qsl, pos, sbt, state, cmp_bt, nb=4, gamma=None, eps=0.0, rope=None, off=0,
          cmp=None):
    T, D = kv.shape
    if gamma is None:
        gamma = np.ones(D, np.float32)
    if rope is None:
        rope = (np.ones((T, 0), np.float32), np.zeros((T, 0), np.float32))
    if cmp is None:
        cmp = np.full((nb, PAGE, D), 0x7FDE, np.uint16)   # sentinel bits
    return oracle.compress_pairs(kv.astype(np.float32), g.astype(np.float32),
                                 np.asarray(qsl, np.int32), np.asarray(pos, np.int32), T,
                                 np.asarray(sbt, np.int32), state, gamma, eps, rope[0], rope[1],
                                 off, cmp, np.asarray(cmp_bt, np.int32))


def test_pooling_rmsnorm_and_rope_by_hand():
    D = 4
    state = np.zeros((2, 4, 2 * D), np.float32)
    kv = np.array([[1, 5, 1, 5], [3, 1, 3, 1]], np.float64)
    # equal gates: the pair's mean, 2 and 3 -> x = [2, 3, 2, 3]
    g = np.zeros((2, D))
    cmp, st, err = _call(kv, g, [0, 2], [6, 7], [1], state, [[2]])
    assert err == 0
    x = np.array([2.0, 3.0, 2.0, 3.0])
    y = x / math.sqrt(np.mean(x * x))
    assert np.array_equal(cmp[2, 3], oracle.f64_to_bf16(y))       # compressed position 7 // 2
    assert np.all(cmp[2, :3] == 0x7FDE) and np.all(cmp[2, 4:] == 0x7FDE)
    # gates ln 3 apart (token 7 higher): weights 1/4, 3/4 -> x = [2.5, 2, 2.5, 2]
    g = np.zeros((2, D))
    g[1] = math.log(3.0)
    cmp, _, _ = _call(kv, g, [0, 2], [6, 7], [1], state, [[2]])
    x = np.array([2.5, 2.0, 2.5, 2.0])
    y = x / math.sqrt(np.mean(x * x))                               # mean(x^2) = 5.125
    assert np.array_equal(cmp[2, 3], oracle.f64_to_bf16(y))
    # a quarter-turn rope row on channels 2..3: (x, y) -> (-y, x); gamma 2, eps 1
    rope = (np.array([[1.0], [0.0]], np.float32), np.array([[0.0], [1.0]], np.float32))
    cmp, _, _ = _call(kv, g, [0, 2], [6, 7], [1], state, [[2]], gamma=np.full(D, 2.0, np.float32),
                      eps=1.0, rope=rope, off=2)
    z = 2.0 * x / math.sqrt(np.mean(x * x) + 1.0)
    assert np.array_equal(cmp[2, 3], oracle.f64_to_bf16([z[0], z[1], -z[3], z[2]]))
    # the identity rope row changes nothing
    ident = (np.ones((2, 1), np.float32), np.zeros((2, 1), np.float32))
    a, _, _ = _call(kv, g, [0, 2], [6, 7], [1], state, [[2]], rope=ident, off=2)
    b, _, _ = _call(kv, g, [0, 2], [6, 7], [1], state, [[2]])
    assert np.array_equal(a, b)


def test_ring_slots_last_rows_and_read_before_write():
    rng = np.random.default_rng(50)
    D, cap = 4, 4
    state = rng.standard_normal((3, cap, 2 * D)).astype(np.float32)
    # request 0: chunk at positions 13..17 (5 rows > CAP), block 2
    kv = rng.standard_normal((5, D))
    g = rng.standard_normal((5, D))
    cmp, st, err = _call(kv, g, [0, 5], list(range(13, 18)), [2], state, [[0]])
    assert err == 0
    # rows 14..17 written at slots 2, 3, 0, 1; row 13 (not among the last 4) is not
    for t, p in enumerate(range(13, 18)):
        if p >= 14:
            assert np.array_equal(st[2, p % cap], np.concatenate([kv[t], g[t]]).astype(np.float32))
    assert np.array_equal(st[:2], state[:2])                   # other blocks untouched
    # 13 is odd and first: its predecessor (12) came from slot 0 *before* 16 overwrote it
    prev = state[2, 12 % cap].astype(np.float64)
    one = _call(np.stack([prev[:D], kv[0]]), np.stack([prev[D:], g[0]]), [0, 2], [12, 13], [0],
                np.zeros((1, cap, 2 * D), np.float32), [[0]])[0]
    assert np.array_equal(cmp[0, 6], one[0, 6])                # compressed position 13 // 2
    # 15 and 17 closed their pairs inside the chunk
    assert not np.any(cmp[0, 7] == 0x7FDE) and not np.any(cmp[0, 8] == 0x7FDE)
    assert np.all(cmp[0, 9:] == 0x7FDE) and np.all(cmp[0, :6] == 0x7FDE)
    # a 2-row chunk writes both rows
    _, st2, _ = _call(kv[:2], g[:2], [0, 2], [20, 21], [1], state, [[0]])
    assert np.array_equal(st2[1, 0], np.concatenate([kv[0], g[0]]).astype(np.float32))
    assert np.array_equal(st2[1, 1], np.concatenate([kv[1], g[1]]).astype(np.float32))
    assert np.array_equal(st2[1, 2:], state[1, 2:])


def test_chunking_invariance():
    rng = np.random.default_rng(51)
    D, cap, n = 8, 4, 14
    kv = rng.standard_normal((n, D))
    g = rng.standard_normal((n, D))
    gamma = rng.uniform(0.5, 2.0, D).astype(np.float32)
    ang = rng.uniform(-3, 3, (n, 2))
    rope = (np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32))
    state0 = rng.standard_normal((1, cap, 2 * D)).astype(np.float32)
    whole, st_whole, e = _call(kv, g, [0, n], range(n), [0], state0, [[1]], nb=2, gamma=gamma,
                               eps=1e-6, rope=rope, off=4)
    assert e == 0
    cmp = np.full((2, PAGE, D), 0x7FDE, np.uint16)
    st = state0
    t0 = 0
    for chunk in (3, 1, 4, 2, 4):
        sl = slice(t0, t0 + chunk)
        cmp, st, e = _call(kv[sl], g[sl], [0, chunk], range(t0, t0 + chunk), [0], st, [[1]],
                           gamma=gamma, eps=1e-6, rope=(rope[0][sl], rope[1][sl]), off=4, cmp=cmp)
        assert e == 0
        t0 += chunk
    assert np.array_equal(cmp, whole)
    assert np.array_equal(st, st_whole)
    assert not np.any(whole[1, :n // 2] == 0x7FDE) and np.all(whole[1, n // 2:] == 0x7FDE)


def test_contract_cases():
    rng = np.random.default_rng(52)
    D, cap = 4, 4
    state = rng.standard_normal((2, cap, 2 * D)).astype(np.float32)
    kv = rng.standard_normal((6, D))
    g = rng.standard_normal((6, D))
    # request 0 disabled (block -1); request 1 has a negative position row
    cmp, st, err = _call(kv[:4], g[:4], [0, 2, 4], [4, 5, 3, -1], [-1, 1], state, [[0], [1]])
    assert err == 0
    assert np.all(cmp[0] == 0x7FDE)                          # nothing from request 0
    assert np.array_equal(st[0], state[0])
    # request 1: position 3 (first, odd) reads slot 2 and publishes compressed
    # position 1; -1 neither publishes nor writes
    prev = state[1, 2].astype(np.float64)
    one = _call(np.stack([prev[:D], kv[2]]), np.stack([prev[D:], g[2]]), [0, 2], [2, 3], [0],
                np.zeros((1, cap, 2 * D), np.float32), [[0]])[0]
    assert np.array_equal(cmp[1, 1], one[0, 1])
    assert np.array_equal(st[1, 3], np.concatenate([kv[2], g[2]]).astype(np.float32))
    assert np.array_equal(np.delete(st[1], 3, axis=0), np.delete(state[1], 3, axis=0))
    # a state block past the pool, a publication page past the table, an unowned row
    _, st, err = _call(kv[:2], g[:2], [0, 2], [8, 9], [5], state, [[0]])
    assert err == oracle.EFLAG_BLOCK_RANGE and np.array_equal(st, state)
    cmp, st, err = _call(kv[:2], g[:2], [0, 2], [300, 301], [1], state, [[0]])
    assert err == oracle.EFLAG_BLOCK_RANGE and np.all(cmp == 0x7FDE)
    assert np.array_equal(st[1, 0], np.concatenate([kv[0], g[0]]).astype(np.float32))
    _, _, err = _call(kv[:3], g[:3], [0, 2], [8, 9, 10], [1], state, [[0]])
    assert err == oracle.EFLAG_META
