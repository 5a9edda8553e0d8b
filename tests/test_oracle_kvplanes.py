"""Pins of the low-bit KV planes of the oracle ([V41] cache ABI: window KV
MXFP8 E4M3 with E8M0 group-of-32 scales; compressed KV packed MXFP4 E2M1 with
E4M3 group-of-16 scales; dequantised on cache reads).

* decode_e4m3 against values worked by hand from the format definition
  (tests/golden/e4m3_codes.json) and, for all 256 codes, against torch's
  float8_e4m3fn decode (a library routine written independently of this one);
* the group-to-channel mapping of both planes on hand-built rows;
* attention over the planes reduces exactly to attention over BF16 caches
  holding the same values (every dequantised value is exactly a BF16 value).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_e4m3_hand_table():
    d = json.load(open(os.path.join(HERE, "golden", "e4m3_codes.json")))["codes"]
    codes = np.array([int(k, 16) for k in d], dtype=np.uint8)
    got = oracle.decode_e4m3(codes)
    for c, g, (k, v) in zip(codes, got, d.items()):
        if v == "nan":
            assert math.isnan(g), k
        else:
            assert g == v and math.copysign(1.0, g) == math.copysign(1.0, v), (k, g, v)


def test_e4m3_all_codes_match_torch():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_mxfp8_plane_group_scales():
    # one row, D = 64: channel c holds code 0x38 (1.0) and group g of 32
    # channels the scale byte 127 + 3g + 1 (2^(3g+1)): the value of channel c
    # is 2^(3 * (c // 32) + 1)
    payload = np.full((1, 128, 64), 0x38, np.uint8)
    scales = np.zeros((1, 128, 2), np.uint8)
    scales[0, 5] = [128, 131]
    payload[0, 5, 40] = 0xC4   # -3.0 in the second group
    plane = oracle.mxfp8_plane(payload, scales)
    row = plane.rows([5])[0]
    want = np.where(np.arange(64) < 32, 2.0, 16.0)
    want[40] = -3.0 * 16.0
    assert np.array_equal(row, want)


def test_mxfp4_plane_nibbles_and_group16_scales():
    # D = 32: byte i holds elements 2i (bits 0-3) and 2i + 1 (bits 4-7);
    # code 0x2 is 1.0, 0xB is -1.5; scales: group 0 -> 0x39 (1.125), group 1
    # -> 0x4c (6.0)
    payload = np.zeros((1, 128, 16), np.uint8)
    payload[0, 9, :] = 0x22             # every element 1.0
    payload[0, 9, 3] = 0xB2             # element 6: 1.0, element 7: -1.5
    payload[0, 9, 12] = 0x2B            # element 24: -1.5, element 25: 1.0
    scales = np.zeros((1, 128, 2), np.uint8)
    scales[0, 9] = [0x39, 0x4C]
    row = oracle.mxfp4_e4m3_plane(payload, scales).rows([9])[0]
    want = np.where(np.arange(32) < 16, 1.125, 6.0)
    want[7] = -1.5 * 1.125
    want[24] = -1.5 * 6.0
    assert np.array_equal(row, want)


def _bf16_bits(x):
    f = np.asarray(x, np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(x)), "value not exact in float32"
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in BF16"
    return (u >> 16).astype(np.uint16)


def test_plane_attention_reduces_to_bf16_attention():
    """Random planes; BF16 caches holding exactly the dequantised values; the
    oracle's attention over either gives identical results."""
    rng = np.random.default_rng(3)
    H, D, R, W, k, ratio = 4, 64, 16, 8, 6, 1
    nbw, nbc = 3, 2
    # window plane: E4M3 codes with exponent field 4..10, E8M0 scales 124..129
    e = rng.integers(4, 11, (nbw, 128, D))
    m = rng.integers(0, 8, (nbw, 128, D))
    sgn = rng.integers(0, 2, (nbw, 128, D))
    win_fp8 = ((sgn << 7) | (e << 3) | m).astype(np.uint8)
    win_sc = rng.integers(124, 130, (nbw, 128, D // 32)).astype(np.uint8)
    # compressed plane: any E2M1 nibbles, positive E4M3 scales 2^-2 .. 2^1
    cmp_fp4 = rng.integers(0, 256, (nbc, 128, D // 2)).astype(np.uint8)
    se = rng.integers(5, 9, (nbc, 128, D // 16))
    cmp_sc = ((se << 3) | rng.integers(0, 8, (nbc, 128, D // 16))).astype(np.uint8)
    wplane = oracle.mxfp8_plane(win_fp8, win_sc)
    cplane = oracle.mxfp4_e4m3_plane(cmp_fp4, cmp_sc)
    win_bf16 = _bf16_bits(wplane.rows(np.arange(nbw * 128))).reshape(nbw, 128, D)
    cmp_bf16 = _bf16_bits(cplane.rows(np.arange(nbc * 128))).reshape(nbc, 128, D)
    T = 3
    qsl = np.array([0, 2, 3], np.int32)
    pos = np.array([200, 201, 150], np.int32)
    wbt = np.array([[2, 0], [1, 2]], np.int32)
    cbt = np.array([[1, 0], [0, 1]], np.int32)
    q = _bf16_bits(np.clip(np.round(rng.standard_normal((T, H, D)) * 16), -127, 127) / 16)
    topk = np.array([[5, 130, 17, 199, -1, -1], [0, 1, 2, 3, 4, 150],
                     [149, 2, -1, -1, -1, -1]], np.int32)
    rc = np.cos(rng.uniform(0, 6, (T, R // 2))).astype(np.float32)
    rs = np.sin(rng.uniform(0, 6, (T, R // 2))).astype(np.float32)
    sink = rng.standard_normal(H)
    args = dict(rope_offset=D - R, topk_idx=topk, ratio=ratio, window=W, attn_sink=sink,
                softmax_scale=0.125, query_start_loc=qsl, positions=pos, num_tokens=T)
    o1, l1, e1 = oracle.sparse_attn(q, rc, rs, cmp_kv=cplane, cmp_block_table=cbt,
                                    win_kv=wplane, win_block_table=wbt, **args)
    o2, l2, e2 = oracle.sparse_attn(q, rc, rs, cmp_kv=cmp_bf16, cmp_block_table=cbt,
                                    win_kv=win_bf16, win_block_table=wbt, **args)
    assert e1 == e2 == 0
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.all(np.isfinite(o1))
