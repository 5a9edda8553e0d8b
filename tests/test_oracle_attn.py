"""Pins for the oracle's shared-KV sparse attention with sink.

Checked against: the hand-worked case in tests/golden/attn_hand.json; a sink
of -inf reducing to textbook softmax attention (scipy.special.softmax and
logsumexp over rows gathered by an independent route); the one-key closed
form v * sigmoid(l - a); all-equal rows giving v * (1 - p_sink); invariance
under permuting the selection and shuffling block tables; k covering every
visible compressed row equalling dense causal attention over those rows plus
the window; the relative-position property of the query rotation; the window
extent of gitcode hyper-parallel issue #2 section 7.1; and the union without
dedup of section 9.1.  The layers without an indexer are checked the same
way: the HCA selection (every visible compressed row) against the dense
route and an explicit selection, its bound, and the SWA-only window.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from tests.tiny import PAGE, bf16_bits, bf16_value, paged_pool, random_block_table


def _build(rng, *, B=1, rows=(2,), H=4, D=32, R=8, W=16, ratio=2, k=8, ctx=(300,),
           sink=None, pos=None, topk=None, cmp_dense=None, win_dense=None, rope=None,
           bt_seed=0):
    T = sum(rows)
    qsl = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    if pos is None:
        pos = np.concatenate([np.arange(c - r, c) for r, c in zip(rows, ctx)]).astype(np.int32)
    ncmp = [c // ratio for c in ctx]
    cpages = max(1, max(-(-n // PAGE) for n in ncmp))
    wpages = max(1, max(-(-c // PAGE) for c in ctx))
    if cmp_dense is None:
        cmp_dense = [bf16_bits(rng.standard_normal((cpages * PAGE, D))) for _ in range(B)]
    if win_dense is None:
        win_dense = [bf16_bits(rng.standard_normal((wpages * PAGE, D))) for _ in range(B)]
    brng = np.random.default_rng(bt_seed)
    cbt, ncb = random_block_table(brng, B, cpages, extra=1)
    wbt, nwb = random_block_table(brng, B, wpages, extra=1)
    cmp_kv = paged_pool(cmp_dense, cbt, ncb)
    win_kv = paged_pool(win_dense, wbt, nwb)
    q = bf16_bits(rng.standard_normal((T, H, D)))
    if rope is None:
        ang = rng.uniform(-3, 3, (T, R // 2))
        rope = (np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32))
    if sink is None:
        sink = rng.standard_normal(H).astype(np.float32)
    if topk is None:
        topk = np.full((T, k), -1, np.int32)
        for t in range(T):
            nv = oracle.visible_count(pos[t], ratio)
            m = min(k, nv)
            topk[t, :m] = np.sort(rng.choice(nv, m, replace=False))
    return dict(q=q, rope_cos=rope[0], rope_sin=rope[1], rope_offset=D - R, cmp_kv=cmp_kv,
                cmp_block_table=cbt, topk_idx=topk, ratio=ratio, win_kv=win_kv,
                win_block_table=wbt, window=W, attn_sink=sink,
                softmax_scale=1.0 / math.sqrt(D), query_start_loc=qsl, positions=pos,
                num_tokens=T), cmp_dense, win_dense


def _dense_reference(a, cmp_dense, win_dense, sink_override=None):
    """Independent route: gather logical rows from the dense per-request arrays,
    rotate q with Python complex numbers, softmax with scipy."""
    T, H, D = a["q"].shape
    R = 2 * a["rope_cos"].shape[1]
    off = a["rope_offset"]
    sink = a["attn_sink"].astype(np.float64) if sink_override is None else sink_override
    qsl = a["query_start_loc"]
    out = np.zeros((T, H, D))
    lse = np.zeros((T, H))
    for t in range(T):
        b = int(np.searchsorted(qsl, t, side="right") - 1)
        p = int(a["positions"][t])
        nv = max(0, (p + 1) // a["ratio"])
        rows = [bf16_value(win_dense[b][j]) for j in range(max(0, p - a["window"] + 1), p + 1)]
        rows += [bf16_value(cmp_dense[b][c]) for c in a["topk_idx"][t] if 0 <= c < nv]
        kv = np.array(rows).reshape(-1, D)
        qv = bf16_value(a["q"][t]).copy()
        for h in range(H):
            for i in range(R // 2):
                z = complex(qv[h, off + 2 * i], qv[h, off + 2 * i + 1]) * complex(
                    float(a["rope_cos"][t, i]), float(a["rope_sin"][t, i]))
                qv[h, off + 2 * i], qv[h, off + 2 * i + 1] = z.real, z.imag
        logits = a["softmax_scale"] * qv @ kv.T
        full = np.concatenate([logits, sink[:, None]], axis=1)
        pr = softmax(full, axis=1)
        out[t] = pr[:, :-1] @ kv
        lse[t] = logsumexp(full, axis=1)
    return out, lse


def test_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "attn_hand.json")))
    win = np.zeros((PAGE, 2), np.uint16)
    win[0] = bf16_bits(g["window_row"])
    cmp_ = np.zeros((PAGE, 2), np.uint16)
    cmp_[0] = bf16_bits(g["selected_row"])
    a = dict(q=bf16_bits(np.array(g["q"]))[None, None, :],
             rope_cos=np.array([g["rope_cos"]], np.float32),
             rope_sin=np.array([g["rope_sin"]], np.float32), rope_offset=0,
             cmp_kv=cmp_[None], cmp_block_table=np.array([[0]], np.int32),
             topk_idx=np.array([[0, -1]], np.int32), ratio=1, win_kv=win[None],
             win_block_table=np.array([[0]], np.int32), window=1,
             attn_sink=np.array([g["sink"]], np.float32), softmax_scale=1.0,
             query_start_loc=np.array([0, 1], np.int32), positions=np.array([0], np.int32),
             num_tokens=1)
    out, lse, err = oracle.sparse_attn(**a)
    assert err == 0
    assert out[0, 0].tolist() == pytest.approx(g["expected_out"], rel=1e-14)
    assert lse[0, 0] == pytest.approx(g["expected_lse"], rel=1e-14)


def test_matches_textbook_softmax_attention():
    rng = np.random.default_rng(20)
    a, cd, wd = _build(rng, B=2, rows=(2, 3), ctx=(300, 700), k=12, W=16)
    out, lse, err = oracle.sparse_attn(**a)
    assert err == 0
    ro, rl = _dense_reference(a, cd, wd)
    assert np.allclose(out, ro, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_sink_minus_inf_is_plain_softmax():
    rng = np.random.default_rng(21)
    a, cd, wd = _build(rng, rows=(3,), ctx=(260,))
    a["attn_sink"] = np.full(4, -np.inf, np.float32)
    out, lse, _ = oracle.sparse_attn(**a)
    ro, rl = _dense_reference(a, cd, wd, sink_override=np.full(4, -np.inf))
    assert np.allclose(out, ro, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_one_key_closed_form():
    rng = np.random.default_rng(22)
    a, cd, wd = _build(rng, rows=(1,), ctx=(1,), W=1, ratio=2, k=4)  # p=0: window {0}, nothing visible
    out, lse, _ = oracle.sparse_attn(**a)
    v = bf16_value(wd[0][0])
    qv = bf16_value(a["q"][0])
    off, R = a["rope_offset"], 2 * a["rope_cos"].shape[1]
    for h in range(4):
        qh = qv[h].copy()
        for i in range(R // 2):
            z = complex(qh[off + 2 * i], qh[off + 2 * i + 1]) * complex(
                float(a["rope_cos"][0, i]), float(a["rope_sin"][0, i]))
            qh[off + 2 * i], qh[off + 2 * i + 1] = z.real, z.imag
        l = a["softmax_scale"] * float(qh @ v)
        s = float(a["attn_sink"][h])
        sig = 1.0 / (1.0 + math.exp(s - l))
        assert np.allclose(out[0, h], v * sig, rtol=1e-12, atol=1e-14)
        assert lse[0, h] == pytest.approx(math.log(math.exp(s) + math.exp(l)), rel=1e-12)


def test_equal_rows_give_one_minus_sink_mass():
    rng = np.random.default_rng(23)
    D = 32
    row = bf16_bits(rng.standard_normal(D))
    cd = [np.tile(row, (3 * PAGE, 1))]
    wd = [np.tile(row, (3 * PAGE, 1))]
    a, _, _ = _build(rng, rows=(2,), ctx=(300,), cmp_dense=cd, win_dense=wd)
    out, lse, _ = oracle.sparse_attn(**a)
    v = bf16_value(row)
    for t in range(2):
        for h in range(4):
            p_sink = math.exp(float(a["attn_sink"][h]) - lse[t, h])
            assert np.allclose(out[t, h], v * (1.0 - p_sink), rtol=1e-12, atol=1e-14)


def test_selection_permutation_and_table_shuffle_invariance():
    rng = np.random.default_rng(24)
    a, cd, wd = _build(rng, B=2, rows=(2, 2), ctx=(400, 500), k=10)
    out0, lse0, _ = oracle.sparse_attn(**a)
    b = dict(a)
    b["topk_idx"] = np.ascontiguousarray(a["topk_idx"][:, ::-1])
    out1, lse1, _ = oracle.sparse_attn(**b)
    assert np.allclose(out0, out1, rtol=1e-13, atol=1e-14) and np.allclose(lse0, lse1)
    c, _, _ = _build(np.random.default_rng(24), B=2, rows=(2, 2), ctx=(400, 500), k=10,
                     cmp_dense=cd, win_dense=wd, bt_seed=5, topk=a["topk_idx"],
                     rope=(a["rope_cos"], a["rope_sin"]), sink=a["attn_sink"])
    c["q"] = a["q"]
    out2, lse2, _ = oracle.sparse_attn(**c)
    assert np.allclose(out0, out2, rtol=1e-13, atol=1e-14) and np.allclose(lse0, lse2)


def test_k_covering_all_visible_is_dense_causal_attention():
    rng = np.random.default_rng(25)
    ctx, ratio, W = 200, 2, 16
    a, cd, wd = _build(rng, rows=(3,), ctx=(ctx,), ratio=ratio, W=W, k=128)
    for t in range(3):
        nv = oracle.visible_count(a["positions"][t], ratio)
        a["topk_idx"][t, :nv] = np.arange(nv)
        a["topk_idx"][t, nv:] = -1
    out, lse, _ = oracle.sparse_attn(**a)
    D = a["q"].shape[2]
    for t in range(3):
        # dense route: score every raw and every compressed row, then mask causally
        p = int(a["positions"][t])
        nv = (p + 1) // ratio
        allrows = np.concatenate([bf16_value(wd[0][:ctx]), bf16_value(cd[0][:ctx // ratio])])
        keep = np.zeros(allrows.shape[0], bool)
        keep[max(0, p - W + 1):p + 1] = True
        keep[ctx:ctx + nv] = True
        r = _one_row(a, t)
        qv = bf16_value(r["q"][0]).copy()
        off = r["rope_offset"]
        for h in range(qv.shape[0]):
            for i in range(r["rope_cos"].shape[1]):
                z = complex(qv[h, off + 2 * i], qv[h, off + 2 * i + 1]) * complex(
                    float(r["rope_cos"][0, i]), float(r["rope_sin"][0, i]))
                qv[h, off + 2 * i], qv[h, off + 2 * i + 1] = z.real, z.imag
        logits = a["softmax_scale"] * qv @ allrows.T
        logits[:, ~keep] = -np.inf
        full = np.concatenate([logits, a["attn_sink"].astype(np.float64)[:, None]], axis=1)
        pr = softmax(full, axis=1)
        assert np.allclose(out[t], pr[:, :-1] @ allrows, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[t], logsumexp(full, axis=1), rtol=1e-12)


def _one_row(a, t):
    r = dict(a)
    r["q"] = a["q"][t:t + 1]
    r["rope_cos"] = a["rope_cos"][t:t + 1]
    r["rope_sin"] = a["rope_sin"][t:t + 1]
    r["topk_idx"] = a["topk_idx"][t:t + 1]
    r["positions"] = a["positions"][t:t + 1]
    r["query_start_loc"] = np.array([0, 1], np.int32)
    r["num_tokens"] = 1
    return r


def test_rotation_relative_position_property():
    # pre-rotating the rope channels of every key by the query's angle makes
    # the rotated-query logits equal the unrotated-query logits on raw keys
    rng = np.random.default_rng(26)
    D, R, H = 16, 8, 2
    off = D - R
    ang = rng.uniform(-3, 3, R // 2)
    keys = rng.standard_normal((4, D))
    keys_rot = keys.copy()
    keys_rot[:, off:] = oracle.rotate_adjacent_pairs(keys[:, off:], np.cos(ang), np.sin(ang))
    q = rng.standard_normal((H, D))
    q_rot = q.copy()
    q_rot[:, off:] = oracle.rotate_adjacent_pairs(q[:, off:], np.cos(ang), np.sin(ang))
    assert np.allclose(q_rot @ keys_rot.T, q @ keys.T)


def test_identity_rope_row_equals_unrotated_query():
    rng = np.random.default_rng(27)
    a, cd, wd = _build(rng, rows=(2,), ctx=(300,))
    a["rope_cos"] = np.ones_like(a["rope_cos"])
    a["rope_sin"] = np.zeros_like(a["rope_sin"])
    out, lse, _ = oracle.sparse_attn(**a)
    D = a["q"].shape[2]
    # with the rope slice at offset D (no rotary channels) the answer is the same
    b = dict(a)
    b["rope_cos"] = a["rope_cos"][:, :0]
    b["rope_sin"] = a["rope_sin"][:, :0]
    b["rope_offset"] = D
    out2, lse2, _ = oracle.sparse_attn(**b)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_window_extent_and_no_dedup(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "visibility.json")))["window"]["cases"][0]
    rng = np.random.default_rng(28)
    D = 8
    a, cd, wd = _build(rng, rows=(1,), ctx=(g["p"] + 1,), W=g["window"], ratio=1, k=2, D=D, R=2,
                       H=1)
    a["topk_idx"][0] = [g["p"], -1]         # the query's own position, selected again
    wr, cr, err = oracle.kv_rows_for_query(0, 0, g["p"], a["topk_idx"][0], 1, g["window"],
                                           a["cmp_block_table"], a["cmp_kv"].shape[0],
                                           a["win_block_table"], a["win_kv"].shape[0])
    assert err == 0
    win_flat = a["win_kv"].reshape(-1, D)
    got = [bf16_value(win_flat[r]).tolist() for r in wr]
    assert got == [bf16_value(wd[0][j]).tolist() for j in g["sees"]]
    assert len(cr) == 1  # same position from the other cache is kept, not merged


def test_contract_flags_and_empty_set():
    rng = np.random.default_rng(29)
    a, cd, wd = _build(rng, rows=(2,), ctx=(300,), k=4)
    a["topk_idx"][0, 0] = 10_000              # not visible
    out, lse, err = oracle.sparse_attn(**a)
    assert err == oracle.EFLAG_TOPK_RANGE
    # the first invisible slot, exactly (p + 1) // ratio, is out as well
    nv = oracle.visible_count(a["positions"][0], a["ratio"])
    a["topk_idx"][0, 0] = nv
    out_b, lse_b, err = oracle.sparse_attn(**a)
    assert err == oracle.EFLAG_TOPK_RANGE
    assert np.array_equal(out_b, out) and np.array_equal(lse_b, lse)
    # an empty key set: position -1 sees no window and no compressed row
    a["positions"] = np.array([-1, -1], np.int32)
    a["topk_idx"][:] = -1
    out, lse, err = oracle.sparse_attn(**a)
    assert err == 0 and np.all(out == 0) and np.allclose(lse, a["attn_sink"][None, :])
    # unowned row
    a["query_start_loc"] = np.array([0, 1], np.int32)
    out, lse, err = oracle.sparse_attn(**a)
    assert err == oracle.EFLAG_META and np.all(out[1] == 0)


# ---- layers without an indexer: HCA (every visible compressed row) and
#      SWA-only (the window alone)

def test_hca_selection_is_dense_causal_attention():
    """No selection array: every causally visible compressed row plus the
    window, checked by the independent dense route (scipy softmax) and
    against the same rows passed as an explicit selection."""
    rng = np.random.default_rng(41)
    ctx, ratio, W = 1100, 128, 16     # ratio 128: 7 .. 8 visible compressed rows
    a, cd, wd = _build(rng, rows=(2, 3), B=2, ctx=(ctx, 900), ratio=ratio, W=W, k=16)
    a["topk_idx"] = None
    out, lse, err = oracle.sparse_attn(**a, k=16)
    assert err == 0
    explicit = np.full((a["num_tokens"], 16), -1, np.int32)
    for t in range(a["num_tokens"]):
        nv = oracle.visible_count(a["positions"][t], ratio)
        assert 1 <= nv <= 16
        explicit[t, :nv] = np.arange(nv)
    b = dict(a, topk_idx=explicit)
    out2, lse2, err2 = oracle.sparse_attn(**b)
    assert err2 == 0 and np.array_equal(out, out2) and np.array_equal(lse, lse2)
    ro, rl = _dense_reference(b, cd, wd)
    assert np.allclose(out, ro, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, rl, rtol=1e-12)


def test_hca_selection_bound():
    """A row with more visible compressed rows than the bound keeps the first
    k of them and reports TOPK_RANGE."""
    assert oracle.deterministic_selection(1279, 128, 16)[1] == 0
    sel, e = oracle.deterministic_selection(1279, 128, 16)
    assert np.array_equal(sel, np.arange(10)) and e == 0
    sel, e = oracle.deterministic_selection(1279, 128, 4)
    assert np.array_equal(sel, np.arange(4)) and e == oracle.EFLAG_TOPK_RANGE
    sel, e = oracle.deterministic_selection(126, 128, 4)
    assert sel.size == 0 and e == 0
    sel, e = oracle.deterministic_selection(1279, 128, 0)   # k = 0: the window alone
    assert sel.size == 0 and e == 0
    rng = np.random.default_rng(43)
    a, cd, wd = _build(rng, rows=(1,), ctx=(1100,), ratio=128, W=8, k=4)
    a["topk_idx"] = None
    out, lse, err = oracle.sparse_attn(**a, k=4)
    assert err == oracle.EFLAG_TOPK_RANGE
    b = dict(a, topk_idx=np.arange(4, dtype=np.int32)[None, :])
    out2, lse2, _ = oracle.sparse_attn(**b)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_swa_only_is_window_softmax_attention():
    """A selection with no columns attends over the window alone: the
    independent dense route over the window rows."""
    rng = np.random.default_rng(47)
    a, cd, wd = _build(rng, rows=(3,), ctx=(400,), ratio=4, W=32, k=4)
    a["topk_idx"] = np.zeros((a["num_tokens"], 0), np.int32)
    out, lse, err = oracle.sparse_attn(**a)
    assert err == 0
    ro, rl = _dense_reference(a, cd, wd)
    assert np.allclose(out, ro, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, rl, rtol=1e-12)
