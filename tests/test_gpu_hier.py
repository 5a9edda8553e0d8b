"""GPU parity of the hierarchical selection entry points against the oracle.

csa_candidate_blocks is compared exactly (the block score is a max of the
same FP32 scores, so the ranking is the same); csa_index_score_candidates to
the score tolerance, its -inf pattern and prefix counts exactly, and bit for
bit against csa_index_score at the same positions; csa_topk_candidates
exactly on the GPU's own scores.  The whole hierarchical chain (full layer
scores -> candidate mask -> reindex scores -> top-k -> attention) runs on C2
shapes against the oracle's chain.
"""
import numpy as np
import pytest

import oracle
import synthetic
from tests import harness as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _csa():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


def _dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda()


def _gpu_candidate_blocks(scores, positions, ratio, block, kb):
    csa = _csa()
    T, stride = scores.shape
    s = _dev(scores.astype(np.float32))
    pos = _dev(positions.astype(np.int32))
    cb = torch.full((T, kb), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(16, csa.csa_candidate_blocks_workspace_bytes(T, stride, block, kb)),
                     dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    csa.csa_candidate_blocks(s, pos, ratio, T, block, cb, ws, err=err)
    torch.cuda.synchronize()
    return cb.cpu().numpy(), int(err.item())


@pytest.mark.parametrize("T,stride,block,kb,ties", [
    (6, 300, 8, 7, False),
    (6, 300, 8, 7, True),
    (5, 4096, 1, 512, True),
    (4, 2048, 128, 3, False),
    (4, 131072, 8, 2048, False),
    (4, 131072, 8, 2048, True),
    (2, 1 << 20, 8, 2048, False),
])
def test_candidate_blocks_parity(T, stride, block, kb, ties):
    rng = np.random.default_rng(stride + block + kb + int(ties))
    s = rng.standard_normal((T, stride)).astype(np.float32)
    if ties:
        s = (np.round(s * 4) / 4).astype(np.float32)
    pos = rng.integers(0, stride, size=T).astype(np.int32)
    pos[0] = stride - 1            # the whole row
    if T > 2:
        pos[1] = -1                # nothing visible
    if T > 3:
        pos[2] = stride + 500      # past the row: POS_RANGE, cut to the row
    print(f"[hier] candidate_blocks T={T} stride={stride} block={block} kb={kb}", flush=True)
    g, ge = _gpu_candidate_blocks(s, pos, 1, block, kb)
    o, oe = oracle.candidate_blocks(s.astype(np.float64), pos, 1, T, block, kb)
    np.testing.assert_array_equal(g, o)
    assert ge == oe


def _paged_case(name, seed=0):
    cfg = synthetic.get(name)
    x = synthetic.make_inputs(cfg, seed=seed, with_tables=False).t
    return cfg, x


def _random_masks(rng, positions, ratio, block, kb, extra_bad_row=None):
    T = len(positions)
    cand = np.full((T, kb), -1, np.int32)
    for t in range(T):
        nb = -(-oracle.visible_count(int(positions[t]), ratio) // block)
        m = min(kb - 1, nb)
        if t == 0:
            m = min(kb, nb)            # a full mask
        pick = set(rng.choice(nb, size=m, replace=False).tolist()) if m else set()
        if t == 0 and nb > 0 and (nb - 1) not in pick:
            # the row's last (possibly partial) block at the end of the mask
            if len(pick) == kb:
                pick.discard(min(pick))
            pick.add(nb - 1)
        pick = sorted(pick)
        cand[t, :len(pick)] = pick
    if extra_bad_row is not None:
        t = extra_bad_row
        nb = -(-oracle.visible_count(int(positions[t]), ratio) // block)
        cand[t] = -1
        cand[t, :2] = [0, nb + 3]      # a block past the span
    return cand


def _gpu_index_candidates(x, cfg, cand, block, stride=None):
    csa = _csa()
    T, kb = cand.shape
    stride = stride or (kb * block + 3) // 4 * 4
    d = {k: _dev(x[k]) for k in ("q_idx", "q_scale", "head_w", "idx_kv", "idx_scale",
                                 "cmp_block_table", "query_start_loc", "positions")}
    cs = torch.full((T, stride), 12345.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((T,), -5, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    cb = _dev(cand)
    csa.csa_index_score_candidates(d["q_idx"], d["q_scale"], d["head_w"], d["idx_kv"],
                                   d["idx_scale"], d["cmp_block_table"], d["query_start_loc"],
                                   d["positions"], T, cfg.ratio, cb, block, cs, cnt, err=err)
    torch.cuda.synchronize()
    return d, cb, cs, cnt, err


@pytest.mark.parametrize("name,kb", [("c1", 5), ("c1", 40), ("c2", 256), ("c3", 2048)])
def test_index_score_candidates_parity(name, kb):
    block = 8
    cfg, x = _paged_case(name)
    rng = np.random.default_rng(kb)
    T = cfg.T
    cand = _random_masks(rng, x["positions"], cfg.ratio, block, kb,
                         extra_bad_row=T - 1 if T > 2 else None)
    print(f"[hier] index_score_candidates {name} kb={kb}", flush=True)
    d, cb, cs, cnt, err = _gpu_index_candidates(x, cfg, cand, block)
    g = cs.cpu().numpy().astype(np.float64)[:, :kb * block]
    o, oe = oracle.index_scores_in_candidates(x["q_idx"], x["q_scale"], x["head_w"], x["idx_kv"],
                                              x["idx_scale"], x["cmp_block_table"],
                                              x["query_start_loc"], x["positions"], T, cfg.ratio,
                                              cand, block)
    H.check_scores(g, o, f"{name} candidate scores")
    assert int(err.item()) == oe
    # the eligible prefix of every well-formed row
    cnt = cnt.cpu().numpy()
    for t in range(T):
        nv = oracle.visible_count(int(x["positions"][t]), cfg.ratio)
        _, elig = oracle.candidate_positions(cand[t], block, nv)
        first_bad = int(np.argmin(elig)) if not elig.all() else len(elig)
        assert cnt[t] == first_bad, (t, cnt[t], first_bad)
    # bit for bit the full scorer's value at the same position
    full = torch.empty((T, cfg.score_stride), dtype=torch.float32, device="cuda")
    _csa().csa_index_score(d["q_idx"], d["q_scale"], d["head_w"], d["idx_kv"], d["idx_scale"],
                           d["cmp_block_table"], d["query_start_loc"], d["positions"], T,
                           cfg.ratio, full)
    torch.cuda.synchronize()
    f = full.cpu().numpy()
    gb = cs.cpu().numpy()
    for t in range(T):
        nv = oracle.visible_count(int(x["positions"][t]), cfg.ratio)
        pos, elig = oracle.candidate_positions(cand[t], block, nv)
        sl = np.nonzero(elig)[0]
        np.testing.assert_array_equal(gb[t, sl].view(np.uint32), f[t, pos[sl]].view(np.uint32))


@pytest.mark.parametrize("name,kb,k", [("c1", 40, 32), ("c2", 256, 512), ("c2", 2048, 512),
                                       ("c3", 2048, 512), ("c3", 4096, 2048)])
def test_topk_candidates_parity(name, kb, k):
    block = 8
    cfg, x = _paged_case(name)
    rng = np.random.default_rng(7 * kb + k)
    T = cfg.T
    cand = _random_masks(rng, x["positions"], cfg.ratio, block, kb)
    print(f"[hier] topk_candidates {name} kb={kb} k={k}", flush=True)
    _, cb, cs, cnt, _ = _gpu_index_candidates(x, cfg, cand, block)
    csa = _csa()
    stride = cs.shape[1]
    idx = torch.full((T, k), -9, dtype=torch.int32, device="cuda")
    val = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, csa.csa_topk_candidates_workspace_bytes(T, stride, k)),
                     dtype=torch.uint8, device="cuda")
    csa.csa_topk_candidates(cs, cnt, cb, block, T, k, idx, val, ws)
    torch.cuda.synchronize()
    gs = cs.cpu().numpy().astype(np.float64)[:, :kb * block]
    oi, ov, _ = oracle.topk_in_candidates(gs, cand, block, x["positions"], cfg.ratio, T, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(val.cpu().numpy().astype(np.float64), ov)


def _block_scores(scores, positions, ratio, block):
    T, n = scores.shape
    nb = -(-n // block)
    out = np.full((T, nb), -np.inf)
    for t in range(T):
        nv = min(oracle.visible_count(int(positions[t]), ratio), n)
        for j in range(-(-nv // block)):
            out[t, j] = np.max(scores[t, j * block:min(nv, (j + 1) * block)])
    return out


def test_hierarchical_chain_c2():
    """Full layer scores -> candidate mask (256 blocks of 8) -> a reindex
    layer's own scores inside the mask -> its top-512 -> attention."""
    csa = _csa()
    cfg = synthetic.get("c2")
    x = synthetic.make_inputs(cfg, seed=0).t
    T, block, kb = cfg.T, 8, 256
    step = csa.step_for_config(cfg, x)
    step.rope()
    step.index()
    cb = torch.empty((T, kb), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(16, csa.csa_candidate_blocks_workspace_bytes(
        T, step.score_stride, block, kb)), dtype=torch.uint8, device="cuda")
    csa.csa_candidate_blocks(step.scores, step.t["positions"], cfg.ratio, T, block, cb, ws)
    torch.cuda.synchronize()
    g_full = step.scores.cpu().numpy().astype(np.float64)
    g_cb = cb.cpu().numpy()
    # exact on the GPU's own scores; against the oracle's scores only block
    # scores within 1e-5 of the kb-th may trade places
    ref_cb, _ = oracle.candidate_blocks(g_full, x["positions"], cfg.ratio, T, block, kb)
    np.testing.assert_array_equal(g_cb, ref_cb)
    o_full, _ = oracle.index_scores(x["q_idx"], x["q_scale"], x["head_w"], x["idx_kv"],
                                    x["idx_scale"], x["cmp_block_table"], x["query_start_loc"],
                                    x["positions"], T, cfg.ratio, cfg.score_stride)
    o_cb, _ = oracle.candidate_blocks(o_full, x["positions"], cfg.ratio, T, block, kb)
    o_bs = _block_scores(o_full, x["positions"], cfg.ratio, block)
    for t in range(T):
        diff = np.setxor1d(g_cb[t][g_cb[t] >= 0], o_cb[t][o_cb[t] >= 0])
        if diff.size:
            sk = np.min(o_bs[t, o_cb[t][o_cb[t] >= 0]])
            assert np.all(np.abs(o_bs[t, diff] - sk) <= 1e-5 * abs(sk)), t

    # the reindex layer: its own index query, scored inside the GPU's mask
    rng = np.random.default_rng(11)
    q2 = rng.integers(-127, 128, size=x["q_idx"].shape).astype(np.int8)
    x2 = dict(x, q_idx=q2)
    _, _, cs, cnt, err = _gpu_index_candidates(x2, cfg, g_cb, block)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    csa.csa_topk_candidates(cs, cnt, cb, block, T, cfg.k, idx)
    step.attn(topk_idx=idx)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    o_sc, _ = oracle.index_scores_in_candidates(q2, x["q_scale"], x["head_w"], x["idx_kv"],
                                                x["idx_scale"], x["cmp_block_table"],
                                                x["query_start_loc"], x["positions"], T,
                                                cfg.ratio, g_cb, block)
    g_sc = cs.cpu().numpy().astype(np.float64)[:, :kb * block]
    H.check_scores(g_sc, o_sc, "reindex scores")
    g_idx = idx.cpu().numpy()
    g_ref, _, _ = oracle.topk_in_candidates(g_sc, g_cb, block, x["positions"], cfg.ratio, T,
                                            cfg.k)
    np.testing.assert_array_equal(g_idx, g_ref)
    # against the oracle's scores: ties within 1e-5 of the k-th may trade places
    o_idx, _, _ = oracle.topk_in_candidates(o_sc, g_cb, block, x["positions"], cfg.ratio, T,
                                            cfg.k)
    o_by_pos = np.full((T, cfg.score_stride), -np.inf)
    for t in range(T):
        nv = oracle.visible_count(int(x["positions"][t]), cfg.ratio)
        pos, elig = oracle.candidate_positions(g_cb[t], block, nv)
        o_by_pos[t, pos[elig]] = o_sc[t, elig]
    H.check_topk(g_idx, o_idx, o_by_pos, x["positions"], cfg.ratio, "reindex top-k")
    # attention on the reindex selection
    o = H.oracle_step(x, cfg, topk_override=g_idx)
    H.check_attn(H.bf16_to_f64(step.out), o["out"], step.lse.cpu().numpy().astype(np.float64),
                 o["lse"], "reindex attention")


def _oracle_attn_on(x, cfg, sel):
    T = cfg.T
    half = cfg.R // 2
    rc = np.zeros((T, half), np.float32)
    rs = np.zeros((T, half), np.float32)
    oracle.materialize_rope_rows(x["freqs_cos"], x["freqs_sin"], x["position_ids"], T, rc, rs)
    out, lse, _ = oracle.sparse_attn(x["q"], rc, rs, cfg.rope_offset, x["cmp_kv"],
                                     x["cmp_block_table"], sel, cfg.ratio, x["win_kv"],
                                     x["win_block_table"], cfg.W, x["attn_sink"],
                                     cfg.softmax_scale, x["query_start_loc"], x["positions"], T,
                                     k=cfg.k)
    return out, lse


def test_reindex_layer_step_parity():
    """C8, the reindex layer's whole step (RoPE rows, scores inside the
    supplied mask, top-512 there, attention) through CsaStep."""
    csa = _csa()
    cfg = synthetic.get("c8")
    x = synthetic.make_inputs(cfg, seed=0).t
    print("[hier] c8 step", flush=True)
    step = csa.step_for_config(cfg, x)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    T, kb, blk = cfg.T, cfg.cand_kb, cfg.cand_block
    cand = x["cand_blocks"]
    g_sc = step.scores.cpu().numpy().astype(np.float64)[:, :kb * blk]
    o_sc, oe = oracle.index_scores_in_candidates(x["q_idx"], x["q_scale"], x["head_w"],
                                                 x["idx_kv"], x["idx_scale"],
                                                 x["cmp_block_table"], x["query_start_loc"],
                                                 x["positions"], T, cfg.ratio, cand, blk)
    assert oe == 0
    H.check_scores(g_sc, o_sc, "c8 scores")
    g_idx = step.topk_idx.cpu().numpy()
    g_ref, _, _ = oracle.topk_in_candidates(g_sc, cand, blk, x["positions"], cfg.ratio, T, cfg.k)
    np.testing.assert_array_equal(g_idx, g_ref)
    o_idx, _, _ = oracle.topk_in_candidates(o_sc, cand, blk, x["positions"], cfg.ratio, T, cfg.k)
    o_by_pos = np.full((T, cfg.score_stride), -np.inf)
    for t in range(T):
        nv = oracle.visible_count(int(x["positions"][t]), cfg.ratio)
        pos, elig = oracle.candidate_positions(cand[t], blk, nv)
        o_by_pos[t, pos[elig]] = o_sc[t, elig]
    H.check_topk(g_idx, o_idx, o_by_pos, x["positions"], cfg.ratio, "c8 top-k")
    out, lse = _oracle_attn_on(x, cfg, g_idx)
    H.check_attn(H.bf16_to_f64(step.out), out, step.lse.cpu().numpy().astype(np.float64), lse,
                 "c8 attention")


def test_full_layer_publishes_mask():
    """C9: the full layer's step also writes the candidate mask; it is exactly
    the oracle's selection over the GPU's own scores."""
    csa = _csa()
    cfg = synthetic.get("c9")
    x = synthetic.make_inputs(cfg, seed=0, with_tables=True).t
    print("[hier] c9 step", flush=True)
    step = csa.step_for_config(cfg, x)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    g_full = step.scores.cpu().numpy().astype(np.float64)
    ref, _ = oracle.candidate_blocks(g_full, x["positions"], cfg.ratio, cfg.T, cfg.cand_block,
                                     cfg.cand_kb)
    np.testing.assert_array_equal(step.cand_blocks.cpu().numpy(), ref)


def test_full_layer_mask_against_oracle_scores():
    """C9's published mask against the oracle's mask over the oracle's own
    float64 scores: the same blocks, except where block scores tie within
    1e-5 of the kb-th best block score (the top-k rule of the task, applied
    to the block scores)."""
    csa = _csa()
    cfg = synthetic.get("c9")
    x = synthetic.make_inputs(cfg, seed=2, with_tables=True).t
    print("[hier] c9 mask vs oracle scores", flush=True)
    step = csa.step_for_config(cfg, x)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    T, blk, kb = cfg.T, cfg.cand_block, cfg.cand_kb
    o_sc, oe = oracle.index_scores(x["q_idx"], x["q_scale"], x["head_w"], x["idx_kv"],
                                   x["idx_scale"], x["cmp_block_table"], x["query_start_loc"],
                                   x["positions"], T, cfg.ratio, cfg.score_stride)
    assert oe == 0
    o_mask, _ = oracle.candidate_blocks(o_sc, x["positions"], cfg.ratio, T, blk, kb)
    g_mask = step.cand_blocks.cpu().numpy()
    differing = 0
    for t in range(T):
        nv = oracle.visible_count(int(x["positions"][t]), cfg.ratio)
        nb = -(-nv // blk)
        row = np.full(nb * blk, -np.inf)
        row[:nv] = o_sc[t, :nv]
        bs = row.reshape(nb, blk).max(axis=1)          # a block is as good as its best slot
        o, g = o_mask[t], g_mask[t]
        m = int((o >= 0).sum())
        assert np.all(g[m:] == -1), f"row {t}: tail not -1"
        gs = g[:m]
        assert np.all(np.diff(gs) > 0) and np.all((gs >= 0) & (gs < nb)), f"row {t}: invalid mask"
        if np.array_equal(g, o):
            continue
        differing += 1
        sk = np.min(bs[o[:m]])
        diff = np.setxor1d(gs, o[:m])
        assert np.all(np.abs(bs[diff] - sk) <= 1e-5 * abs(sk)), (
            f"row {t}: mask differs beyond ties ({len(diff)} blocks)")
    print(f"[hier] c9 mask rows differing only at ties: {differing}/{T}", flush=True)
