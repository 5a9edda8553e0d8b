"""The bench's algorithmic-byte model (host logic, no GPU): the FP4 index
plane moves Di/2 + Di/32 bytes per key instead of Di + 4 and nothing else
changes; a reindex layer counts each key of its mask once per request; the
full layer that publishes a mask adds the block maxima and the mask."""
import dataclasses

import numpy as np

import bench
import oracle
import synthetic


def _sel(cfg, x):
    s, _ = oracle.index_scores(x["q_idx"], x["q_scale"], x["head_w"], x["idx_kv"], x["idx_scale"],
                               x["cmp_block_table"], x["query_start_loc"], x["positions"], cfg.T,
                               cfg.ratio, cfg.score_stride)
    idx, _, _ = oracle.topk(s, x["positions"], cfg.ratio, cfg.T, cfg.k)
    return idx


def test_fp4_plane_moves_fewer_index_bytes():
    c2, c11 = synthetic.get("c2"), synthetic.get("c11")
    x2 = synthetic.make_inputs(c2, seed=0, with_tables=False).t
    sel = np.tile(np.arange(c2.k, dtype=np.int32), (c2.T, 1))   # any valid selection
    a = bench.work_model(c2, x2, sel)
    b = bench.work_model(c11, x2, sel)      # same shapes; only the key format differs
    assert a["idx_keys"] == b["idx_keys"] > 0
    per_key = (c2.Di + 4) - (c11.Di // 2 + c11.Di // 32)
    assert per_key == 64
    q_side = c2.T * c2.Hi * per_key
    assert a["step_bytes"] - b["step_bytes"] == a["idx_keys"] * per_key + q_side
    assert a["stage_bytes"]["attn"] == b["stage_bytes"]["attn"]


def test_reindex_counts_mask_keys_once_per_request():
    cfg = dataclasses.replace(synthetic.get("c1"), name="c1_reindex_test", mode="reindex",
                              cand_kb=8, k=16)
    x = synthetic.make_inputs(cfg, seed=0).t
    cand = x["cand_blocks"]
    assert cand.shape == (cfg.T, 8)
    pos = x["positions"]
    qsl = x["query_start_loc"]
    keys = 0
    for b in range(len(qsl) - 1):
        u = set()
        for t in range(qsl[b], qsl[b + 1]):
            nv = oracle.visible_count(int(pos[t]), cfg.ratio)
            for c in cand[t]:
                if c >= 0:
                    u.update(p for p in range(int(c) * 8, int(c) * 8 + 8) if p < nv)
        keys += len(u)
    sel = np.full((cfg.T, cfg.k), -1, np.int32)
    wm = bench.work_model(cfg, x, sel)
    assert wm["idx_keys"] == keys
    assert wm["stage_bytes"]["index"] >= keys * (cfg.Di + 4)


def test_full_layer_with_mask_adds_the_mask_stage():
    base = synthetic.get("c1")
    cfg = dataclasses.replace(base, name="c1_hier_test", mode="hier_full", cand_kb=8)
    x = synthetic.make_inputs(base, seed=0, with_tables=False).t
    sel = _sel(base, x)
    a = bench.work_model(base, x, sel)
    b = bench.work_model(cfg, x, sel)
    assert "cand" in b["stage_bytes"] and "cand" not in a["stage_bytes"]
    assert b["step_bytes"] - a["step_bytes"] == 4 * base.T * 8
