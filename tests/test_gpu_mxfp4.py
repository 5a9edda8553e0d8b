"""GPU parity of the MXFP4 index plane (csa_index_score_mxfp4) against the
oracle: edge cases on small paged pools, the whole C11 step (C2's shapes
with FP4 index keys), and the 1M-position C10 rows sampled."""
import numpy as np
import pytest

import oracle
import synthetic
from tests import harness as H
from tests.tiny import PAGE, paged_pool

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _csa():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


def _dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda()


def _gpu_scores(c, T, stride):
    csa = _csa()
    s = torch.full((T, stride), 777.0, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    csa.csa_index_score_mxfp4(_dev(c["q_fp4"]), _dev(c["q_sc"]), _dev(c["head_w"]),
                              _dev(c["idx_fp4"]), _dev(c["idx_sc"]), _dev(c["block_table"]),
                              _dev(c["query_start_loc"]), _dev(c["positions"]),
                              c["num_tokens"], c["ratio"], s, err=err)
    torch.cuda.synchronize()
    return s.cpu().numpy(), int(err.item())


@pytest.mark.parametrize("Hi", [64, 5])
def test_mxfp4_edges(Hi):
    rng = np.random.default_rng(Hi)
    Di, ratio, B = 128, 2, 2
    n = [700, 300]                       # compressed rows per request
    pages = [-(-x // PAGE) for x in n]
    maxp = max(pages)
    nblk = sum(pages) + 2
    perm = rng.permutation(nblk).astype(np.int32)
    bt = np.full((B, maxp), -1, np.int32)
    bt[0, :pages[0]] = perm[:pages[0]]
    bt[1, :pages[1]] = perm[pages[0]:pages[0] + pages[1]]
    kc = [rng.integers(0, 256, size=(x, Di // 2), dtype=np.uint8) for x in n]
    ks = [rng.integers(118, 131, size=(x, Di // 32)).astype(np.uint8) for x in n]
    idx_fp4 = paged_pool(kc, bt, nblk)
    idx_sc = paged_pool(ks, bt, nblk, fill=127)
    # request 0: rows 0-2, request 1: rows 3-5; row 6 is active but unowned
    pos = np.array([-1, 5, 1399, 2, 599, 4000, 10], np.int32)   # 4000: past request 1's table
    T = len(pos)
    qsl = np.array([0, 3, 6], np.int32)
    c = dict(q_fp4=rng.integers(0, 256, size=(T, Hi, Di // 2), dtype=np.uint8),
             q_sc=rng.integers(118, 131, size=(T, Hi, Di // 32)).astype(np.uint8),
             head_w=(rng.standard_normal((T, Hi)) / 2).astype(np.float32),
             idx_fp4=idx_fp4, idx_sc=idx_sc, block_table=bt, query_start_loc=qsl,
             positions=pos, num_tokens=T, ratio=ratio)
    stride = maxp * PAGE
    print(f"[mxfp4] edges Hi={Hi}", flush=True)
    g, ge = _gpu_scores(c, T, stride)
    o, oe = oracle.index_scores_mxfp4(score_stride=stride, **c)
    H.check_scores(g.astype(np.float64), o, f"mxfp4 edges Hi={Hi}")
    assert ge == oe
    # padding rows past num_tokens are never written
    c2 = dict(c, num_tokens=5)
    g2, _ = _gpu_scores(c2, T, stride)
    assert np.all(g2[5:] == 777.0)


def test_mxfp4_step_parity_c11():
    csa = _csa()
    cfg = synthetic.get("c11")
    x = synthetic.make_inputs(cfg, seed=0).t
    print("[mxfp4] c11 step", flush=True)
    step = csa.step_for_config(cfg, x)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    T = cfg.T
    g_s = step.scores.cpu().numpy().astype(np.float64)
    o_s, oe = oracle.index_scores_mxfp4(x["q_idx"], x["q_scale"], x["head_w"], x["idx_kv"],
                                        x["idx_scale"], x["cmp_block_table"],
                                        x["query_start_loc"], x["positions"], T, cfg.ratio,
                                        cfg.score_stride)
    assert oe == 0
    H.check_scores(g_s, o_s, "c11 scores")
    o_idx, _, _ = oracle.topk(o_s, x["positions"], cfg.ratio, T, cfg.k)
    g_idx = step.topk_idx.cpu().numpy()
    H.check_topk(g_idx, o_idx, o_s, x["positions"], cfg.ratio, "c11 top-k")
    # attention on the GPU's selection
    half = cfg.R // 2
    rc = np.zeros((T, half), np.float32)
    rs = np.zeros((T, half), np.float32)
    oracle.materialize_rope_rows(x["freqs_cos"], x["freqs_sin"], x["position_ids"], T, rc, rs)
    out, lse, _ = oracle.sparse_attn(x["q"], rc, rs, cfg.rope_offset, x["cmp_kv"],
                                     x["cmp_block_table"], g_idx, cfg.ratio, x["win_kv"],
                                     x["win_block_table"], cfg.W, x["attn_sink"],
                                     cfg.softmax_scale, x["query_start_loc"], x["positions"], T,
                                     k=cfg.k)
    H.check_attn(H.bf16_to_f64(step.out), out, step.lse.cpu().numpy().astype(np.float64), lse,
                 "c11 attention")


@pytest.mark.timeout(600)
def test_mxfp4_c10_sampled_rows():
    csa = _csa()
    cfg = synthetic.get("c10")
    x = synthetic.make_inputs(cfg, seed=0, with_tables=False).t
    print("[mxfp4] c10 scores", flush=True)
    c = dict(q_fp4=x["q_idx"], q_sc=x["q_scale"], head_w=x["head_w"], idx_fp4=x["idx_kv"],
             idx_sc=x["idx_scale"], block_table=x["cmp_block_table"],
             query_start_loc=x["query_start_loc"], positions=x["positions"], num_tokens=cfg.T,
             ratio=cfg.ratio)
    g, ge = _gpu_scores(c, cfg.T, cfg.score_stride)
    assert ge == 0
    rows = [0, cfg.T - 1]
    xs = H.sub_batch(x, rows)
    print("[mxfp4] c10 oracle on 2 rows", flush=True)
    o, oe = oracle.index_scores_mxfp4(xs["q_idx"], xs["q_scale"], xs["head_w"], xs["idx_kv"],
                                      xs["idx_scale"], xs["cmp_block_table"],
                                      xs["query_start_loc"], xs["positions"], len(rows),
                                      cfg.ratio, cfg.score_stride)
    H.check_scores(g[rows].astype(np.float64), o, "c10 sampled scores")
