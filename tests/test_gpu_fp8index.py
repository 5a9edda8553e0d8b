"""GPU parity of the FP8 index plane (csa_index_score_fp8) against the oracle.

* Edge cases on small paged pools (unowned rows, nothing visible, a span past
  the table, padding rows), every head count and several head widths, with
  every non-NaN E4M3 code.
* Integer-valued codes give the INT8 scorer's bits: both kernels form the same
  FP32 products (w * qs) * relu(dot) of exact dots and sum them in the same
  order.
* The whole C15 step (C2's shapes with the FP8 plane) and sampled rows of the
  1M-position C14.
"""
import numpy as np
import pytest

import oracle
import synthetic
from tests import harness as H
from tests.tiny import PAGE, paged_pool

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NON_NAN = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def _csa():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


def _dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda()


def _gpu_scores(c, T, stride, fn="csa_index_score_fp8"):
    csa = _csa()
    s = torch.full((T, stride), 777.0, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    getattr(csa, fn)(_dev(c["q"]), _dev(c["q_scale"]), _dev(c["head_w"]), _dev(c["keys"]),
                     _dev(c["idx_scale"]), _dev(c["block_table"]), _dev(c["query_start_loc"]),
                     _dev(c["positions"]), c["num_tokens"], c["ratio"], s, err=err)
    torch.cuda.synchronize()
    return s.cpu().numpy(), int(err.item())


def _pools(rng, n, Di, keys_of):
    B = len(n)
    pages = [-(-x // PAGE) for x in n]
    maxp = max(pages)
    nblk = sum(pages) + 2
    perm = rng.permutation(nblk).astype(np.int32)
    bt = np.full((B, maxp), -1, np.int32)
    o = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[o:o + pages[b]]
        o += pages[b]
    keys = paged_pool([keys_of(x) for x in n], bt, nblk)
    ks = paged_pool([rng.uniform(0.005, 0.02, size=x).astype(np.float32) for x in n], bt, nblk)
    return bt, keys, ks, maxp * PAGE


@pytest.mark.parametrize("Hi,Di", [(64, 128), (5, 128), (37, 64), (1, 32)])
def test_fp8_edges(Hi, Di):
    rng = np.random.default_rng(Hi * 131 + Di)
    bt, keys, ks, stride = _pools(rng, [700, 300], Di,
                                  lambda x: rng.choice(NON_NAN, size=(x, Di)).astype(np.uint8))
    # request 0: rows 0-2, request 1: rows 3-5; row 6 is active but unowned
    pos = np.array([-1, 5, 1399, 2, 599, 4000, 10], np.int32)   # 4000: past request 1's table
    T = len(pos)
    c = dict(q=rng.choice(NON_NAN, size=(T, Hi, Di)).astype(np.uint8),
             q_scale=rng.uniform(0.001, 0.01, size=(T, Hi)).astype(np.float32),
             head_w=(rng.standard_normal((T, Hi)) / 2).astype(np.float32),
             keys=keys, idx_scale=ks, block_table=bt, query_start_loc=np.array([0, 3, 6], np.int32),
             positions=pos, num_tokens=T, ratio=2)
    print(f"[fp8idx] edges Hi={Hi} Di={Di}", flush=True)
    g, ge = _gpu_scores(c, T, stride)
    args = (c["q"], c["q_scale"], c["head_w"], keys, ks, bt, c["query_start_loc"], pos, T, 2,
            stride)
    o, oe = oracle.index_scores_fp8(*args)
    H.check_scores(g.astype(np.float64), o, f"fp8 edges Hi={Hi} Di={Di}",
                   extra_tol=H.fp8_dot_tolerance(*args))
    assert ge == oe and oe & oracle.EFLAG_META and oe & oracle.EFLAG_POS_RANGE
    # padding rows past num_tokens are never written
    g2, _ = _gpu_scores(dict(c, num_tokens=5), T, stride)
    assert np.all(g2[5:] == 777.0)


def _e4m3_of_int(v):
    v = int(v)
    if v == 0:
        return 0
    a = abs(v)
    e = a.bit_length() - 1
    return (0x80 if v < 0 else 0) | ((e + 7) << 3) | ((a - (1 << e)) * 8 // (1 << e))


@pytest.mark.parametrize("Hi,Di", [(64, 128), (17, 64)])
def test_fp8_integer_codes_give_the_int8_bits(Hi, Di):
    rng = np.random.default_rng(7 + Di)
    ints = {}
    bt, k8, ks, stride = _pools(rng, [1000, 260], Di,
                                lambda x: ints.setdefault(x, rng.integers(-16, 17, size=(x, Di))
                                                          ).astype(np.int8))
    enc = np.vectorize(_e4m3_of_int)
    kf = paged_pool([enc(ints[x]).astype(np.uint8) for x in (1000, 260)], bt, k8.shape[0])
    pos = np.array([999, 998, 259, 100], np.int32)
    T = len(pos)
    q = rng.integers(-16, 17, size=(T, Hi, Di))
    common = dict(q_scale=rng.uniform(0.001, 0.01, size=(T, Hi)).astype(np.float32),
                  head_w=(rng.standard_normal((T, Hi)) / 2).astype(np.float32), idx_scale=ks,
                  block_table=bt, query_start_loc=np.array([0, 2, 4], np.int32), positions=pos,
                  num_tokens=T, ratio=1)
    print(f"[fp8idx] integer codes Hi={Hi} Di={Di}", flush=True)
    g8, e8 = _gpu_scores(dict(common, q=enc(q).astype(np.uint8), keys=kf), T, stride)
    gi, ei = _gpu_scores(dict(common, q=q.astype(np.int8), keys=k8), T, stride,
                         fn="csa_index_score")
    assert e8 == ei == 0
    assert np.array_equal(g8.view(np.uint32), gi.view(np.uint32))


def test_fp8_step_parity_c15():
    csa = _csa()
    cfg = synthetic.get("c15")
    x = synthetic.make_inputs(cfg, seed=0).t
    print("[fp8idx] c15 step", flush=True)
    step = csa.step_for_config(cfg, x)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    o = H.oracle_step(x, cfg)
    assert o["err"] == 0
    tol = H.fp8_dot_tolerance(x["q_idx"], x["q_scale"], x["head_w"], x["idx_kv"],
                              x["idx_scale"], x["cmp_block_table"], x["query_start_loc"],
                              x["positions"], cfg.T, cfg.ratio, cfg.score_stride)
    H.check_scores(step.scores.cpu().numpy().astype(np.float64), o["scores"], "c15 scores",
                   extra_tol=tol)
    same = H.check_topk(step.topk_idx.cpu().numpy(), o["topk_idx"], o["scores"], x["positions"],
                        cfg.ratio, "c15 top-k", extra_tol=tol)
    assert same.sum() >= cfg.T // 2
    H.check_attn(H.bf16_to_f64(step.out)[same], o["out"][same],
                 step.lse.cpu().numpy()[same], o["lse"][same], "c15 attention")


@pytest.mark.timeout(600)
def test_fp8_c14_sampled_rows():
    csa = _csa()
    cfg = synthetic.get("c14")
    x = synthetic.make_inputs(cfg, seed=0, with_tables=False).t
    print("[fp8idx] c14 scores", flush=True)
    c = dict(q=x["q_idx"], q_scale=x["q_scale"], head_w=x["head_w"], keys=x["idx_kv"],
             idx_scale=x["idx_scale"], block_table=x["cmp_block_table"],
             query_start_loc=x["query_start_loc"], positions=x["positions"], num_tokens=cfg.T,
             ratio=cfg.ratio)
    g, ge = _gpu_scores(c, cfg.T, cfg.score_stride)
    assert ge == 0
    rows = [0, cfg.T - 1]
    xs = H.sub_batch(x, rows)
    print("[fp8idx] c14 oracle on 2 rows", flush=True)
    args = (xs["q_idx"], xs["q_scale"], xs["head_w"], xs["idx_kv"], xs["idx_scale"],
            xs["cmp_block_table"], xs["query_start_loc"], xs["positions"], len(rows), cfg.ratio,
            cfg.score_stride)
    o, oe = oracle.index_scores_fp8(*args)
    assert oe == 0
    H.check_scores(g[rows].astype(np.float64), o, "c14 sampled scores",
                   extra_tol=H.fp8_dot_tolerance(*args))
