"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Every workload config runs the whole step (RoPE rows, indexer scores, top-k,
sparse attention) on the GPU; the oracle runs on the same seeded inputs (all
rows, or a fixed sample of the 8,192-row prefill).  Attention is also checked
on the oracle's own selection, so a selection that differs only at ties never
hides an attention error.  The layers without an indexer (HCA: every visible
compressed row; SWA-only: the window) run their RoPE rows and attention.
"""
import numpy as np
import pytest

import oracle
import synthetic
from tests import harness as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _lib():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


_CACHE = {}


def _run_config(name):
    if name in _CACHE:
        return _CACHE[name]
    csa = _lib()
    cfg = synthetic.get(name)
    print(f"[parity] {cfg.name}: generating inputs", flush=True)
    x = synthetic.make_inputs(cfg, seed=0).t
    step = csa.step_for_config(cfg, x)
    print(f"[parity] {cfg.name}: GPU step", flush=True)
    step.run()
    torch.cuda.synchronize()
    g = dict(rope_cos=step.rope_cos.cpu().numpy(), rope_sin=step.rope_sin.cpu().numpy(),
             scores=step.scores.cpu().numpy().astype(np.float64),
             topk_idx=step.topk_idx.cpu().numpy(), out=H.bf16_to_f64(step.out),
             lse=step.lse.cpu().numpy().astype(np.float64), err=int(step.err.item()))
    if cfg.T > 256:
        rows = sorted(set([0, 1, 2, 3, 126, 127, 128, 129, 255, 256, 511, 512, 4095, 4096,
                           cfg.T - 2, cfg.T - 1] +
                          list(np.random.default_rng(1).choice(cfg.T, 48, replace=False))))
    else:
        rows = list(range(cfg.T))
    xs = H.sub_batch(x, rows) if len(rows) < cfg.T else x
    print(f"[parity] {cfg.name}: oracle on {len(rows)} rows", flush=True)
    o = H.oracle_step(xs, cfg)
    # attention of the GPU on the oracle's selection (input flows oracle -> GPU only)
    sel_full = step.topk_idx.clone()
    sel_full[torch.as_tensor(rows, device="cuda")] = torch.as_tensor(o["topk_idx"], device="cuda")
    step.attn(topk_idx=sel_full)
    torch.cuda.synchronize()
    g_attn_on_o = dict(out=H.bf16_to_f64(step.out)[rows], lse=step.lse.cpu().numpy()[rows])
    res = (cfg, x, step, g, o, rows, g_attn_on_o)
    _CACHE[name] = res
    return res


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_config_parity(name):
    cfg, x, step, g, o, rows, ga = _run_config(name)
    assert g["err"] == 0 and o["err"] == 0
    r = np.asarray(rows)
    # RoPE rows: bit-exact
    assert np.array_equal(g["rope_cos"][r].view(np.uint32), o["rope_cos"].view(np.uint32))
    assert np.array_equal(g["rope_sin"][r].view(np.uint32), o["rope_sin"].view(np.uint32))
    # scores
    H.check_scores(g["scores"][r], o["scores"], cfg.name)
    # top-k
    same = H.check_topk(g["topk_idx"][r], o["topk_idx"], o["scores"], o_positions(x, rows),
                        cfg.ratio, cfg.name)
    # attention on the oracle's selection: the task's elementwise bar, then
    # the pages' per-row RMS / peak budget
    H.check_attn(ga["out"], o["out"], ga["lse"], o["lse"], cfg.name + " attn")
    bud = H.check_budgets(ga["out"], o["out"], cfg.name + " attn budget")
    # end to end where the selections agree
    if same.any():
        H.check_attn(g["out"][r][same], o["out"][same], g["lse"][r][same], o["lse"][same],
                     cfg.name + " step")
        H.check_budgets(g["out"][r][same], o["out"][same], cfg.name + " step budget")
    print(f"[parity] {cfg.name}: rows with identical selection {same.sum()}/{len(rows)}; "
          f"worst budget use rms {bud['rms']:.3f}, peak {bud['peak']:.3f}", flush=True)


def o_positions(x, rows):
    return np.asarray(x["positions"])[np.asarray(rows)]


@pytest.mark.timeout(900)
def test_c5_max_context_parity():
    cfg, x, step, g, o, rows, ga = _run_config("c5")
    assert g["err"] == 0 and o["err"] == 0
    H.check_scores(g["scores"], o["scores"], cfg.name)
    same = H.check_topk(g["topk_idx"], o["topk_idx"], o["scores"], x["positions"], cfg.ratio,
                        cfg.name)
    H.check_attn(ga["out"], o["out"], ga["lse"], o["lse"], cfg.name + " attn")
    bud = H.check_budgets(ga["out"], o["out"], cfg.name + " attn budget")
    if same.any():
        H.check_attn(g["out"][same], o["out"][same], g["lse"][same], o["lse"][same],
                     cfg.name + " step")
        H.check_budgets(g["out"][same], o["out"][same], cfg.name + " step budget")
    print(f"[parity] {cfg.name}: worst budget use rms {bud['rms']:.3f}, "
          f"peak {bud['peak']:.3f}", flush=True)
    _CACHE.pop("c5", None)


def test_determinism_c2():
    csa = _lib()
    cfg = synthetic.get("c2")
    x = synthetic.make_inputs(cfg, seed=3).t
    step = csa.step_for_config(cfg, x)
    outs = []
    for _ in range(2):
        step.run()
        torch.cuda.synchronize()
        outs.append((step.scores.clone(), step.topk_idx.clone(), step.out.clone(),
                     step.lse.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("name", ["c6", "c7"])
def test_indexerless_layer_parity(name):
    """The layers without an indexer at their full sizes: HCA ratio-128 decode
    (every visible compressed row of a 1,048,576-token context plus the
    window, no selection array) and SWA-only decode (the window alone),
    against the oracle's deterministic selection."""
    csa = _lib()
    cfg = synthetic.get(name)
    print(f"[parity] {cfg.name}", flush=True)
    x = synthetic.make_inputs(cfg, seed=11).t
    step = csa.step_for_config(cfg, x)
    step.out.view(torch.int16).fill_(0x7FDE)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    half = cfg.R // 2
    rc = np.zeros((cfg.T, half), np.float32)
    rs = np.zeros_like(rc)
    oracle.materialize_rope_rows(x["freqs_cos"], x["freqs_sin"], x["position_ids"], cfg.T, rc, rs)
    assert np.array_equal(step.rope_cos.cpu().numpy().view(np.uint32), rc.view(np.uint32))
    sel = None if cfg.mode == "hca" else np.zeros((cfg.T, 0), np.int32)
    oo, ol, oe = oracle.sparse_attn(x["q"], rc, rs, cfg.rope_offset, x["cmp_kv"],
                                    x["cmp_block_table"], sel, cfg.ratio, x["win_kv"],
                                    x["win_block_table"], cfg.W, x["attn_sink"],
                                    cfg.softmax_scale, x["query_start_loc"], x["positions"],
                                    cfg.T, k=cfg.k)
    assert oe == 0
    H.check_attn(H.bf16_to_f64(step.out), oo, step.lse.cpu().numpy(), ol, cfg.name)


def test_hca_prefill_and_bound():
    """HCA through the prefill (ring) schedule, and a bound k below the
    visible count: the first k compressed rows and TOPK_RANGE, as the
    oracle."""
    from synthetic.configs import CsaConfig
    csa = _lib()
    cfg = CsaConfig(name="hca_small", description="HCA prefill rows and a short bound",
                    rows_per_request=(300, 2), positions=(tuple(range(4000, 4300)), (9000, 9001)),
                    H=16, D=128, R=32, Hi=4, Di=32, W=64, ratio=128, k=80, context=9100,
                    rope_capacity=16384, mode="hca")
    x = synthetic.make_inputs(cfg, seed=13).t
    for fn, k, expect in (("prefill", 80, 0), ("decode", 80, 0), ("decode", 40, oracle.EFLAG_TOPK_RANGE)):
        step = csa.CsaStep(x, ratio=cfg.ratio, k=k, window=cfg.W, rope_offset=cfg.rope_offset,
                           softmax_scale=cfg.softmax_scale, prefill=(fn == "prefill"), mode="hca")
        step.run()
        torch.cuda.synchronize()
        half = cfg.R // 2
        rc = np.zeros((cfg.T, half), np.float32)
        rs = np.zeros_like(rc)
        oracle.materialize_rope_rows(x["freqs_cos"], x["freqs_sin"], x["position_ids"], cfg.T,
                                     rc, rs)
        oo, ol, oe = oracle.sparse_attn(x["q"], rc, rs, cfg.rope_offset, x["cmp_kv"],
                                        x["cmp_block_table"], None, cfg.ratio, x["win_kv"],
                                        x["win_block_table"], cfg.W, x["attn_sink"],
                                        cfg.softmax_scale, x["query_start_loc"], x["positions"],
                                        cfg.T, k=k)
        assert oe == expect and int(step.err.item()) == expect, (fn, k)
        H.check_attn(H.bf16_to_f64(step.out), oo, step.lse.cpu().numpy(), ol, f"hca {fn} k{k}")


def test_hca_many_spans():
    """Two rows over a 5,000,000-token HCA context: 39,062 visible compressed
    rows plus the window per row, split into more spans than the 64 a merge
    wave holds one per lane."""
    from synthetic.configs import CsaConfig
    csa = _lib()
    ctx = 5_000_000
    cfg = CsaConfig(name="hca_many", description="HCA rows with more than 64 spans",
                    rows_per_request=(2,), positions=((ctx - 2, ctx - 1),), H=16, D=128, R=32,
                    Hi=4, Di=32, W=128, ratio=128, k=40000, context=ctx,
                    rope_neg_rows=(0, 1), rope_capacity=4096, mode="hca")   # identity rope rows
    x = synthetic.make_inputs(cfg, seed=17).t
    step = csa.step_for_config(cfg, x)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    half = cfg.R // 2
    rc = np.zeros((cfg.T, half), np.float32)
    rs = np.zeros_like(rc)
    oracle.materialize_rope_rows(x["freqs_cos"], x["freqs_sin"], x["position_ids"], cfg.T, rc, rs)
    oo, ol, oe = oracle.sparse_attn(x["q"], rc, rs, cfg.rope_offset, x["cmp_kv"],
                                    x["cmp_block_table"], None, cfg.ratio, x["win_kv"],
                                    x["win_block_table"], cfg.W, x["attn_sink"],
                                    cfg.softmax_scale, x["query_start_loc"], x["positions"],
                                    cfg.T, k=cfg.k)
    assert oe == 0
    H.check_attn(H.bf16_to_f64(step.out), oo, step.lse.cpu().numpy(), ol, cfg.name)
