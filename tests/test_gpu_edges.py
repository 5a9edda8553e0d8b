"""Edge cases of the HIP path against the oracle, through the C ABI: crafted
top-k rows on both selection paths (ties, NaN, signed zeros, -inf, spans
shorter than k, the candidate-overflow fallback, workspace reuse), a ragged
batch with an empty request and padding rows, num_tokens = 0, device error
flags, and other head counts / widths."""
import numpy as np
import pytest

import oracle
import synthetic
from synthetic.configs import CsaConfig
from tests import harness as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENT_I = 0x7EEEEEEE


def _csa():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


def _topk_gpu(scores: np.ndarray, positions, ratio, k, num_tokens=None, ws=None):
    csa = _csa()
    T, stride = scores.shape
    nt = T if num_tokens is None else num_tokens
    s = torch.as_tensor(scores.astype(np.float32), device="cuda")
    p = torch.as_tensor(np.asarray(positions, np.int32), device="cuda")
    idx = torch.full((T, k), SENT_I, dtype=torch.int32, device="cuda")
    val = torch.full((T, k), 7.0, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wsb = csa.csa_topk_workspace_bytes(T, stride, k)
    if ws is None and wsb:
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    csa.csa_topk(s, p, ratio, nt, k, idx, val, workspace=ws, err=err)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy(), int(err.item()), ws


def _compare_topk(scores, positions, ratio, k, what):
    gi, gv, gerr, _ = _topk_gpu(scores, positions, ratio, k)
    oi, ov, oerr = oracle.topk(scores.astype(np.float32).astype(np.float64), positions, ratio,
                               scores.shape[0], k)
    assert gerr == oerr, what
    assert np.array_equal(gi, oi), f"{what}: indices differ"
    assert np.array_equal(gv.astype(np.float64), ov.astype(np.float32).astype(np.float64),
                          equal_nan=True), f"{what}: values differ"


@pytest.mark.parametrize("stride,k", [(256, 1), (256, 32), (16384, 512), (16384, 4096),
                                      (32768, 2048), (65536, 2048), (1 << 20, 2048),
                                      (1 << 20, 4096), (40960, 7)])
def test_topk_random_rows(stride, k):
    print(f"[edges] topk random stride={stride} k={k}", flush=True)
    rng = np.random.default_rng(stride + k)
    T = 6
    sc = rng.standard_normal((T, stride)).astype(np.float32) * 50
    pos = np.array([stride - 1, stride // 2, 5, k - 2, -1, 32767 if stride > 32768 else 3])
    _compare_topk(sc, pos, 1, k, f"stride {stride} k {k}")


@pytest.mark.parametrize("stride", [4096, 65536])
def test_topk_ties_nan_zero_inf(stride):
    print(f"[edges] topk ties stride={stride}", flush=True)
    rng = np.random.default_rng(7)
    T = 5
    sc = rng.integers(-3, 4, (T, stride)).astype(np.float32)  # few distinct values
    sc[1] = 0.0
    sc[1, ::3] = -0.0                                           # signed zeros tie
    sc[2, ::5] = np.nan
    sc[2, 1::5] = -np.inf
    sc[3] = 1.0                                                 # all equal (overflow path)
    sc[4, : stride // 2] = np.nan
    pos = np.full(T, stride - 1)
    _compare_topk(sc, pos, 1, 512, f"ties stride {stride}")


def test_topk_long_rows_with_ties():
    """1M-position rows of few distinct values, signed zeros, infinities and
    NaN: the sampled threshold's small-rank path sees thousands of keys at its
    bound and hands over to the selection core; exact as the oracle."""
    print("[edges] topk long rows with ties", flush=True)
    rng = np.random.default_rng(77)
    T, stride, k = 5, 1 << 20, 2048
    sc = rng.integers(-3, 4, (T, stride)).astype(np.float32)
    sc[1] = 2.0                                    # every key equal
    sc[1, ::7] = -0.0
    sc[2, ::97] = np.inf                           # more +inf keys than k
    sc[2, 1::13] = np.nan
    sc[3] = rng.standard_normal(stride).astype(np.float32)
    sc[3, ::3] = np.nan                            # a third NaN
    sc[4] = np.where(rng.random(stride) < 0.003, 5.0, sc[4])   # a tied top band near k
    pos = np.full(T, stride - 1)
    _compare_topk(sc, pos, 1, k, "long rows with ties")


@pytest.mark.parametrize("case", ["ascending", "clustered", "outliers", "few_groups"])
def test_topk_long_row_group_bound(case):
    """Long rows take a threshold from the maxima of 32-score groups: rows
    whose best keys pack into few groups (ascending, clustered), heavy-tailed
    rows, and a row with more keys to choose than groups, exactly as the
    oracle."""
    print(f"[edges] topk long row {case}", flush=True)
    rng = np.random.default_rng(31)
    T, stride, k = 4, 1 << 18, 2048
    sc = rng.standard_normal((T, stride)).astype(np.float32)
    pos = np.full(T, stride - 1)
    if case == "ascending":
        sc[0] = np.arange(stride, dtype=np.float32)
        sc[1] = np.sort(sc[1])
    elif case == "clustered":
        sc[:, 1000:1000 + 3 * k] += 6.0        # the best keys in one run of groups
        sc[2, ::64] += 9.0                      # one high key in every other group
    elif case == "outliers":
        out = rng.random((T, stride)) < 0.05
        sc[out] *= 4.0
    else:
        pos[:] = [40000, 50000, 65535, 32768]   # fewer groups than k at 40000 and 50000
    _compare_topk(sc, pos, 1, k, f"long row {case}")


def test_topk_workspace_needs_no_clearing():
    """The long-row workspace carries no state between calls: garbage in it
    (here 0xff bytes, then the leftovers of a previous call) changes nothing."""
    rng = np.random.default_rng(9)
    stride, k = 1 << 17, 2048
    a = rng.standard_normal((4, stride)).astype(np.float32)
    pos = np.full(4, stride - 1)
    wsb = _csa().csa_topk_workspace_bytes(4, stride, k)
    ws = torch.full((wsb,), 255, dtype=torch.uint8, device="cuda")
    gi, _, _, ws = _topk_gpu(a, pos, 1, k, ws=ws)
    oi, _, _ = oracle.topk(a.astype(np.float64), pos, 1, 4, k)
    assert np.array_equal(gi, oi)
    b = rng.standard_normal((4, stride)).astype(np.float32)
    gi2, _, _, ws = _topk_gpu(b, pos, 1, k, num_tokens=2, ws=ws)
    oi2, _, _ = oracle.topk(b[:2].astype(np.float64), pos[:2], 1, 2, k)
    assert np.array_equal(gi2[:2], oi2)
    assert np.all(gi2[2:] == SENT_I), "padding rows written"


def _ragged_cfg():
    return CsaConfig(
        name="ragged", description="ragged decode/prefill mix with an empty request",
        rows_per_request=(3, 0, 1, 4, 2),
        positions=((300, 301, 302), (), (0,), (5, 127, 128, 511), (254, 255)),
        rope_neg_rows=(1,), H=8, D=64, R=16, Hi=4, Di=32, W=16, ratio=2, k=32, context=512,
        rope_capacity=1024)


def _fill_sentinels(step):
    for t in (step.rope_cos, step.rope_sin, step.scores, step.topk_val, step.lse):
        t.view(torch.int32).fill_(0x7FC0DEAD)
    step.topk_idx.fill_(SENT_I)
    step.out.view(torch.int16).fill_(0x7FDE)


def test_ragged_batch_with_padding_rows():
    csa = _csa()
    cfg = _ragged_cfg()
    x = synthetic.make_inputs(cfg, seed=5).t
    nt = cfg.T - 1  # last row is storage padding
    step = csa.CsaStep(x, ratio=cfg.ratio, k=cfg.k, window=cfg.W, rope_offset=cfg.rope_offset,
                       softmax_scale=cfg.softmax_scale, num_tokens=nt)
    _fill_sentinels(step)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    rows = list(range(nt))
    xs = H.sub_batch(x, rows)
    o = H.oracle_step(xs, cfg)
    assert np.array_equal(step.rope_cos.cpu().numpy()[:nt].view(np.uint32),
                          o["rope_cos"].view(np.uint32))
    H.check_scores(step.scores.cpu().numpy()[:nt].astype(np.float64), o["scores"], "ragged")
    gi = step.topk_idx.cpu().numpy()[:nt]
    same = H.check_topk(gi, o["topk_idx"], o["scores"], xs["positions"], cfg.ratio, "ragged")
    assert same.all()
    H.check_attn(H.bf16_to_f64(step.out)[:nt], o["out"], step.lse.cpu().numpy()[:nt],
                 o["lse"], "ragged")
    # the padding row is untouched everywhere
    assert np.all(step.rope_cos.cpu().numpy()[nt:].view(np.uint32) == 0x7FC0DEAD)
    assert np.all(step.scores.cpu().numpy()[nt:].view(np.uint32) == 0x7FC0DEAD)
    assert np.all(step.topk_idx.cpu().numpy()[nt:] == SENT_I)
    assert np.all(step.out.view(torch.int16).cpu().numpy()[nt:] == 0x7FDE)
    assert np.all(step.lse.cpu().numpy()[nt:].view(np.uint32) == 0x7FC0DEAD)


def test_zero_tokens_writes_nothing():
    csa = _csa()
    cfg = synthetic.get("c1")
    x = synthetic.make_inputs(cfg, seed=1).t
    step = csa.step_for_config(cfg, x, num_tokens=0)
    _fill_sentinels(step)
    step.run()
    torch.cuda.synchronize()
    assert np.all(step.scores.cpu().numpy().view(np.uint32) == 0x7FC0DEAD)
    assert np.all(step.topk_idx.cpu().numpy() == SENT_I)
    assert np.all(step.out.view(torch.int16).cpu().numpy() == 0x7FDE)


@pytest.mark.parametrize("fuse_rope", [True, False])
def test_device_error_flags_match_oracle(fuse_rope):
    csa = _csa()
    cfg = _ragged_cfg()
    x = dict(synthetic.make_inputs(cfg, seed=6).t)
    x["cmp_block_table"] = x["cmp_block_table"].copy()
    x["cmp_block_table"][0, 1] = 10_000          # visible page of request 0 -> invalid block
    x["position_ids"] = x["position_ids"].copy()
    x["position_ids"][2] = cfg.rope_capacity + 3  # past the RoPE table
    step = csa.step_for_config(cfg, x, fuse_rope=fuse_rope)
    assert step.fuse_rope == fuse_rope
    _fill_sentinels(step)
    step.run()
    torch.cuda.synchronize()
    o = H.oracle_step(x, cfg)
    assert int(step.err.item()) == o["err"] == (oracle.EFLAG_BLOCK_RANGE | oracle.EFLAG_POS_RANGE)
    H.check_scores(step.scores.cpu().numpy().astype(np.float64), o["scores"], "flags")
    # row 2's rope row stayed untouched
    assert np.all(step.rope_cos.cpu().numpy()[2].view(np.uint32) == 0x7FC0DEAD)
    # attention given an invisible selected index and a row no request owns
    sel = torch.as_tensor(o["topk_idx"], device="cuda").clone()
    sel[0, 0] = oracle.visible_count(int(x["positions"][0]), cfg.ratio)
    qsl_bad = x["query_start_loc"].copy()
    qsl_bad[-1] -= 1                              # the last row loses its request
    step.t["query_start_loc"].copy_(torch.as_tensor(qsl_bad))
    step.err.zero_()
    # RoPE rows of the oracle: row 2 is untouched there too; use identity for it
    # (the fused call gathers the rows again, flags row 2 again and rotates it
    # by the identity)
    rc = torch.as_tensor(np.nan_to_num(o["rope_cos"], nan=1.0), device="cuda")
    rs = torch.as_tensor(np.nan_to_num(o["rope_sin"], nan=0.0), device="cuda")
    step.rope_cos.copy_(rc)
    step.rope_sin.copy_(rs)
    step.attn(topk_idx=sel)
    torch.cuda.synchronize()
    oo, ol, oe = oracle.sparse_attn(x["q"], rc.cpu().numpy(), rs.cpu().numpy(), cfg.rope_offset,
                                    x["cmp_kv"], x["cmp_block_table"], sel.cpu().numpy(),
                                    cfg.ratio, x["win_kv"], x["win_block_table"], cfg.W,
                                    x["attn_sink"], cfg.softmax_scale, qsl_bad, x["positions"],
                                    cfg.T)
    assert int(step.err.item()) == oe | (oracle.EFLAG_POS_RANGE if fuse_rope else 0)
    assert oe & oracle.EFLAG_TOPK_RANGE and oe & oracle.EFLAG_META
    H.check_attn(H.bf16_to_f64(step.out), oo, step.lse.cpu().numpy(), ol, "flags attn")


@pytest.mark.parametrize("H_,D,R,off", [(1, 64, 16, 48), (16, 128, 64, 0), (33, 256, 64, 192),
                                        (64, 512, 0, 512), (64, 512, 64, 448)])
def test_attention_shapes(H_, D, R, off):
    print(f"[edges] attention H={H_} D={D} R={R} off={off}", flush=True)
    csa = _csa()
    cfg = CsaConfig(name="shape", description="attention shape sweep",
                    rows_per_request=(3, 2), positions=((1000, 1001, 1002), (130, 131)),
                    H=H_, D=D, R=max(R, 2), Hi=8, Di=64, W=128, ratio=1, k=300, context=1100,
                    rope_capacity=2048)
    x = synthetic.make_inputs(cfg, seed=11).t
    rng = np.random.default_rng(3)
    sel = np.full((cfg.T, cfg.k), -1, np.int32)
    for t, p in enumerate(cfg.flat_positions):
        nv = p + 1
        m = min(cfg.k - 7, nv)
        sel[t, :m] = np.sort(rng.choice(nv, m, replace=False))
    half = R // 2
    ang = rng.uniform(-3, 3, (cfg.T, half))
    rc = np.cos(ang).astype(np.float32)
    rs = np.sin(ang).astype(np.float32)
    dev = lambda a: torch.as_tensor(a, device="cuda")
    q = torch.from_numpy(x["q"].view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty((cfg.T, H_, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((cfg.T, H_), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for fn in ("decode", "prefill"):
        ws_n = csa.csa_sparse_attn_workspace_bytes(cfg.T, H_, D, cfg.k, cfg.W)
        ws = torch.zeros(max(ws_n, 1), dtype=torch.uint8, device="cuda")
        getattr(csa, "csa_sparse_attn_" + fn)(
            q, dev(rc), dev(rs), off, torch.from_numpy(x["cmp_kv"].view(np.int16)).cuda(),
            dev(x["cmp_block_table"]), dev(sel), cfg.ratio,
            torch.from_numpy(x["win_kv"].view(np.int16)).cuda(), dev(x["win_block_table"]),
            cfg.W, dev(x["attn_sink"]), cfg.softmax_scale, dev(x["query_start_loc"]),
            dev(x["positions"]), cfg.T, out, lse=lse, workspace=ws, err=err)
        torch.cuda.synchronize()
        oo, ol, oe = oracle.sparse_attn(x["q"], rc, rs, off, x["cmp_kv"], x["cmp_block_table"],
                                        sel, cfg.ratio, x["win_kv"], x["win_block_table"], cfg.W,
                                        x["attn_sink"], cfg.softmax_scale, x["query_start_loc"],
                                        x["positions"], cfg.T)
        assert int(err.item()) == oe == 0
        H.check_attn(H.bf16_to_f64(out), oo, lse.cpu().numpy(), ol, f"{fn} H{H_} D{D}")
        if ws_n:
            # the same workspace, dirty from the first call, serves a second
            first = out.clone()
            getattr(csa, "csa_sparse_attn_" + fn)(
                q, dev(rc), dev(rs), off, torch.from_numpy(x["cmp_kv"].view(np.int16)).cuda(),
                dev(x["cmp_block_table"]), dev(sel), cfg.ratio,
                torch.from_numpy(x["win_kv"].view(np.int16)).cuda(), dev(x["win_block_table"]),
                cfg.W, dev(x["attn_sink"]), cfg.softmax_scale, dev(x["query_start_loc"]),
                dev(x["positions"]), cfg.T, out, lse=lse, workspace=ws, err=err)
            torch.cuda.synchronize()
            assert torch.equal(first, out), "second call on the same workspace differs"


@pytest.mark.parametrize("Hi,Di", [(1, 16), (5, 48), (37, 80), (64, 96), (17, 112), (64, 128)])
def test_index_shapes(Hi, Di):
    """Indexer widths that leave partial 32-channel MFMA steps and partial
    32-head tiles, against the oracle's scores."""
    print(f"[edges] index Hi={Hi} Di={Di}", flush=True)
    cfg = CsaConfig(name="ishape", description="indexer shape sweep",
                    rows_per_request=(3, 2), positions=((1000, 1001, 1002), (300, 301)),
                    H=8, D=64, R=16, Hi=Hi, Di=Di, W=16, ratio=1, k=64, context=1100,
                    rope_capacity=2048)
    x = synthetic.make_inputs(cfg, seed=5).t
    csa = _csa()
    step = csa.step_for_config(cfg, x)
    step.index()
    torch.cuda.synchronize()
    o, oe = oracle.index_scores(x["q_idx"], x["q_scale"], x["head_w"], x["idx_kv"], x["idx_scale"],
                                x["cmp_block_table"], x["query_start_loc"], x["positions"],
                                cfg.T, cfg.ratio, step.score_stride)
    assert int(step.err.item()) == oe == 0
    H.check_scores(step.scores.cpu().numpy().astype(np.float64), o, f"index Hi{Hi} Di{Di}")


@pytest.mark.parametrize("rows", [(6, 6), (1, 1, 1, 1), (3, 1), (2, 2, 2), (5,), (4, 0, 4)])
def test_index_group_layouts(rows):
    """Row groups of the indexer: requests of equal length (whose groups the
    kernel derives without scanning query_start_loc, including requests of
    more than four rows), and divisible or empty-request batches where that
    guess is wrong and the scan decides."""
    print(f"[edges] index rows={rows}", flush=True)
    positions = tuple(tuple(300 + 97 * b + 5 * i for i in range(n)) for b, n in enumerate(rows))
    cfg = CsaConfig(name="igroups", description="indexer row-group layouts",
                    rows_per_request=rows, positions=positions, H=8, D=64, R=16, Hi=8, Di=64,
                    W=16, ratio=1, k=64, context=1100, rope_capacity=2048)
    x = synthetic.make_inputs(cfg, seed=9).t
    csa = _csa()
    step = csa.step_for_config(cfg, x)
    step.index()
    torch.cuda.synchronize()
    o, oe = oracle.index_scores(x["q_idx"], x["q_scale"], x["head_w"], x["idx_kv"], x["idx_scale"],
                                x["cmp_block_table"], x["query_start_loc"], x["positions"],
                                cfg.T, cfg.ratio, step.score_stride)
    assert int(step.err.item()) == oe == 0
    H.check_scores(step.scores.cpu().numpy().astype(np.float64), o, f"index rows {rows}")
