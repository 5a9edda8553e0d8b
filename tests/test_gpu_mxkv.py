"""GPU parity of the low-bit KV decode (csa_sparse_attn_decode_mx) against the
oracle, through the C ABI.

The planes are those of pypto-lib "DeepSeek V4.1 Flash", the paragraph on the
production cache ABI: window rows MXFP8 E4M3 with E8M0 group-of-32 scales,
compressed rows packed MXFP4 E2M1 with E4M3 group-of-16 scales, dequantised on
read.  The oracle reads the same codes through its plane row sources.

* every head width (D = 64 .. 512; below 512 one load instruction carries
  several rows, mixing window and compressed rows) on a supplied selection;
* the dequantised planes through the BF16 decode entry point give the same
  bits (the same kernel once the tile is in LDS);
* extreme scale bytes and every non-NaN code, and NaN codes, which propagate;
* the whole step at C3's shapes (c12) and at max context with every cache
  low-bit (c13: MXFP4 index plane too), against the oracle.
"""
import numpy as np
import pytest

import oracle
import synthetic
from synthetic.configs import CsaConfig
from tests import harness as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _csa():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _selection(cfg, seed, short=7):
    rng = np.random.default_rng(seed)
    sel = np.full((cfg.T, cfg.k), -1, np.int32)
    for t, p in enumerate(cfg.flat_positions):
        nv = oracle.visible_count(p, cfg.ratio)
        m = min(cfg.k - short, nv)
        sel[t, :m] = np.sort(rng.choice(nv, m, replace=False))
    return sel


def _run_mx(csa, cfg, x, sel, rc, rs, off=None):
    T, H_, D = cfg.T, cfg.H, cfg.D
    out = torch.empty((T, H_, D), dtype=torch.bfloat16, device="cuda")
    out.view(torch.int16).fill_(0x7FDE)
    lse = torch.empty((T, H_), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wsn = csa.csa_sparse_attn_mx_workspace_bytes(T, H_, D, cfg.k, cfg.W)
    ws = torch.empty(max(wsn, 1), dtype=torch.uint8, device="cuda") if wsn else None
    csa.csa_sparse_attn_decode_mx(
        _dev(x["q"]), _dev(rc), _dev(rs), cfg.rope_offset if off is None else off,
        _dev(x["cmp_fp4"]), _dev(x["cmp_scale"]), _dev(x["cmp_block_table"]), _dev(sel),
        cfg.ratio, _dev(x["win_fp8"]), _dev(x["win_scale"]), _dev(x["win_block_table"]), cfg.W,
        _dev(x["attn_sink"]), cfg.softmax_scale, _dev(x["query_start_loc"]),
        _dev(x["positions"]), T, out, lse=lse, workspace=ws, err=err)
    torch.cuda.synchronize()
    return out, lse, int(err.item())


def _oracle_attn(cfg, x, sel, rc, rs, off=None):
    cmp_src, win_src = H.kv_sources(x, cfg)
    return oracle.sparse_attn(x["q"], rc, rs, cfg.rope_offset if off is None else off, cmp_src,
                              x["cmp_block_table"], sel, cfg.ratio, win_src,
                              x["win_block_table"], cfg.W, x["attn_sink"], cfg.softmax_scale,
                              x["query_start_loc"], x["positions"], cfg.T)


def _rope(cfg, seed):
    rng = np.random.default_rng(seed)
    ang = rng.uniform(-3, 3, (cfg.T, cfg.R // 2))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _shape_cfg(H_, D, R, k=300, ratio=1):
    return CsaConfig(name="mx_shape", description="low-bit KV attention shape sweep",
                     rows_per_request=(3, 2), positions=((1000, 1001, 1002), (130, 131)),
                     H=H_, D=D, R=R, Hi=8, Di=64, W=128, ratio=ratio, k=k, context=1100,
                     rope_capacity=2048, kv_format="mx")


@pytest.mark.parametrize("H_,D,R", [(8, 64, 16), (16, 128, 64), (33, 256, 64), (64, 512, 64)])
def test_mx_attention_shapes(H_, D, R):
    print(f"[mxkv] shapes H={H_} D={D} R={R}", flush=True)
    csa = _csa()
    cfg = _shape_cfg(H_, D, R)
    x = synthetic.make_inputs(cfg, seed=5).t
    sel = _selection(cfg, 2)
    rc, rs = _rope(cfg, 3)
    out, lse, err = _run_mx(csa, cfg, x, sel, rc, rs)
    oo, ol, oe = _oracle_attn(cfg, x, sel, rc, rs)
    assert err == oe == 0
    H.check_attn(H.bf16_to_f64(out), oo, lse.cpu().numpy(), ol, f"mx H{H_} D{D}")
    H.check_budgets(H.bf16_to_f64(out), oo, f"mx H{H_} D{D} budget")


def _bf16_bits(values):
    """float64 values that are BF16 numbers -> their uint16 bit patterns."""
    f = np.asarray(values, dtype=np.float32)
    assert np.array_equal(f.astype(np.float64), values)
    b = f.view(np.uint32)
    assert not np.any(b & 0xFFFF)
    return (b >> 16).astype(np.uint16)


def _same_as_bf16_decode(csa, cfg, x, sel, rc, rs, what):
    """The low-bit call against the BF16 decode entry point on the pools the
    oracle's planes dequantise: both entry points run the same schedule and
    kernels once a tile is in LDS, so the bits must agree."""
    out, lse, err = _run_mx(csa, cfg, x, sel, rc, rs)
    assert err == 0
    cmp_src, win_src = H.kv_sources(x, cfg)
    ncb, nwb, D = x["cmp_fp4"].shape[0], x["win_fp8"].shape[0], cfg.D
    cmp_kv = _bf16_bits(cmp_src.rows(np.arange(ncb * 128))).reshape(ncb, 128, D)
    win_kv = _bf16_bits(win_src.rows(np.arange(nwb * 128))).reshape(nwb, 128, D)
    out_b = torch.empty_like(out)
    lse_b = torch.empty_like(lse)
    errb = torch.zeros(1, dtype=torch.int32, device="cuda")
    wsn = csa.csa_sparse_attn_workspace_bytes(cfg.T, cfg.H, D, cfg.k, cfg.W)
    ws = torch.empty(wsn, dtype=torch.uint8, device="cuda") if wsn else None
    csa.csa_sparse_attn_decode(
        _dev(x["q"]), _dev(rc), _dev(rs), cfg.rope_offset, _dev(cmp_kv),
        _dev(x["cmp_block_table"]), _dev(sel), cfg.ratio, _dev(win_kv),
        _dev(x["win_block_table"]), cfg.W, _dev(x["attn_sink"]), cfg.softmax_scale,
        _dev(x["query_start_loc"]), _dev(x["positions"]), cfg.T, out_b, lse=lse_b, workspace=ws,
        err=errb)
    torch.cuda.synchronize()
    assert int(errb.item()) == 0
    assert torch.isfinite(out.float()).all(), what
    assert torch.equal(out.view(torch.int16), out_b.view(torch.int16)), what
    assert torch.equal(lse, lse_b), what


@pytest.mark.parametrize("H_,D,R,k", [(8, 64, 16, 500), (64, 512, 64, 500), (8, 64, 16, 1000),
                                      (64, 512, 64, 1000)])
def test_mx_equals_bf16_decode_on_dequantised_planes(H_, D, R, k):
    """k = 500: the decode kernel (128-entry spans per 16-head group);
    k = 1000: lists past 1024 entries, the ring kernel over spans."""
    print(f"[mxkv] vs bf16 H={H_} D={D} k={k}", flush=True)
    csa = _csa()
    cfg = _shape_cfg(H_, D, R, k=k)
    x = synthetic.make_inputs(cfg, seed=8).t
    _same_as_bf16_decode(csa, cfg, x, _selection(cfg, 4), *_rope(cfg, 6), f"D{D}")


@pytest.mark.parametrize("D,k", [(64, 500), (512, 500), (512, 1000)])
def test_mx_extreme_scales_and_every_code(D, k):
    """Every non-NaN E4M3 window code beside E8M0 bytes over 10 .. 150 (the
    products stay normal BF16 numbers), every E2M1 nibble beside every
    non-NaN E4M3 group scale of either sign (subnormals and zero included):
    the same bits as the BF16 decode on the oracle's dequantised pools."""
    print(f"[mxkv] extreme scales D={D} k={k}", flush=True)
    csa = _csa()
    cfg = _shape_cfg(8 if D == 64 else 64, D, 16 if D == 64 else 64, k=k)
    x = dict(synthetic.make_inputs(cfg, seed=9).t)
    rng = np.random.default_rng(10)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    x["win_fp8"] = rng.choice(codes, size=x["win_fp8"].shape).astype(np.uint8)
    x["win_scale"] = rng.integers(10, 151, size=x["win_scale"].shape, dtype=np.uint8)
    x["cmp_fp4"] = rng.integers(0, 256, size=x["cmp_fp4"].shape, dtype=np.uint8)
    x["cmp_scale"] = rng.choice(codes, size=x["cmp_scale"].shape).astype(np.uint8)
    _same_as_bf16_decode(csa, cfg, x, _selection(cfg, 12), *_rope(cfg, 13),
                         f"extreme D{D} k{k}")


def test_mx_nan_codes_propagate():
    """A NaN E4M3 code in one window row, and a NaN E4M3 group scale in one
    selected compressed row: the query rows that read them give NaN outputs
    and lse, as in the oracle; the others stay finite and match."""
    print("[mxkv] NaN codes", flush=True)
    csa = _csa()
    cfg = _shape_cfg(8, 64, 16)
    x = dict(synthetic.make_inputs(cfg, seed=14).t)
    sel = _selection(cfg, 15)
    rc, rs = _rope(cfg, 16)
    # request 1 (positions 130, 131): window position 131 -> only row 4 reads it
    wbt = x["win_block_table"]
    blk = int(wbt[1, 131 // 128])
    wf = x["win_fp8"].copy()
    wf[blk, 131 % 128, 5] = 0x7F
    x["win_fp8"] = wf
    # request 0 row 0: its first selected compressed row gets a NaN scale
    c = int(sel[0, 0])
    cbt = x["cmp_block_table"]
    cs = x["cmp_scale"].copy()
    cs[int(cbt[0, c // 128]), c % 128, 1] = 0xFF
    x["cmp_scale"] = cs
    out, lse, err = _run_mx(csa, cfg, x, sel, rc, rs)
    oo, ol, oe = _oracle_attn(cfg, x, sel, rc, rs)
    assert err == oe == 0
    g = H.bf16_to_f64(out)
    gl = lse.cpu().numpy()
    nan_rows = np.isnan(oo).all(axis=(1, 2))
    # rows 1 and 2 of request 0 may select the same compressed row
    assert nan_rows[0] and nan_rows[4]
    assert np.array_equal(np.isnan(g).all(axis=(1, 2)), nan_rows)
    assert np.isnan(gl[nan_rows]).all()
    ok = ~nan_rows
    H.check_attn(g[ok], oo[ok], gl[ok], ol[ok], "mx finite rows")


def _step_parity(name, rows=None, seed=0):
    csa = _csa()
    cfg = synthetic.get(name)
    print(f"[mxkv] {cfg.name}: generating inputs", flush=True)
    x = synthetic.make_inputs(cfg, seed=seed).t
    step = csa.step_for_config(cfg, x)
    assert step.kv_format == "mx"
    print(f"[mxkv] {cfg.name}: GPU step", flush=True)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    rows = list(range(cfg.T)) if rows is None else rows
    xs = H.sub_batch(x, rows) if len(rows) < cfg.T else x
    print(f"[mxkv] {cfg.name}: oracle on {len(rows)} rows", flush=True)
    o = H.oracle_step(xs, cfg)
    assert o["err"] == 0
    r = np.asarray(rows)
    H.check_scores(step.scores.cpu().numpy()[r].astype(np.float64), o["scores"], cfg.name)
    same = H.check_topk(step.topk_idx.cpu().numpy()[r], o["topk_idx"], o["scores"],
                        np.asarray(x["positions"])[r], cfg.ratio, cfg.name)
    # attention on the oracle's selection, then end to end where they agree
    sel = step.topk_idx.clone()
    sel[torch.as_tensor(r, device="cuda")] = torch.as_tensor(o["topk_idx"], device="cuda")
    step.attn(topk_idx=sel)
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    g = H.bf16_to_f64(step.out)[r]
    gl = step.lse.cpu().numpy()[r]
    H.check_attn(g, o["out"], gl, o["lse"], cfg.name + " attn")
    bud = H.check_budgets(g, o["out"], cfg.name + " attn budget")
    print(f"[mxkv] {cfg.name}: selections identical on {same.sum()}/{len(rows)} rows; "
          f"budget use rms {bud['rms']:.3f}, peak {bud['peak']:.3f}", flush=True)


@pytest.mark.timeout(600)
def test_c12_step_parity():
    _step_parity("c12")


@pytest.mark.timeout(900)
def test_c13_max_context_low_bit_step():
    _step_parity("c13", rows=[0, 5])
