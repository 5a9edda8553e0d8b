"""The decode attention that gathers its rope rows from the full tables
(csa_sparse_attn_decode_rope and, over the low-bit KV planes,
csa_sparse_attn_decode_mx_rope: pypto-lib "DeepSeek V4.1 Flash", section
"Serving-owned full RoPE tables" folded into the attention launch), through
the C ABI: the rope rows it writes equal the oracle's materialisation bit for
bit, and its output and lse equal, bit for bit, those of the separate
launches (csa_materialize_rope_rows, then the attention call) on the same
inputs -- on the short-list and split-ring schedules, HCA and SWA layers,
the low-bit planes, a padded batch, rows whose RoPE position is -1, and rows
past the tables."""
import numpy as np
import pytest

import oracle
import synthetic
from tests import harness as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENT = 0x7FC0DEAD


def _csa():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


def _fill(step):
    for t in (step.rope_cos, step.rope_sin, step.lse):
        t.view(torch.int32).fill_(SENT)
    step.out.view(torch.int16).fill_(0x7FDE)


def _bits(t):
    return t.contiguous().view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy()


def _oracle_rows(x, T, nt, half):
    rc = np.full((T, half), np.nan, np.float32)
    rs = np.full((T, half), np.nan, np.float32)
    err = oracle.materialize_rope_rows(x["freqs_cos"], x["freqs_sin"], x["position_ids"], nt,
                                       rc, rs)
    return rc, rs, err


def _pair(cfg, x, nt=None):
    csa = _csa()
    sep = csa.step_for_config(cfg, x, num_tokens=nt, fuse_rope=False)
    fused = csa.step_for_config(cfg, x, num_tokens=nt)
    assert fused.fuse_rope and not sep.fuse_rope
    assert "rope" not in fused.stages and "rope" in sep.stages
    for s in (sep, fused):
        _fill(s)
        s.run()
    torch.cuda.synchronize()
    return sep, fused


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5", "c6", "c7", "c8", "c12", "c13", "c14"])
def test_fused_rope_equals_separate_launches(name):
    print(f"[rope-fused] {name}", flush=True)
    cfg = synthetic.get(name)
    x = synthetic.make_inputs(cfg, seed=21).t
    sep, fused = _pair(cfg, x)
    assert int(fused.err.item()) == int(sep.err.item()) == 0
    rc, rs, oerr = _oracle_rows(x, cfg.T, cfg.T, cfg.R // 2)
    assert oerr == 0
    assert np.array_equal(_bits(fused.rope_cos), rc.view(np.int32))
    assert np.array_equal(_bits(fused.rope_sin), rs.view(np.int32))
    assert np.array_equal(_bits(fused.out), _bits(sep.out)), f"{name}: output differs"
    assert np.array_equal(_bits(fused.lse), _bits(sep.lse)), f"{name}: lse differs"
    if hasattr(fused, "topk_idx") and fused.mode in ("csa", "reindex"):
        assert torch.equal(fused.topk_idx, sep.topk_idx)


def test_fused_rope_padded_batch():
    """Storage padding rows (t >= num_tokens) keep their rope rows, output and
    lse untouched; active rows (some at RoPE position -1) match."""
    cfg = synthetic.get("c3")   # a request's first row has RoPE position -1
    x = synthetic.make_inputs(cfg, seed=22).t
    nt = cfg.T - 3
    sep, fused = _pair(cfg, x, nt=nt)
    assert int(fused.err.item()) == int(sep.err.item()) == 0
    rc, rs, _ = _oracle_rows(x, cfg.T, nt, cfg.R // 2)
    assert (np.asarray(x["position_ids"])[:nt] < 0).any()
    assert np.array_equal(_bits(fused.rope_cos)[:nt], rc[:nt].view(np.int32))
    assert np.array_equal(_bits(fused.rope_sin)[:nt], rs[:nt].view(np.int32))
    assert np.all(_bits(fused.rope_cos)[nt:] == SENT)
    assert np.all(_bits(fused.rope_sin)[nt:] == SENT)
    assert np.all(_bits(fused.out)[nt:] == 0x7FDE)
    assert np.all(_bits(fused.lse)[nt:] == SENT)
    assert np.array_equal(_bits(fused.out)[:nt], _bits(sep.out)[:nt])
    assert np.array_equal(_bits(fused.lse)[:nt], _bits(sep.lse)[:nt])


def test_fused_rope_rows_past_the_tables():
    """A RoPE position past the tables raises CSA_EFLAG_POS_RANGE and leaves
    that rope row untouched, as the materialisation does; the row itself
    attends with the identity rotation, and every other row is unaffected."""
    csa = _csa()
    cfg = synthetic.get("c2")
    x = dict(synthetic.make_inputs(cfg, seed=23).t)
    x["position_ids"] = np.asarray(x["position_ids"]).copy()
    bad = 3
    x["position_ids"][bad] = cfg.rope_capacity + 5
    fused = csa.step_for_config(cfg, x)
    _fill(fused)
    fused.run()
    torch.cuda.synchronize()
    assert int(fused.err.item()) == oracle.EFLAG_POS_RANGE
    assert np.all(_bits(fused.rope_cos)[bad] == SENT)
    assert np.all(_bits(fused.rope_sin)[bad] == SENT)
    rc, rs, oerr = _oracle_rows(x, cfg.T, cfg.T, cfg.R // 2)
    assert oerr == oracle.EFLAG_POS_RANGE
    others = [t for t in range(cfg.T) if t != bad]
    assert np.array_equal(_bits(fused.rope_cos)[others], rc[others].view(np.int32))
    # the separate attention call on the oracle's rows, identity for the bad row
    rc[bad], rs[bad] = 1.0, 0.0
    sep = csa.step_for_config(cfg, x, fuse_rope=False)
    _fill(sep)
    sep.index()
    sep.topk()
    sep.rope_cos.copy_(torch.as_tensor(rc))
    sep.rope_sin.copy_(torch.as_tensor(rs))
    sep.attn()
    torch.cuda.synchronize()
    assert int(sep.err.item()) == 0
    assert torch.equal(sep.topk_idx, fused.topk_idx)
    assert np.array_equal(_bits(fused.out), _bits(sep.out))
    assert np.array_equal(_bits(fused.lse), _bits(sep.lse))
    # and the oracle agrees with the result to the attention tolerance
    o_out, o_lse, _ = oracle.sparse_attn(x["q"], rc, rs, cfg.rope_offset, x["cmp_kv"],
                                         x["cmp_block_table"], fused.topk_idx.cpu().numpy(),
                                         cfg.ratio, x["win_kv"], x["win_block_table"], cfg.W,
                                         x["attn_sink"], cfg.softmax_scale,
                                         x["query_start_loc"], x["positions"], cfg.T)
    H.check_attn(H.bf16_to_f64(fused.out), o_out, fused.lse.cpu().numpy(), o_lse, "past tables")


def test_fused_rope_without_row_outputs():
    """rope_cos / rope_sin NULL: the rows are used but not written."""
    csa = _csa()
    cfg = synthetic.get("c2")
    x = synthetic.make_inputs(cfg, seed=24).t
    sep = csa.step_for_config(cfg, x, fuse_rope=False)
    _fill(sep)
    sep.run()
    t = sep.t
    out = torch.empty_like(sep.out)
    lse = torch.empty_like(sep.lse)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    csa.csa_sparse_attn_decode_rope(
        t["q"], t["freqs_cos"], t["freqs_sin"], t["position_ids"], cfg.rope_offset, t["cmp_kv"],
        t["cmp_block_table"], sep.topk_idx, cfg.ratio, t["win_kv"], t["win_block_table"], cfg.W,
        t["attn_sink"], cfg.softmax_scale, t["query_start_loc"], t["positions"], cfg.T, out,
        lse=lse, workspace=sep.attn_ws, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(out.view(torch.int16), sep.out.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), sep.lse.view(torch.int32))


def test_fused_rope_repeat_is_bitwise():
    """Two runs of the fused step on one input give the same bits."""
    csa = _csa()
    cfg = synthetic.get("c5")
    x = synthetic.make_inputs(cfg, seed=25).t
    st = csa.step_for_config(cfg, x)
    st.run()
    torch.cuda.synchronize()
    a = [st.out.clone(), st.lse.clone(), st.rope_cos.clone()]
    _fill(st)
    st.run()
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), st.out.view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), st.lse.view(torch.int32))
    assert torch.equal(a[2].view(torch.int32), st.rope_cos.view(torch.int32))
