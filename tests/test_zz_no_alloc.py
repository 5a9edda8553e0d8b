"""The allocation-free decode entry point against the workspace one.

csa_sparse_attn_decode_noalloc runs the same kernels as
csa_sparse_attn_decode, with the split partials in the library's static
device array instead of a caller workspace, so its outputs must equal the
workspace call's bit for bit.  Two calls in a row on one GPU: a ratio-1 decode
batch of eight rows whose key lists are split into spans (the larger
partials), then three active rows of another draw, which must not see
anything the first call left in the array.
"""
import numpy as np
import pytest

import synthetic

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _csa():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


def _attn_args(step, num_tokens):
    t = step.t
    return (t["q"], step.rope_cos, step.rope_sin, step.rope_offset, t["cmp_kv"],
            t["cmp_block_table"], step.topk_idx, step.ratio, t["win_kv"], t["win_block_table"],
            step.window, t["attn_sink"], step.softmax_scale, t["query_start_loc"],
            t["positions"], num_tokens)


def _compare(csa, name, num_tokens):
    cfg = synthetic.get(name)
    print(f"[noalloc] {cfg.name}: num_tokens={num_tokens}", flush=True)
    x = synthetic.make_inputs(cfg, seed=8 + num_tokens).t
    step = csa.step_for_config(cfg, x, num_tokens=num_tokens)
    step.rope()
    step.index()
    step.topk()
    torch.cuda.synchronize()
    need = csa.csa_sparse_attn_workspace_bytes(num_tokens, cfg.H, cfg.D, cfg.k, cfg.W)
    assert 0 < need <= csa.csa_sparse_attn_noalloc_max_bytes()
    # the workspace entry point
    out_ws = torch.full_like(step.out, 0)
    out_ws.view(torch.int16).fill_(0x7FDE)
    lse_ws = torch.full_like(step.lse, float("nan"))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    err_ws = torch.zeros(1, dtype=torch.int32, device="cuda")
    csa.csa_sparse_attn_decode(*_attn_args(step, num_tokens), out_ws, lse=lse_ws, workspace=ws,
                               err=err_ws, k=cfg.k)
    # the allocation-free one
    out_na = torch.full_like(step.out, 0)
    out_na.view(torch.int16).fill_(0x7FDE)
    lse_na = torch.full_like(step.lse, float("nan"))
    err_na = torch.zeros(1, dtype=torch.int32, device="cuda")
    csa.csa_sparse_attn_decode_noalloc(*_attn_args(step, num_tokens), out_na, lse=lse_na,
                                       err=err_na, k=cfg.k)
    torch.cuda.synchronize()
    assert int(err_ws.item()) == 0 and int(err_na.item()) == 0
    assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16)), f"{name}: out"
    assert torch.equal(lse_ws.view(torch.int32), lse_na.view(torch.int32)), f"{name}: lse"
    # rows past num_tokens stay untouched
    assert np.all(out_na.view(torch.int16).cpu().numpy()[num_tokens:] == 0x7FDE)
    return need


def test_noalloc_matches_workspace_call_twice():
    csa = _csa()
    big = _compare(csa, "c3", 8)     # 17 spans of 128 entries per row, merged
    small = _compare(csa, "c3", 3)   # the same lists, fewer rows
    assert small < big
