"""Two GPU checks of the library's contract beyond single-call parity.

* A padded decode batch (pypto-lib "DeepSeek V4.1 Flash", "Compressor state
  ownership": T may include trailing storage padding): 8 active rows of the
  ratio-1 decode layer in a 300-row extent, every workspace sized by its
  helper from the extent T, runs without a workspace error, matches the oracle
  on the active rows and leaves the padding rows untouched.
* Repeat runs are bitwise identical for every kernel family: the prefill ring
  kernel (C4), the decode spans with their merge and the three-kernel
  long-row top-k (C5), the hierarchical selection (C8 reindex, C9 mask
  publication) and the MXFP4 scorer (C11).  Each workload runs twice on the same inputs and
  buffers; the first differing output fails the test.
"""
import numpy as np
import pytest

import synthetic
from tests import harness as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENT_I = 0x7EEEEEEE


def _csa():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


PER_ROW = ("q", "q_idx", "q_scale", "head_w", "positions", "position_ids")


def test_padded_decode_batch_uses_helper_sized_workspaces():
    csa = _csa()
    cfg = synthetic.get("c3")   # 2048 + 128 entries per row: 17 spans, merged
    x = synthetic.make_inputs(cfg, seed=21).t
    T_store, nt = 300, cfg.T
    xp = dict(x)
    for k in PER_ROW:
        a = np.asarray(x[k])
        pad = np.repeat(a[-1:], T_store - nt, axis=0)   # finite bytes in the padding rows
        xp[k] = np.ascontiguousarray(np.concatenate([a, pad], axis=0))
    print(f"[repeat] padded decode: T={T_store}, num_tokens={nt}", flush=True)
    need = csa.csa_sparse_attn_workspace_bytes(T_store, cfg.H, cfg.D, cfg.k, cfg.W)
    assert need >= csa.csa_sparse_attn_workspace_bytes(nt, cfg.H, cfg.D, cfg.k, cfg.W) > 0
    step = csa.step_for_config(cfg, xp, num_tokens=nt)
    assert step.T == T_store and step.attn_ws is not None and step.attn_ws.numel() == need
    for t in (step.rope_cos, step.rope_sin, step.scores, step.topk_val, step.lse):
        t.view(torch.int32).fill_(0x7FC0DEAD)
    step.topk_idx.fill_(SENT_I)
    step.out.view(torch.int16).fill_(0x7FDE)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    o = H.oracle_step(x, cfg)
    H.check_scores(step.scores.cpu().numpy()[:nt].astype(np.float64), o["scores"], "padded")
    gi = step.topk_idx.cpu().numpy()[:nt]
    same = H.check_topk(gi, o["topk_idx"], o["scores"], x["positions"], cfg.ratio, "padded")
    assert same.sum() >= nt // 2
    # attention where the selections agree (elsewhere they differ only at ties)
    H.check_attn(H.bf16_to_f64(step.out)[:nt][same], o["out"][same],
                 step.lse.cpu().numpy()[:nt][same], o["lse"][same], "padded")
    assert np.all(step.out.view(torch.int16).cpu().numpy()[nt:] == 0x7FDE)
    assert np.all(step.lse.cpu().numpy()[nt:].view(np.uint32) == 0x7FC0DEAD)
    assert np.all(step.topk_idx.cpu().numpy()[nt:] == SENT_I)
    assert np.all(step.scores.cpu().numpy()[nt:].view(np.uint32) == 0x7FC0DEAD)


def _outputs(step):
    outs = {"rope_cos": step.rope_cos, "out": step.out, "err": step.err}
    if step.lse is not None:
        outs["lse"] = step.lse
    if step.mode in ("csa", "reindex", "hier_full"):
        outs["scores"] = step.scores
        outs["topk_idx"] = step.topk_idx
        if step.topk_val is not None:
            outs["topk_val"] = step.topk_val
    if step.mode == "hier_full":
        outs["cand_blocks"] = step.cand_blocks
    if step.mode == "reindex":
        outs["cand_count"] = step.cand_count
    return {k: v.view(torch.uint8) if v.dtype == torch.bfloat16 else v for k, v in outs.items()}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c4", "c5", "c8", "c9", "c11"])
def test_repeat_runs_are_bitwise_identical(name):
    csa = _csa()
    cfg = synthetic.get(name)
    print(f"[repeat] {cfg.name}: generating inputs", flush=True)
    x = synthetic.make_inputs(cfg, seed=4).t
    step = csa.step_for_config(cfg, x)
    first = None
    for run in range(2):
        step.err.zero_()
        print(f"[repeat] {cfg.name}: run {run}", flush=True)
        step.run()
        torch.cuda.synchronize()
        cur = {k: v.clone() for k, v in _outputs(step).items()}
        if first is None:
            first = cur
            # scrub every output between the runs, so the second run must
            # write all of it again
            for v in _outputs(step).values():
                v.fill_(0x5A if v.dtype == torch.uint8 else -7)
            continue
        for k in first:
            assert torch.equal(first[k], cur[k]), f"{cfg.name}: {k} differs between runs"
    assert int(first["err"].item()) == 0
