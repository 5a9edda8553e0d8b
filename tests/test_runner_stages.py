"""The step driver's launch plan, checked on the host (no GPU: the buffers are
CPU tensors and no kernel is launched): decode steps gather their RoPE rows
inside the attention launch and the compressor inside its own, so only
prefill attention keeps the separate RoPE-row launch; fuse_rope=False gives
the one-call-per-step plan back."""
import pytest

import synthetic

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_attention_csa_amd as m
    try:
        m.load()
    except m.CsaError as e:  # pragma: no cover - build first
        pytest.fail(f"libcsa.so not built: {e}")
    return m


@pytest.mark.parametrize("name,fused,separate", [
    ("c1", ("index", "topk", "attn"), ("rope", "index", "topk", "attn")),
    ("c4", ("rope", "index", "topk", "attn"), ("rope", "index", "topk", "attn")),
    ("c6", ("attn",), ("rope", "attn")),
    ("c9", ("index", "topk", "cand", "attn"), ("rope", "index", "topk", "cand", "attn")),
    ("c11", ("index", "topk", "attn"), ("rope", "index", "topk", "attn")),
    ("c16", ("compress_pairs", "index", "topk", "attn"),
     ("rope", "compress_pairs", "index", "topk", "attn")),
    ("c17", ("compress_pairs",), ("rope", "compress_pairs")),
])
def test_stage_plan(csa, name, fused, separate):
    cfg = synthetic.get(name)
    x = synthetic.make_inputs(cfg, seed=0).t
    a = csa.step_for_config(cfg, x, device="cpu")
    b = csa.step_for_config(cfg, x, device="cpu", fuse_rope=False)
    assert a.stages == fused
    assert b.stages == separate
    if cfg.mode != "compress":
        # the query rope rows exist either way (written by the fused attention)
        assert tuple(a.rope_cos.shape) == (cfg.T, cfg.R // 2)
