"""GPU parity of the ratio-2 compressor publication (csa_compress_pairs).

Published rows against the oracle, with a tolerance from the arithmetic: the
FP32 pooling differs from the exact value by a few FP32 ulps, so its BF16
rounding can land one BF16 ulp (at most 2^-7 relative) away from the
oracle's; the norm factor moves by far less; each side's output rounding adds
at most half an ulp (2^-8 relative).  Where the pooled value cancels, the
FP32 rounding is relative to the pair's inputs instead: an absolute
2^-18 RMS(row) covers inputs up to 16 times the row's RMS.  Off the rope span that bounds
|g - o| by 2^-6 |o| up to second-order terms (the test allows 1.05 times
that).  A rope pair mixes two channels: the rotation carries the 2^-7
errors of both inputs into each output, at most sqrt(2) 2^-7 (|o_c| + |o_p|),
plus the two output roundings, under 2^-5 (|o_c| + |o_p|).  Ring rows and
every untouched byte are bit-exact.  Chunking invariance is bitwise: a pair
pools the same FP32 inputs whether its predecessor comes from the chunk or
from the ring.
"""
import numpy as np
import pytest

import oracle
import synthetic
from tests import harness as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PAGE = 128
SENT = 0x7FDE


def _csa():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


def _dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda()


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _case(rng, chunks, starts, D=512, R=64, cap=4, disabled=(), neg_rows=()):
    B = len(chunks)
    T = sum(chunks)
    qsl = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    pos = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, chunks)]).astype(np.int32)
    for r in neg_rows:
        pos[r] = -1
    kv = rng.standard_normal((T, D)).astype(np.float32)
    gate = rng.standard_normal((T, D)).astype(np.float32)
    nsb = B + 2
    sbt = rng.permutation(nsb)[:B].astype(np.int32)
    for b in disabled:
        sbt[b] = -1
    state = rng.standard_normal((nsb, cap, 2 * D)).astype(np.float32)
    pages = max(1, max((s + n) // 2 // PAGE + 1 for s, n in zip(starts, chunks)))
    ncb = B * pages + 1
    cbt = rng.permutation(ncb)[:B * pages].astype(np.int32).reshape(B, pages)
    gamma = rng.uniform(0.5, 2.0, D).astype(np.float32)
    ang = rng.uniform(-3, 3, (T, R // 2))
    c = np.cos(ang).astype(np.float32)
    s = np.sin(ang).astype(np.float32)
    cmp = np.full((ncb, PAGE, D), SENT, np.uint16)
    return dict(kv_proj=kv, gate=gate, query_start_loc=qsl, positions=pos, num_tokens=T,
                state_block_table=sbt, state_cache=state, rms_gamma=gamma, rms_eps=1e-6,
                rope_cos=c, rope_sin=s, rope_offset=D - R, cmp_kv=cmp, cmp_block_table=cbt)


def _run(a):
    csa = _csa()
    state = _dev(a["state_cache"])
    cmp = _bf16_dev(a["cmp_kv"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    csa.csa_compress_pairs(_dev(a["kv_proj"]), _dev(a["gate"]), _dev(a["query_start_loc"]),
                           _dev(a["positions"]), a["num_tokens"], _dev(a["state_block_table"]),
                           state, _dev(a["rms_gamma"]), a["rms_eps"], _dev(a["rope_cos"]),
                           _dev(a["rope_sin"]), a["rope_offset"], cmp, _dev(a["cmp_block_table"]),
                           err=err)
    torch.cuda.synchronize()
    return (cmp.view(torch.int16).cpu().numpy().view(np.uint16), state.cpu().numpy(),
            int(err.item()))


def _check_rows(g_bits, o_bits, off, half, what):
    """Published BF16 rows against the oracle's, to the tolerance above."""
    g = oracle.bf16_to_f64(g_bits)
    o = oracle.bf16_to_f64(o_bits)
    tol = 1.05 * 2.0 ** -6 * np.abs(o)
    span = slice(off, off + 2 * half)
    mag = np.abs(o[..., span])
    partner = mag.reshape(mag.shape[:-1] + (-1, 2))[..., ::-1].reshape(mag.shape)
    tol[..., span] = 2.0 ** -5 * (mag + partner)
    # the FP32 pooling's rounding is relative to the pair's inputs, not to a
    # pooled value that cancels: a few FP32 ulps of inputs up to 16x the row
    # RMS, carried through the norm factor
    tol += 2.0 ** -18 * np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    assert np.all(np.abs(g - o) <= tol + 1e-30), (
        f"{what}: worst {np.max(np.abs(g - o) - tol):.3g} over, rows {o.shape[0]}")


def _compare(a, what):
    g_cmp, g_st, g_err = _run(a)
    o_cmp, o_st, o_err = oracle.compress_pairs(**a)
    assert g_err == o_err, (g_err, o_err)
    assert np.array_equal(g_st.view(np.uint32), o_st.view(np.uint32)), f"{what}: ring differs"
    untouched = np.all(o_cmp == SENT, axis=-1)
    assert np.array_equal(g_cmp[untouched], o_cmp[untouched]), f"{what}: stray writes"
    assert not np.any(np.all(g_cmp == SENT, axis=-1) & ~untouched), f"{what}: missing rows"
    if untouched.all():
        return 0
    _check_rows(g_cmp[~untouched], o_cmp[~untouched], a["rope_offset"], a["rope_cos"].shape[1],
                what)
    return int((~untouched).sum())


def test_mixed_chunks_against_the_oracle():
    rng = np.random.default_rng(60)
    # chunk lengths and start positions: decode pairs, a single odd token
    # reading the ring, a chunk longer than the ring starting at an odd position
    a = _case(rng, chunks=[2, 1, 5, 7, 3], starts=[10, 13, 21, 100, 6], disabled=(4,),
              neg_rows=())
    print("[compress] mixed chunks", flush=True)
    n = _compare(a, "mixed")
    assert n == 1 + 1 + 3 + 3   # 11; 13; 21, 23, 25; 101, 103, 105


@pytest.mark.parametrize("D,R", [(96, 32), (256, 0), (1000, 64), (2048, 64)])
def test_head_widths(D, R):
    """Every channel-chunk count the kernel instantiates, partial chunks
    (lanes past D) and a layer without a rope span."""
    rng = np.random.default_rng(D + R)
    a = _case(rng, chunks=[3, 4, 1], starts=[5, 20, 9], D=D, R=R)
    print(f"[compress] D={D} R={R}", flush=True)
    assert _compare(a, f"D={D}") == 2 + 2 + 1


def test_repeated_slots_keep_the_later_row():
    """Non-consecutive positions whose slots repeat among a chunk's last CAP
    rows: the later row wins each slot (the oracle writes in row order)."""
    rng = np.random.default_rng(64)
    a = _case(rng, chunks=[6], starts=[0])
    a["positions"] = np.array([3, 8, 13, 17, 21, 24], np.int32)   # last 4: slots 1, 1, 1, 0
    print("[compress] repeated slots", flush=True)
    _compare(a, "repeated slots")


def test_contract_flags_and_negative_positions():
    rng = np.random.default_rng(61)
    # request 0: positions 7, -1, 9 (9 pools with the negative row's input);
    # request 1's state block is past the pool: its in-chunk pair still
    # publishes, its ring accesses are skipped
    a = _case(rng, chunks=[3, 2], starts=[7, 4], neg_rows=(1,))
    a["state_block_table"][1] = 99
    print("[compress] flags", flush=True)
    assert _compare(a, "flags") == 3                    # 7, 9; 5
    # an active row no request owns
    b = _case(rng, chunks=[2, 2], starts=[3, 400])
    b["query_start_loc"] = np.array([0, 2, 3], np.int32)
    _compare(b, "unowned")
    # a publication page past the table: position 301 -> compressed 150, page 1
    c = _case(rng, chunks=[2, 2], starts=[300, 10])
    c["cmp_block_table"] = c["cmp_block_table"][:, :1].copy()
    c["cmp_block_table"][1, 0] = -1                     # and an unmapped page
    assert _compare(c, "pages") == 0


def test_decode_shapes_c2_like():
    """4 requests x S = 2 decode rows at positions (p - 1, p), p odd, D = 512:
    each request closes one pair per step."""
    rng = np.random.default_rng(62)
    a = _case(rng, chunks=[2, 2, 2, 2], starts=[32766, 1000, 2, 77])
    print("[compress] decode", flush=True)
    assert _compare(a, "decode") == 4


def test_chunking_invariance_bitwise():
    rng = np.random.default_rng(63)
    n = 40
    whole = _case(rng, chunks=[n], starts=[0])
    g_whole, st_whole, e = _run(whole)
    assert e == 0
    cmp = whole["cmp_kv"].copy()
    state = whole["state_cache"].copy()
    t0 = 0
    print("[compress] chunking", flush=True)
    for chunk in (3, 1, 7, 2, 5, 1, 1, 9, 11):
        sl = slice(t0, t0 + chunk)
        part = dict(whole, kv_proj=whole["kv_proj"][sl], gate=whole["gate"][sl],
                    positions=whole["positions"][sl], num_tokens=chunk,
                    query_start_loc=np.array([0, chunk], np.int32),
                    rope_cos=whole["rope_cos"][sl], rope_sin=whole["rope_sin"][sl],
                    cmp_kv=cmp, state_cache=state)
        cmp, state, e = _run(part)
        assert e == 0
        t0 += chunk
    assert t0 == n
    assert np.array_equal(cmp, g_whole)
    assert np.array_equal(state.view(np.uint32), st_whole.view(np.uint32))


def _step(cfg_name):
    import compressed_sparse_attention_csa_amd as csa
    cfg = synthetic.get(cfg_name)
    x = synthetic.make_inputs(cfg, seed=0).t
    step = csa.step_for_config(cfg, x)
    return cfg, x, step


def _published_rows(cfg, x, cmp_bits):
    """(request, compressed position, pool row) of every pair the chunk closes."""
    qsl, pos, bt = x["query_start_loc"], x["positions"], x["cmp_block_table"]
    out = []
    for b in range(cfg.B):
        for t in range(qsl[b], qsl[b + 1]):
            p = int(pos[t])
            if p >= 0 and p % 2 == 1:
                c = p // 2
                out.append(cmp_bits[bt[b, c // PAGE], c % PAGE])
    return np.stack(out)


def test_c16_decode_step_with_the_compressor():
    """C2's decode step with the publication first: the published rows, the
    ring, the step's scores / top-k / attention, and attention over a
    selection that holds the freshly published row."""
    cfg, x, step = _step("c16")
    print("[compress] c16 step", flush=True)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    o = H.oracle_step(x, cfg)
    assert o["err"] == 0
    g_cmp = step.t["cmp_kv"].view(torch.int16).cpu().numpy().view(np.uint16)
    g_rows = _published_rows(cfg, x, g_cmp)
    assert g_rows.shape[0] == cfg.B
    _check_rows(g_rows, _published_rows(cfg, x, o["cmp_kv"]), cfg.rope_offset, cfg.R // 2,
                "c16 published rows")
    # every other row of the pool is untouched
    mask = np.ones(g_cmp.shape[:2], bool)
    for b in range(cfg.B):
        mask[x["cmp_block_table"][b, 16383 // PAGE], 16383 % PAGE] = False
    assert np.array_equal(g_cmp[mask], x["cmp_kv"][mask])
    g_st = step.t["state_cache"].cpu().numpy()
    assert np.array_equal(g_st.view(np.uint32), o["state_cache"].view(np.uint32))
    H.check_scores(step.scores.cpu().numpy().astype(np.float64), o["scores"], "c16 scores")
    same = H.check_topk(step.topk_idx.cpu().numpy(), o["topk_idx"], o["scores"], x["positions"],
                        cfg.ratio, "c16 top-k")
    H.check_attn(H.bf16_to_f64(step.out)[same], o["out"][same],
                 step.lse.cpu().numpy()[same], o["lse"][same], "c16 attention")
    # the freshly published row inside the selection of the rows that see it
    # (the odd rows: position 32767 sees compressed positions 0..16383): the
    # oracle's selection with one entry replaced by 16383, re-sorted
    sel = o["topk_idx"].copy()
    for t in range(cfg.T):
        if x["positions"][t] % 2 == 0:
            continue
        row = [c for c in sel[t] if c != 16383][:cfg.k - 1] + [16383]
        sel[t] = np.sort(np.asarray(row, np.int32))
    step.attn(topk_idx=torch.from_numpy(sel).cuda())
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    o2 = H.oracle_step(x, cfg, topk_override=sel)
    H.check_attn(H.bf16_to_f64(step.out), o2["out"], step.lse.cpu().numpy(), o2["lse"],
                 "c16 attention over the published row")


def test_c17_prefill_chunk_publication():
    """The 8,192-token prefill chunk: all 4,096 published rows and the ring."""
    cfg, x, step = _step("c17")
    print("[compress] c17 chunk", flush=True)
    step.run()
    torch.cuda.synchronize()
    assert int(step.err.item()) == 0
    o_cmp, o_st, oe = H.oracle_compress(x, cfg)
    assert oe == 0
    g_cmp = step.t["cmp_kv"].view(torch.int16).cpu().numpy().view(np.uint16)
    _check_rows(g_cmp.reshape(-1, cfg.D), o_cmp.reshape(-1, cfg.D), cfg.rope_offset, cfg.R // 2,
                "c17 published rows")
    g_st = step.t["state_cache"].cpu().numpy()
    assert np.array_equal(g_st.view(np.uint32), o_st.view(np.uint32))


def _run_tables(a, tc, ts, rope_pos):
    """csa_compress_pairs_rope: the rope rows gathered from full tables."""
    csa = _csa()
    state = _dev(a["state_cache"])
    cmp = _bf16_dev(a["cmp_kv"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    csa.csa_compress_pairs_rope(_dev(a["kv_proj"]), _dev(a["gate"]), _dev(a["query_start_loc"]),
                                _dev(a["positions"]), a["num_tokens"],
                                _dev(a["state_block_table"]), state, _dev(a["rms_gamma"]),
                                a["rms_eps"], _dev(tc), _dev(ts), _dev(rope_pos),
                                a["rope_offset"], cmp, _dev(a["cmp_block_table"]), err=err)
    torch.cuda.synchronize()
    return (cmp.view(torch.int16).cpu().numpy().view(np.uint16), state.cpu().numpy(),
            int(err.item()))


def _with_tables(a, rng, cap, rope_pos):
    """Full tables of `cap` rows and the rope rows the materialisation makes
    of them for rope_pos (identity for negative positions; rows past the
    tables get the identity too, which the table call uses for them)."""
    half = a["rope_cos"].shape[1]
    ang = rng.uniform(-3, 3, (cap, half))
    tc, ts = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    T = a["num_tokens"]
    rc = np.full((T, half), np.nan, np.float32)
    rs = np.full((T, half), np.nan, np.float32)
    err = oracle.materialize_rope_rows(tc, ts, rope_pos, T, rc, rs)
    rc = np.nan_to_num(rc, nan=1.0)
    rs = np.nan_to_num(rs, nan=0.0)
    return tc, ts, dict(a, rope_cos=rc, rope_sin=rs), err


def test_table_rope_rows_equal_materialised_rows():
    """csa_compress_pairs_rope publishes, bit for bit, what csa_compress_pairs
    publishes from the materialised rows of the same positions (pair starts,
    -1 rows included), and leaves the same ring."""
    rng = np.random.default_rng(71)
    a = _case(rng, chunks=[2, 1, 5, 7, 3, 6], starts=[10, 13, 21, 100, 6, 40], disabled=(4,),
              neg_rows=(5,))
    pos = a["positions"]
    rope_pos = np.where(pos >= 0, pos - pos % 2, -1).astype(np.int32)
    tc, ts, a_rows, e0 = _with_tables(a, rng, 256, rope_pos)
    assert e0 == 0
    print("[compress] table rope rows", flush=True)
    g_cmp, g_st, g_err = _run_tables(a, tc, ts, rope_pos)
    r_cmp, r_st, r_err = _run(a_rows)
    assert g_err == r_err
    assert np.array_equal(g_cmp, r_cmp), "published rows differ"
    assert np.array_equal(g_st.view(np.uint32), r_st.view(np.uint32)), "ring differs"
    assert _compare(a_rows, "table rope rows, against the oracle") > 0


def test_table_rope_position_past_the_tables():
    """A pair start past the tables flags POS_RANGE and that publication
    rotates by the identity; the other rows are unaffected."""
    rng = np.random.default_rng(72)
    a = _case(rng, chunks=[4, 4], starts=[20, 61])
    pos = a["positions"]
    rope_pos = np.where(pos >= 0, pos - pos % 2, -1).astype(np.int32)
    cap = 64
    assert pos[6] == 63 and pos[2] == 22
    rope_pos[6] = cap + 7                 # an odd row: its publication
    rope_pos[2] = cap + 1                 # an even row: flagged, nothing published
    tc, ts, a_rows, e0 = _with_tables(a, rng, cap, rope_pos)
    assert e0 == oracle.EFLAG_POS_RANGE
    g_cmp, g_st, g_err = _run_tables(a, tc, ts, rope_pos)
    r_cmp, r_st, r_err = _run(a_rows)
    assert g_err == r_err | oracle.EFLAG_POS_RANGE == oracle.EFLAG_POS_RANGE
    assert np.array_equal(g_cmp, r_cmp)
    assert np.array_equal(g_st.view(np.uint32), r_st.view(np.uint32))


@pytest.mark.parametrize("name", ["c16", "c17"])
def test_step_with_table_rope_equals_separate_rope_launch(name):
    """The compressor steps without a RoPE launch (the compressor and the
    decode attention gather their rows) give the same bits as with it."""
    csa = _csa()
    cfg = synthetic.get(name)
    x = synthetic.make_inputs(cfg, seed=31).t
    sep = csa.step_for_config(cfg, x, fuse_rope=False)
    fused = csa.step_for_config(cfg, x)
    assert "rope" in sep.stages and "rope" not in fused.stages
    print(f"[compress] {name}: stages {fused.stages} vs {sep.stages}", flush=True)
    for s in (sep, fused):
        s.run()
    torch.cuda.synchronize()
    assert int(fused.err.item()) == int(sep.err.item()) == 0
    assert torch.equal(fused.t["cmp_kv"].view(torch.int16), sep.t["cmp_kv"].view(torch.int16))
    assert torch.equal(fused.t["state_cache"].view(torch.int32),
                       sep.t["state_cache"].view(torch.int32))
    if cfg.mode != "compress":
        assert torch.equal(fused.topk_idx, sep.topk_idx)
        assert torch.equal(fused.out.view(torch.int16), sep.out.view(torch.int16))
        assert torch.equal(fused.lse.view(torch.int32), sep.lse.view(torch.int32))
        assert torch.equal(fused.rope_cos.view(torch.int32), sep.rope_cos.view(torch.int32))
