"""GPU parity of the ratio-2 compressor publication (csa_compress_pairs).

Published rows against the oracle, with a tolerance from the arithmetic: the
FP32 pooling differs from the exact value by a few FP32 ulps, so its BF16
rounding can land one BF16 ulp (at most 2^-7 relative) away from the
oracle's; the norm factor moves by far less; each side's output rounding adds
at most half an ulp (2^-8 relative).  Off the rope span that bounds
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
    g = oracle.bf16_to_f64(g_cmp[~untouched])
    o = oracle.bf16_to_f64(o_cmp[~untouched])
    off = a["rope_offset"]
    tol = 1.05 * 2.0 ** -6 * np.abs(o)
    span = slice(off, off + 2 * a["rope_cos"].shape[1])
    mag = np.abs(o[:, span])
    partner = mag.reshape(mag.shape[0], -1, 2)[:, :, ::-1].reshape(mag.shape)
    tol[:, span] = 2.0 ** -5 * (mag + partner)
    assert np.all(np.abs(g - o) <= tol + 1e-30), (
        f"{what}: worst {np.max(np.abs(g - o) - tol):.3g} over, rows {int((~untouched).sum())}")
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
