"""Shared pieces of the GPU parity tests: run the oracle on (a subset of) the
rows of a synthetic workload, run the HIP path through the C ABI, and compare
with the stated tolerances.

Tolerances (derived in the design notes):
  * RoPE rows, top-k indices: bit-exact; top-k may differ only where the
    oracle's own scores tie within 1e-5 relative of the k-th score;
  * scores: |g - o| <= 1e-5 * |o| + 2e-6 * max|o_row| (FP32 epilogue over 64
    heads against float64);
  * attention output and lse: |g - o| <= 1e-2 + 2e-2 * |o|.
"""
from __future__ import annotations

import numpy as np

import oracle

SENTINEL_U32 = 0x7FC0DEAD
SENTINEL_BF16 = 0x7FDE


def sub_batch(x: dict, rows) -> dict:
    """The same requests restricted to the given rows (row independence lets
    the oracle score a sample of a large batch)."""
    rows = np.asarray(sorted(rows), dtype=np.int64)
    qsl = np.asarray(x["query_start_loc"])
    owner = np.searchsorted(qsl, rows, side="right") - 1
    counts = np.bincount(owner, minlength=len(qsl) - 1)
    y = dict(x)
    y["query_start_loc"] = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    for k in ("q_idx", "q_scale", "head_w", "positions", "position_ids", "q"):
        y[k] = np.ascontiguousarray(np.asarray(x[k])[rows])
    return y


def kv_sources(x: dict, cfg):
    """The oracle's (compressed, window) KV arguments for a config's format."""
    if getattr(cfg, "kv_format", "bf16") == "mx":
        return (oracle.mxfp4_e4m3_plane(x["cmp_fp4"], x["cmp_scale"]),
                oracle.mxfp8_plane(x["win_fp8"], x["win_scale"]))
    return x["cmp_kv"], x["win_kv"]


def oracle_compress(x: dict, cfg, cmp_kv=None):
    """The oracle's compressor publication for a config carrying one: its
    rope rows (the pair starts), then compress_pairs.  Returns (cmp_kv,
    state_cache, err)."""
    T = x["kv_proj"].shape[0]
    half = cfg.R // 2
    rc = np.full((T, half), np.nan, np.float32)
    rs = np.full((T, half), np.nan, np.float32)
    e0 = oracle.materialize_rope_rows(x["freqs_cos"], x["freqs_sin"], x["cmp_position_ids"], T,
                                      rc, rs)
    c, st, e1 = oracle.compress_pairs(x["kv_proj"], x["gate"], x["query_start_loc"],
                                      x["positions"], T, x["state_block_table"],
                                      x["state_cache"], x["rms_gamma"], cfg.rms_eps, rc, rs,
                                      cfg.rope_offset,
                                      x["cmp_kv"] if cmp_kv is None else cmp_kv,
                                      x["cmp_block_table"])
    return c, st, e0 | e1


def oracle_step(x: dict, cfg, topk_override=None) -> dict:
    T = x["q"].shape[0]
    half = cfg.R // 2
    ec, cst = 0, None
    if getattr(cfg, "compress", False):   # the publication comes first
        cmp_pub, cst, ec = oracle_compress(x, cfg)
        x = dict(x, cmp_kv=cmp_pub)
    rc = np.full((T, half), np.nan, np.float32)
    rs = np.full((T, half), np.nan, np.float32)
    e0 = oracle.materialize_rope_rows(x["freqs_cos"], x["freqs_sin"], x["position_ids"], T, rc, rs)
    score_fn = {"mxfp4": oracle.index_scores_mxfp4, "fp8": oracle.index_scores_fp8}.get(
        getattr(cfg, "index_format", "int8"), oracle.index_scores)
    s, e1 = score_fn(x["q_idx"], x["q_scale"], x["head_w"], x["idx_kv"], x["idx_scale"],
                     x["cmp_block_table"], x["query_start_loc"], x["positions"], T, cfg.ratio,
                     cfg.score_stride)
    idx, val, e2 = oracle.topk(s, x["positions"], cfg.ratio, T, cfg.k)
    sel = idx if topk_override is None else topk_override
    cmp_kv, win_kv = kv_sources(x, cfg)
    out, lse, e3 = oracle.sparse_attn(x["q"], rc, rs, cfg.rope_offset, cmp_kv,
                                      x["cmp_block_table"], sel, cfg.ratio, win_kv,
                                      x["win_block_table"], cfg.W, x["attn_sink"],
                                      cfg.softmax_scale, x["query_start_loc"], x["positions"], T)
    return dict(rope_cos=rc, rope_sin=rs, scores=s, topk_idx=idx, topk_val=val, out=out,
                lse=lse, err=e0 | e1 | e2 | e3 | ec, cmp_kv=x.get("cmp_kv"), state_cache=cst)


def bf16_to_f64(t) -> np.ndarray:
    a = t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp8_dot_tolerance(q_fp8, q_scale, head_w, idx_fp8, idx_scale, block_table,
                      query_start_loc, positions, num_tokens, ratio, score_stride):
    """Extra absolute score tolerance of the FP8 index plane (the INT8 plane's
    dots are exact).  gfx950's block-scaled FP8 MFMA sums each group of eight
    products in fixed point aligned to the group's largest product, keeping 13
    bits below that product's leading bit and truncating the rest (measured
    with single-MFMA probes: one 448 * 1 product beside seven products of
    2^-5 .. 2^-4 keeps them to multiples of 2^-5; seven of 2^-6 or less
    vanish).  A group's error is then below 8 * 2^-13 of its largest product,
    so a head's dot is off by at most 2^-10 * sum_i |q_i k_i|, plus
    Di * 2^-24 of it for the FP32 accumulation across groups.  Summed over
    the heads with |w qs ks|, that is the factor times the score of the
    absolute values, which the oracle computes on codes with their sign bits
    cleared."""
    Di = np.asarray(idx_fp8).shape[2]
    b, _ = oracle.index_scores_fp8(np.asarray(q_fp8) & 0x7F, np.abs(q_scale), np.abs(head_w),
                                   np.asarray(idx_fp8) & 0x7F, np.abs(idx_scale), block_table,
                                   query_start_loc, positions, num_tokens, ratio, score_stride)
    return np.where(np.isfinite(b), b * (2.0 ** -10 + Di * 2.0 ** -24), 0.0)


def check_scores(g: np.ndarray, o: np.ndarray, what="", extra_tol=None):
    """extra_tol: an absolute tolerance added per score (the FP8 plane's)."""
    assert g.shape == o.shape, (g.shape, o.shape)
    ninf_o = np.isneginf(o)
    assert np.array_equal(np.isneginf(g), ninf_o), f"{what}: -inf pattern differs"
    fin = ~ninf_o
    for t in range(o.shape[0]):
        f = fin[t]
        if not f.any():
            continue
        scale = np.max(np.abs(o[t, f]))
        d = np.abs(g[t, f] - o[t, f])
        tol = 1e-5 * np.abs(o[t, f]) + 2e-6 * scale
        if extra_tol is not None:
            tol = tol + extra_tol[t, f]
        bad = d > tol
        assert not bad.any(), (f"{what} row {t}: {bad.sum()} scores off; worst "
                               f"{np.max(d / np.maximum(tol, 1e-30)):.3g}x tolerance")


def check_topk(g_idx: np.ndarray, o_idx: np.ndarray, o_scores: np.ndarray, positions, ratio,
               what="", extra_tol=None):
    """Exact, or differing only at oracle ties within 1e-5 relative of the k-th
    score (plus, with extra_tol, twice the larger score tolerance of the two
    entries a swap exchanges)."""
    T, k = o_idx.shape
    assert g_idx.shape == o_idx.shape
    rows_equal = np.zeros(T, bool)
    for t in range(T):
        o = o_idx[t]
        g = g_idx[t]
        m = int((o >= 0).sum())
        assert np.all(g[m:] == -1), f"{what} row {t}: tail not -1"
        gs = g[:m]
        assert np.all(np.diff(gs) > 0), f"{what} row {t}: not ascending/unique"
        nv = oracle.visible_count(positions[t], ratio)
        assert np.all((gs >= 0) & (gs < nv)), f"{what} row {t}: ineligible index"
        if np.array_equal(g, o):
            rows_equal[t] = True
            continue
        sk = np.min(o_scores[t, o[:m]])  # the oracle's m-th best score
        diff = np.setxor1d(gs, o[:m])
        tie = 1e-5 * abs(sk)
        if extra_tol is not None:
            tie = tie + 2.0 * np.max(extra_tol[t, np.concatenate([diff, o[:m]])])
        assert np.all(np.abs(o_scores[t, diff] - sk) <= tie), (
            f"{what} row {t}: selection differs beyond ties ({len(diff)} entries)")
    return rows_equal


def check_attn(g_out, o_out, g_lse=None, o_lse=None, what=""):
    d = np.abs(g_out - o_out)
    tol = 1e-2 + 2e-2 * np.abs(o_out)
    bad = d > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outputs off; worst "
                           f"{np.max(d / tol):.3g}x tolerance")
    if g_lse is not None:
        dl = np.abs(g_lse - o_lse)
        tl = 1e-2 + 2e-2 * np.abs(o_lse)
        assert not (dl > tl).any(), f"{what}: lse off, worst {np.max(dl / tl):.3g}x"


def check_budgets(g, o, what=""):
    """The pages' per-row precision budget for attention outputs (pypto-lib
    "DeepSeek V4.1 Flash", "Compressor state ownership": every token's output
    row meets RMS(err) <= 1e-6 + 0.01 RMS(ref) and max|err| <= 1e-5 +
    0.05 RMS(ref); non-finite values fail).  A second check beside the
    elementwise tolerance."""
    g = np.asarray(g, np.float64).reshape(g.shape[0], -1)
    o = np.asarray(o, np.float64).reshape(o.shape[0], -1)
    assert np.isfinite(g).all(), f"{what}: non-finite outputs"
    rms_ref = np.sqrt(np.mean(o * o, axis=1))
    err = g - o
    rms_err = np.sqrt(np.mean(err * err, axis=1))
    peak = np.max(np.abs(err), axis=1)
    bad_rms = rms_err > 1e-6 + 0.01 * rms_ref
    bad_peak = peak > 1e-5 + 0.05 * rms_ref
    assert not bad_rms.any(), (f"{what}: rows {np.flatnonzero(bad_rms)[:8]} over the RMS "
                               f"budget; worst {np.max(rms_err / (1e-6 + 0.01 * rms_ref)):.3g}x")
    assert not bad_peak.any(), (f"{what}: rows {np.flatnonzero(bad_peak)[:8]} over the peak "
                                f"budget; worst {np.max(peak / (1e-5 + 0.05 * rms_ref)):.3g}x")
    return dict(rms=float(np.max(rms_err / (1e-6 + 0.01 * rms_ref))),
                peak=float(np.max(peak / (1e-5 + 0.05 * rms_ref))))


def rel_stats(g, o):
    """Diagnostics of the pages' precision budgets (per-row RMS / peak)."""
    g = g.reshape(g.shape[0], -1)
    o = o.reshape(o.shape[0], -1)
    rms_ref = np.sqrt(np.mean(o * o, axis=1))
    rms_err = np.sqrt(np.mean((g - o) ** 2, axis=1))
    peak = np.max(np.abs(g - o), axis=1)
    return dict(rms_ratio=float(np.max(rms_err / np.maximum(rms_ref, 1e-30))),
                peak_ratio=float(np.max(peak / np.maximum(rms_ref, 1e-30))))
