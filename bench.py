#!/usr/bin/env python3
"""Throughput of one CSA layer step on one MI355X.

A step is the whole hot path on one batch: RoPE rows -> INT8 indexer scores ->
top-k -> shared-KV sparse attention (four library calls on one stream).  The
default workload is the largest single-GPU decode configuration, the
max-context ratio-1 decode layer (8 rows = 2 requests x 4, 64 heads x 512,
1,048,576 compressed rows per request in 128-token pages, top-k 2048, window
128, about 5% heavy-tailed index-key outliers); --config picks another.

Timing: W untimed warmup steps, then exactly K steps bracketed by
torch.cuda.synchronize(); inputs are resident in HBM.  A step is one replay of
a captured HIP graph of the four calls.  To keep the layer's working set out
of the 256 MB Infinity Cache (as it would be when 40 layers run between two
steps of this one), successive steps rotate through enough independent copies
of the inputs to exceed 512 MiB.  Each stage's per-launch duration (for the
roofline) comes from HIP events around a graph of back-to-back launches of
that stage over the same rotating copies.

Prints ONE JSON line (rank 0).  --gpus N with N > 1 exits: this build runs on
one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense BF16 MFMA
INT8_PEAK_TOPS = 5000.0        # dense INT8 MFMA

KERNEL_SOURCES = {
    "rope": "csa_rope.hip", "index": "csa_index.hip", "topk": "csa_topk.hip",
    "attn": "csa_attn.hip", "cand": "csa_topk.hip", "compress_pairs": "csa_compress.hip",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c5",
                    help="c1..c15 (default c5: max-context ratio-1 decode)")
    ap.add_argument("--copies", type=int, default=0, help="input copies (0 = auto, cold L2/MALL)")
    ap.add_argument("--warm", action="store_true", help="one input copy (cache-warm timing)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy five times (the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE counts)")
    return ap.parse_args()


def copy_calibration():
    """Five plain device-to-device copies of 256 MiB: each reads and writes
    exactly 268,435,456 bytes, so FETCH_SIZE / WRITE_SIZE per dispatch of this
    copy give the counters' scale factor."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


# ---------------------------------------------------------------------------
# algorithmic bytes / flops (counting only; the pages' data movement per unit)
# ---------------------------------------------------------------------------

def visible(p, ratio):
    return max(0, (int(p) + 1) // ratio)


def compress_bytes(cfg, x):
    """The compressor's bytes: every token's FP32 KV projection and gate row
    once, each published BF16 row, the ring rows it reads (a chunk's odd first
    row) and writes (the chunk's last min(chunk, CAP) rows), the RMSNorm
    weights and each publishing row's rope row."""
    D, R, cap = cfg.D, cfg.R, cfg.state_capacity
    qsl = np.asarray(x["query_start_loc"])
    pos = np.asarray(x["positions"])
    pub = ring_rd = ring_wr = 0
    for b in range(len(qsl) - 1):
        lo, hi = int(qsl[b]), int(qsl[b + 1])
        if hi <= lo:
            continue
        pub += int(sum(1 for t in range(lo, hi) if pos[t] >= 0 and pos[t] % 2 == 1))
        ring_rd += int(pos[lo] >= 0 and pos[lo] % 2 == 1)
        ring_wr += int(sum(1 for t in range(max(lo, hi - cap), hi) if pos[t] >= 0))
    T = len(pos)
    return (8 * T * D + 2 * D * pub + 8 * D * (ring_rd + ring_wr) + 4 * D + 4 * R * pub
            + 4 * T)


def work_model(cfg, x, topk_idx: np.ndarray, fused_rope: bool = False):
    """Bytes each stage must move once, and the step total (decode formula:
    index keys of every visible position once per request, every unique
    gathered KV row once per request, Q, O, lse and small metadata; with the
    compressor, its bytes on top).  fused_rope: the attention launch gathers
    the query rope rows from the tables and writes them, and the compressor
    reads its table rows itself (no rope stage)."""
    T, H, D, R, Hi, Di, k = cfg.T, cfg.H, cfg.D, cfg.R, cfg.Hi, cfg.Di, cfg.k
    mode = getattr(cfg, "mode", "csa")
    if mode == "compress":   # the publication alone: rope rows of the pair starts, then it
        cb = compress_bytes(cfg, x)
        st = {"compress_pairs": cb} if fused_rope else {"rope": 8 * T * R + 4 * T,
                                                        "compress_pairs": cb}
        return dict(stage_bytes=st, step_bytes=cb, flops={}, kv_rows=0, kv_bytes=0,
                    idx_keys=0, pairs=0)
    qsl = np.asarray(x["query_start_loc"])
    pos = np.asarray(x["positions"])
    nv = np.array([visible(p, cfg.ratio) for p in pos])
    idx_keys = 0
    kv_rows = 0
    kv_bytes = 0   # KV bytes of those rows (window and compressed rows differ in the MX planes)
    win_rb, cmp_rb = cfg.kv_row_bytes
    pairs = 0
    scored = 0   # index scores written (score rows, or the mask's slots)
    kb, blk = getattr(cfg, "cand_kb", 0), getattr(cfg, "cand_block", 8)
    for b in range(len(qsl) - 1):
        rows = range(qsl[b], qsl[b + 1])
        if not len(rows):
            continue
        if mode in ("csa", "hier_full"):
            idx_keys += int(max(nv[t] for t in rows))
        elif mode == "reindex":   # every key of the request's candidate slots, once
            cand = np.asarray(x["cand_blocks"])
            keys = set()
            for t in rows:
                for c in cand[t]:
                    if c >= 0:
                        keys.update(range(int(c) * blk, min(int(nv[t]), (int(c) + 1) * blk)))
            idx_keys += len(keys)
        win, sel = set(), set()
        for t in rows:
            p = int(pos[t])
            w = list(range(max(0, p - cfg.W + 1), p + 1))
            if mode in ("csa", "reindex", "hier_full"):
                s = [int(c) for c in topk_idx[t] if c >= 0]
            elif mode == "hca":   # every visible compressed row, bounded by k
                s = list(range(min(int(nv[t]), k)))
            else:                 # swa: the window alone
                s = []
            win.update(w)
            sel.update(s)
            pairs += len(w) + len(s)
        kv_rows += len(win) + len(sel)
        kv_bytes += len(win) * win_rb + len(sel) * cmp_rb
    indexed = mode in ("csa", "reindex", "hier_full")
    kbytes = cfg.index_key_bytes           # one index key: payload + scales
    qbytes = kbytes + 4                     # one query head: payload + scales + weight
    q_side = T * Hi * qbytes if indexed else 0
    sel_bytes = 4 * T * k if indexed else 0   # the selection array the attention reads
    mask_bytes = 4 * T * kb if mode in ("reindex", "hier_full") else 0
    if mode == "reindex":
        scored = T * kb * blk
        ranked = 0
        for t in range(T):
            c = np.asarray(x["cand_blocks"])[t]
            ranked += sum(min(blk, max(0, int(nv[t]) - int(b) * blk)) for b in c if b >= 0)
    else:
        scored = T * cfg.score_stride
        ranked = int(nv.clip(max=cfg.score_stride).sum())
    st = {
        "rope": 8 * T * R + 4 * T,   # read + write cos and sin rows (R/2 FP32 each), positions
        "index": idx_keys * kbytes + q_side + 4 * scored + mask_bytes * (mode == "reindex"),
        "topk": 4 * ranked + 8 * T * k + mask_bytes * (mode == "reindex"),
        "attn": kv_bytes + 4 * T * H * D + 4 * T * H + sel_bytes + 4 * T * R,
    }
    if mode == "hier_full":   # block maxima over every visible score, then the mask
        st["cand"] = 4 * int(nv.clip(max=cfg.score_stride).sum()) + mask_bytes
    if not indexed:
        st = {"rope": st["rope"], "attn": st["attn"]}
    step = (idx_keys * kbytes + kv_bytes + 4 * T * H * D + 4 * T * H + q_side
            + 2 * sel_bytes + 4 * T * R + mask_bytes)
    if fused_rope:   # table rows read in place of rope rows; the rows written, position ids
        st["attn"] += 4 * T * R + 4 * T
        del st["rope"]
    if getattr(cfg, "compress", False):
        if "rope" in st:
            st["rope"] += 8 * T * R + 4 * T      # the pair starts' rope rows, same launch
        st["compress_pairs"] = compress_bytes(cfg, x)
        step += st["compress_pairs"]
    flops = {"attn": pairs * H * D * 4,
             "index": int(sum(nv[t] for t in range(T))) * Hi * Di * 2}
    return dict(stage_bytes=st, step_bytes=step, flops=flops, kv_rows=kv_rows,
                kv_bytes=kv_bytes, idx_keys=idx_keys, pairs=pairs)


def source_hash(name: str) -> str:
    p = os.path.join(ROOT, "compressed_sparse_attention_csa_amd", "csrc", KERNEL_SOURCES[name])
    h = hashlib.sha256()
    for q in (p, os.path.join(ROOT, "compressed_sparse_attention_csa_amd", "csrc",
                              "csa_common.h")):
        h.update(open(q, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(stage: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get("source_hash") != source_hash(stage):
        return None
    return d.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on host cores
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(cfg, x, budget_s: float):
    import oracle  # the cpu_baseline leg is the one place bench.py uses the oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = min(blas_threads, len(os.sched_getaffinity(0)))
    T = cfg.T
    mode = getattr(cfg, "mode", "csa")
    compress = getattr(cfg, "compress", False)

    def oracle_compress(sub, n, cmp_kv):
        rc = np.zeros((n, cfg.R // 2), np.float32)
        rs = np.zeros_like(rc)
        oracle.materialize_rope_rows(sub["freqs_cos"], sub["freqs_sin"], sub["cmp_position_ids"],
                                     n, rc, rs)
        return oracle.compress_pairs(sub["kv_proj"], sub["gate"], sub["query_start_loc"],
                                     sub["positions"], n, sub["state_block_table"],
                                     sub["state_cache"], sub["rms_gamma"], cfg.rms_eps, rc, rs,
                                     cfg.rope_offset, cmp_kv, sub["cmp_block_table"])[0]

    if mode == "compress":
        # sample: the whole chunk, repeated until the budget is spent
        done, t0 = 0, time.perf_counter()
        while True:
            oracle_compress(x, T, x["cmp_kv"])
            done += T
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
        return {"value": done / el, "unit": "rows/s", "cores": int(cores), "kind": "oracle",
                "cpu_model": cpu_model(),
                "sample": f"{done // T} x the whole {T}-token chunk (rope rows of the pair "
                          f"starts and the compressor, float64 NumPy) in {el:.1f} s"}
    # sample: whole rows of the workload; all of them when they fit the budget
    rows_per_call = T if T <= 16 else 16
    if compress and rows_per_call != T:
        raise ValueError("the compressor's baseline samples whole chunks")
    done_rows = 0
    t0 = time.perf_counter()
    stage = dict(rope=0.0, index=0.0, topk=0.0, attn=0.0)
    if mode == "hier_full":
        stage["cand"] = 0.0
    if compress:
        stage["compress_pairs"] = 0.0
    rng = np.random.default_rng(0)
    while True:
        rows = np.arange(T) if rows_per_call == T else np.sort(rng.choice(T, rows_per_call, False))
        qsl = np.asarray(x["query_start_loc"])
        owner = np.searchsorted(qsl, rows, side="right") - 1
        cnt = np.bincount(owner, minlength=len(qsl) - 1)
        sub = dict(x)
        sub["query_start_loc"] = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
        for key in ("q_idx", "q_scale", "head_w", "positions", "position_ids", "q", "cand_blocks"):
            if key in x:
                sub[key] = np.ascontiguousarray(np.asarray(x[key])[rows])
        n = len(rows)
        if compress:   # the publication first (whole chunks: rows_per_call == T)
            z = time.perf_counter()
            sub["cmp_kv"] = oracle_compress(sub, n, x["cmp_kv"])
            stage["compress_pairs"] += time.perf_counter() - z
        a = time.perf_counter()
        cand_before = stage.get("cand", 0.0)
        rc = np.zeros((n, cfg.R // 2), np.float32)
        rs = np.zeros_like(rc)
        oracle.materialize_rope_rows(sub["freqs_cos"], sub["freqs_sin"], sub["position_ids"], n,
                                     rc, rs)
        b_ = time.perf_counter()
        if mode in ("csa", "hier_full") and cfg.index_format == "fp8":
            s, _ = oracle.index_scores_fp8(sub["q_idx"], sub["q_scale"], sub["head_w"],
                                           sub["idx_kv"], sub["idx_scale"],
                                           sub["cmp_block_table"], sub["query_start_loc"],
                                           sub["positions"], n, cfg.ratio, cfg.score_stride)
            c_ = time.perf_counter()
            idx, _, _ = oracle.topk(s, sub["positions"], cfg.ratio, n, cfg.k)
        elif mode in ("csa", "hier_full") and cfg.index_format == "mxfp4":
            s, _ = oracle.index_scores_mxfp4(sub["q_idx"], sub["q_scale"], sub["head_w"],
                                             sub["idx_kv"], sub["idx_scale"],
                                             sub["cmp_block_table"], sub["query_start_loc"],
                                             sub["positions"], n, cfg.ratio, cfg.score_stride)
            c_ = time.perf_counter()
            idx, _, _ = oracle.topk(s, sub["positions"], cfg.ratio, n, cfg.k)
        elif mode in ("csa", "hier_full"):
            s, _ = oracle.index_scores(sub["q_idx"], sub["q_scale"], sub["head_w"], sub["idx_kv"],
                                       sub["idx_scale"], sub["cmp_block_table"],
                                       sub["query_start_loc"], sub["positions"], n, cfg.ratio,
                                       cfg.score_stride)
            c_ = time.perf_counter()
            idx, _, _ = oracle.topk(s, sub["positions"], cfg.ratio, n, cfg.k)
            if mode == "hier_full":
                m_ = time.perf_counter()
                oracle.candidate_blocks(s, sub["positions"], cfg.ratio, n, cfg.cand_block,
                                        cfg.cand_kb)
                stage["cand"] += time.perf_counter() - m_
        elif mode == "reindex":
            s, _ = oracle.index_scores_in_candidates(
                sub["q_idx"], sub["q_scale"], sub["head_w"], sub["idx_kv"], sub["idx_scale"],
                sub["cmp_block_table"], sub["query_start_loc"], sub["positions"], n, cfg.ratio,
                sub["cand_blocks"], cfg.cand_block)
            c_ = time.perf_counter()
            idx, _, _ = oracle.topk_in_candidates(s, sub["cand_blocks"], cfg.cand_block,
                                                  sub["positions"], cfg.ratio, n, cfg.k)
        else:   # hca: every visible compressed row; swa: no compressed row
            c_ = time.perf_counter()
            idx = None if mode == "hca" else np.zeros((n, 0), np.int32)
        d_ = time.perf_counter()
        if cfg.kv_format == "mx":   # the oracle dequantises the low-bit planes on read
            cmp_kv = oracle.mxfp4_e4m3_plane(sub["cmp_fp4"], sub["cmp_scale"])
            win_kv = oracle.mxfp8_plane(sub["win_fp8"], sub["win_scale"])
        else:
            cmp_kv, win_kv = sub["cmp_kv"], sub["win_kv"]
        oracle.sparse_attn(sub["q"], rc, rs, cfg.rope_offset, cmp_kv,
                           sub["cmp_block_table"], idx, cfg.ratio, win_kv,
                           sub["win_block_table"], cfg.W, sub["attn_sink"], cfg.softmax_scale,
                           sub["query_start_loc"], sub["positions"], n, k=cfg.k)
        e_ = time.perf_counter()
        stage["rope"] += b_ - a
        stage["index"] += c_ - b_
        stage["topk"] += d_ - c_ - (stage.get("cand", 0.0) - cand_before)
        stage["attn"] += e_ - d_
        done_rows += n
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done_rows / el, "unit": "rows/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done_rows} query rows of this workload ({rows_per_call} per oracle call, "
                      f"{'every stage' if mode in ('csa', 'reindex', 'hier_full') else 'rope rows and attention'}, "
                      f"float64 NumPy) in {el:.1f} s",
            "stage_seconds": {k: round(v, 3) for k, v in stage.items()
                              if mode in ("csa", "reindex", "hier_full")
                              or k in ("rope", "attn", "compress_pairs")}}


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs the CSA step on one GPU; --gpus {args.gpus} is not "
              "supported (the multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)
    import torch
    import synthetic
    import compressed_sparse_attention_csa_amd as csa

    cfg = synthetic.get(args.config)
    x = synthetic.make_inputs(cfg, seed=0).t
    shared_names = ("freqs_cos", "freqs_sin")
    first = csa.step_for_config(cfg, x)
    shared = {n: first.t[n] for n in shared_names}
    idx_touch = (cfg.T * cfg.cand_kb * cfg.cand_block if cfg.mode == "reindex"
                 else cfg.B * cfg.n_cmp_per_request)
    per_copy_touch = (idx_touch * cfg.index_key_bytes +
                      cfg.T * (cfg.k * cfg.kv_row_bytes[1] + cfg.W * cfg.kv_row_bytes[0]) +
                      4 * cfg.T * cfg.H * cfg.D)
    if cfg.mode == "compress":
        per_copy_touch = 9 * cfg.T * cfg.D
    if args.warm:
        copies = 1
    elif args.copies > 0:
        copies = args.copies
    else:
        copies = int(min(48, max(1, -(-(512 << 20) // max(per_copy_touch, 1)))))
    steps = [first] + [csa.step_for_config(cfg, x, shared=shared) for _ in range(copies - 1)]

    stages = first.stages
    for i in range(args.warmup):
        steps[i % copies].run()
    torch.cuda.synchronize()

    # one captured graph per input copy: a step is one graph replay, so host
    # launch overhead stays out of the step time (as under decode graph capture)
    cap = torch.cuda.Stream()
    graphs = []
    for st in steps:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            st.run()
        graphs.append(g)
    for i in range(max(2, args.warmup)):
        graphs[i % copies].replay()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # the same steps with one input copy: the working set stays in the
    # Infinity Cache (reported beside the cold figure, which is the value)
    ms_warm = None
    if copies > 1:
        for _ in range(2):
            graphs[0].replay()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for _ in range(args.steps):
            graphs[0].replay()
        torch.cuda.synchronize()
        ms_warm = (time.perf_counter() - w0) * 1e3 / args.steps

    # per-launch duration of each stage: a graph of back-to-back launches of
    # that stage over the rotating copies, timed with HIP events on the stream
    # the graph runs on
    stage_ms = {}
    reps = max(8, copies)
    for s in stages:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for i in range(reps):
                getattr(steps[i % copies], s)()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream()
        e0.record(stream)
        n_rep = 5
        for _ in range(n_rep):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        stage_ms[s] = e0.elapsed_time(e1) / (n_rep * reps)
    errs = [int(s.err.item()) for s in steps]
    topk_host = first.topk_idx.cpu().numpy() if cfg.mode != "compress" else None

    wm = work_model(cfg, x, topk_host, fused_rope=("rope" not in stages))
    rows = cfg.T
    value = rows / (ms_per_step / 1e3)
    step_gbs = wm["step_bytes"] / (ms_per_step / 1e3) / 1e9

    # dominant kernel: the stage with the largest share of the step
    dom = max(stages, key=lambda s: stage_ms[s])
    if dom == "attn" and cfg.T > 256:
        ach = wm["flops"]["attn"] / (stage_ms[dom] / 1e3) / 1e12
        roof = {"kernel": "attn_kernel (csa_sparse_attn_prefill)", "bound": "mfma",
                "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(dom, cfg.name),
                "algorithmic_per_launch": wm["flops"]["attn"], "avg_launch_ms": stage_ms[dom]}
    else:
        long_rows = cfg.score_stride > 32768
        if first.mode == "reindex":
            long_rows = first.score_stride > 32768
        split_ring = (not first.prefill and cfg.W + cfg.k >= 1024 and cfg.kv_format == "bf16")
        names = {"rope": "rope_rows_kernel",
                 "index": "index_cand_kernel" if first.mode == "reindex" else "index_score_kernel",
                 "topk": ("topk_sample_kernel + topk_filter_kernel + topk_final_kernel" if long_rows
                          else "topk_small_kernel"),
                 "cand": "block_max_kernel + top-k of the block scores",
                 "compress_pairs": "compress_pairs_kernel",
                 "attn": ("attn_kernel + attn_merge_kernel" if split_ring
                          else ("attn_decode_kernel (low-bit KV) + attn_merge_kernel"
                                if cfg.kv_format == "mx"
                                else "attn_decode_kernel + attn_merge_kernel"))}
        ach = wm["stage_bytes"][dom] / (stage_ms[dom] / 1e3) / 1e9
        roof = {"kernel": names[dom], "bound": "hbm", "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom, cfg.name),
                "algorithmic_per_launch": wm["stage_bytes"][dom], "avg_launch_ms": stage_ms[dom]}

    # the indexer's dot products against the matrix-core peak of its dtype
    # (the INT8 and FP8 planes 5 POPS dense, MXFP4 10): at C5 the kernel is
    # bound by its MFMAs and VALU epilogue together, so this figure sits
    # beside the HBM one
    compute_roof = None
    if first.mode in ("csa", "hier_full") and wm["flops"].get("index"):
        pk = 10000.0 if cfg.index_format == "mxfp4" else INT8_PEAK_TOPS
        ach_c = wm["flops"]["index"] / (stage_ms["index"] / 1e3) / 1e12
        compute_roof = {"kernel": "index_score_kernel", "bound": "mfma",
                        "achieved": round(ach_c, 1), "peak": pk, "unit": "TOP/s",
                        "frac": round(ach_c / pk, 4), "dtype": cfg.index_format,
                        "algorithmic_ops_per_launch": wm["flops"]["index"]}
    rec = {
        "metric": "CSA decode rows/s per layer + achieved HBM GB/s (% of MI355X peak)",
        "value": round(value, 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp32+bf16" if cfg.mode == "compress" else
                  {"mxfp4": "mxfp4+bf16", "fp8": "fp8+bf16"}.get(cfg.index_format, "int8+bf16")),
        "data": "synthetic",
        "config": {"workload": cfg.name, "rows": cfg.T, "requests": cfg.B, "heads": cfg.H,
                   "head_dim": cfg.D, "ratio": cfg.ratio, "top_k": cfg.k, "window": cfg.W,
                   "compressed_rows_per_request": cfg.n_cmp_per_request,
                   "kv_cache": ("window MXFP8 E4M3 + E8M0/32, compressed MXFP4 E2M1 + E4M3/16"
                                if cfg.kv_format == "mx" else "bf16"),
                   "indexer": ((f"{cfg.Hi}x{cfg.Di}" +
                                " " + cfg.index_format)
                               if first.mode in ("csa", "reindex", "hier_full") else "none"),
                   "compressor": ("ratio-2 publication, FP32 state ring of "
                                  f"{cfg.state_capacity}" if cfg.compress else "none"),
                   "selection": {"csa": "indexer top-k", "hca": "every visible compressed row",
                                 "compress": "none (the compressor alone)",
                                 "swa": "window only",
                                 "reindex": f"indexer top-k inside {cfg.cand_kb} candidate blocks "
                                            f"of {cfg.cand_block}",
                                 "hier_full": f"indexer top-k, publishing {cfg.cand_kb} candidate "
                                              f"blocks of {cfg.cand_block}"}[first.mode],
                   "input_copies": copies,
                   "cache": "warm" if copies == 1 else "cold (rotating copies > 512 MiB)"},
        "step_hbm": {"algorithmic_bytes": wm["step_bytes"], "achieved_gbs": round(step_gbs, 1),
                     "frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4)},
        "stage_ms": {s: round(v, 5) for s, v in stage_ms.items()},
        "ms_per_step_warm": None if ms_warm is None else round(ms_warm, 5),
        "stage_bytes_algorithmic": wm["stage_bytes"],
        "roofline": roof,
        "roofline_compute": compute_roof,
        "device_errors": errs[0],
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
