"""Device buffers for one CSA layer step and the calls that run it.

``CsaStep`` uploads host arrays (NumPy) once, allocates every output and
workspace up front, and then runs the path as four library calls on one
stream: RoPE rows -> indexer scores -> top-k -> sparse attention (RoPE rows ->
attention for the layers without an indexer), with the ratio-2 compressor's
publication after the RoPE rows when the step carries it.  Decode steps
gather the RoPE rows inside the attention launch instead, and the compressor
inside its own launch, so only prefill keeps the separate RoPE launch.  It only moves memory and passes pointers; all
arithmetic runs in libcsa.so.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import _lib

PAGE = _lib.PAGE

def _to_dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # BF16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


class CsaStep:
    def __init__(self, arrays: Dict[str, np.ndarray], *, ratio: int, k: int, window: int,
                 rope_offset: int, softmax_scale: float, num_tokens: Optional[int] = None,
                 prefill: bool = False, device: str = "cuda", with_values: bool = True,
                 with_lse: bool = True, shared: Optional[Dict[str, torch.Tensor]] = None,
                 mode: str = "csa", cand_kb: int = 0, cand_block: int = 8,
                 index_format: str = "int8", kv_format: str = "bf16", compress: bool = False,
                 rms_eps: float = 1e-6, fuse_rope: bool = True):
        # mode "csa": indexer scores and top-k select the compressed rows;
        # "hca": no indexer, every visible compressed row (k bounds them);
        # "swa": the window alone (k = 0); "reindex": scores and top-k only
        # inside the supplied candidate mask arrays["cand_blocks"];
        # "hier_full": the csa step, then the candidate mask of cand_kb blocks
        # of cand_block positions it publishes; "compress": the ratio-2
        # compressor's publication alone.  compress=True runs that
        # publication first in any mode (its rope rows share the rope launch).
        if mode not in ("csa", "hca", "swa", "reindex", "hier_full", "compress"):
            raise ValueError(f"unknown mode {mode!r}")
        if mode in ("reindex", "hier_full") and cand_kb < 1:
            raise ValueError(f"mode {mode!r} needs cand_kb >= 1")
        self.mode = mode
        if index_format not in ("int8", "mxfp4", "fp8"):
            raise ValueError(f"unknown index format {index_format!r}")
        if index_format != "int8" and mode == "reindex":
            raise ValueError("the reindex scorer takes the INT8 index plane")
        self.index_format = index_format
        # "bf16": arrays cmp_kv / win_kv; "mx": the low-bit planes cmp_fp4 +
        # cmp_scale and win_fp8 + win_scale (decode only)
        if kv_format not in ("bf16", "mx"):
            raise ValueError(f"unknown KV format {kv_format!r}")
        if kv_format == "mx" and prefill:
            raise ValueError("the low-bit KV planes have a decode entry point only")
        self.kv_format = kv_format
        self.ratio, self.k, self.window = int(ratio), int(k), int(window)
        self.rope_offset, self.softmax_scale = int(rope_offset), float(softmax_scale)
        self.prefill = prefill
        dev = torch.device(device)
        self.t: Dict[str, torch.Tensor] = {}
        for name, a in arrays.items():
            if shared is not None and name in shared:
                self.t[name] = shared[name]   # e.g. read-only RoPE tables reused by copies
            else:
                self.t[name] = _to_dev(a, dev)
        self.compress = bool(compress) or mode == "compress"
        if self.compress and (kv_format != "bf16" or ratio != 2):
            raise ValueError("the compressor publishes BF16 rows at ratio 2")
        self.rms_eps = float(rms_eps)
        # fuse_rope: the launches that use RoPE rows gather them from the full
        # tables themselves -- the decode attention (csa_sparse_attn_decode_rope
        # / _mx_rope, which also writes the query rows out) and the compressor
        # (csa_compress_pairs_rope) -- so no separate RoPE launch remains
        # except for prefill attention
        self.fuse_rope = bool(fuse_rope) and not prefill and mode != "compress"
        self.fuse_rope_cmp = bool(fuse_rope) and self.compress
        f32 = dict(dtype=torch.float32, device=dev)
        half = self.t["freqs_cos"].shape[1]
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        if mode == "compress":
            T, D = self.t["kv_proj"].shape
            self.T, self.H, self.D = T, 0, D
        else:
            T, H, D = self.t["q"].shape
            self.T, self.H, self.D = T, H, D
        self.num_tokens = T if num_tokens is None else int(num_tokens)
        # RoPE rows: the queries' rows, then (with the compressor) the rows of
        # each token's pair start; those that no fused launch gathers are
        # materialised by one launch when no row is padding
        need_q = mode != "compress" and not self.fuse_rope
        need_c = self.compress and not self.fuse_rope_cmp
        pos_ids = (([self.t["position_ids"]] if need_q else [])
                   + ([self.t["cmp_position_ids"]] if need_c else []))
        self.rope_pos = None
        if pos_ids:
            self.rope_pos = pos_ids[0] if len(pos_ids) == 1 else torch.cat(pos_ids)
            self.rope_all_cos = torch.empty((len(pos_ids) * T, half), **f32)
            self.rope_all_sin = torch.empty((len(pos_ids) * T, half), **f32)
        if need_q:
            self.rope_cos, self.rope_sin = self.rope_all_cos[:T], self.rope_all_sin[:T]
        elif mode != "compress":   # written by the fused attention
            self.rope_cos = torch.empty((T, half), **f32)
            self.rope_sin = torch.empty((T, half), **f32)
        if need_c:
            self.cmp_rope_cos, self.cmp_rope_sin = self.rope_all_cos[-T:], self.rope_all_sin[-T:]
        if mode == "compress":
            return
        q = self.t["q"]
        self.score_stride = self.t["cmp_block_table"].shape[1] * PAGE
        self.cand_kb, self.cand_block = int(cand_kb), int(cand_block)
        if mode == "reindex":
            # the scores of the mask's slots replace the full score rows
            self.score_stride = (self.cand_kb * self.cand_block + 3) // 4 * 4
            self.cand_blocks = self.t["cand_blocks"]
            self.cand_count = torch.empty((T,), dtype=torch.int32, device=dev)
        elif mode == "hier_full":
            self.cand_blocks = torch.empty((T, self.cand_kb), dtype=torch.int32, device=dev)
            cw = _lib.csa_candidate_blocks_workspace_bytes(T, self.score_stride, self.cand_block,
                                                           self.cand_kb)
            self.cand_ws = torch.empty(cw, dtype=torch.uint8, device=dev)
        self.scores = torch.empty((T, self.score_stride), **f32)
        self.topk_idx = torch.empty((T, self.k), dtype=torch.int32, device=dev)
        self.topk_val = torch.empty((T, self.k), **f32) if with_values else None
        self.out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((T, H), **f32) if with_lse else None
        tw = _lib.csa_topk_workspace_bytes(T, self.score_stride, self.k)
        self.topk_ws = torch.empty(tw, dtype=torch.uint8, device=dev) if tw else None
        if kv_format == "mx":
            aw = _lib.csa_sparse_attn_mx_workspace_bytes(T, H, D, self.k, self.window)
        else:
            aw = 0 if prefill else _lib.csa_sparse_attn_workspace_bytes(T, H, D, self.k,
                                                                        self.window)
        self.attn_ws = torch.empty(aw, dtype=torch.uint8, device=dev) if aw else None

    # ---- the four stages -------------------------------------------------
    def rope(self, stream=None):
        if self.rope_pos is None:   # every user gathers its own rows
            return
        T, n = self.T, self.rope_pos.shape[0]
        if self.num_tokens == T:
            _lib.csa_materialize_rope_rows(self.t["freqs_cos"], self.t["freqs_sin"],
                                           self.rope_pos, n, self.rope_all_cos,
                                           self.rope_all_sin, err=self.err, stream=stream)
            return
        for i in range(0, n, T):   # each part keeps its padding rows untouched
            _lib.csa_materialize_rope_rows(self.t["freqs_cos"], self.t["freqs_sin"],
                                           self.rope_pos[i:i + T], self.num_tokens,
                                           self.rope_all_cos[i:i + T],
                                           self.rope_all_sin[i:i + T], err=self.err,
                                           stream=stream)

    def compress_pairs(self, stream=None):
        """The ratio-2 compressor: every pair an odd row closes is published
        into cmp_kv, the state ring keeps the chunk's last rows."""
        t = self.t
        if self.fuse_rope_cmp:
            _lib.csa_compress_pairs_rope(
                t["kv_proj"], t["gate"], t["query_start_loc"], t["positions"], self.num_tokens,
                t["state_block_table"], t["state_cache"], t["rms_gamma"], self.rms_eps,
                t["freqs_cos"], t["freqs_sin"], t["cmp_position_ids"], self.rope_offset,
                t["cmp_kv"], t["cmp_block_table"], err=self.err, stream=stream)
            return
        _lib.csa_compress_pairs(t["kv_proj"], t["gate"], t["query_start_loc"], t["positions"],
                                self.num_tokens, t["state_block_table"], t["state_cache"],
                                t["rms_gamma"], self.rms_eps, self.cmp_rope_cos,
                                self.cmp_rope_sin, self.rope_offset, t["cmp_kv"],
                                t["cmp_block_table"], err=self.err, stream=stream)

    def index(self, stream=None):
        t = self.t
        if self.mode == "reindex":
            _lib.csa_index_score_candidates(
                t["q_idx"], t["q_scale"], t["head_w"], t["idx_kv"], t["idx_scale"],
                t["cmp_block_table"], t["query_start_loc"], t["positions"], self.num_tokens,
                self.ratio, self.cand_blocks, self.cand_block, self.scores, self.cand_count,
                err=self.err, stream=stream)
            return
        if self.index_format == "mxfp4":
            _lib.csa_index_score_mxfp4(t["q_idx"], t["q_scale"], t["head_w"], t["idx_kv"],
                                       t["idx_scale"], t["cmp_block_table"],
                                       t["query_start_loc"], t["positions"], self.num_tokens,
                                       self.ratio, self.scores, err=self.err, stream=stream)
            return
        if self.index_format == "fp8":
            _lib.csa_index_score_fp8(t["q_idx"], t["q_scale"], t["head_w"], t["idx_kv"],
                                     t["idx_scale"], t["cmp_block_table"], t["query_start_loc"],
                                     t["positions"], self.num_tokens, self.ratio, self.scores,
                                     err=self.err, stream=stream)
            return
        _lib.csa_index_score(t["q_idx"], t["q_scale"], t["head_w"], t["idx_kv"], t["idx_scale"],
                             t["cmp_block_table"], t["query_start_loc"], t["positions"],
                             self.num_tokens, self.ratio, self.scores, err=self.err,
                             stream=stream)

    def topk(self, stream=None):
        if self.mode == "reindex":
            _lib.csa_topk_candidates(self.scores, self.cand_count, self.cand_blocks,
                                     self.cand_block, self.num_tokens, self.k, self.topk_idx,
                                     self.topk_val, workspace=self.topk_ws, err=self.err,
                                     stream=stream)
            return
        _lib.csa_topk(self.scores, self.t["positions"], self.ratio, self.num_tokens, self.k,
                      self.topk_idx, self.topk_val, workspace=self.topk_ws, err=self.err,
                      stream=stream)

    def attn(self, stream=None, topk_idx: Optional[torch.Tensor] = None):
        t = self.t
        fn = _lib.csa_sparse_attn_prefill if self.prefill else _lib.csa_sparse_attn_decode
        if topk_idx is None and self.mode in ("csa", "reindex", "hier_full"):
            topk_idx = self.topk_idx
        if self.kv_format == "mx" and self.fuse_rope:
            _lib.csa_sparse_attn_decode_mx_rope(
                t["q"], t["freqs_cos"], t["freqs_sin"], t["position_ids"], self.rope_offset,
                t["cmp_fp4"], t["cmp_scale"], t["cmp_block_table"], topk_idx, self.ratio,
                t["win_fp8"], t["win_scale"], t["win_block_table"], self.window, t["attn_sink"],
                self.softmax_scale, t["query_start_loc"], t["positions"], self.num_tokens,
                self.out, lse=self.lse, rope_cos=self.rope_cos, rope_sin=self.rope_sin,
                workspace=self.attn_ws, err=self.err, stream=stream, k=self.k)
            return
        if self.kv_format == "mx":
            _lib.csa_sparse_attn_decode_mx(
                t["q"], self.rope_cos, self.rope_sin, self.rope_offset, t["cmp_fp4"],
                t["cmp_scale"], t["cmp_block_table"], topk_idx, self.ratio, t["win_fp8"],
                t["win_scale"], t["win_block_table"], self.window, t["attn_sink"],
                self.softmax_scale, t["query_start_loc"], t["positions"], self.num_tokens,
                self.out, lse=self.lse, workspace=self.attn_ws, err=self.err, stream=stream,
                k=self.k)
            return
        if self.fuse_rope:
            _lib.csa_sparse_attn_decode_rope(
                t["q"], t["freqs_cos"], t["freqs_sin"], t["position_ids"], self.rope_offset,
                t["cmp_kv"], t["cmp_block_table"], topk_idx, self.ratio, t["win_kv"],
                t["win_block_table"], self.window, t["attn_sink"], self.softmax_scale,
                t["query_start_loc"], t["positions"], self.num_tokens, self.out, lse=self.lse,
                rope_cos=self.rope_cos, rope_sin=self.rope_sin, workspace=self.attn_ws,
                err=self.err, stream=stream, k=self.k)
            return
        fn(t["q"], self.rope_cos, self.rope_sin, self.rope_offset, t["cmp_kv"],
           t["cmp_block_table"], topk_idx, self.ratio, t["win_kv"], t["win_block_table"],
           self.window, t["attn_sink"], self.softmax_scale, t["query_start_loc"],
           t["positions"], self.num_tokens, self.out, lse=self.lse, workspace=self.attn_ws,
           err=self.err, stream=stream, k=self.k)

    @property
    def stages(self):
        pre = (("rope",) if self.rope_pos is not None else ()) + (
            ("compress_pairs",) if self.compress else ())
        if self.mode == "compress":
            return pre
        if self.mode == "hier_full":
            return pre + ("index", "topk", "cand", "attn")
        if self.mode in ("csa", "reindex"):
            return pre + ("index", "topk", "attn")
        return pre + ("attn",)

    def inv_rope(self, stream=None, out=None):
        """The output's rope span rotated back by each row's angles (into
        `out`, by default a buffer of the step's own, leaving self.out as the
        attention result)."""
        if out is None:
            if getattr(self, "out_inv", None) is None:
                self.out_inv = torch.empty_like(self.out)
            out = self.out_inv
        _lib.csa_inverse_rope(self.out, out, self.rope_cos, self.rope_sin, self.rope_offset,
                              self.num_tokens, stream=stream)

    def cand(self, stream=None):
        """The candidate mask the full layer publishes (mode hier_full)."""
        _lib.csa_candidate_blocks(self.scores, self.t["positions"], self.ratio,
                                  self.num_tokens, self.cand_block, self.cand_blocks,
                                  self.cand_ws, err=self.err, stream=stream)

    def run(self, stream=None):
        for s in self.stages:
            getattr(self, s)(stream)


def step_for_config(cfg, arrays: Dict[str, np.ndarray], **kw) -> CsaStep:
    """CsaStep with the scalar parameters of a workload config."""
    return CsaStep(arrays, ratio=cfg.ratio, k=cfg.k, window=cfg.W, rope_offset=cfg.rope_offset,
                   softmax_scale=cfg.softmax_scale, prefill=(cfg.T > 256),
                   mode=getattr(cfg, "mode", "csa"), cand_kb=getattr(cfg, "cand_kb", 0),
                   cand_block=getattr(cfg, "cand_block", 8),
                   index_format=getattr(cfg, "index_format", "int8"),
                   kv_format=getattr(cfg, "kv_format", "bf16"),
                   compress=getattr(cfg, "compress", False),
                   rms_eps=getattr(cfg, "rms_eps", 1e-6), **kw)
