"""ctypes binding of libcsa.so (argument marshalling only).

Every function keeps the C entry point's name and semantics (see
``include/csa.h``); tensor arguments are torch tensors on the GPU, whose
shapes give the sizes the C call takes.  All arithmetic runs in the HIP
kernels; if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

PAGE = 128
EFLAG_POS_RANGE = 1
EFLAG_BLOCK_RANGE = 2
EFLAG_TOPK_RANGE = 4
EFLAG_META = 8

_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float

_SIGS = {
    "csa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "csa_materialize_rope_rows": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _I32, _I32, _P, _P, _P, _P]),
    "csa_index_score": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _P, _I32, _P, _P, _I32, _I32,
                                       _I32, _I32, _I32, _I32, _P, _I64, _P, _P]),
    "csa_topk_workspace_bytes": (_SZ, [_I32, _I64, _I32]),
    "csa_topk": (ctypes.c_int, [_P, _I64, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _SZ, _P, _P]),
    "csa_sparse_attn_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "csa_sparse_attn_decode": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _P, _I32, _P, _I32, _P, _I32,
                                              _I32, _P, _I32, _P, _I32, _I32, _P, _F32, _P, _P,
                                              _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _SZ, _P,
                                              _P]),
    "csa_index_score_mxfp4": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _P, _I32, _P, _P, _I32,
                                             _I32, _I32, _I32, _I32, _I32, _P, _I64, _P, _P]),
    "csa_candidate_blocks_workspace_bytes": (_SZ, [_I32, _I64, _I32, _I32]),
    "csa_candidate_blocks": (ctypes.c_int, [_P, _I64, _P, _I32, _I32, _I32, _I32, _I32, _P, _P,
                                            _SZ, _P, _P]),
    "csa_index_score_candidates": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _P, _I32, _P, _P,
                                                  _I32, _I32, _I32, _I32, _I32, _I32, _P, _I32,
                                                  _I32, _P, _I64, _P, _P, _P]),
    "csa_topk_candidates_workspace_bytes": (_SZ, [_I32, _I64, _I32]),
    "csa_topk_candidates": (ctypes.c_int, [_P, _I64, _P, _P, _I32, _I32, _I32, _I32, _I32, _P,
                                           _P, _P, _SZ, _P, _P]),
}
_SIGS["csa_sparse_attn_prefill"] = _SIGS["csa_sparse_attn_decode"]
_SIGS["csa_index_score_fp8"] = _SIGS["csa_index_score"]
_SIGS["csa_compress_pairs"] = (ctypes.c_int, [_P, _P, _I32, _P, _P, _I32, _I32, _I32, _P, _P,
                                              _I32, _I32, _P, _F32, _P, _P, _I32, _I32, _P, _I32,
                                              _P, _I32, _P, _P])
# the compressor's arguments with (freqs_cos, freqs_sin, table_capacity,
# rope_position_ids) in place of the rope rows
_SIGS["csa_compress_pairs_rope"] = (
    ctypes.c_int, _SIGS["csa_compress_pairs"][1][:14] + [_P, _P, _I32, _P]
    + _SIGS["csa_compress_pairs"][1][16:])
_SIGS["csa_inverse_rope"] = (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                            _P])
_SIGS["csa_sparse_attn_mx_workspace_bytes"] = _SIGS["csa_sparse_attn_workspace_bytes"]
# the decode arguments with a scale plane after each payload plane
_SIGS["csa_sparse_attn_decode_mx"] = (
    ctypes.c_int, _SIGS["csa_sparse_attn_decode"][1][:6] + [_P]
    + _SIGS["csa_sparse_attn_decode"][1][6:13] + [_P] + _SIGS["csa_sparse_attn_decode"][1][13:])
# the decode arguments with (freqs_cos, freqs_sin, table_capacity) in place
# of the rope rows, and the rope rows it writes after lse
_SIGS["csa_sparse_attn_decode_rope"] = (
    ctypes.c_int, [_P, _P, _P, _I32, _P] + _SIGS["csa_sparse_attn_decode"][1][3:28] + [_P, _P]
    + _SIGS["csa_sparse_attn_decode"][1][28:])
# the low-bit decode arguments with the same replacement
_SIGS["csa_sparse_attn_decode_mx_rope"] = (
    ctypes.c_int, [_P, _P, _P, _I32, _P] + _SIGS["csa_sparse_attn_decode_mx"][1][3:30] + [_P, _P]
    + _SIGS["csa_sparse_attn_decode_mx"][1][30:])
_SIGS["csa_sparse_attn_noalloc_max_bytes"] = (_SZ, [])
# the decode arguments without (workspace, workspace_bytes)
_SIGS["csa_sparse_attn_decode_noalloc"] = (
    ctypes.c_int, _SIGS["csa_sparse_attn_decode"][1][:28] + _SIGS["csa_sparse_attn_decode"][1][30:])

EXPORTS = tuple(_SIGS)


class CsaError(RuntimeError):
    pass


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcsa.so; raises when it is missing (the HIP path has no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise CsaError(f"{path} is missing: build it with __graft_entry__.build() "
                       "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise CsaError("tensor arguments must live on the GPU")
    if not t.is_contiguous():
        raise CsaError("tensor arguments must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = load().csa_status_string(status).decode()
        raise CsaError(f"{what}: {msg} ({status})")


def _need(t: torch.Tensor, dtypes, ndim: int, name: str):
    if t.dtype not in dtypes:
        raise CsaError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != ndim:
        raise CsaError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def csa_status_string(status: int) -> str:
    return load().csa_status_string(status).decode()


def csa_materialize_rope_rows(freqs_cos, freqs_sin, position_ids, num_tokens, rope_cos,
                              rope_sin, err=None, stream=None) -> None:
    _need(freqs_cos, (torch.float32,), 2, "freqs_cos")
    _need(rope_cos, (torch.float32,), 2, "rope_cos")
    st = load().csa_materialize_rope_rows(
        _ptr(freqs_cos), _ptr(freqs_sin), freqs_cos.shape[0], freqs_cos.shape[1],
        _ptr(position_ids), position_ids.shape[0], int(num_tokens), _ptr(rope_cos),
        _ptr(rope_sin), _ptr(err), _stream(stream))
    _check(st, "csa_materialize_rope_rows")


def csa_compress_pairs(kv_proj, gate, query_start_loc, positions, num_tokens, state_block_table,
                       state_cache, rms_gamma, rms_eps, rope_cos, rope_sin, rope_offset, cmp_kv,
                       cmp_block_table, err=None, stream=None) -> None:
    """Ratio-2 compressor publication into cmp_kv (BF16 [blocks, 128, D]) and
    the FP32 state ring state_cache [blocks, capacity, 2 D] (both in place)."""
    _need(kv_proj, (torch.float32,), 2, "kv_proj")
    _need(gate, (torch.float32,), 2, "gate")
    _need(state_cache, (torch.float32,), 3, "state_cache")
    _need(cmp_kv, _BF16, 3, "cmp_kv")
    T, D = kv_proj.shape
    if tuple(gate.shape) != (T, D) or state_cache.shape[2] != 2 * D or cmp_kv.shape[2] != D:
        raise CsaError("kv_proj, gate, state_cache and cmp_kv disagree on D")
    st = load().csa_compress_pairs(
        _ptr(kv_proj), _ptr(gate), D, _ptr(query_start_loc), _ptr(positions),
        query_start_loc.shape[0] - 1, T, int(num_tokens), _ptr(state_block_table),
        _ptr(state_cache), state_cache.shape[0], state_cache.shape[1], _ptr(rms_gamma),
        float(rms_eps), _ptr(rope_cos), _ptr(rope_sin), 2 * rope_cos.shape[1], int(rope_offset),
        _ptr(cmp_kv), cmp_kv.shape[0], _ptr(cmp_block_table), cmp_block_table.shape[1],
        _ptr(err), _stream(stream))
    _check(st, "csa_compress_pairs")


def csa_compress_pairs_rope(kv_proj, gate, query_start_loc, positions, num_tokens,
                            state_block_table, state_cache, rms_gamma, rms_eps, freqs_cos,
                            freqs_sin, rope_position_ids, rope_offset, cmp_kv, cmp_block_table,
                            err=None, stream=None) -> None:
    """csa_compress_pairs with each token's rope row taken from the full tables
    (FP32 [capacity, rope_dim / 2]) at rope_position_ids[t]."""
    _need(kv_proj, (torch.float32,), 2, "kv_proj")
    _need(gate, (torch.float32,), 2, "gate")
    _need(state_cache, (torch.float32,), 3, "state_cache")
    _need(cmp_kv, _BF16, 3, "cmp_kv")
    T, D = kv_proj.shape
    if tuple(gate.shape) != (T, D) or state_cache.shape[2] != 2 * D or cmp_kv.shape[2] != D:
        raise CsaError("kv_proj, gate, state_cache and cmp_kv disagree on D")
    half = _rope_tables_check(freqs_cos, freqs_sin, None, None, T)
    st = load().csa_compress_pairs_rope(
        _ptr(kv_proj), _ptr(gate), D, _ptr(query_start_loc), _ptr(positions),
        query_start_loc.shape[0] - 1, T, int(num_tokens), _ptr(state_block_table),
        _ptr(state_cache), state_cache.shape[0], state_cache.shape[1], _ptr(rms_gamma),
        float(rms_eps), _ptr(freqs_cos), _ptr(freqs_sin), freqs_cos.shape[0],
        _ptr(rope_position_ids), 2 * half, int(rope_offset), _ptr(cmp_kv), cmp_kv.shape[0],
        _ptr(cmp_block_table), cmp_block_table.shape[1], _ptr(err), _stream(stream))
    _check(st, "csa_compress_pairs_rope")


def csa_inverse_rope(inp, out, rope_cos, rope_sin, rope_offset, num_tokens, stream=None) -> None:
    """out (BF16 [T, H, D], may be inp) = inp with the rope span of each
    active row rotated by the conjugate of its rope row."""
    _need(inp, _BF16, 3, "in")
    _need(out, _BF16, 3, "out")
    T, H, D = inp.shape
    if tuple(out.shape) != (T, H, D):
        raise CsaError(f"out {tuple(out.shape)} does not match in {tuple(inp.shape)}")
    st = load().csa_inverse_rope(_ptr(inp), _ptr(out), _ptr(rope_cos), _ptr(rope_sin),
                                 2 * rope_cos.shape[1], int(rope_offset), T, int(num_tokens), H,
                                 D, _stream(stream))
    _check(st, "csa_inverse_rope")


def csa_index_score(q_idx, q_scale, head_w, idx_kv, idx_scale, block_table, query_start_loc,
                    positions, num_tokens, ratio, scores, err=None, stream=None) -> None:
    _need(q_idx, (torch.int8,), 3, "q_idx")
    _need(idx_kv, (torch.int8,), 3, "idx_kv")
    _need(scores, (torch.float32,), 2, "scores")
    T, Hi, Di = q_idx.shape
    st = load().csa_index_score(
        _ptr(q_idx), _ptr(q_scale), _ptr(head_w), _ptr(idx_kv), _ptr(idx_scale),
        idx_kv.shape[0], _ptr(block_table), block_table.shape[1], _ptr(query_start_loc),
        _ptr(positions), query_start_loc.shape[0] - 1, T, int(num_tokens), Hi, Di, int(ratio),
        _ptr(scores), scores.shape[1], _ptr(err), _stream(stream))
    _check(st, "csa_index_score")


def csa_index_score_mxfp4(q_fp4, q_sc, head_w, idx_fp4, idx_sc, block_table, query_start_loc,
                          positions, num_tokens, ratio, scores, err=None, stream=None) -> None:
    _need(q_fp4, (torch.uint8,), 3, "q_fp4")
    _need(idx_fp4, (torch.uint8,), 3, "idx_fp4")
    _need(scores, (torch.float32,), 2, "scores")
    T, Hi, Db = q_fp4.shape
    st = load().csa_index_score_mxfp4(
        _ptr(q_fp4), _ptr(q_sc), _ptr(head_w), _ptr(idx_fp4), _ptr(idx_sc), idx_fp4.shape[0],
        _ptr(block_table), block_table.shape[1], _ptr(query_start_loc), _ptr(positions),
        query_start_loc.shape[0] - 1, T, int(num_tokens), Hi, 2 * Db, int(ratio), _ptr(scores),
        scores.shape[1], _ptr(err), _stream(stream))
    _check(st, "csa_index_score_mxfp4")


def csa_index_score_fp8(q_fp8, q_scale, head_w, idx_fp8, idx_scale, block_table,
                        query_start_loc, positions, num_tokens, ratio, scores, err=None,
                        stream=None) -> None:
    _need(q_fp8, (torch.uint8,), 3, "q_fp8")
    _need(idx_fp8, (torch.uint8,), 3, "idx_fp8")
    _need(scores, (torch.float32,), 2, "scores")
    T, Hi, Di = q_fp8.shape
    st = load().csa_index_score_fp8(
        _ptr(q_fp8), _ptr(q_scale), _ptr(head_w), _ptr(idx_fp8), _ptr(idx_scale),
        idx_fp8.shape[0], _ptr(block_table), block_table.shape[1], _ptr(query_start_loc),
        _ptr(positions), query_start_loc.shape[0] - 1, T, int(num_tokens), Hi, Di, int(ratio),
        _ptr(scores), scores.shape[1], _ptr(err), _stream(stream))
    _check(st, "csa_index_score_fp8")


def csa_topk_workspace_bytes(T: int, score_stride: int, k: int) -> int:
    return int(load().csa_topk_workspace_bytes(T, score_stride, k))


def csa_topk(scores, positions, ratio, num_tokens, k, topk_idx, topk_val=None, workspace=None,
             err=None, stream=None) -> None:
    _need(scores, (torch.float32,), 2, "scores")
    _need(topk_idx, (torch.int32,), 2, "topk_idx")
    T = scores.shape[0]
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().csa_topk(_ptr(scores), scores.shape[1], _ptr(positions), int(ratio), T,
                         int(num_tokens), int(k), _ptr(topk_idx), _ptr(topk_val),
                         _ptr(workspace), wsb, _ptr(err), _stream(stream))
    _check(st, "csa_topk")


def csa_candidate_blocks_workspace_bytes(T: int, score_stride: int, block: int, kb: int) -> int:
    return int(load().csa_candidate_blocks_workspace_bytes(T, score_stride, block, kb))


def csa_candidate_blocks(scores, positions, ratio, num_tokens, block, cand_blocks, workspace,
                         err=None, stream=None) -> None:
    _need(scores, (torch.float32,), 2, "scores")
    _need(cand_blocks, (torch.int32,), 2, "cand_blocks")
    T = scores.shape[0]
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().csa_candidate_blocks(_ptr(scores), scores.shape[1], _ptr(positions), int(ratio),
                                     T, int(num_tokens), int(block), cand_blocks.shape[1],
                                     _ptr(cand_blocks), _ptr(workspace), wsb, _ptr(err),
                                     _stream(stream))
    _check(st, "csa_candidate_blocks")


def csa_index_score_candidates(q_idx, q_scale, head_w, idx_kv, idx_scale, block_table,
                               query_start_loc, positions, num_tokens, ratio, cand_blocks,
                               block, cand_scores, cand_count, err=None, stream=None) -> None:
    _need(q_idx, (torch.int8,), 3, "q_idx")
    _need(idx_kv, (torch.int8,), 3, "idx_kv")
    _need(cand_blocks, (torch.int32,), 2, "cand_blocks")
    _need(cand_scores, (torch.float32,), 2, "cand_scores")
    _need(cand_count, (torch.int32,), 1, "cand_count")
    T, Hi, Di = q_idx.shape
    st = load().csa_index_score_candidates(
        _ptr(q_idx), _ptr(q_scale), _ptr(head_w), _ptr(idx_kv), _ptr(idx_scale),
        idx_kv.shape[0], _ptr(block_table), block_table.shape[1], _ptr(query_start_loc),
        _ptr(positions), query_start_loc.shape[0] - 1, T, int(num_tokens), Hi, Di, int(ratio),
        _ptr(cand_blocks), cand_blocks.shape[1], int(block), _ptr(cand_scores),
        cand_scores.shape[1], _ptr(cand_count), _ptr(err), _stream(stream))
    _check(st, "csa_index_score_candidates")


def csa_topk_candidates_workspace_bytes(T: int, cand_stride: int, k: int) -> int:
    return int(load().csa_topk_candidates_workspace_bytes(T, cand_stride, k))


def csa_topk_candidates(cand_scores, cand_count, cand_blocks, block, num_tokens, k, topk_idx,
                        topk_val=None, workspace=None, err=None, stream=None) -> None:
    _need(cand_scores, (torch.float32,), 2, "cand_scores")
    _need(cand_blocks, (torch.int32,), 2, "cand_blocks")
    _need(topk_idx, (torch.int32,), 2, "topk_idx")
    T = cand_scores.shape[0]
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().csa_topk_candidates(_ptr(cand_scores), cand_scores.shape[1], _ptr(cand_count),
                                    _ptr(cand_blocks), cand_blocks.shape[1], int(block), T,
                                    int(num_tokens), int(k), _ptr(topk_idx), _ptr(topk_val),
                                    _ptr(workspace), wsb, _ptr(err), _stream(stream))
    _check(st, "csa_topk_candidates")


def csa_sparse_attn_workspace_bytes(T: int, H: int, D: int, k: int, window: int) -> int:
    return int(load().csa_sparse_attn_workspace_bytes(T, H, D, k, window))


def _attn(fn_name, q, rope_cos, rope_sin, rope_offset, cmp_kv, cmp_block_table, topk_idx, ratio,
          win_kv, win_block_table, window, attn_sink, softmax_scale, query_start_loc, positions,
          num_tokens, out, lse=None, workspace=None, err=None, stream=None, k=None,
          noalloc=False):
    """topk_idx None selects every visible compressed row, with k (required
    then) bounding their count; k = 0 attends over the window alone, and the
    compressed pool and table may then be None."""
    _need(q, _BF16, 3, "q")
    _need(out, _BF16, 3, "out")
    T, H, D = q.shape
    if topk_idx is not None:
        k = topk_idx.shape[1]
    elif k is None:
        raise CsaError("k is required when topk_idx is None")
    rope_dim = 2 * rope_cos.shape[1]
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [
        _ptr(q), _ptr(rope_cos), _ptr(rope_sin), rope_dim, int(rope_offset), _ptr(cmp_kv),
        0 if cmp_kv is None else cmp_kv.shape[0], _ptr(cmp_block_table),
        0 if cmp_block_table is None else cmp_block_table.shape[1], _ptr(topk_idx), int(k),
        int(ratio), _ptr(win_kv), win_kv.shape[0], _ptr(win_block_table),
        win_block_table.shape[1], int(window), _ptr(attn_sink), float(softmax_scale),
        _ptr(query_start_loc), _ptr(positions), query_start_loc.shape[0] - 1, T,
        int(num_tokens), H, D, _ptr(out), _ptr(lse)]
    args += [_ptr(err), _stream(stream)] if noalloc else [_ptr(workspace), wsb, _ptr(err),
                                                          _stream(stream)]
    st = getattr(load(), fn_name)(*args)
    _check(st, fn_name)


def csa_sparse_attn_decode(*args, **kw) -> None:
    _attn("csa_sparse_attn_decode", *args, **kw)


def _rope_tables_check(freqs_cos, freqs_sin, rope_cos, rope_sin, T):
    """Full RoPE tables FP32 [capacity, half]; rope rows FP32 [T, half] or None."""
    _need(freqs_cos, (torch.float32,), 2, "freqs_cos")
    _need(freqs_sin, (torch.float32,), 2, "freqs_sin")
    half = freqs_cos.shape[1]
    if tuple(freqs_sin.shape) != tuple(freqs_cos.shape):
        raise CsaError("freqs_cos and freqs_sin differ in shape")
    for name, r in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        if r is not None:
            _need(r, (torch.float32,), 2, name)
            if tuple(r.shape) != (T, half):
                raise CsaError(f"{name}: expected {(T, half)}, got {tuple(r.shape)}")
    return half


def csa_sparse_attn_decode_rope(q, freqs_cos, freqs_sin, position_ids, rope_offset, cmp_kv,
                                cmp_block_table, topk_idx, ratio, win_kv, win_block_table, window,
                                attn_sink, softmax_scale, query_start_loc, positions, num_tokens,
                                out, lse=None, rope_cos=None, rope_sin=None, workspace=None,
                                err=None, stream=None, k=None) -> None:
    """csa_sparse_attn_decode that gathers each row's rope row (table row
    position_ids[t] of freqs_cos / freqs_sin, FP32 [capacity, rope_dim / 2])
    itself and, when rope_cos / rope_sin (FP32 [T, rope_dim / 2]) are given,
    writes them as csa_materialize_rope_rows would."""
    _need(q, _BF16, 3, "q")
    _need(out, _BF16, 3, "out")
    T, H, D = q.shape
    half = _rope_tables_check(freqs_cos, freqs_sin, rope_cos, rope_sin, T)
    if topk_idx is not None:
        k = topk_idx.shape[1]
    elif k is None:
        raise CsaError("k is required when topk_idx is None")
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().csa_sparse_attn_decode_rope(
        _ptr(q), _ptr(freqs_cos), _ptr(freqs_sin), freqs_cos.shape[0], _ptr(position_ids),
        2 * half,
        int(rope_offset), _ptr(cmp_kv), 0 if cmp_kv is None else cmp_kv.shape[0],
        _ptr(cmp_block_table), 0 if cmp_block_table is None else cmp_block_table.shape[1],
        _ptr(topk_idx), int(k), int(ratio), _ptr(win_kv), win_kv.shape[0], _ptr(win_block_table),
        win_block_table.shape[1], int(window), _ptr(attn_sink), float(softmax_scale),
        _ptr(query_start_loc), _ptr(positions), query_start_loc.shape[0] - 1, T,
        int(num_tokens), H, D, _ptr(out), _ptr(lse), _ptr(rope_cos), _ptr(rope_sin),
        _ptr(workspace), wsb, _ptr(err), _stream(stream))
    _check(st, "csa_sparse_attn_decode_rope")


def csa_sparse_attn_noalloc_max_bytes() -> int:
    return int(load().csa_sparse_attn_noalloc_max_bytes())


def csa_sparse_attn_decode_noalloc(*args, **kw) -> None:
    """csa_sparse_attn_decode with the library's static scratch instead of a
    workspace (no workspace argument)."""
    if kw.get("workspace") is not None:
        raise CsaError("csa_sparse_attn_decode_noalloc takes no workspace")
    kw.pop("workspace", None)
    _attn("csa_sparse_attn_decode_noalloc", *args, noalloc=True, **kw)


def csa_sparse_attn_prefill(*args, **kw) -> None:
    _attn("csa_sparse_attn_prefill", *args, **kw)


def csa_sparse_attn_mx_workspace_bytes(T: int, H: int, D: int, k: int, window: int) -> int:
    return int(load().csa_sparse_attn_mx_workspace_bytes(T, H, D, k, window))


def _mx_planes(q, out, cmp_fp4, cmp_scale, win_fp8, win_scale):
    _need(q, _BF16, 3, "q")
    _need(out, _BF16, 3, "out")
    _need(win_fp8, (torch.uint8,), 3, "win_fp8")
    _need(win_scale, (torch.uint8,), 3, "win_scale")
    T, H, D = q.shape
    if win_fp8.shape[2] != D or tuple(win_scale.shape) != (win_fp8.shape[0], PAGE, D // 32):
        raise CsaError(f"window planes {tuple(win_fp8.shape)} / {tuple(win_scale.shape)} do not "
                       f"match D = {D}")
    if cmp_fp4 is not None:
        _need(cmp_fp4, (torch.uint8,), 3, "cmp_fp4")
        _need(cmp_scale, (torch.uint8,), 3, "cmp_scale")
        if (cmp_fp4.shape[2] != D // 2
                or tuple(cmp_scale.shape) != (cmp_fp4.shape[0], PAGE, D // 16)):
            raise CsaError(f"compressed planes {tuple(cmp_fp4.shape)} / "
                           f"{tuple(cmp_scale.shape)} do not match D = {D}")
    return T, H, D


def _mx_tail(cmp_fp4, cmp_scale, cmp_block_table, topk_idx, k, ratio, win_fp8, win_scale,
             win_block_table, window, attn_sink, softmax_scale, query_start_loc, positions, T,
             num_tokens, H, D):
    """The arguments from cmp_fp4 to D, shared by both low-bit decode calls."""
    if topk_idx is not None:
        k = topk_idx.shape[1]
    elif k is None:
        raise CsaError("k is required when topk_idx is None")
    return [_ptr(cmp_fp4), _ptr(cmp_scale), 0 if cmp_fp4 is None else cmp_fp4.shape[0],
            _ptr(cmp_block_table), 0 if cmp_block_table is None else cmp_block_table.shape[1],
            _ptr(topk_idx), int(k), int(ratio), _ptr(win_fp8), _ptr(win_scale), win_fp8.shape[0],
            _ptr(win_block_table), win_block_table.shape[1], int(window), _ptr(attn_sink),
            float(softmax_scale), _ptr(query_start_loc), _ptr(positions),
            query_start_loc.shape[0] - 1, T, int(num_tokens), H, D]


def csa_sparse_attn_decode_mx(q, rope_cos, rope_sin, rope_offset, cmp_fp4, cmp_scale,
                              cmp_block_table, topk_idx, ratio, win_fp8, win_scale,
                              win_block_table, window, attn_sink, softmax_scale, query_start_loc,
                              positions, num_tokens, out, lse=None, workspace=None, err=None,
                              stream=None, k=None) -> None:
    """Decode attention over the low-bit KV planes: cmp_fp4 uint8 [blocks, 128,
    D/2] with cmp_scale uint8 [blocks, 128, D/16] (E4M3), win_fp8 uint8
    [blocks, 128, D] with win_scale uint8 [blocks, 128, D/32] (E8M0).  The
    other arguments are csa_sparse_attn_decode's."""
    T, H, D = _mx_planes(q, out, cmp_fp4, cmp_scale, win_fp8, win_scale)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().csa_sparse_attn_decode_mx(
        _ptr(q), _ptr(rope_cos), _ptr(rope_sin), 2 * rope_cos.shape[1], int(rope_offset),
        *_mx_tail(cmp_fp4, cmp_scale, cmp_block_table, topk_idx, k, ratio, win_fp8, win_scale,
                  win_block_table, window, attn_sink, softmax_scale, query_start_loc, positions,
                  T, num_tokens, H, D),
        _ptr(out), _ptr(lse), _ptr(workspace), wsb, _ptr(err), _stream(stream))
    _check(st, "csa_sparse_attn_decode_mx")


def csa_sparse_attn_decode_mx_rope(q, freqs_cos, freqs_sin, position_ids, rope_offset, cmp_fp4,
                                   cmp_scale, cmp_block_table, topk_idx, ratio, win_fp8,
                                   win_scale, win_block_table, window, attn_sink, softmax_scale,
                                   query_start_loc, positions, num_tokens, out, lse=None,
                                   rope_cos=None, rope_sin=None, workspace=None, err=None,
                                   stream=None, k=None) -> None:
    """csa_sparse_attn_decode_mx gathering each row's rope row from the full
    tables (as csa_sparse_attn_decode_rope), writing them to rope_cos /
    rope_sin when given."""
    T, H, D = _mx_planes(q, out, cmp_fp4, cmp_scale, win_fp8, win_scale)
    half = _rope_tables_check(freqs_cos, freqs_sin, rope_cos, rope_sin, T)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().csa_sparse_attn_decode_mx_rope(
        _ptr(q), _ptr(freqs_cos), _ptr(freqs_sin), freqs_cos.shape[0], _ptr(position_ids),
        2 * half, int(rope_offset),
        *_mx_tail(cmp_fp4, cmp_scale, cmp_block_table, topk_idx, k, ratio, win_fp8, win_scale,
                  win_block_table, window, attn_sink, softmax_scale, query_start_loc, positions,
                  T, num_tokens, H, D),
        _ptr(out), _ptr(lse), _ptr(rope_cos), _ptr(rope_sin), _ptr(workspace), wsb, _ptr(err),
        _stream(stream))
    _check(st, "csa_sparse_attn_decode_mx_rope")
