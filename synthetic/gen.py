"""Seeded synthetic inputs for one CSA layer step (shared by the oracle tests,
the GPU parity tests, smoke() and the benchmark).

Everything is drawn on the host with NumPy PCG64.  Each tensor owns its own
stream, ``SeedSequence(seed, spawn_key=(tensor_id, chunk))``, so adding a tensor
or changing the chunking of another never changes the bytes of this one.

Distributions follow the tiny decode config of the workload list and are reused
for the larger ones:

* Q and KV rows: float32 N(0,1) rounded to BF16 (round-to-nearest-even), kept as
  raw uint16 bit patterns.
* indexer keys: integers uniform on [-127, 127]; per-row FP32 key scales
  U(0.005, 0.02); with ``outlier_frac`` > 0 each compressed position is an
  outlier with that probability and its key scale is multiplied by 4.
* FP8 index plane (``index_format`` "fp8"): key and query E4M3 codes drawn
  like the window plane's below (exponent field 4..10, never NaN), the INT8
  plane's FP32 key scales, query scales U(0.01, 0.05).
* indexer query: float32 N(0,1) quantised per (row, head) to INT8 with the
  per-token amax rule of pypto-lib "DeepSeek V4-Flash, MTP point", section
  "What is quantized" (amax floored at 1e-4, mapped to 127).  This is input
  shaping upstream of the scorer, which receives the INT8 codes and scales.
* per-head weights N(0,1)/2, attention sinks N(0,1).
* block tables: a seeded permutation of one pool's blocks.  The window pool
  only holds the pages that some window touches; every other table entry is -1.
* RoPE tables: FP32 half-width [capacity, R/2], angle = pos * theta^(-2i/R)
  evaluated in float64 (no YaRN).  Tables are caller inputs of the path.
* low-bit KV planes (``kv_format`` "mx"), codes drawn directly, no quantiser:
  window E4M3 codes with uniform sign and mantissa and exponent field 4..10
  (magnitudes 2^-3 .. 2^3 times 1 + m/8, never NaN) beside E8M0 bytes
  122..125 (2^-5 .. 2^-2); compressed packed E2M1 bytes uniform over all 256
  (every nibble uniform over the 16 codes) beside positive E4M3 scales with
  exponent field 3..6 (2^-4 .. 2^-1 times 1 + m/8).  The dequantised values
  have an RMS near 0.6 (window) and 1.0 (compressed), the scale of the BF16
  rows.  These planes replace the BF16 pools.
* compressor inputs (``compress``): FP32 KV projections and gate scores
  N(0,1) per token, an FP32 state ring N(0,1) (the tokens before the chunk),
  state blocks a seeded permutation of one per request, RMSNorm weights
  U(0.5, 1.5), and the rope positions the caller gives the compressor: each
  token's pair start (its position rounded down to even), -1 for negative
  positions.

No arithmetic of the method (scores, selection, attention, rotation) lives here.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict

import numpy as np

from .configs import PAGE, CsaConfig

_TENSOR_IDS = {
    "q": 1, "cmp_kv": 2, "win_kv": 3, "q_idx_f": 4, "head_w": 5, "idx_kv": 6,
    "idx_scale": 7, "outlier": 8, "attn_sink": 9, "cmp_perm": 10, "win_perm": 11,
    "cand_blocks": 12, "q_fp4": 13, "q_e8m0": 14, "idx_fp4": 15, "idx_e8m0": 16,
    "win_fp8_bits": 17, "win_fp8_exp": 18, "win_e8m0": 19, "cmp_fp4": 20, "cmp_sc_m": 21,
    "cmp_sc_e": 22, "idx_fp8_bits": 23, "idx_fp8_exp": 24, "q_fp8_bits": 25, "q_fp8_exp": 26,
    "q_fp8_scale": 27, "kv_proj": 28, "gate": 29, "state_cache": 30, "state_perm": 31,
    "rms_gamma": 32,
}

_CHUNK_ELEMS = 1 << 24  # fixed chunk so the draws never depend on the caller


def _rng(seed: int, name: str, chunk: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(_TENSOR_IDS[name], chunk))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite normal draws, so no NaN handling is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + bias) >> 16).astype(np.uint16)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _bf16_normal(seed: int, name: str, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def fill(ci: int) -> None:
        s = ci * _CHUNK_ELEMS
        e = min(n, s + _CHUNK_ELEMS)
        g = _rng(seed, name, ci)
        out[s:e] = f32_to_bf16_bits(g.standard_normal(e - s, dtype=np.float32))

    nchunks = -(-n // _CHUNK_ELEMS)
    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _u8_uniform(seed: int, name: str, shape, lo: int, hi: int) -> np.ndarray:
    """uint8 integers uniform on [lo, hi], drawn in fixed chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)

    def fill(ci: int) -> None:
        s = ci * _CHUNK_ELEMS
        e = min(n, s + _CHUNK_ELEMS)
        out[s:e] = _rng(seed, name, ci).integers(lo, hi + 1, size=e - s, dtype=np.uint8)

    nchunks = -(-n // _CHUNK_ELEMS)
    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def quantize_rows_int8(x: np.ndarray):
    """Per-row symmetric INT8: scale = max(amax, 1e-4) / 127, code = RNE(x/scale)
    clipped to [-127, 127].  Returns (codes int8, scale float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (np.maximum(amax, np.float32(1e-4)) / np.float32(127.0)).astype(np.float32)
    codes = np.clip(np.rint(x / scale[..., None]), -127, 127).astype(np.int8)
    return codes, scale


def rope_tables(capacity: int, rope_dim: int, theta: float):
    """Caller-owned FP32 half-width cos/sin tables, [capacity, rope_dim/2]."""
    half = rope_dim // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / rope_dim)
    ang = np.arange(capacity, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@dataclasses.dataclass
class CsaInputs:
    cfg: CsaConfig
    t: Dict[str, np.ndarray]

    def __getitem__(self, k):
        return self.t[k]


def _f32_normal(seed: int, name: str, shape) -> np.ndarray:
    return _rng(seed, name).standard_normal(shape, dtype=np.float32)


def _compressor_inputs(t: Dict[str, np.ndarray], cfg: CsaConfig, seed: int, pos: np.ndarray):
    T, B, D = cfg.T, cfg.B, cfg.D
    t["kv_proj"] = _f32_normal(seed, "kv_proj", (T, D))
    t["gate"] = _f32_normal(seed, "gate", (T, D))
    t["state_cache"] = _f32_normal(seed, "state_cache", (B, cfg.state_capacity, 2 * D))
    t["state_block_table"] = _rng(seed, "state_perm").permutation(B).astype(np.int32)
    t["rms_gamma"] = _rng(seed, "rms_gamma").uniform(0.5, 1.5, D).astype(np.float32)
    t["cmp_position_ids"] = np.where(pos >= 0, pos - pos % 2, -1).astype(np.int32)


def make_inputs(cfg: CsaConfig, seed: int = 0, with_tables: bool = True) -> CsaInputs:
    T, B, H, D, R = cfg.T, cfg.B, cfg.H, cfg.D, cfg.R
    Hi, Di = cfg.Hi, cfg.Di
    t: Dict[str, np.ndarray] = {}

    qsl = np.asarray(cfg.query_start_loc, dtype=np.int32)
    pos = np.asarray(cfg.flat_positions, dtype=np.int32)
    rope_pos = pos.copy()
    for b in range(B):
        for off in cfg.rope_neg_rows:
            if off < cfg.rows_per_request[b]:
                rope_pos[qsl[b] + off] = -1
    t["query_start_loc"] = qsl
    t["positions"] = pos
    t["position_ids"] = rope_pos

    if with_tables:
        t["freqs_cos"], t["freqs_sin"] = rope_tables(cfg.rope_capacity, R, cfg.theta)
    if cfg.compress:
        _compressor_inputs(t, cfg, seed, pos)
    if cfg.mode == "compress":   # the publication alone: the compressed pool and its table
        pages = cfg.cmp_pages_per_request
        perm = _rng(seed, "cmp_perm").permutation(B * pages).astype(np.int32)
        t["cmp_block_table"] = perm.reshape(B, pages)
        t["cmp_kv"] = _bf16_normal(seed, "cmp_kv", (B * pages, PAGE, D))
        return CsaInputs(cfg, t)

    # ---- query side
    t["q"] = _bf16_normal(seed, "q", (T, H, D))
    qf = _rng(seed, "q_idx_f").standard_normal((T, Hi, Di), dtype=np.float32)
    t["q_idx"], t["q_scale"] = quantize_rows_int8(qf)
    t["head_w"] = (_rng(seed, "head_w").standard_normal((T, Hi)) / 2.0).astype(np.float32)
    t["attn_sink"] = _rng(seed, "attn_sink").standard_normal(H).astype(np.float32)

    # ---- compressed pool (KV + index keys share one block table)
    pages = cfg.cmp_pages_per_request
    nbc = B * pages
    perm = _rng(seed, "cmp_perm").permutation(nbc).astype(np.int32)
    t["cmp_block_table"] = perm.reshape(B, pages)
    if cfg.kv_format == "mx":
        t["cmp_fp4"] = _u8_uniform(seed, "cmp_fp4", (nbc, PAGE, D // 2), 0, 255)
        t["cmp_scale"] = ((_u8_uniform(seed, "cmp_sc_e", (nbc, PAGE, D // 16), 3, 6) << 3)
                          | _u8_uniform(seed, "cmp_sc_m", (nbc, PAGE, D // 16), 0, 7))
    else:
        t["cmp_kv"] = _bf16_normal(seed, "cmp_kv", (nbc, PAGE, D))
    t["idx_kv"] = _rng(seed, "idx_kv").integers(-127, 128, size=(nbc, PAGE, Di),
                                                 dtype=np.int8)
    sc = _rng(seed, "idx_scale").uniform(0.005, 0.02, size=(nbc, PAGE)).astype(np.float32)
    if cfg.outlier_frac > 0:
        hit = _rng(seed, "outlier").random((nbc, PAGE)) < cfg.outlier_frac
        sc = np.where(hit, sc * np.float32(4.0), sc).astype(np.float32)
    t["idx_scale"] = sc
    if cfg.index_format == "fp8":
        # the FP8 plane replaces the INT8 one (same names, same FP32 scales):
        # E4M3 codes with uniform sign and mantissa and exponent field 4..10,
        # never NaN; query scales U(0.01, 0.05)
        def e4m3_codes(bits_name, exp_name, shape):
            bits = _u8_uniform(seed, bits_name, shape, 0, 255)
            return (bits & 0x87) | (_u8_uniform(seed, exp_name, shape, 4, 10) << 3)
        t["q_idx"] = e4m3_codes("q_fp8_bits", "q_fp8_exp", (T, Hi, Di))
        t["q_scale"] = _rng(seed, "q_fp8_scale").uniform(0.01, 0.05, size=(T, Hi)).astype(np.float32)
        t["idx_kv"] = e4m3_codes("idx_fp8_bits", "idx_fp8_exp", (nbc, PAGE, Di))
    if cfg.index_format == "mxfp4":
        # the FP4 plane replaces the INT8 one (same names): packed E2M1 codes,
        # every nibble uniform over the 16 codes, and E8M0 group scales
        # 2^-6 .. 2^1 (bytes 121 .. 128)
        t["q_idx"] = _rng(seed, "q_fp4").integers(0, 256, size=(T, Hi, Di // 2), dtype=np.uint8)
        t["q_scale"] = _rng(seed, "q_e8m0").integers(121, 129, size=(T, Hi, Di // 32),
                                                     dtype=np.uint8)
        t["idx_kv"] = _rng(seed, "idx_fp4").integers(0, 256, size=(nbc, PAGE, Di // 2),
                                                     dtype=np.uint8)
        t["idx_scale"] = _rng(seed, "idx_e8m0").integers(121, 129, size=(nbc, PAGE, Di // 32),
                                                         dtype=np.uint8)

    # ---- window pool: only the pages some window touches are backed
    wpages = cfg.win_pages_per_request
    touched = []
    for b in range(B):
        s = set()
        for p in cfg.positions[b]:
            lo = max(0, p - cfg.W + 1)
            for pg in range(lo // PAGE, p // PAGE + 1):
                s.add(pg)
        touched.append(sorted(s))
    nbw = sum(len(x) for x in touched)
    wperm = _rng(seed, "win_perm").permutation(nbw).astype(np.int32)
    wbt = np.full((B, wpages), -1, dtype=np.int32)
    i = 0
    for b in range(B):
        for pg in touched[b]:
            wbt[b, pg] = wperm[i]
            i += 1
    t["win_block_table"] = wbt
    if cfg.kv_format == "mx":
        bits = _u8_uniform(seed, "win_fp8_bits", (nbw, PAGE, D), 0, 255)
        t["win_fp8"] = (bits & 0x87) | (_u8_uniform(seed, "win_fp8_exp", (nbw, PAGE, D), 4, 10) << 3)
        t["win_scale"] = _u8_uniform(seed, "win_e8m0", (nbw, PAGE, D // 32), 122, 125)
    else:
        t["win_kv"] = _bf16_normal(seed, "win_kv", (nbw, PAGE, D))

    # ---- a reindex layer's candidate mask (the full layer's output, supplied
    #      as an input): per row, cand_kb distinct blocks of cand_block
    #      positions drawn uniformly from the blocks its position reaches,
    #      ascending, padded with -1
    if cfg.mode == "reindex":
        kb, blk = cfg.cand_kb, cfg.cand_block
        g = _rng(seed, "cand_blocks")
        cand = np.full((T, kb), -1, dtype=np.int32)
        for r in range(T):
            reach = -(-max(0, (int(pos[r]) + 1) // cfg.ratio) // blk)
            m = min(kb, reach)
            if m:
                cand[r, :m] = np.sort(g.choice(reach, size=m, replace=False))
        t["cand_blocks"] = cand
    return CsaInputs(cfg, t)
