"""Workload shapes for one compressed-sparse-attention (CSA) layer step.

Each config is a synthetic stand-in for a V4/V4.1-Flash attention layer as the
pages describe it (pypto-lib "DeepSeek V4.1 Flash", checkpoint-shape table: 64
heads of width 512, maximum position 1,048,576; pypto-lib "DeepSeek V4-Flash,
MTP point", deployment table: 4 requests x S=2 decode rows per card, prefill up
to 8,192 tokens walked in 128-token tiles).  No dataset is involved.

This module holds shapes only; no arithmetic of the method lives here.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Tuple

PAGE = 128  # tokens per cache block (the pages' 128-token scheduler block)


@dataclasses.dataclass(frozen=True)
class CsaConfig:
    name: str
    description: str
    # query side
    rows_per_request: Tuple[int, ...]   # decode/prefill rows of each request
    positions: Tuple[Tuple[int, ...], ...]  # causal position of every row, per request
    rope_neg_rows: Tuple[int, ...] = ()  # row offsets (within each request) whose rope position is -1
    H: int = 64
    D: int = 512
    R: int = 64                 # rope_dim (rotated channels, adjacent pairs)
    Hi: int = 64                # indexer heads
    Di: int = 128               # indexer head dim
    W: int = 128                # sliding window
    ratio: int = 2
    k: int = 512
    context: int = 32768        # raw tokens per request already in the caches
    rope_capacity: int = 1 << 20
    theta: float = 10000.0
    outlier_frac: float = 0.0   # fraction of compressed positions whose key scale is x4
    shared_pool: bool = False   # all requests page into one pool (C5)
    # "csa": indexer + top-k select the compressed rows; "hca": no indexer,
    # every causally visible compressed row (k bounds them); "swa": the
    # window alone (k = 0); "reindex": a layer that scores only the positions
    # of a supplied candidate mask (cand_kb blocks of cand_block positions)
    # and selects its k there; "hier_full": the csa step that also publishes
    # such a mask for the reindex layers; "compress": the compressor's
    # publication alone (no query side)
    mode: str = "csa"
    cand_kb: int = 0
    cand_block: int = 8
    # index plane: "int8" (INT8 keys and query, FP32 per-row scales), "fp8"
    # (E4M3 codes in the same layout) or "mxfp4" (packed E2M1 keys and query,
    # one E8M0 scale per 32 dims)
    index_format: str = "int8"
    # KV planes: "bf16" (one BF16 cache per pool) or "mx" (the low-bit cache
    # ABI: window rows MXFP8 E4M3 with one E8M0 byte per 32 channels,
    # compressed rows packed MXFP4 E2M1 with one E4M3 byte per 16 channels)
    kv_format: str = "bf16"
    # the ratio-2 compressor's publication ahead of the step (pypto-lib
    # "DeepSeek V4.1 Flash", "Compressor state ownership": an FP32 state ring
    # of state_capacity slots per request, pairs closed by odd positions);
    # mode "compress" runs that publication alone
    compress: bool = False
    state_capacity: int = 4
    rms_eps: float = 1e-6

    @property
    def kv_row_bytes(self):
        """(window, compressed) bytes of one KV row, payload + scales."""
        if self.kv_format == "mx":
            return self.D + self.D // 32, self.D // 2 + self.D // 16
        return 2 * self.D, 2 * self.D

    @property
    def index_key_bytes(self) -> int:
        """Bytes of one index key (payload + scales)."""
        return self.Di // 2 + self.Di // 32 if self.index_format == "mxfp4" else self.Di + 4

    # ---- derived sizes -------------------------------------------------
    @property
    def B(self) -> int:
        return len(self.rows_per_request)

    @property
    def T(self) -> int:
        return int(sum(self.rows_per_request))

    @property
    def query_start_loc(self) -> List[int]:
        out = [0]
        for r in self.rows_per_request:
            out.append(out[-1] + r)
        return out

    @property
    def flat_positions(self) -> List[int]:
        return [p for req in self.positions for p in req]

    @property
    def n_cmp_per_request(self) -> int:
        """Compressed rows each request holds: context // ratio."""
        return self.context // self.ratio

    @property
    def cmp_pages_per_request(self) -> int:
        return -(-self.n_cmp_per_request // PAGE)

    @property
    def win_pages_per_request(self) -> int:
        return -(-self.context // PAGE)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def rope_offset(self) -> int:
        return self.D - self.R

    @property
    def score_stride(self) -> int:
        return self.cmp_pages_per_request * PAGE


def _decode(name, desc, n_req, s, context, **kw) -> CsaConfig:
    pos = tuple(tuple(range(context - s, context)) for _ in range(n_req))
    return CsaConfig(name=name, description=desc, rows_per_request=(s,) * n_req,
                     positions=pos, context=context, **kw)


C1 = _decode(
    "c1_tiny_decode",
    "tiny decode: 2 rows, 8 heads x 64, rope 16, 512 raw tokens at ratio 2 -> 256 "
    "compressed rows, window 16, indexer 4x32, top-k 32, positions 510/511",
    n_req=1, s=2, context=512, H=8, D=64, R=16, Hi=4, Di=32, W=16, ratio=2, k=32,
    rope_capacity=1024)

C2 = _decode(
    "c2_ratio2_decode",
    "V4.1 ratio-2 decode: 8 rows (4 requests x S=2), 64x512 heads, 32,768 tokens "
    "-> 16,384 compressed rows per request, window 128, indexer 64x128, top-k 512",
    n_req=4, s=2, context=32768, ratio=2, k=512)

C3 = _decode(
    "c3_ratio1_decode",
    "V4.1 ratio-1 decode: 8 rows (4 x 2), 131,072 compressed rows per request, "
    "window 128, indexer 64x128, top-k 2048, first row of each request at rope "
    "position -1",
    n_req=4, s=2, context=131072, ratio=1, k=2048, rope_neg_rows=(0,))

C4 = CsaConfig(
    name="c4_ratio2_prefill",
    description="V4.1 ratio-2 prefill: 1 request, 8,192 causal queries at positions "
                "0..8191, 4,096 compressed rows, window 128, indexer 64x128, top-k 512",
    rows_per_request=(8192,), positions=(tuple(range(8192)),), context=8192,
    ratio=2, k=512)

C5 = _decode(
    "c5_maxctx_ratio1_decode",
    "max-context ratio-1 decode: 8 rows (2 requests x 4), 1,048,576 positions per "
    "request in 8,192 pages of one shared pool, window 128, top-k 2048, 5% of "
    "positions carry x4 key scales",
    n_req=2, s=4, context=1 << 20, ratio=1, k=2048, outlier_frac=0.05,
    shared_pool=True)

# Layers without an indexer (the layer schedule of the pages' MTP-point
# model): HCA at ratio 128 attends over every visible compressed row plus the
# window, SWA over the window alone.
C6 = _decode(
    "c6_hca_ratio128_decode",
    "HCA ratio-128 decode: 8 rows (4 requests x S=2), 1,048,576 tokens -> 8,192 "
    "compressed rows per request, all of them attended with the 128-token window",
    n_req=4, s=2, context=1 << 20, ratio=128, k=8192, mode="hca")

C7 = _decode(
    "c7_swa_decode",
    "SWA-only decode: 8 rows (4 requests x S=2), 32,768 tokens, the 128-token "
    "window alone",
    n_req=4, s=2, context=32768, ratio=128, k=0, mode="swa")

# The hierarchical indexer of the ratio-1 layers (pypto-lib "DeepSeek V4.1
# Flash", section "Decode composition"): the full layer keeps 2,048 blocks of
# eight compressed positions, a reindex layer picks its final 512 inside them.
C8 = _decode(
    "c8_reindex_ratio1_decode",
    "ratio-1 reindex decode: 8 rows (4 x 2), 131,072 compressed rows per request, "
    "a supplied mask of 2,048 blocks of 8 per row, indexer 64x128 scored inside "
    "it, top-k 512, window 128",
    n_req=4, s=2, context=131072, ratio=1, k=512, mode="reindex", cand_kb=2048)

C9 = _decode(
    "c9_full_hier_ratio1_decode",
    "ratio-1 full decode that also publishes the candidate mask: C3's step (top-k "
    "2048) plus 2,048 blocks of 8 per row",
    n_req=4, s=2, context=131072, ratio=1, k=2048, mode="hier_full", cand_kb=2048)

# The FP4 index plane of the production cache ABI (pypto-lib "DeepSeek V4.1
# Flash": index keys packed MXFP4 E2M1 with group-of-32 E8M0 scales) on the
# max-context and the ratio-2 decode shapes.
C10 = _decode(
    "c10_maxctx_mxfp4_decode",
    "max-context ratio-1 decode with the MXFP4 index plane: C5's shapes, index keys "
    "and queries packed E2M1 with one E8M0 scale per 32 dims (68 bytes per key)",
    n_req=2, s=4, context=1 << 20, ratio=1, k=2048, shared_pool=True, index_format="mxfp4")

C11 = _decode(
    "c11_ratio2_mxfp4_decode",
    "V4.1 ratio-2 decode with the MXFP4 index plane: C2's shapes",
    n_req=4, s=2, context=32768, ratio=2, k=512, index_format="mxfp4")

# The low-bit KV planes of the production cache ABI (pypto-lib "DeepSeek V4.1
# Flash", the paragraph on the production cache ABI: MXFP8 window KV, MXFP4
# compressed KV with E4M3 group-of-16 scales) on the ratio-1 decode shapes;
# the max-context one also takes the MXFP4 index plane, so every cache it
# reads is in its production format.
C12 = _decode(
    "c12_ratio1_mxkv_decode",
    "ratio-1 decode over the low-bit KV planes: C3's shapes, window rows MXFP8 E4M3 "
    "(528 bytes), compressed rows MXFP4 E2M1 with E4M3 group-16 scales (288 bytes)",
    n_req=4, s=2, context=131072, ratio=1, k=2048, rope_neg_rows=(0,), kv_format="mx")

C13 = _decode(
    "c13_maxctx_lowbit_decode",
    "max-context ratio-1 decode with every cache low-bit: C5's shapes, MXFP4 index "
    "keys, MXFP8 window KV and MXFP4 compressed KV",
    n_req=2, s=4, context=1 << 20, ratio=1, k=2048, shared_pool=True, index_format="mxfp4",
    kv_format="mx")

# The FP8 index plane, ROCm ATOM's default index cache dtype ("DeepSeek-V4.1
# native paged runtime", "Current execution scope"), on the max-context and
# the ratio-2 decode shapes.
C14 = _decode(
    "c14_maxctx_fp8index_decode",
    "max-context ratio-1 decode with the FP8 index plane: C5's shapes, index keys and "
    "queries as E4M3 codes with FP32 per-row / per-head scales (132 bytes per key)",
    n_req=2, s=4, context=1 << 20, ratio=1, k=2048, shared_pool=True, index_format="fp8")

C15 = _decode(
    "c15_ratio2_fp8index_decode",
    "V4.1 ratio-2 decode with the FP8 index plane: C2's shapes",
    n_req=4, s=2, context=32768, ratio=2, k=512, index_format="fp8")

# The ratio-2 compressor (pypto-lib "DeepSeek V4.1 Flash", "Compressor state
# ownership"): each decode step first publishes the pair its odd row closes,
# then scores, selects and attends; a prefill chunk publishes every pair it
# closes (the compressor alone, at the 8,192-token prefill shape).
C16 = _decode(
    "c16_ratio2_decode_compress",
    "V4.1 ratio-2 decode with the compressor ahead of it: C2's shapes, each request's "
    "rows (32766, 32767) close one pair, published at compressed position 16383 from "
    "FP32 KV projections and gate scores, FP32 state ring of 4 slots",
    n_req=4, s=2, context=32768, ratio=2, k=512, compress=True)

C17 = CsaConfig(
    name="c17_ratio2_prefill_compress",
    description="ratio-2 compressor over an 8,192-token prefill chunk: 1 request, "
                "positions 0..8191, FP32 KV projections and gate scores of width 512, "
                "4,096 pairs published into 32 pages, the last 4 rows to the ring",
    rows_per_request=(8192,), positions=(tuple(range(8192)),), context=8192, ratio=2,
    k=0, mode="compress", compress=True)

CONFIGS: Dict[str, CsaConfig] = {c.name: c for c in (C1, C2, C3, C4, C5, C6, C7, C8, C9, C10,
                                                     C11, C12, C13, C14, C15, C16, C17)}
SHORT = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5, "c6": C6, "c7": C7, "c8": C8,
         "c9": C9, "c10": C10, "c11": C11, "c12": C12, "c13": C13, "c14": C14, "c15": C15,
         "c16": C16, "c17": C17}


def get(name: str) -> CsaConfig:
    if name in SHORT:
        return SHORT[name]
    return CONFIGS[name]
