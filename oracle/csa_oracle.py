"""CPU oracle for one compressed-sparse-attention (CSA) layer step.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow reference that the
HIP path is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the library and its
Python binding never do.  It shares no code, header, table or helper with the
HIP sources.

Arithmetic is float64 NumPy, row by row, in the order the pages state it.
Integer dot products of the indexer are formed with a float64 matrix product
of INT8-valued operands, which is exact: every partial sum is an integer of
magnitude at most 128 * 127 * 127 < 2**53.

Sources (the pages are cited by title and section):

* [V41]  pypto-lib "DeepSeek V4.1 Flash" -- sections "Serving-owned full RoPE
  tables", "Compressor state ownership" (metadata contract, index checks
  before table indexing), "Decode composition" (Top-K checks, -1 padding).
* [HP]   gitcode hyper-parallel issue #2, "Hyper-Parallel 支持 MindFormers
  DeepSeek V4 CP 并行方案" -- Stage-2 operator calls (sinks, softmax scale,
  ori_win_left=127 / ori_win_right=0), section 7.1 (window example), 8.2
  (causal compressed visibility, worked example p=300), 9.1 (kv_full is the
  window KV followed by the compressed KV; indices are the union), 10.2
  (indexer indices are compressed slot ids), 10.3 (causal mask).
* [MTP]  pypto-lib "DeepSeek V4-Flash, MTP point" -- section "What is
  quantized" (INT8 index-key cache with an FP32 per-row scale; BF16 KV;
  FP32 attn_sink).
* [ATOM] ROCm ATOM "DeepSeek-V4.1 native paged runtime" -- section "Current
  execution scope" (per-row bounds, 128-token PAGE, padding sentinels).

Readings where the pages are silent (listed with reasons in the design notes):

* the score is sum_h w[t,h] * relu(qs[t,h] * ks[c] * <q8[t,h], k8[c]>): ReLU on
  each dequantised head dot, weights after the ReLU, no extra 1/sqrt scaling;
* top-k ties break toward the lower position; the output is ascending by
  position, padded with -1 (value -inf) when fewer than k positions are visible;
* the window of a query at position p is raw positions [max(0, p-W+1), p];
  window rows and selected compressed rows are concatenated with no dedup;
* the sink is one unscaled logit per head in the softmax denominator with no
  value row; lse includes it; an empty key set gives out = 0, lse = sink;
* only the query is rotated (adjacent pairs (2i, 2i+1) of channels
  [rope_offset, rope_offset + rope_dim) by rope row t); cached rows are used as
  stored.

Device-error flags mirror the library's documented bit values (restated here,
not shared): rows that violate the metadata contract are handled as listed in
each function.
"""
from __future__ import annotations

import numpy as np

PAGE = 128

EFLAG_POS_RANGE = 1     # position past a table / a row's visible span past its storage
EFLAG_BLOCK_RANGE = 2   # block id outside the pool (or page outside the table)
EFLAG_TOPK_RANGE = 4    # selected index not visible to the row
EFLAG_META = 8          # active row that no request owns


# ----------------------------------------------------------------------------
# small exact helpers
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of BF16 bit patterns: the top 16 bits of an IEEE float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """BF16 bit patterns of float64 values, rounded to nearest even in one
    step from the float64 value (8 significant bits kept).  Finite values in
    BF16's normal range only."""
    b = np.asarray(x, dtype=np.float64).view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = (b + np.uint64(0x0FFFFFFFFFFF) + lsb) & ~np.uint64((1 << 45) - 1)
    return (r.view(np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def visible_count(pos: int, ratio: int) -> int:
    """Compressed slots a query at absolute position ``pos`` may see.

    [HP] 8.2 / 10.3: slot c is visible to position p iff c < (p + 1) // ratio
    (worked example: p = 300, ratio = 128 sees slots 0 and 1, not 2).
    A negative position sees nothing."""
    return max(0, (int(pos) + 1) // int(ratio))


def window_positions(pos: int, window: int) -> range:
    """Raw positions in the sliding window of a query at ``pos``:
    [max(0, p - W + 1), p] -- ori_win_left = W - 1 tokens to the left, none to
    the right ([HP] Stage-2 calls; worked example in section 7.1: with W = 4,
    token 4 sees tokens 1..4)."""
    p = int(pos)
    if p < 0:
        return range(0)
    return range(max(0, p - window + 1), p + 1)


def owner_request(t: int, query_start_loc: np.ndarray) -> int:
    """Request b with query_start_loc[b] <= t < query_start_loc[b+1]; -1 if none.
    [V41] "Compressor state ownership": packed, nondecreasing query starts;
    equal neighbours are an empty request."""
    qsl = np.asarray(query_start_loc)
    for b in range(len(qsl) - 1):
        if qsl[b] <= t < qsl[b + 1]:
            return b
    return -1


def rotate_adjacent_pairs(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate channel pairs (2i, 2i+1) of ``x`` by the angle whose cosine and
    sine are cos[i], sin[i] (multiplication by e^{i theta} with x[2i] the real
    part).  [V41] "Serving-owned full RoPE tables": FP32 half-width tables are
    kept for adjacent-pair rotation."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    re = x[..., 0::2]
    im = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = re * c - im * s
    out[..., 1::2] = re * s + im * c
    return out


# ----------------------------------------------------------------------------
# a1: RoPE rows
# ----------------------------------------------------------------------------

def inverse_rope(out, rope_cos, rope_sin, rope_offset, num_tokens):
    """Inverse RoPE of the attention output ([ATOM] "DeepSeek-V4.1 native paged
    runtime", introduction and "Current execution scope": the V4 attention is
    followed by an inverse RoPE kernel; the pages do not define it).  Reading:
    shared K = V rows carry their rope span rotated by their own positions, so
    the output's rope span is a mix of rotated values; the inverse rotates
    that span of every head of active row t back by row t's angles -- the
    conjugate of its rope row, multiplication by e^{-i theta} in the pair
    convention of ``rotate_adjacent_pairs``.  Channels outside
    [rope_offset, rope_offset + 2 * half) are unchanged; rows >= num_tokens
    are returned as given.  Returns float64 [T, H, D]."""
    o = np.array(out, dtype=np.float64, copy=True)
    c = np.asarray(rope_cos, dtype=np.float64)
    s = np.asarray(rope_sin, dtype=np.float64)
    half = c.shape[1]
    for t in range(int(num_tokens)):
        span = o[t, :, rope_offset:rope_offset + 2 * half]
        o[t, :, rope_offset:rope_offset + 2 * half] = rotate_adjacent_pairs(span, c[t], -s[t])
    return o


def materialize_rope_rows(freqs_cos, freqs_sin, position_ids, num_tokens,
                          rope_cos, rope_sin) -> int:
    """[V41] "Serving-owned full RoPE tables": for each active row t < num_tokens
    copy row position_ids[t] of the FP32 half-width tables; a negative position
    writes the identity rotation (cos 1, sin +0); rows >= num_tokens are left
    untouched.  A nonnegative position at or past the table capacity is a
    contract violation: the row is left untouched and POS_RANGE is flagged.

    Writes ``rope_cos`` / ``rope_sin`` (float32 [T, R/2]) in place; returns the
    error flags."""
    cap = freqs_cos.shape[0]
    err = 0
    for t in range(int(num_tokens)):
        p = int(position_ids[t])
        if p < 0:
            rope_cos[t, :] = np.float32(1.0)
            rope_sin[t, :] = np.float32(0.0)
        elif p < cap:
            rope_cos[t, :] = freqs_cos[p, :]
            rope_sin[t, :] = freqs_sin[p, :]
        else:
            err |= EFLAG_POS_RANGE
    return err


# ----------------------------------------------------------------------------
# a2 + a4: lightning-indexer scores
# ----------------------------------------------------------------------------

def _physical_rows(block_table_row, num_blocks, positions):
    """Translate request-local positions to flat pool rows through a 128-token
    block table ([V41] cache ABI; [ATOM] "Current execution scope").  Returns
    (rows, ok) where ok marks positions whose page and block id are valid."""
    positions = np.asarray(positions, dtype=np.int64)
    page = positions // PAGE
    in_table = page < len(block_table_row)
    blk = np.full(positions.shape, -1, dtype=np.int64)
    blk[in_table] = np.asarray(block_table_row, dtype=np.int64)[page[in_table]]
    ok = in_table & (blk >= 0) & (blk < num_blocks)
    rows = np.where(ok, blk * PAGE + positions % PAGE, 0)
    return rows, ok


def index_scores(q_idx, q_scale, head_w, idx_kv, idx_scale, block_table,
                 query_start_loc, positions, num_tokens, ratio, score_stride,
                 key_chunk: int = 1 << 16):
    """Lightning-indexer score of every causally visible compressed position.

    For active row t of request b at position p, and c < (p + 1) // ratio:

        score[t, c] = sum_h w[t,h] * relu( qs[t,h] * ks[c] * <q8[t,h,:], k8[c,:]> )

    with k8 / ks the INT8 key row and FP32 scale of compressed position c,
    found through the request's block table ([MTP] "What is quantized": INT8
    index keys with an FP32 per-row scale; [HP] 10.2: scores over compressed
    slot ids; 10.3: causal mask).  Positions c >= (p + 1) // ratio score -inf.

    Contract checks (flags; never an out-of-range read):
      * a row no request owns: META, the whole row is -inf;
      * visible span larger than score_stride or than the block table covers:
        POS_RANGE, the span is cut to what fits;
      * a visible position whose page holds an invalid block id: BLOCK_RANGE,
        that position scores -inf.

    Returns (scores float64 [num_tokens, score_stride], err)."""
    qsl = np.asarray(query_start_loc)
    num_blocks = idx_kv.shape[0]
    Di = idx_kv.shape[2]
    keys_flat = idx_kv.reshape(num_blocks * PAGE, Di)
    scales_flat = np.asarray(idx_scale, dtype=np.float64).reshape(-1)
    scores = np.full((int(num_tokens), int(score_stride)), -np.inf, dtype=np.float64)
    err = 0
    max_blocks = block_table.shape[1]
    for t in range(int(num_tokens)):
        b = owner_request(t, qsl)
        if b < 0:
            err |= EFLAG_META
            continue
        n = visible_count(positions[t], ratio)
        if n > score_stride or n > PAGE * max_blocks:
            err |= EFLAG_POS_RANGE
            n = min(n, int(score_stride), PAGE * max_blocks)
        q = np.asarray(q_idx[t], dtype=np.float64)          # [Hi, Di], integer valued
        qs = np.asarray(q_scale[t], dtype=np.float64)        # [Hi]
        w = np.asarray(head_w[t], dtype=np.float64)          # [Hi]
        for c0 in range(0, n, key_chunk):
            cs = np.arange(c0, min(n, c0 + key_chunk))
            rows, ok = _physical_rows(block_table[b], num_blocks, cs)
            if not ok.all():
                err |= EFLAG_BLOCK_RANGE
            k8 = keys_flat[rows].astype(np.float64)         # [n_c, Di]
            ks = scales_flat[rows]                           # [n_c]
            dots = q @ k8.T                                  # [Hi, n_c], exact integers
            per_head = qs[:, None] * ks[None, :] * dots
            s = (w[:, None] * np.maximum(per_head, 0.0)).sum(axis=0)
            s[~ok] = -np.inf
            scores[t, cs] = s
    return scores, err


def index_scores_fp8(q_fp8, q_scale, head_w, idx_fp8, idx_scale, block_table,
                     query_start_loc, positions, num_tokens, ratio, score_stride,
                     key_chunk: int = 1 << 16):
    """The indexer score with the FP8 index plane ([ATOM] "Current execution
    scope": FP8 is the default index cache dtype; its layout is not given).
    Reading: the INT8 plane's layout with E4M3 codes in place of INT8 ones --
    key rows [blocks, 128, Di] of OCP E4M3FN codes with one FP32 scale per
    row, the query [T, Hi, Di] of E4M3 codes with one FP32 scale per (row,
    head) -- and the score formula of ``index_scores`` over the decoded values:

        score[t, c] = sum_h w[t,h] * relu( qs[t,h] * ks[c] * <e4m3(q[t,h]), e4m3(k[c])> )

    Every product of two E4M3 values, and every sum of Di <= 128 of them, is
    exact in float64.  Visibility, contract checks and flags are those of
    ``index_scores``.  Returns (scores float64 [num_tokens, score_stride], err)."""
    qsl = np.asarray(query_start_loc)
    num_blocks = idx_fp8.shape[0]
    Di = idx_fp8.shape[2]
    keys_flat = np.asarray(idx_fp8, dtype=np.uint8).reshape(num_blocks * PAGE, Di)
    scales_flat = np.asarray(idx_scale, dtype=np.float64).reshape(-1)
    scores = np.full((int(num_tokens), int(score_stride)), -np.inf, dtype=np.float64)
    err = 0
    max_blocks = block_table.shape[1]
    for t in range(int(num_tokens)):
        b = owner_request(t, qsl)
        if b < 0:
            err |= EFLAG_META
            continue
        n = visible_count(positions[t], ratio)
        if n > score_stride or n > PAGE * max_blocks:
            err |= EFLAG_POS_RANGE
            n = min(n, int(score_stride), PAGE * max_blocks)
        q = decode_e4m3(q_fp8[t])                             # [Hi, Di]
        qs = np.asarray(q_scale[t], dtype=np.float64)         # [Hi]
        w = np.asarray(head_w[t], dtype=np.float64)           # [Hi]
        for c0 in range(0, n, key_chunk):
            cs = np.arange(c0, min(n, c0 + key_chunk))
            rows, ok = _physical_rows(block_table[b], num_blocks, cs)
            if not ok.all():
                err |= EFLAG_BLOCK_RANGE
            k = decode_e4m3(keys_flat[rows])                  # [n_c, Di]
            ks = scales_flat[rows]                            # [n_c]
            dots = q @ k.T                                    # [Hi, n_c], exact
            per_head = qs[:, None] * ks[None, :] * dots
            s = (w[:, None] * np.maximum(per_head, 0.0)).sum(axis=0)
            s[~ok] = -np.inf
            scores[t, cs] = s
    return scores, err


# ----------------------------------------------------------------------------
# the step before the path: ratio-2 compressor publication
# ----------------------------------------------------------------------------

def compress_pairs(kv_proj, gate, query_start_loc, positions, num_tokens, state_block_table,
                   state_cache, rms_gamma, rms_eps, rope_cos, rope_sin, rope_offset, cmp_kv,
                   cmp_block_table):
    """Ratio-2 compressor publication with its FP32 state ring ([V41]
    "Compressor state ownership" and the paragraph on the production cache
    ABI: the state ring [num_state_blocks, CAP, 2D] holds each token's KV
    projection then its gate score; a valid token at position p lives in slot
    block * CAP + p % CAP with block = state_block_table[b]; an odd position
    closes a pair; the first token of a chunk reads its predecessor from the
    ring, later ones take the preceding input row; every ring read comes
    before every ring write; only the last min(chunk, CAP) rows of a chunk are
    written; negative positions neither publish nor write; block -1 disables
    the request's compressor; one compressed row covers two tokens).

    Readings (the pages name the pooling softmax, the BF16 rounding before
    RMSNorm and group-start RoPE rows without formulas): for a pair (p - 1, p)
    with projections kv_j and gate scores g_j,
        pooled[c] = sum_j e^{g_j[c]} kv_j[c] / sum_j e^{g_j[c]}     (per channel)
        x = bf16(pooled);  y = x / sqrt(mean(x^2) + eps) * gamma
        y[off:off+R] rotated by the rope row of the pair's start p - 1
    (rope_cos / rope_sin row t holds that row for token t), and bf16(y) is
    published at compressed position p // 2 of the request's BF16 pool.

    Flags: a state block or publication page outside its pool -> BLOCK_RANGE
    (the access is skipped); a row no request owns -> META.
    Returns (cmp_kv after, state_cache after, err); the inputs are not changed."""
    qsl = np.asarray(query_start_loc)
    pos = np.asarray(positions)
    kv = np.asarray(kv_proj, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    state_in = np.asarray(state_cache, dtype=np.float32)
    state = state_in.copy()
    cmp_out = np.array(cmp_kv, copy=True)
    nsb, cap, two_d = state_in.shape
    D = two_d // 2
    nb = cmp_out.shape[0]
    gamma = np.asarray(rms_gamma, dtype=np.float64)
    c = np.asarray(rope_cos, dtype=np.float64)
    sn = np.asarray(rope_sin, dtype=np.float64)
    half = c.shape[1]
    err = 0
    nt = int(num_tokens)
    writes = []   # (slot index tuple, row) applied after every read
    for t in range(nt):
        if owner_request(t, qsl) < 0:
            err |= EFLAG_META
    for b in range(len(qsl) - 1):
        lo, hi = min(int(qsl[b]), nt), min(int(qsl[b + 1]), nt)
        if hi <= lo:
            continue
        blk = int(state_block_table[b])
        if blk < 0:
            continue                                   # compressor disabled
        blk_ok = blk < nsb
        if not blk_ok:
            err |= EFLAG_BLOCK_RANGE
        for t in range(lo, hi):
            p = int(pos[t])
            if p < 0 or p % 2 == 0:
                continue
            if t > lo:
                prev_kv, prev_g = kv[t - 1], g[t - 1]
            elif blk_ok:
                row = state_in[blk, (p - 1) % cap].astype(np.float64)
                prev_kv, prev_g = row[:D], row[D:]
            else:
                continue
            gg = np.stack([prev_g, g[t]])
            w = np.exp(gg - gg.max(axis=0))
            w = w / w.sum(axis=0)
            pooled = w[0] * prev_kv + w[1] * kv[t]
            x = bf16_to_f64(f64_to_bf16(pooled))
            y = x / np.sqrt(np.mean(x * x) + float(rms_eps)) * gamma
            if half:
                y[rope_offset:rope_offset + 2 * half] = rotate_adjacent_pairs(
                    y[rope_offset:rope_offset + 2 * half], c[t], sn[t])
            rows, ok = _physical_rows(cmp_block_table[b], nb, np.array([p // 2]))
            if not ok[0]:
                err |= EFLAG_BLOCK_RANGE
                continue
            r = int(rows[0])
            cmp_out[r // PAGE, r % PAGE] = f64_to_bf16(y)
        if not blk_ok:
            continue
        for t in range(max(lo, hi - cap), hi):
            p = int(pos[t])
            if p < 0:
                continue
            writes.append(((blk, p % cap), np.concatenate([kv[t], g[t]]).astype(np.float32)))
    for (bi, si), row in writes:
        state[bi, si] = row
    return cmp_out, state, err


# ----------------------------------------------------------------------------
# a2 with the low-bit index plane: MXFP4 keys and queries
# ----------------------------------------------------------------------------

def decode_e2m1(codes):
    """Values of packed E2M1 (FP4) codes.  Each byte holds two elements, the
    one with the lower index in bits 0-3.  A 4-bit code is sign | 2-bit
    exponent | 1-bit mantissa: exponent 0 is subnormal (mantissa * 0.5),
    otherwise 2^(e-1) * (1 + mantissa / 2) -- the magnitudes 0, 0.5, 1, 1.5,
    2, 3, 4, 6 ([V41] cache ABI: packed MXFP4 E2M1 index keys).  Returns
    float64 with the last axis doubled."""
    b = np.asarray(codes, dtype=np.uint8)
    nib = np.stack([b & 0xF, b >> 4], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))
    sign = np.where(nib & 8, -1.0, 1.0)
    e = (nib >> 1) & 3
    m = (nib & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e.astype(np.int64) - 1))
    return sign * mag


def decode_e8m0(scale_bytes):
    """Value of an E8M0 block scale: 2^(byte - 127) (the pages settle this
    convention: a scale byte reads as 2^(byte - 127), the same as torch's
    float8_e8m0fnu; byte 255 is NaN)."""
    b = np.asarray(scale_bytes, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def mx_rows(codes, scale_bytes, group=32):
    """Dequantised rows of an MX plane: E2M1 values times the E8M0 scale of
    their group of `group` consecutive elements."""
    v = decode_e2m1(codes)
    sc = decode_e8m0(scale_bytes)
    return v * np.repeat(sc, group, axis=-1)


def decode_e4m3(codes):
    """Values of FP8 E4M3 codes in the OCP "E4M3FN" form: sign | 4-bit
    exponent (bias 7) | 3-bit mantissa; exponent 0 is subnormal
    (mantissa / 8 * 2^-6), otherwise (1 + mantissa / 8) * 2^(e - 7); there is
    no infinity, and S.1111.111 is NaN, so the largest magnitude is 448 ([V41]
    cache ABI: the window KV payload is MXFP8 E4M3 and the compressed KV
    scales are E4M3).  Returns float64 of the same shape."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & ((b & 7) == 7), np.nan, mag)
    return sign * mag


def index_scores_mxfp4(q_fp4, q_sc, head_w, idx_fp4, idx_sc, block_table, query_start_loc,
                       positions, num_tokens, ratio, score_stride, key_chunk: int = 1 << 15):
    """The indexer score with the FP4 index plane ([ATOM] "Current execution
    scope": the FP4 index arithmetic is E2M1 with one E8M0 scale per 32
    dims; [V41] cache ABI: index keys packed MXFP4 E2M1 with group-of-32
    E8M0 scales).  Reading: the query side uses the same MX format, and the
    score keeps the formula of ``index_scores`` with each head's dot taken
    over the dequantised rows (the block scales replace the per-row scales):

        score[t, c] = sum_h w[t,h] * relu( <mx(q[t,h]), mx(k[c])> )

    Visibility, contract checks and flags are those of ``index_scores``.
    Returns (scores float64 [num_tokens, score_stride], err)."""
    qsl = np.asarray(query_start_loc)
    num_blocks = idx_fp4.shape[0]
    Db = idx_fp4.shape[2]
    keys_flat = np.asarray(idx_fp4).reshape(num_blocks * PAGE, Db)
    sc_flat = np.asarray(idx_sc).reshape(num_blocks * PAGE, -1)
    scores = np.full((int(num_tokens), int(score_stride)), -np.inf, dtype=np.float64)
    err = 0
    max_blocks = block_table.shape[1]
    for t in range(int(num_tokens)):
        b = owner_request(t, qsl)
        if b < 0:
            err |= EFLAG_META
            continue
        n = visible_count(positions[t], ratio)
        if n > score_stride or n > PAGE * max_blocks:
            err |= EFLAG_POS_RANGE
            n = min(n, int(score_stride), PAGE * max_blocks)
        q = mx_rows(q_fp4[t], q_sc[t])                     # [Hi, Di]
        w = np.asarray(head_w[t], dtype=np.float64)
        for c0 in range(0, n, key_chunk):
            cs = np.arange(c0, min(n, c0 + key_chunk))
            rows, ok = _physical_rows(block_table[b], num_blocks, cs)
            if not ok.all():
                err |= EFLAG_BLOCK_RANGE
            k = mx_rows(keys_flat[rows], sc_flat[rows])     # [n_c, Di]
            dots = q @ k.T                                  # [Hi, n_c]
            s = (w[:, None] * np.maximum(dots, 0.0)).sum(axis=0)
            s[~ok] = -np.inf
            scores[t, cs] = s
    return scores, err


# ----------------------------------------------------------------------------
# a3: top-k
# ----------------------------------------------------------------------------

def topk(scores, positions, ratio, num_tokens, k):
    """Per active row, the k best visible positions.

    The visible span of row t is n = (p + 1) // ratio ([HP] 10.3), cut to the
    score row width (flag POS_RANGE if cut); the width of the selection is
    m = min(k, n) ([HP] 7.4: top-k width capped by the key length).  Order:
    score descending, ties toward the lower position, NaN below everything.
    Output ([V41] "Decode composition": eligibility, uniqueness, logical
    position order, trailing -1): the m chosen positions ascending, then -1 up
    to k; values are the chosen scores, -inf for padding.

    Returns (idx int32 [num_tokens, k], val float64 [num_tokens, k], err)."""
    scores = np.asarray(scores, dtype=np.float64)
    nt = int(num_tokens)
    idx = np.full((nt, int(k)), -1, dtype=np.int32)
    val = np.full((nt, int(k)), -np.inf, dtype=np.float64)
    err = 0
    width = scores.shape[1]
    for t in range(nt):
        n = visible_count(positions[t], ratio)
        if n > width:
            err |= EFLAG_POS_RANGE
            n = width
        m = min(int(k), n)
        if m == 0:
            continue
        s = scores[t, :n]
        chosen = _best_ascending(s, m)
        idx[t, :m] = chosen
        val[t, :m] = s[chosen]
    return idx, val, err


def _best_ascending(s, m):
    """Indices of the m best entries of s -- score descending, the lower
    index first among equal scores, NaN below everything -- in ascending
    index order."""
    s = np.asarray(s, dtype=np.float64)
    nan = np.isnan(s)
    primary = np.where(nan, np.inf, -s)          # ascending sort = descending score
    order = np.lexsort((np.arange(len(s)), nan, primary))
    return np.sort(order[:m])


# ----------------------------------------------------------------------------
# Hierarchical selection: the full layer's candidate blocks, then a reindex
# layer's selection inside them
# ----------------------------------------------------------------------------

def candidate_blocks(scores, positions, ratio, num_tokens, block, kb):
    """The full layer's candidate mask ([V41] "Decode composition": the
    hierarchical indexer first picks 2,048 blocks of eight compressed
    positions; later reindex layers select only inside that mask, which stays
    in request-local compressed-position space).

    Reading (the pages name the block selection but not the block score):
    block j of row t covers positions j*block .. j*block + block - 1, and its
    score is the largest score among its visible positions (c < n_vis, the
    span cut to the score row width as in ``topk``).  A block with no visible
    position is not eligible.  The min(kb, eligible) best blocks -- block score
    descending, lower block id first, NaN below everything -- are returned in
    ascending block order, padded with -1.

    Returns (blocks int32 [num_tokens, kb], err)."""
    scores = np.asarray(scores, dtype=np.float64)
    nt = int(num_tokens)
    out = np.full((nt, int(kb)), -1, dtype=np.int32)
    err = 0
    width = scores.shape[1]
    for t in range(nt):
        n = visible_count(positions[t], ratio)
        if n > width:
            err |= EFLAG_POS_RANGE
            n = width
        nb = -(-n // block)
        bs = np.empty(nb, dtype=np.float64)
        for j in range(nb):
            part = scores[t, j * block:min(n, (j + 1) * block)]
            finite = part[~np.isnan(part)]
            bs[j] = finite.max() if finite.size else np.nan
        m = min(int(kb), nb)
        if m:
            out[t, :m] = _best_ascending(bs, m)
    return out, err


def candidate_positions(cand_row, block, n_vis):
    """Positions of one row's candidate slots: slot i is position
    cand_row[i // block] * block + i % block.  Returns (pos int64 [kb*block],
    eligible bool) -- a slot is eligible when its block entry is not -1 and
    its position is visible (c < n_vis)."""
    cand_row = np.asarray(cand_row, dtype=np.int64)
    slots = np.arange(len(cand_row) * block)
    blk = cand_row[slots // block]
    pos = blk * block + slots % block
    eligible = (blk >= 0) & (pos < n_vis)
    return np.where(blk >= 0, pos, -1), eligible


def index_scores_in_candidates(q_idx, q_scale, head_w, idx_kv, idx_scale, block_table,
                               query_start_loc, positions, num_tokens, ratio,
                               cand_blocks, block):
    """A reindex layer's scores: the ``index_scores`` formula with the layer's
    own index query, evaluated only at the positions of row t's candidate
    blocks ([V41] "Decode composition": reindex layers compute a new index
    query and read the supplied candidate mask).

    Slot i of row t is position cand_blocks[t, i // block] * block + i % block.
    A slot that is not eligible (block -1, or position not visible) scores
    -inf.  A candidate block past the visible span is a selection the row may
    not see: TOPK_RANGE.  Page / block-id problems flag as in
    ``index_scores``; a row no request owns flags META and scores -inf.

    Returns (scores float64 [num_tokens, kb*block], err)."""
    qsl = np.asarray(query_start_loc)
    cand_blocks = np.asarray(cand_blocks)
    num_blocks = idx_kv.shape[0]
    Di = idx_kv.shape[2]
    keys_flat = idx_kv.reshape(num_blocks * PAGE, Di)
    scales_flat = np.asarray(idx_scale, dtype=np.float64).reshape(-1)
    nslot = cand_blocks.shape[1] * block
    scores = np.full((int(num_tokens), nslot), -np.inf, dtype=np.float64)
    err = 0
    for t in range(int(num_tokens)):
        b = owner_request(t, qsl)
        if b < 0:
            err |= EFLAG_META
            continue
        n = visible_count(positions[t], ratio)
        row = cand_blocks[t]
        if np.any(row[row >= 0].astype(np.int64) * block >= n):
            err |= EFLAG_TOPK_RANGE
        pos, eligible = candidate_positions(row, block, n)
        sl = np.nonzero(eligible)[0]
        if sl.size == 0:
            continue
        rows, ok = _physical_rows(block_table[b], num_blocks, pos[sl])
        if not ok.all():
            err |= EFLAG_BLOCK_RANGE
        q = np.asarray(q_idx[t], dtype=np.float64)
        qs = np.asarray(q_scale[t], dtype=np.float64)
        w = np.asarray(head_w[t], dtype=np.float64)
        k8 = keys_flat[rows].astype(np.float64)
        ks = scales_flat[rows]
        dots = q @ k8.T
        s = (w[:, None] * np.maximum(qs[:, None] * ks[None, :] * dots, 0.0)).sum(axis=0)
        s[~ok] = -np.inf
        scores[t, sl] = s
    return scores, err


def topk_in_candidates(cand_scores, cand_blocks, block, positions, ratio, num_tokens, k):
    """A reindex layer's final selection: per active row, the k best eligible
    candidate slots, reported as compressed positions ([V41] "Decode
    composition": the final 512 positions come only from inside the candidate
    mask).  Same order and output contract as ``topk``: score descending, the
    lower position first, NaN below everything; m = min(k, eligible slots);
    the chosen positions ascending, then -1 (value -inf).

    Returns (idx int32 [num_tokens, k], val float64 [num_tokens, k], err)."""
    cand_scores = np.asarray(cand_scores, dtype=np.float64)
    cand_blocks = np.asarray(cand_blocks)
    nt = int(num_tokens)
    idx = np.full((nt, int(k)), -1, dtype=np.int32)
    val = np.full((nt, int(k)), -np.inf, dtype=np.float64)
    for t in range(nt):
        n = visible_count(positions[t], ratio)
        pos, eligible = candidate_positions(cand_blocks[t], block, n)
        sl = np.nonzero(eligible)[0]
        m = min(int(k), sl.size)
        if m == 0:
            continue
        by_pos = sl[np.argsort(pos[sl], kind="stable")]
        chosen = by_pos[_best_ascending(cand_scores[t, by_pos], m)]
        idx[t, :m] = pos[chosen]
        val[t, :m] = cand_scores[t, chosen]
    return idx, val, 0


# ----------------------------------------------------------------------------
# a5 + a6/a7: shared-KV sparse attention with sink
# ----------------------------------------------------------------------------

def deterministic_selection(p, ratio, k):
    """The compressed rows of a layer without an indexer (the ratio-128 HCA
    layers): every causally visible compressed row, positions 0 .. n_vis - 1.
    [HP] Stage-2 call for ratio=128 passes no sparse indices (attention over
    the whole causally visible compressed KV plus the window); [MTP] sections
    "Layer schedule" and "Attention paths" give the HCA layers a
    deterministic top-k and no indexer.  k bounds the count:
    a row with more visible rows keeps the first k and reports TOPK_RANGE;
    k = 0 selects nothing and reports nothing (the SWA-only layers: the
    window alone).  Returns (positions, err)."""
    n = visible_count(p, ratio)
    m = min(n, int(k))
    return np.arange(m, dtype=np.int64), (EFLAG_TOPK_RANGE if int(k) > 0 and n > m else 0)


class KvPlane:
    """A paged KV cache, read row by row: ``num_blocks`` pages of 128 rows and
    ``rows(flat)`` -> float64 [len(flat), D], the values of flat pool rows
    (page * 128 + slot).  Attention reads keys/values only through this, so
    the BF16 cache and the low-bit caches of [V41]'s cache ABI share the
    attention arithmetic; the low-bit planes are dequantised on read (the
    pages' references quantise on cache publication and dequantise on cache
    reads)."""

    def __init__(self, num_blocks, d, rows):
        self.num_blocks = int(num_blocks)
        self.d = int(d)
        self._rows = rows

    def rows(self, flat):
        return self._rows(np.asarray(flat, dtype=np.int64))


def bf16_plane(kv):
    """BF16 KV cache [blocks, 128, D] (uint16 bit patterns)."""
    kv = np.asarray(kv)
    nb, _, d = kv.shape
    flat = kv.reshape(nb * PAGE, d)
    return KvPlane(nb, d, lambda r: bf16_to_f64(flat[r]))


def mxfp8_plane(payload, scales):
    """The window KV plane of [V41]'s cache ABI: payload [blocks, 128, D] MXFP8
    E4M3 codes, scales [blocks, 128, D / 32] E8M0 bytes; channel c of a row is
    e4m3(payload[c]) * 2^(scales[c // 32] - 127)."""
    payload = np.asarray(payload, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    nb, _, d = payload.shape
    pf = payload.reshape(nb * PAGE, d)
    sf = scales.reshape(nb * PAGE, d // 32)
    return KvPlane(nb, d, lambda r: decode_e4m3(pf[r]) * np.repeat(decode_e8m0(sf[r]), 32, axis=-1))


def mxfp4_e4m3_plane(payload, scales):
    """The compressed KV plane of [V41]'s cache ABI: payload [blocks, 128, D / 2]
    of packed E2M1 codes (element 2i in bits 0-3 of byte i), scales
    [blocks, 128, D / 16] E4M3 codes; channel c of a row is
    e2m1(c) * e4m3(scales[c // 16])."""
    payload = np.asarray(payload, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    nb, _, half = payload.shape
    pf = payload.reshape(nb * PAGE, half)
    sf = scales.reshape(nb * PAGE, (2 * half) // 16)
    return KvPlane(nb, 2 * half,
                   lambda r: decode_e2m1(pf[r]) * np.repeat(decode_e4m3(sf[r]), 16, axis=-1))


def kv_rows_for_query(t, b, p, topk_row, ratio, window, cmp_block_table, num_cmp_blocks,
                      win_block_table, num_win_blocks, k=None):
    """The key/value rows of one query, window first then selected compressed
    rows, as (pool, flat_row) pairs -- [HP] 9.1: kv_full = [window KV,
    compressed KV], topk_idxs = [window_idxs, compressed_idxs]; the two caches
    are separate, so nothing is deduplicated.  topk_row None takes the
    deterministic selection (every visible compressed row, bounded by k).
    Returns (win_rows, cmp_rows, err)."""
    err = 0
    wpos = np.asarray(list(window_positions(p, window)), dtype=np.int64)
    wrows, wok = _physical_rows(win_block_table[b], num_win_blocks, wpos)
    if not wok.all():
        err |= EFLAG_BLOCK_RANGE
    n = visible_count(p, ratio)
    if topk_row is None:
        sel, e = deterministic_selection(p, ratio, k)
        err |= e
    else:
        sel = np.asarray([int(c) for c in topk_row if int(c) >= 0], dtype=np.int64)
    if np.any(sel >= n):
        err |= EFLAG_TOPK_RANGE
    sel = sel[sel < n]
    crows, cok = _physical_rows(cmp_block_table[b], num_cmp_blocks, sel)
    if not cok.all():
        err |= EFLAG_BLOCK_RANGE
    return wrows[wok], crows[cok], err


def sparse_attn(q, rope_cos, rope_sin, rope_offset, cmp_kv, cmp_block_table,
                topk_idx, ratio, win_kv, win_block_table, window, attn_sink,
                softmax_scale, query_start_loc, positions, num_tokens, k=None):
    """Shared-KV multi-head attention over the window rows and the selected
    compressed rows, with one sink logit per head.

    [HP] Stage-2 call (sinks = attn_sink, softmax_scale, ori_win_left = 127,
    ori_win_right = 0) and 9.1 (union of window and compressed rows); all
    heads share one KV row, which serves as both key and value ([MTP]: one
    BF16 KV cache per layer).  For each head h of active row t:

        q      = BF16 query with channels [off, off + R) rotated by rope row t
        l_j    = softmax_scale * <q, K_j>          for each row j of the set
        M      = max(sink_h, max_j l_j)
        Z      = exp(sink_h - M) + sum_j exp(l_j - M)
        out    = sum_j exp(l_j - M) / Z * K_j
        lse    = M + log Z

    topk_idx None (with the bound k) selects every causally visible
    compressed row (deterministic_selection: the HCA layers); a selection
    with no columns leaves the window alone (the SWA-only layers of [MTP]
    "Layer schedule": sliding window only, no compressor, no indexer).

    Contract checks: an active row that no request owns flags META and is
    treated as having no keys; window pages with invalid block ids, and
    selected entries that are not visible (TOPK_RANGE) or sit on invalid
    pages (BLOCK_RANGE), are flagged and left out; negative selected entries
    are padding.

    cmp_kv and win_kv are BF16 caches [blocks, 128, D] (uint16 bit patterns)
    or KvPlane row sources (the low-bit planes, dequantised on read).

    Returns (out float64 [num_tokens, H, D], lse float64 [num_tokens, H], err)."""
    nt = int(num_tokens)
    T, H, D = q.shape
    half = rope_cos.shape[1]
    qsl = np.asarray(query_start_loc)
    cmp_src = cmp_kv if isinstance(cmp_kv, KvPlane) else bf16_plane(cmp_kv)
    win_src = win_kv if isinstance(win_kv, KvPlane) else bf16_plane(win_kv)
    ncb = cmp_src.num_blocks
    nwb = win_src.num_blocks
    sink = np.asarray(attn_sink, dtype=np.float64)
    out = np.zeros((nt, H, D), dtype=np.float64)
    lse = np.zeros((nt, H), dtype=np.float64)
    err = 0
    for t in range(nt):
        b = owner_request(t, qsl)
        if b < 0:
            err |= EFLAG_META
            out[t] = 0.0
            lse[t] = sink
            continue
        p = int(positions[t])
        wrows, crows, e = kv_rows_for_query(t, b, p, None if topk_idx is None else topk_idx[t],
                                            ratio, window, cmp_block_table, ncb,
                                            win_block_table, nwb, k)
        err |= e
        kv = np.concatenate([win_src.rows(wrows).reshape(-1, D),
                             cmp_src.rows(crows).reshape(-1, D)], axis=0)
        qt = bf16_to_f64(q[t])                                          # [H, D]
        qt[:, rope_offset:rope_offset + 2 * half] = rotate_adjacent_pairs(
            qt[:, rope_offset:rope_offset + 2 * half], rope_cos[t], rope_sin[t])
        if kv.shape[0] == 0:
            out[t] = 0.0
            lse[t] = sink
            continue
        logits = softmax_scale * (qt @ kv.T)                            # [H, n]
        m = np.maximum(sink, logits.max(axis=1))                        # [H]
        e_kv = np.exp(logits - m[:, None])
        z = np.exp(sink - m) + e_kv.sum(axis=1)
        out[t] = (e_kv / z[:, None]) @ kv
        lse[t] = m + np.log(z)
    return out, lse, err
