"""Helpers that build small paged inputs from dense logical arrays (tests only).

They lay logical rows into 128-row pages through a block table, so a test can
compute the expected result on the dense rows by an independent route.
"""
from __future__ import annotations

import numpy as np

PAGE = 128


def paged_pool(dense_per_request, block_tables, num_blocks, fill=0):
    """dense_per_request[b]: array [n_b, ...] of logical rows of request b.
    block_tables: int array [B, max_blocks].  Returns pool [num_blocks, 128, ...]
    with row c of request b stored at block block_tables[b][c // 128], slot c % 128.
    Rows past what the table covers are dropped."""
    sample = np.asarray(dense_per_request[0])
    pool = np.full((num_blocks, PAGE) + sample.shape[1:], fill, dtype=sample.dtype)
    for b, rows in enumerate(dense_per_request):
        rows = np.asarray(rows)
        for c in range(min(rows.shape[0], PAGE * len(block_tables[b]))):
            pool[block_tables[b][c // PAGE], c % PAGE] = rows[c]
    return pool


def bf16_bits(x):
    """float -> bf16 bits, round to nearest even (finite inputs)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_value(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def random_block_table(rng, B, pages, extra=0):
    """Disjoint shuffled pages for B requests in one pool of B*pages+extra blocks."""
    nb = B * pages + extra
    perm = rng.permutation(nb).astype(np.int32)
    return perm[: B * pages].reshape(B, pages), nb
