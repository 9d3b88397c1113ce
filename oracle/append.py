"""Paged KV append on the CPU: the oracle.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library neither
imports nor calls it, and it shares no code with the GPU path.

What it computes. Before a decode step reads the cache, the step's new
tokens are written into it: the KV cache is kept in 64-token pages (FlashMLA
blog, "기술 기반"), token j of sequence b living in physical page
block_table[b, j // 64], slot j % 64 (PagedAttention, among the related
techniques of the Flash Attention wiki note, "지식 연결 (Graph)"). The lengths
passed to decode already count the T new tokens, so new token t of sequence
b is position p = L_b - T + t, the same alignment as causal decode (see
attention.py).

Readings where the pages are silent (listed in the design notes):
  * A token with p < 0 (a sequence holding fewer than T tokens) is not
    written.
  * A block-table entry outside [0, num_pages) is not written through.

Arrays are numpy: the cache as bf16 bit patterns uint16 [P, 64, G, D], the
new rows [B, T, G, D] of the same dtype, int32 block_table [B, max_pages],
int32 seqlens [B]. Bytes are copied, nothing is computed.
"""
from __future__ import annotations

import numpy as np

PAGE = 64


def new_token_slots(block_table, seqlens, T):
    """The (b, t, page, slot) of every new token that is written, in order."""
    out = []
    for b in range(len(seqlens)):
        L = int(seqlens[b])
        for t in range(T):
            p = L - T + t
            if p < 0:
                continue
            out.append((b, t, int(block_table[b, p // PAGE]), p % PAGE))
    return out


def append_rows(cache, new, block_table, seqlens):
    """A copy of `cache` with the new tokens' rows written into their slots."""
    cache = np.array(cache, copy=True)
    num_pages = cache.shape[0]
    T = new.shape[1]
    for b, t, page, slot in new_token_slots(block_table, seqlens, T):
        if 0 <= page < num_pages:
            cache[page, slot] = new[b, t]
    return cache
