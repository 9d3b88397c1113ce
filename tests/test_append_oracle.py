"""Pins of the paged-KV-append oracle (CPU): the generator's page layout
rebuilt token by token, exactly the new tokens' slots changing, short
sequences, out-of-cache block-table entries, and a hand-worked example."""
import numpy as np
import pytest

import oracle
from workloads import CONFIGS, make_inputs

SENTINEL = 0xFFFF


def _row(cache, bt, b, j):
    return cache[bt[b, j // 64], j % 64]


@pytest.mark.parametrize("cfg_id", [1, 3])
@pytest.mark.parametrize("T", [1, 3, 64])
def test_appending_a_sequence_chunk_by_chunk_rebuilds_the_generated_cache(cfg_id, T):
    """The generator lays token j of sequence b at page bt[b, j // 64], slot
    j % 64. Starting from a cache of sentinels and appending every sequence's
    tokens T at a time (lengths counting the new tokens) must give back the
    generated cache on every live slot and leave every other slot alone."""
    cfg = CONFIGS[cfg_id]
    if cfg_id == 3:  # keep the fp64-free check quick: the first 12 sequences
        cfg = cfg.with_(batch=12)
    d = make_inputs(cfg)
    gen, bt, L = d["kv"], d["block_table"], d["cache_seqlens"]
    cache = np.full_like(gen, SENTINEL)
    for b in range(cfg.batch):
        cur = 0
        while cur < L[b]:
            n = min(T, int(L[b]) - cur)
            new = np.stack([_row(gen, bt, b, j) for j in range(cur, cur + n)])[None]
            cache = oracle.append_rows(cache, new, bt[b:b + 1], np.array([cur + n], np.int32))
            cur += n
    live = np.zeros(gen.shape[:2], bool)
    for b in range(cfg.batch):
        for j in range(int(L[b])):
            live[bt[b, j // 64], j % 64] = True
    assert np.array_equal(cache[live], gen[live])
    assert (cache[~live] == SENTINEL).all()


def test_only_the_new_tokens_slots_change():
    rng = np.random.default_rng(0)
    P, G, D, B, T = 24, 2, 8, 5, 3
    cache = rng.integers(0, 1 << 16, size=(P, 64, G, D), dtype=np.uint16)
    L = np.array([1, 3, 64, 65, 130], np.int32)
    bt = rng.permutation(P)[:B * 3].reshape(B, 3).astype(np.int32)
    new = (rng.integers(0, 1 << 15, size=(B, T, G, D), dtype=np.uint16) | 0x8000).astype(np.uint16)
    out = oracle.append_rows(cache, new, bt, L)
    expect = {}
    for b in range(B):
        for t in range(T):
            p = int(L[b]) - T + t
            if p >= 0:
                expect[(int(bt[b, p // 64]), p % 64)] = new[b, t]
    changed = {(int(pg), int(sl)) for pg, sl in zip(*np.nonzero((out != cache).any(axis=(2, 3))))}
    assert changed == set(expect)
    for (pg, sl), row in expect.items():
        assert np.array_equal(out[pg, sl], row)


def test_a_sequence_shorter_than_the_new_tokens_keeps_only_its_last_ones():
    cache = np.zeros((2, 64, 1, 4), np.uint16)
    new = np.arange(1, 21, dtype=np.uint16).reshape(1, 5, 1, 4)  # 5 new tokens
    out = oracle.append_rows(cache, new, np.array([[1, 0]], np.int32), np.array([2], np.int32))
    # L = 2 < T = 5: positions 0 and 1 hold new tokens 3 and 4
    assert np.array_equal(out[1, 0, 0], new[0, 3, 0])
    assert np.array_equal(out[1, 1, 0], new[0, 4, 0])
    assert (out[1, 2:] == 0).all() and (out[0] == 0).all()


def test_block_table_entries_outside_the_cache_are_not_written():
    cache = np.zeros((2, 64, 1, 4), np.uint16)
    new = np.ones((2, 1, 1, 4), np.uint16)
    bt = np.array([[-1, 0], [7, 1]], np.int32)
    out = oracle.append_rows(cache, new, bt, np.array([1, 1], np.int32))
    assert (out == 0).all()


def test_worked_example_crossing_a_page_boundary():
    """Two new tokens after 63 cached ones: lengths 65, positions 63 and 64,
    i.e. the last slot of the first page and the first slot of the second."""
    cache = np.zeros((3, 64, 1, 2), np.uint16)
    new = np.array([[[[11, 12]], [[21, 22]]]], np.uint16)  # [B=1, T=2, 1, 2]
    out = oracle.append_rows(cache, new, np.array([[2, 0]], np.int32), np.array([65], np.int32))
    assert out[2, 63, 0].tolist() == [11, 12]
    assert out[0, 0, 0].tolist() == [21, 22]
    assert int((out != 0).sum()) == 4
