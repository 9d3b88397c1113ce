"""The device-side precondition check (mla_check_pages) against the plain
rule it enforces: every length in [0, 64 * max_pages], every block-table
entry a valid length uses in [0, num_pages); entries past a sequence's last
page (pads) and the pages of a sequence with an invalid length are not
checked. Violations are planted in host arrays; the check kernel reads the
table only where a valid length reaches, so no decode runs on them."""
import numpy as np
import pytest

from workloads import CONFIGS, make_inputs
from gpu_helpers import log

pytestmark = pytest.mark.gpu


def expected(block_table, seqlens, num_pages):
    B, max_pages = block_table.shape
    count, first = 0, None
    for b in range(B):
        L = int(seqlens[b])
        if not 0 <= L <= 64 * max_pages:
            count += 1
            first = first or (b, -1, L)
            continue
        for j in range((L + 63) // 64):
            page = int(block_table[b, j])
            if not 0 <= page < num_pages:
                count += 1
                first = first or (b, j, page)
    return [count, *(first if first else (-1, 0, 0))]


def run(block_table, seqlens, num_pages, dev):
    import torch
    import mla_paged_kv_03_amd as lib
    st = lib.mla_check_pages(torch.from_numpy(block_table).to(dev),
                             torch.from_numpy(seqlens).to(dev), num_pages)
    torch.cuda.synchronize()
    return st.cpu().tolist()


def _inputs():
    cfg = CONFIGS[3].with_(batch=40)
    d = make_inputs(cfg, seed=21)
    return (np.ascontiguousarray(d["block_table"]), np.ascontiguousarray(d["cache_seqlens"]),
            d["kv"].shape[0])


def test_clean_inputs_report_nothing(dev):
    bt, sl, P = _inputs()
    log(f"[case] check pages clean: B={len(sl)} max_pages={bt.shape[1]}")
    assert run(bt, sl, P, dev) == [0, -1, 0, 0] == expected(bt, sl, P)


def test_planted_violations_are_counted_and_the_first_is_named(dev):
    bt, sl, P = _inputs()
    B, max_pages = bt.shape
    used = [b for b in range(B) if sl[b] > 64]
    b1, b2 = used[2], used[5]
    bt[b1, 0] = P               # one past the pool
    bt[b2, 1] = -7              # negative entry in a used slot
    short = [b for b in range(B) if 0 < sl[b] < 64 * (max_pages - 1)]
    bt[short[0], (sl[short[0]] + 63) // 64] = 10 ** 9   # a pad: never checked
    sl[used[7]] = 64 * max_pages + 1                     # a length the table cannot hold
    sl[used[9]] = -3
    want = expected(bt, sl, P)
    log(f"[case] check pages planted: expect {want}")
    assert want[0] == 4
    assert run(bt, sl, P, dev) == want


def test_length_at_the_table_limit_and_empty_batch(dev):
    bt, sl, P = _inputs()
    sl[0] = 64 * bt.shape[1]                 # exactly fills the row: valid
    bt[0, :] = np.arange(bt.shape[1]) % P
    assert run(bt, sl, P, dev) == expected(bt, sl, P) == [0, -1, 0, 0]
    empty = np.zeros((0, 4), np.int32)
    assert run(empty, np.zeros(0, np.int32), P, dev) == [0, -1, 0, 0]
