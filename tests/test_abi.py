"""The C interface without a GPU: the library loads and exports every symbol
the header declares, argument errors come back as status codes before any
device work, and the split-KV schedule covers every page exactly once."""
import ctypes
import os

import numpy as np
import pytest

from mla_paged_kv_03_amd import _lib, mla_decode_plan_host, PlanInfo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REC = 8
HDR = 8  # plan signature words ahead of the worker records
FIX_DEFAULT, FIX_LATENT128 = 2, 6  # schedule.h


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_every_declared_function_is_exported(L):
    names = _lib.header_functions()
    assert {"mla_decode_plan", "mla_decode", "gqa_decode", "attn_combine", "mla_kv_append",
            "gqa_kv_append", "gqla_expand_kv", "gqla_absorb_query", "gqla_absorb_output",
            "gqla_decode", "mla_decode_fp8", "mla_kv_append_fp8",
            "mla_kv_quantize_fp8", "mla_check_pages", "mla_decode_noalloc",
            "mla_check_fp8_scales", "mla_decode_plan_fp8"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.mla_status_string(code) != b"unknown status"
    assert L.mla_status_string(7) == b"unknown status"


NULL = None


def _mla(L, **kw):
    args = dict(q=ctypes.c_void_p(16), kv=ctypes.c_void_p(32), bt=ctypes.c_void_p(48),
                sl=ctypes.c_void_p(64), B=2, T=1, H=8, P=5, maxp=4, scale=0.07, causal=0,
                meta=ctypes.c_void_p(80), splits=ctypes.c_void_p(96), ws=None, wsb=0,
                out=ctypes.c_void_p(112), lse=ctypes.c_void_p(128))
    args.update(kw)
    a = args
    return L.mla_decode(a["q"], a["kv"], a["bt"], a["sl"], a["B"], a["T"], a["H"], a["P"],
                        a["maxp"], a["scale"], a["causal"], a["meta"], a["splits"], a["ws"],
                        a["wsb"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(kv=None), -1), (dict(bt=None), -1), (dict(sl=None), -1),
    (dict(meta=None), -1), (dict(splits=None), -1), (dict(out=None), -1), (dict(lse=None), -1),
    (dict(B=-1), -2), (dict(T=0), -2), (dict(H=0), -2), (dict(P=0), -2), (dict(maxp=0), -2),
    (dict(causal=2), -2), (dict(scale=float("nan")), -2), (dict(scale=float("inf")), -2),
    (dict(q=ctypes.c_void_p(18)), -2), (dict(out=ctypes.c_void_p(8)), -2),
    (dict(T=1 << 11, H=1 << 10), -3),
])
def test_mla_decode_rejects_bad_arguments_before_device_work(L, kw, code):
    assert _mla(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(kv=None), -1), (dict(bt=None), -1), (dict(sl=None), -1),
    (dict(out=None), -1), (dict(lse=None), -1), (dict(B=-1), -2), (dict(T=0), -2),
    (dict(P=0), -2), (dict(causal=2), -2), (dict(scale=float("nan")), -2),
    (dict(q=ctypes.c_void_p(18)), -2), (dict(T=1 << 11, H=1 << 10), -3), (dict(B=0), 0),
])
def test_noalloc_rejects_bad_arguments_before_device_work(L, kw, code):
    a = dict(q=ctypes.c_void_p(16), kv=ctypes.c_void_p(32), bt=ctypes.c_void_p(48),
             sl=ctypes.c_void_p(64), B=2, T=1, H=8, P=5, maxp=4, scale=0.07, causal=0,
             out=ctypes.c_void_p(112), lse=ctypes.c_void_p(128))
    a.update(kw)
    assert L.mla_decode_noalloc(a["q"], a["kv"], a["bt"], a["sl"], a["B"], a["T"], a["H"],
                                a["P"], a["maxp"], a["scale"], a["causal"], a["out"], a["lse"],
                                None) == code


def test_gqa_rejects_bad_group_count(L):
    p = ctypes.c_void_p(16)
    rc = L.gqa_decode(p, p, p, p, p, 2, 1, 12, 5, 3, 4, 0.1, 0, p, p, None, 0, p, p, None)
    assert rc == -2  # 12 heads are not a multiple of 5 KV heads
    rc = L.gqa_decode(p, p, None, p, p, 2, 1, 16, 4, 3, 4, 0.1, 0, p, p, None, 0, p, p, None)
    assert rc == -1  # no V cache


def test_plan_rejects_unsupported_shapes(L):
    info = PlanInfo()
    assert L.mla_decode_plan(None, 2, 1, 8, 1, 512, None, None, None, None) == -1
    assert L.mla_decode_plan(None, 2, 1, 8, 2, 512, None, None, ctypes.byref(info), None) == -3
    assert L.mla_decode_plan(None, 2, 1, 8, 1, 256, None, None, ctypes.byref(info), None) == -3
    assert L.mla_decode_plan(None, 2, 1, 8, 3, 128, None, None, ctypes.byref(info), None) == -2
    p = ctypes.c_void_p(64)
    assert L.mla_decode_plan(None, 2, 1, 8, 1, 512, p, p, ctypes.byref(info), None) == -1


def test_attn_combine_argument_checks(L):
    p = ctypes.c_void_p(64)
    assert L.attn_combine(p, p, p, 2, 4, 12, p, p, None) == -2      # dv not a multiple of 8
    assert L.attn_combine(None, p, p, 2, 4, 16, p, p, None) == -1
    assert L.attn_combine(p, p, p, 0, 4, 16, p, p, None) == 0        # nothing to do


def test_check_pages_argument_checks(L):
    p = ctypes.c_void_p(64)
    # block_table, cache_seqlens, batch, num_pages, max_pages, status, stream
    assert L.mla_check_pages(p, p, 2, 10, 4, None, None) == -1          # no status word
    assert L.mla_check_pages(None, p, 2, 10, 4, p, None) == -1
    assert L.mla_check_pages(p, None, 2, 10, 4, p, None) == -1
    assert L.mla_check_pages(p, p, -1, 10, 4, p, None) == -2
    assert L.mla_check_pages(p, p, 2, 0, 4, p, None) == -2
    assert L.mla_check_pages(p, p, 2, 10, 0, p, None) == -2
    assert L.mla_check_pages(p, p, 2, 10, 4, ctypes.c_void_p(66), None) == -2


def test_fp8_plan_argument_checks(L):
    """The FP8 decode's plan checks its arguments as mla_decode_plan does
    (the sizes need a device: tests/test_plan_guard_gpu.py)."""
    info = PlanInfo()
    assert L.mla_decode_plan_fp8(None, 2, 1, 8, None, None, None, None) == -1
    assert L.mla_decode_plan_fp8(None, -1, 1, 8, None, None, ctypes.byref(info), None) == -2
    assert L.mla_decode_plan_fp8(None, 2, 0, 8, None, None, ctypes.byref(info), None) == -2
    p = ctypes.c_void_p(64)
    assert L.mla_decode_plan_fp8(None, 2, 1, 8, p, p, ctypes.byref(info), None) == -1
    assert L.mla_decode_plan_fp8(None, 2, 1, 8, p, None, ctypes.byref(info), None) == -1


def test_check_fp8_scales_argument_checks(L):
    p = ctypes.c_void_p(64)
    assert L.mla_check_fp8_scales(p, 10, None, None) == -1             # no status word
    assert L.mla_check_fp8_scales(None, 10, p, None) == -1
    assert L.mla_check_fp8_scales(p, -1, p, None) == -2
    assert L.mla_check_fp8_scales(ctypes.c_void_p(66), 10, p, None) == -2   # unaligned scales
    assert L.mla_check_fp8_scales(p, 10, ctypes.c_void_p(66), None) == -2   # unaligned status


def test_kv_append_argument_checks(L):
    p = ctypes.c_void_p(64)
    # new_kv, kv_cache, block_table, cache_seqlens, batch, s_q, num_pages, max_pages
    assert L.mla_kv_append(p, p, p, p, 0, 1, 4, 4, None) == 0          # nothing to do
    assert L.mla_kv_append(None, p, p, p, 2, 1, 4, 4, None) == -1
    assert L.mla_kv_append(p, None, p, p, 2, 1, 4, 4, None) == -1
    assert L.mla_kv_append(p, p, p, None, 2, 1, 4, 4, None) == -1
    assert L.mla_kv_append(p, p, p, p, -1, 1, 4, 4, None) == -2
    assert L.mla_kv_append(p, p, p, p, 2, 0, 4, 4, None) == -2
    assert L.mla_kv_append(ctypes.c_void_p(72), p, p, p, 2, 1, 4, 4, None) == -2  # unaligned
    assert L.mla_kv_append(p, p, p, p, 1 << 20, 1 << 12, 4, 4, None) == -3
    # gqa: new_k, new_v, k_cache, v_cache, bt, sl, batch, s_q, h_kv, num_pages, max_pages
    assert L.gqa_kv_append(p, None, p, p, p, p, 2, 1, 8, 4, 4, None) == -1
    assert L.gqa_kv_append(p, p, p, None, p, p, 2, 1, 8, 4, 4, None) == -1
    assert L.gqa_kv_append(p, p, p, p, p, p, 2, 1, 0, 4, 4, None) == -2
    assert L.gqa_kv_append(p, p, p, p, p, p, 0, 1, 8, 4, 4, None) == 0


def test_gqla_argument_checks(L):
    p = ctypes.c_void_p(64)
    # q, w_uk, q_absorbed, n_tokens, h_q, h_kv
    assert L.gqla_absorb_query(p, p, p, 0, 16, 4, None) == 0          # nothing to do
    assert L.gqla_absorb_query(None, p, p, 2, 16, 4, None) == -1
    assert L.gqla_absorb_query(p, p, None, 2, 16, 4, None) == -1
    assert L.gqla_absorb_query(p, p, p, 2, 16, 5, None) == -2        # 16 heads, 5 groups
    assert L.gqla_absorb_query(p, p, p, -1, 16, 4, None) == -2
    assert L.gqla_absorb_query(ctypes.c_void_p(72), p, p, 2, 16, 4, None) == -2
    assert L.gqla_absorb_query(p, p, p, 1 << 30, 16, 1, None) == -3
    assert L.gqla_absorb_output(p, None, p, 2, 16, 4, None) == -1
    assert L.gqla_absorb_output(p, p, p, 2, 0, 1, None) == -2
    # kv_rows, w_uk, w_uv, k_rows, v_rows, n_rows, h_kv
    assert L.gqla_expand_kv(p, p, p, p, p, 0, 8, None) == 0
    assert L.gqla_expand_kv(p, p, None, p, p, 64, 8, None) == -1
    assert L.gqla_expand_kv(p, p, p, p, p, 64, 0, None) == -2
    assert L.gqla_expand_kv(p, p, p, p, p, -1, 8, None) == -2
    assert L.gqla_expand_kv(p, p, p, p, p, 1 << 31, 8, None) == -3
    rc = L.gqla_decode(p, p, None, p, p, 2, 1, 16, 4, 3, 4, 0.1, 0, p, p, None, 0, p, p, None)
    assert rc == -1  # no V cache
    rc = L.gqla_decode(p, p, p, p, p, 2, 1, 12, 5, 3, 4, 0.1, 0, p, p, None, 0, p, p, None)
    assert rc == -2


def test_fp8_argument_checks(L):
    p = ctypes.c_void_p(64)
    args = dict(B=2, T=1, H=8, P=5, maxp=4)
    # q, codes, scales, bt, sl, B, T, H, P, maxp, scale, causal, meta, splits, ws, wsb, out, lse
    rc = L.mla_decode_fp8(p, p, None, p, p, 2, 1, 8, 5, 4, 0.07, 0, p, p, None, 0, p, p, None)
    assert rc == -1                                       # no scales
    rc = L.mla_decode_fp8(p, p, ctypes.c_void_p(66), p, p, 2, 1, 8, 5, 4, 0.07, 0, p, p, None, 0,
                          p, p, None)
    assert rc == -2                                       # misaligned scales
    rc = L.mla_decode_fp8(p, p, p, p, p, 2, 0, 8, 5, 4, 0.07, 0, p, p, None, 0, p, p, None)
    assert rc == -2
    # new_kv, codes, scales, bt, sl, batch, s_q, num_pages, max_pages
    assert L.mla_kv_append_fp8(p, p, p, p, p, 0, 1, 4, 4, None) == 0
    assert L.mla_kv_append_fp8(p, p, None, p, p, 2, 1, 4, 4, None) == -1
    assert L.mla_kv_append_fp8(p, ctypes.c_void_p(72), p, p, p, 2, 1, 4, 4, None) == -2
    assert L.mla_kv_append_fp8(p, p, p, p, p, 2, 0, 4, 4, None) == -2
    assert L.mla_kv_quantize_fp8(p, p, p, 0, None) == 0
    assert L.mla_kv_quantize_fp8(None, p, p, 4, None) == -1
    assert L.mla_kv_quantize_fp8(p, p, p, -1, None) == -2
    assert L.mla_kv_quantize_fp8(p, p, p, 1 << 31, None) == -3


# ------------------------------------------------------------ the schedule
def walk_schedule(seqlens, meta, splits, info):
    """Replay what the decode kernel does with a schedule: which worker
    processes which pages of which sequence, with which split slot."""
    W = info.num_workers
    B = len(seqlens)
    pages = [(int(L) + 63) // 64 for L in seqlens]
    seen = [np.zeros(n, dtype=int) for n in pages]
    owners_empty = [0] * B
    slot_users = {}
    for w in range(W):
        bs, ps, be, pe, split0, owns, lo, hi = meta[HDR + w * REC:HDR + (w + 1) * REC]
        for b in range(bs, be + 1):
            n = pages[b]
            p0 = ps if b == bs else 0
            p1 = pe if b == be else n
            if n == 0:
                if b > bs or owns:
                    owners_empty[b] += 1
                continue
            if p0 >= p1:
                continue
            seen[b][p0:p1] += 1
            nslots = splits[b + 1] - splits[b]
            split = split0 if b == bs else 0
            if nslots:
                assert 0 <= split < nslots
                key = splits[b] + split
                assert key not in slot_users, "two pieces write one slot"
                slot_users[key] = (b, p0, p1)
    return seen, owners_empty, slot_users


SCHEDULES = [
    [64, 200], [4096] * 64, [8192] * 256, [0, 0, 1, 0], [1], [0], [],
    list(np.random.default_rng(3).integers(0, 20000, size=128)),
    list(np.random.default_rng(4).integers(0, 70, size=300)),
    [1] * 1000 + [65536],
]


@pytest.mark.parametrize("seqlens", SCHEDULES)
@pytest.mark.parametrize("shape", [(1, 128, 1, 512), (2, 128, 1, 512), (1, 16, 1, 512),
                                   (1, 8, 1, 512), (1, 128, 8, 128), (3, 7, 1, 512)])
@pytest.mark.parametrize("cus", [256, 304, 7, 1])
def test_schedule_covers_every_page_once(seqlens, shape, cus):
    T, H, G, dv = shape
    meta, splits, info = mla_decode_plan_host(seqlens, T, H, G, dv, num_cus=cus)
    W = info.num_workers
    assert W >= 1 and (W < 8 or W % 8 == 0)
    seen, owners_empty, slot_users = walk_schedule(seqlens, meta, splits, info)
    for b, L in enumerate(seqlens):
        if L == 0:
            assert owners_empty[b] == 1, f"empty sequence {b} owned {owners_empty[b]} times"
        else:
            assert (seen[b] == 1).all(), f"sequence {b} pages covered {seen[b]}"
    # every slot of a split sequence is written, slots are within the bound
    assert splits[0] == 0 and (np.diff(splits) >= 0).all()
    assert splits[-1] <= info.max_split_slots
    assert sorted(slot_users) == list(range(splits[-1]))
    for b in range(len(seqlens)):
        assert splits[b + 1] - splits[b] != 1, "a single piece never uses a slot"
    # the line: each sequence is k blocks of `fix` overhead units and its
    # pages, k its share of the workers by cost (pages + fix), recorded
    # total T in the signature; fix is more for the 128-row latent decode,
    # whose queries and output weigh several pages
    fix = int(meta[6])
    assert fix == (FIX_LATENT128 if (G == 1 and dv == 512 and T * H >= 128) else FIX_DEFAULT)
    pages = [(int(L) + 63) // 64 for L in seqlens]
    cost = sum(p + fix for p in pages)
    assert int(meta[7]) == cost
    units = meta[HDR + W * REC:HDR + W * REC + len(seqlens) + 1]
    assert units[0] == 0
    for b, p in enumerate(pages):
        k = (units[b + 1] - units[b] - p) // fix
        assert units[b + 1] - units[b] == p + k * fix
        share = (2 * (p + fix) * W + cost) // (2 * cost) if cost else 1
        assert k == (1 if p == 0 else min(max(share, 1), p))


def _worker_costs(seqlens, meta, info):
    """Per worker: pages processed plus the overhead units of every piece."""
    W, fix = info.num_workers, int(meta[6])
    pages = [(int(L) + 63) // 64 for L in seqlens]
    costs = []
    for w in range(W):
        bs, ps, be, pe = meta[HDR + w * REC:HDR + w * REC + 4]
        c = 0
        for b in range(bs, be + 1):
            p0 = ps if b == bs else 0
            p1 = min(pe if b == be else pages[b], pages[b])
            if p1 > p0:
                c += p1 - p0 + fix
        costs.append(c)
    return costs


@pytest.mark.parametrize("seqlens", SCHEDULES + [
    list(np.random.default_rng(3).integers(1, 16385, size=128))])
def test_schedule_balances_work(seqlens):
    """Every worker's range is one chunk of the line; a worker pays at most
    one piece's overhead beyond the units in its range (when it starts a
    piece in the middle of a block)."""
    meta, splits, info = mla_decode_plan_host(seqlens, 2, 128, num_cus=256)
    W, fix = info.num_workers, int(meta[6])
    loads = [meta[HDR + w * REC + 7] - meta[HDR + w * REC + 6] for w in range(W)]
    total = int(meta[HDR + W * REC + len(seqlens)])
    chunk = max(-(-total // W), fix + 1)
    assert max(loads) <= chunk and sum(loads) == total
    assert max(_worker_costs(seqlens, meta, info)) <= chunk + fix


def test_equal_sequences_split_into_equal_pieces():
    """The DeepSeek-V3 decode batch (64 sequences of 4096 tokens, 128 heads)
    on 256 workers: every worker gets one piece of 16 pages."""
    seqlens = [4096] * 64
    meta, splits, info = mla_decode_plan_host(seqlens, 1, 128, num_cus=256)
    W = info.num_workers
    assert W == 256
    for w in range(W):
        bs, ps, be, pe = meta[HDR + w * REC:HDR + w * REC + 4]
        assert bs == be and pe - ps == 16, (w, bs, ps, be, pe)
    assert list(np.diff(splits)) == [4] * 64


def test_workspace_size_matches_slot_bound():
    _, _, info = mla_decode_plan_host([100] * 10, 2, 128, num_cus=256)
    rows = 2 * 128
    assert info.max_split_slots == 2 * (info.num_workers - 1)
    assert info.workspace_bytes >= info.max_split_slots * rows * (512 + 1) * 4


@pytest.mark.parametrize("shape", [(1, 128, 1, 512), (2, 128, 1, 512), (1, 128, 8, 128),
                                   (3, 7, 1, 512)])
def test_plan_opens_with_its_geometry(shape):
    """The metadata starts with a signature: a fixed tag, the worker count,
    the batch, the rows per sequence (s_q * h_q), the KV heads, the value
    width, the plan's overhead units per piece and the batch's total cost;
    the decode and merge kernels compare the first six with their own call."""
    T, H, G, dv = shape
    seqlens = [100, 0, 5000]
    meta, splits, info = mla_decode_plan_host(seqlens, T, H, G, dv, num_cus=256)
    assert info.metadata_bytes == 4 * (HDR + info.num_workers * REC + len(seqlens) + 1)
    assert list(meta[:6]) == [0x4D4C4150, info.num_workers, len(seqlens), T * H, G, dv]
    fix = FIX_LATENT128 if (G == 1 and dv == 512 and T * H >= 128) else FIX_DEFAULT
    cost = sum((L + 63) // 64 + fix for L in seqlens)
    assert list(meta[6:8]) == [fix, cost]


def test_page_range_is_clamped_to_current_lengths(tmp_path):
    """A plan reused after the lengths shrank (a stale plan) must never send
    a worker past the pages the current lengths reach: the kernel takes its
    page range from schedule.h's page_range, compiled here for the host and
    run over every worker and sequence of plans made for longer lengths."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    src = tmp_path / "range.cpp"
    csrc = os.path.join(ROOT, "mla_paged_kv_03_amd", "csrc")
    src.write_text(r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "schedule.h"
// argv: W, then B lengths of the plan, then B current lengths
int main(int argc, char** argv) {
  const int W = atoi(argv[1]);
  const int B = (argc - 2) / 2;
  std::vector<int32_t> Lp(B), Lc(B), meta(sched::HDR + W * sched::REC + B + 1);
  for (int b = 0; b < B; ++b) { Lp[b] = atoi(argv[2 + b]); Lc[b] = atoi(argv[2 + B + b]); }
  std::vector<int32_t> splits(B + 1);
  sched::host_plan(Lp.data(), B, W, 128, 1, 512, FIX, meta.data(), splits.data());
  long pairs = 0;
  for (int w = 0; w < W; ++w) {
    int32_t* rec = sched::records(meta.data()) + w * sched::REC;
    for (int b = rec[sched::R_B_START]; b <= rec[sched::R_B_END]; ++b) {
      const int npg = sched::seq_pages(Lc[b]);
      int p0, p1;
      sched::page_range(rec, b, rec[sched::R_B_START], rec[sched::R_B_END], npg, &p0, &p1);
      for (int j = p0; j < p1; ++j) {
        if (j < 0 || j >= npg) { printf("OUT %d %d %d\n", w, b, j); return 1; }
        ++pairs;
      }
    }
  }
  printf("OK %ld\n", pairs);
  return 0;
}
""")
    rng = np.random.default_rng(9)
    for fix, W in [(f, w) for f in (FIX_DEFAULT, FIX_LATENT128) for w in (1, 7, 64, 128)]:
        exe = tmp_path / f"range{fix}"
        if not exe.exists():
            subprocess.run([gxx, "-O1", "-std=c++17", f"-DFIX={fix}", "-I", csrc, str(src), "-o",
                            str(exe)], check=True)
        for _ in range(4):
            B = int(rng.integers(1, 40))
            plan_L = rng.integers(0, 5000, size=B)
            cur_L = (plan_L * rng.uniform(0, 1, size=B)).astype(int)  # shrunk
            res = subprocess.run([str(exe), str(W), *map(str, plan_L), *map(str, cur_L)],
                                 capture_output=True, text=True)
            assert res.returncode == 0, res.stdout
            # with the plan's own lengths every page is visited exactly once
            res = subprocess.run([str(exe), str(W), *map(str, plan_L), *map(str, plan_L)],
                                 capture_output=True, text=True)
            assert res.returncode == 0
            assert int(res.stdout.split()[1]) == int(sum((int(L) + 63) // 64 for L in plan_L))
