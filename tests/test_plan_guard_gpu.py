"""A plan passed to the decode call through the C interface must have been
made for the call's geometry. The plan's metadata opens with a signature
(batch, workers, s_q * h_q, h_kv, value width); the decode and merge kernels
check it on the device and, for a plan made for another shape, leave out
and lse exactly as they were instead of indexing records and slots laid out
for that other shape. The Python binding refuses such plans on the host, so
these tests call the C entry points directly."""
import ctypes

import numpy as np
import pytest

from gpu_helpers import check, inputs, log, run_oracle, to_device
from test_parity_gpu import _gqa, _mla

pytestmark = pytest.mark.gpu

SENTINEL_OUT = 0x7BCD  # a finite bf16 pattern no decode produces here by chance
SENTINEL_LSE = 12345.5


def _call(d, t, plan, T, H, G, ws_bytes):
    """Decode through the C ABI with the given plan; out/lse start as
    sentinels. Returns (status, out bits, lse)."""
    import torch
    import mla_paged_kv_03_amd as lib
    from mla_paged_kv_03_amd import _lib
    cfg = d["cfg"]
    B = cfg.batch
    dv = cfg.d_v
    out = torch.full((B, T, H, dv), 0, dtype=torch.int16, device=t["q"].device)
    out.fill_(SENTINEL_OUT)
    out = out.view(torch.bfloat16)
    lse = torch.full((B, T, H), SENTINEL_LSE, dtype=torch.float32, device=t["q"].device)
    ws = torch.empty(ws_bytes // 4 + 64, dtype=torch.float32, device=t["q"].device)
    p = ws.data_ptr()
    wsp = ctypes.c_void_p(p + (-p) % 256)
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    L = _lib.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if cfg.kind == "mla":
        rc = L.mla_decode(P(t["q"]), P(t["kv"]), P(t["block_table"]), P(t["cache_seqlens"]), B,
                          T, H, t["kv"].shape[0], t["block_table"].shape[1], cfg.scale,
                          int(cfg.causal), P(plan.sched_metadata), P(plan.num_splits), wsp,
                          ws_bytes, P(out), P(lse), stream)
    else:
        rc = L.gqa_decode(P(t["q"]), P(t["k"]), P(t["v"]), P(t["block_table"]),
                          P(t["cache_seqlens"]), B, T, H, G, t["k"].shape[0],
                          t["block_table"].shape[1], cfg.scale, int(cfg.causal),
                          P(plan.sched_metadata), P(plan.num_splits), wsp, ws_bytes, P(out),
                          P(lse), stream)
    torch.cuda.synchronize()
    return rc, out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()


def _untouched(out_bits, lse):
    return bool((out_bits == SENTINEL_OUT).all() and (lse == SENTINEL_LSE).all())


def test_plan_for_another_row_count_leaves_outputs_untouched(dev):
    import mla_paged_kv_03_amd as lib
    cfg = _mla(4, 2, 128, (5000, 64, 3000, 1), True)
    d = inputs(cfg, seed=21)
    t = to_device(d, dev)
    need = lib.plan_info(4, 2, 128).workspace_bytes
    wrong = lib.mla_decode_plan(t["cache_seqlens"], 1, 128)      # made for s_q = 1
    log("[case] mla plan s_q=1 used for s_q=2")
    rc, ob, lse = _call(d, t, wrong, 2, 128, 1, max(need, 256))
    assert rc == 0 and _untouched(ob, lse)
    right = lib.mla_decode_plan(t["cache_seqlens"], 2, 128)
    rc, ob, lse = _call(d, t, right, 2, 128, 1, max(need, 256))
    assert rc == 0
    import torch
    out = torch.from_numpy(ob).view(torch.bfloat16).float().double().numpy()
    ref_out, ref_lse = run_oracle(d)
    check(out, lse.astype(np.float64), ref_out, ref_lse, "right plan after a wrong one")


def test_plan_for_another_batch_leaves_outputs_untouched(dev):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = _mla(5, 1, 128, (4096, 100, 20000, 700, 64), False)
    d = inputs(cfg, seed=22)
    t = to_device(d, dev)
    need = lib.plan_info(5, 1, 128).workspace_bytes
    # made for the first three sequences only: its slot prefix has 4 entries
    wrong = lib.mla_decode_plan(t["cache_seqlens"][:3].contiguous(), 1, 128)
    log("[case] mla plan for batch 3 used for batch 5")
    rc, ob, lse = _call(d, t, wrong, 1, 128, 1, max(need, 256))
    assert rc == 0 and _untouched(ob, lse)


def test_plan_for_other_kv_heads_leaves_outputs_untouched(dev):
    import mla_paged_kv_03_amd as lib
    cfg = _gqa(3, 1, 64, 8, (9000, 70, 2000))
    d = inputs(cfg, seed=23)
    t = to_device(d, dev)
    need = lib.plan_info(3, 1, 64, 8, 128).workspace_bytes
    wrong = lib.mla_decode_plan(t["cache_seqlens"], 1, 64, 4, 128)   # h_kv = 4
    log("[case] gqa plan for h_kv=4 used for h_kv=8")
    rc, ob, lse = _call(d, t, wrong, 1, 64, 8, max(need, 256))
    assert rc == 0 and _untouched(ob, lse)


def test_fp8_decode_takes_its_own_plan_at_128_heads(dev):
    """From 128 query rows per KV head on, the FP8 decode's plan (64-row
    workgroups: a worker per CU and row block) differs from the bf16
    decode's: the bf16 plan leaves the FP8 decode's outputs untouched, the
    FP8 plan gives the binding's result bit for bit. Below 128 rows the two
    plans have the same sizes."""
    import torch
    import mla_paged_kv_03_amd as lib
    from mla_paged_kv_03_amd import _lib
    for s_q, h_q in [(1, 8), (1, 16), (2, 32)]:
        a, b = lib.plan_info(4, s_q, h_q), lib.plan_info(4, s_q, h_q, kv_fp8=True)
        assert (a.num_workers, a.metadata_bytes, a.workspace_bytes) == \
            (b.num_workers, b.metadata_bytes, b.workspace_bytes)
    a, b = lib.plan_info(4, 1, 128), lib.plan_info(4, 1, 128, kv_fp8=True)
    assert b.row_blocks == 2 and 2 * b.num_workers == a.num_workers
    cfg = _mla(4, 1, 128, (5000, 64, 3000, 1), False)
    d = inputs(cfg, seed=24)
    t = to_device(d, dev)
    codes, scales = lib.mla_kv_quantize_fp8(t["kv"])
    B, T, H = 4, 1, 128
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    L = _lib.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(plan):
        need = max(plan.info.workspace_bytes, 256)
        ws = torch.empty(need // 4 + 64, dtype=torch.float32, device=dev)
        p = ws.data_ptr()
        out = torch.full((B, T, H, 512), SENTINEL_OUT, dtype=torch.int16, device=dev)
        lse = torch.full((B, T, H), SENTINEL_LSE, dtype=torch.float32, device=dev)
        rc = L.mla_decode_fp8(P(t["q"]), P(codes), P(scales), P(t["block_table"]),
                              P(t["cache_seqlens"]), B, T, H, codes.shape[0],
                              t["block_table"].shape[1], cfg.scale, int(cfg.causal),
                              P(plan.sched_metadata), P(plan.num_splits),
                              ctypes.c_void_p(p + (-p) % 256), need, P(out), P(lse), stream)
        torch.cuda.synchronize()
        return rc, out.cpu().numpy(), lse.cpu().numpy()

    log("[case] fp8 decode at 128 heads with the bf16 plan")
    rc, ob, lse = call(lib.mla_decode_plan(t["cache_seqlens"], T, H))
    assert rc == 0 and _untouched(ob, lse)
    log("[case] fp8 decode at 128 heads with its own plan")
    rc, ob, lse = call(lib.mla_decode_plan(t["cache_seqlens"], T, H, kv_fp8=True))
    assert rc == 0
    ref_o, ref_l = lib.mla_decode_fp8(t["q"], codes, scales, t["block_table"],
                                      t["cache_seqlens"], cfg.scale, cfg.causal)
    torch.cuda.synchronize()
    assert np.array_equal(ob, ref_o.view(torch.int16).cpu().numpy())
    assert np.array_equal(lse, ref_l.cpu().numpy())
