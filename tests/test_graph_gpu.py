"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph): plan,
decode and split merge (one launch or two), the paged append, the FP8
decode (both page paths) and the GQLA products record no allocation and no
memset, so a captured step replays.
Each replay runs on fresh inputs copied into the captured buffers, with
eager work in between, and must equal the eager result bit for bit."""
import ctypes

import numpy as np
import pytest

from workloads import CONFIGS, GQLA_CONFIGS, make_gqla_inputs, make_inputs
from gpu_helpers import bf16_tensor, log

pytestmark = pytest.mark.gpu


# mixed: 24 sequences, 2 causal tokens, 128 heads (the one-launch merge);
# few_long: two long sequences over 16 heads, split over many workers (the
# two-launch merge)
MLA_SHAPES = {
    "mixed": dict(batch=24, seqlen_rule="fixed",
                  seqlens_fixed=tuple([1, 70, 640, 3000, 64, 0] * 4)),
    "few_long": dict(batch=2, s_q=1, h_q=16, causal=False, seqlen_rule="fixed",
                     seqlens_fixed=(20000, 9000)),
}


def _mla_inputs(dev, seed, shape="mixed"):
    import torch
    cfg = CONFIGS[3].with_(**MLA_SHAPES[shape])
    d = make_inputs(cfg, seed=seed)
    return cfg, {"q": bf16_tensor(d["q"], dev), "kv": bf16_tensor(d["kv"], dev),
                 "bt": torch.from_numpy(d["block_table"]).to(dev),
                 "sl": torch.from_numpy(d["cache_seqlens"]).to(dev)}


@pytest.mark.parametrize("shape", list(MLA_SHAPES))
def test_captured_decode_step_replays_like_eager(dev, shape):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg, live = _mla_inputs(dev, 1, shape)
    B, T, H = cfg.batch, cfg.s_q, cfg.h_q
    plan = lib.mla_decode_plan(live["sl"], T, H, 1, 512)
    new_kv = torch.zeros(B, T, 576, dtype=torch.bfloat16, device=dev)
    out = torch.empty(B, T, H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=dev)

    def step():
        # re-plan, append the new tokens, decode (with the split merge)
        lib._lib.check("mla_decode_plan", lib._lib.lib().mla_decode_plan(
            lib._ptr(live["sl"]), B, T, H, 1, 512, lib._ptr(plan.sched_metadata),
            lib._ptr(plan.num_splits), ctypes.byref(plan.info), lib._stream()))
        lib.mla_kv_append(new_kv, live["kv"], live["bt"], live["sl"])
        lib.mla_decode(live["q"], live["kv"], live["bt"], live["sl"], cfg.scale, cfg.causal,
                       plan=plan, out=out, lse=lse)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        _, fresh = _mla_inputs(dev, 10 + r, shape)
        rng = np.random.default_rng(r)
        nk = torch.from_numpy(rng.standard_normal((B, T, 576)).astype(np.float32)).to(dev)
        for k in ("q", "kv", "bt", "sl"):
            live[k].copy_(fresh[k])
        new_kv.copy_(nk.to(torch.bfloat16))
        kv0 = live["kv"].clone()
        g.replay()
        torch.cuda.synchronize()
        got_out, got_lse, got_kv = out.clone(), lse.clone(), live["kv"].clone()
        # eager on the same inputs, with other work queued in between
        _ = torch.randn(1 << 20, device=dev).sum()
        live["kv"].copy_(kv0)
        step()
        torch.cuda.synchronize()
        log(f"[case] graph replay {shape} {r}")
        assert torch.equal(got_kv, live["kv"])
        assert torch.equal(got_out.view(torch.int16), out.view(torch.int16))
        assert torch.equal(got_lse, lse)


def test_captured_fp8_and_gqla_steps_replay_like_eager(dev):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = GQLA_CONFIGS["small"]
    d = make_gqla_inputs(cfg)
    t = {k: bf16_tensor(d[k], dev) for k in ("q", "kv", "w_uk", "w_uv")}
    bt = torch.from_numpy(d["block_table"]).to(dev)
    sl = torch.from_numpy(d["cache_seqlens"]).to(dev)
    B, T, H, G = cfg.batch, cfg.s_q, cfg.h_q, cfg.h_kv
    plan_a = lib.mla_decode_plan(sl, T, H, 1, 512)
    plan_8 = lib.mla_decode_plan(sl, T, H, 1, 512, kv_fp8=True)
    plan_g = lib.mla_decode_plan(sl, T, H, G, 128)
    codes, scales = lib.mla_kv_quantize_fp8(t["kv"])
    qa = torch.empty(B, T, H, 576, dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty(B, T, H, 512, dtype=torch.bfloat16, device=dev)
    o8 = torch.empty_like(o_lat)
    out_a = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=dev)
    out_g = torch.empty_like(out_a)
    lse = [torch.empty(B, T, H, dtype=torch.float32, device=dev) for _ in range(3)]
    k_rows, v_rows = lib.gqla_expand_kv(t["kv"], t["w_uk"], t["w_uv"])

    def step():
        lib.gqla_absorb_query(t["q"], t["w_uk"], out=qa)
        lib.mla_decode(qa, t["kv"], bt, sl, cfg.scale, cfg.causal, plan=plan_a, out=o_lat,
                       lse=lse[0])
        lib.gqla_absorb_output(o_lat, t["w_uv"], out=out_a)
        lib.gqla_expand_kv(t["kv"], t["w_uk"], t["w_uv"], k_rows, v_rows)
        lib.gqla_decode(t["q"], k_rows, v_rows, bt, sl, cfg.scale, cfg.causal, plan=plan_g,
                        out=out_g, lse=lse[1])
        lib.mla_kv_quantize_fp8(t["kv"], codes, scales)
        lib.mla_decode_fp8(qa, codes, scales, bt, sl, cfg.scale, cfg.causal, plan=plan_8,
                           out=o8, lse=lse[2])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    outs = (out_a, out_g, o8, *lse)
    for r in range(3):
        fresh = make_gqla_inputs(cfg, seed=40 + r)
        for k in ("q", "kv", "w_uk", "w_uv"):
            t[k].copy_(bf16_tensor(fresh[k], dev))
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in outs]
        _ = torch.randn(1 << 20, device=dev).sum()
        step()
        torch.cuda.synchronize()
        log(f"[case] graph replay (fp8, gqla) {r}")
        for a, b in zip(got, outs):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_captured_fp8_decode_at_64_rows_replays_like_eager(dev):
    """FP8 decode with 128 heads: 64 rows per workgroup, pages dequantised by
    the copy waves; quantise, plan and decode in one captured step."""
    import torch
    import mla_paged_kv_03_amd as lib
    cfg, live = _mla_inputs(dev, 2, "mixed")
    B, T, H = cfg.batch, cfg.s_q, cfg.h_q
    plan = lib.mla_decode_plan(live["sl"], T, H, 1, 512, kv_fp8=True)
    codes, scales = lib.mla_kv_quantize_fp8(live["kv"])
    out = torch.empty(B, T, H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=dev)

    def step():
        lib._lib.check("mla_decode_plan_fp8", lib._lib.lib().mla_decode_plan_fp8(
            lib._ptr(live["sl"]), B, T, H, lib._ptr(plan.sched_metadata),
            lib._ptr(plan.num_splits), ctypes.byref(plan.info), lib._stream()))
        lib.mla_kv_quantize_fp8(live["kv"], codes, scales)
        lib.mla_decode_fp8(live["q"], codes, scales, live["bt"], live["sl"], cfg.scale,
                           cfg.causal, plan=plan, out=out, lse=lse)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        _, fresh = _mla_inputs(dev, 20 + r, "mixed")
        for k in ("q", "kv", "bt", "sl"):
            live[k].copy_(fresh[k])
        g.replay()
        torch.cuda.synchronize()
        got_out, got_lse = out.clone(), lse.clone()
        _ = torch.randn(1 << 20, device=dev).sum()
        step()
        torch.cuda.synchronize()
        log(f"[case] graph replay (fp8, 64 rows) {r}")
        assert torch.equal(got_out.view(torch.int16), out.view(torch.int16))
        assert torch.equal(got_lse, lse)
