"""Benchmark of the paged MLA decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
    python bench.py --op append [--config N] [--append-tokens T]
    python bench.py --op gqla
    python bench.py --kv fp8 [--config 2|3|4]    (MLA decode over an FP8 latent cache)


One step is the whole path over one batch: the split-KV plan, the fused
decode kernel and the split merge (mla_decode_plan + mla_decode, or
gqa_decode for config 5), with inputs already resident in HBM. The default
workload is the DeepSeek-V3-shaped decode: batch 64, one query token, 128
heads, 576/512 head dims, every sequence 4096 tokens in 64-token pages.
Three independent input sets rotate between steps so the 256 MB Infinity
Cache cannot hold the working set.

Prints one JSON line: decode tokens/s (value), TFLOP/s and HBM GB/s against
MI355X peaks, the roofline of the dominant (decode) kernel timed by HIP
events on its stream, and the CPU oracle's rate on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode TFLOPS + HBM GB/s (% MI355X peak); decode tokens/s at B=64"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16: 256 CU x 2.4 GHz x 4096 flop/clk
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mla_paged_kv_03_amd", "csrc")


def decode_kernel_of(cfg, fp8=False):
    """(kernel name, source file) of the decode kernel a configuration runs:
    the 128-row latent kernel for a bf16 latent cache with s_q * h_q >= 128,
    else the 64-row kernel (GQA, FP8 cache, fewer rows)."""
    if cfg.kind == "mla" and not fp8 and cfg.s_q * cfg.h_q >= 128:
        return "decode128_kernel", os.path.join(CSRC, "decode128_kernels.hip")
    kind = "gqa" if cfg.kind == "gqa" else "mla fp8" if fp8 else "mla"
    return f"decode_kernel ({kind})", os.path.join(CSRC, "decode_kernels.hip")


def algorithmic_work(d, fp8=False):
    """Bytes and FLOPs an IO-optimal decode must move and compute: every
    valid cached token once (an FP8 latent row: 576 code bytes + a 4-byte
    scale), q, out and lse; 2 (d_qk + d_v) flop per (query row, visible
    key) pair."""
    cfg = d["cfg"]
    L = d["cache_seqlens"].astype(np.int64)
    tok_bytes = cfg.h_kv * (cfg.d_qk * 2 if cfg.kind == "mla" else (cfg.d_qk + cfg.d_v) * 2)
    if fp8:
        tok_bytes = cfg.d_qk + 4
    rows = cfg.batch * cfg.s_q * cfg.h_q
    kv = int(L.sum()) * tok_bytes
    qb = rows * cfg.d_qk * 2
    ob = rows * cfg.d_v * 2 + rows * 4
    pairs = 0
    for t in range(cfg.s_q):
        vis = np.clip(L - cfg.s_q + 1 + t, 0, L) if cfg.causal else L
        pairs += int(vis.sum()) * cfg.h_q
    flops = 2 * (cfg.d_qk + cfg.d_v) * pairs
    return {"bytes": kv + qb + ob, "kv_bytes": kv, "flops": flops, "rows": rows}


def stored_traffic(workload, kernel_src):
    """HBM bytes per decode launch of `workload` from its committed
    rocprofv3 counter summary, if that was taken on the current source of
    the kernel it runs; else None."""
    path = os.path.join(PROFILES, f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m1 = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    m2 = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    if not (m1 and m2):
        return None
    cur = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    return int(m1.group(1)) if m2.group(1) == cur else None


def cpu_baseline(d, budget_s=10.0):
    """The oracle as it stands, on the host cores, over whole sequences of
    the workload, in order and wrapping around, until about budget_s seconds
    of work are done (at least one sequence)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity set
        threads = len(os.sched_getaffinity(0))
    cfg = d["cfg"]
    done, t0 = 0, time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        idx = [done % cfg.batch]
        q = d["q"][idx]
        bt = d["block_table"][idx]
        L = d["cache_seqlens"][idx]
        if cfg.kind == "mla":
            oracle.attend_two_pass(q, d["kv"], bt, L, cfg.scale, cfg.causal, d_v=cfg.d_v)
        else:
            oracle.attend_two_pass(q, d["k"], bt, L, cfg.scale, cfg.causal, v_cache=d["v"])
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done * cfg.s_q / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} sequences of the same workload taken in order "
                      f"(batch {cfg.batch}; {done * cfg.s_q} query tokens, {dt:.1f} s, "
                      f"fp64 numpy)"}


def bench_append(args, cfg):
    """The paged KV append alone: T new tokens per sequence written into the
    config's cache (lengths count them), timed over back-to-back launches
    with events on the stream. Bytes moved: every written row read once and
    written once."""
    import torch
    import mla_paged_kv_03_amd as lib
    from mla_paged_kv_03_amd import _lib
    from workloads import make_inputs, f32_to_bf16_bits

    dev = torch.device("cuda:0")
    L = _lib.lib()
    T = args.append_tokens or cfg.s_q
    d = make_inputs(cfg)
    B = cfg.batch
    rng = np.random.default_rng(123)
    bt = torch.from_numpy(d["block_table"]).to(dev)
    sl = torch.from_numpy(d["cache_seqlens"]).to(dev)
    P = ctypes.c_void_p
    ptr = lambda x: P(x.data_ptr())
    stream = P(torch.cuda.current_stream().cuda_stream)
    tok = lambda shape: torch.from_numpy(
        f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32)).view(np.int16)).to(dev)
    if cfg.kind == "mla":
        new = tok((B, T, cfg.d_qk))
        cache = torch.from_numpy(d["kv"].view(np.int16)).to(dev)
        row_bytes = cfg.d_qk * 2

        def call():
            return L.mla_kv_append(ptr(new), ptr(cache), ptr(bt), ptr(sl), B, T, d["num_pages"],
                                   bt.shape[1], stream)
    else:
        nk, nv = tok((B, T, cfg.h_kv, cfg.d_qk)), tok((B, T, cfg.h_kv, cfg.d_v))
        kc = torch.from_numpy(d["k"].view(np.int16)).to(dev)
        vc = torch.from_numpy(d["v"].view(np.int16)).to(dev)
        row_bytes = cfg.h_kv * (cfg.d_qk + cfg.d_v) * 2

        def call():
            return L.gqa_kv_append(ptr(nk), ptr(nv), ptr(kc), ptr(vc), ptr(bt), ptr(sl), B, T,
                                   cfg.h_kv, d["num_pages"], bt.shape[1], stream)
    written = int(np.minimum(d["cache_seqlens"].astype(np.int64), T).sum())
    nbytes = 2 * written * row_bytes
    for _ in range(args.warmup):
        if call() != 0:
            raise RuntimeError("append failed")
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / args.steps * 1e3
    gbs = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "paged KV append GB/s (rows read + written)", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}_append_t{T}", "batch": B, "new_tokens": T,
                   "rows_written": written, "row_bytes": row_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "kv_append_kernel", "launch_avg_us": round(us, 2),
                     "algorithmic_bytes_per_launch": nbytes}}), flush=True)


def bench_gqla(args):
    """GQLA's two decode paths from one set of synthetic weights, DeepSeek-V3
    decode shape with 8 KV groups (64 sequences of 4096 tokens, 128 heads).

    absorb step: absorbed queries (product with W_UK), plan, decode over the
    latent cache, product with W_UV.  GQA step: plan, decode over the
    expanded per-group caches. The expansion itself (once per cached token,
    at append time) is timed on its own. Each part is timed over back-to-back
    launches with events on the stream; the decode kernels alone with the
    library's profiling events."""
    import torch
    import mla_paged_kv_03_amd as lib
    from mla_paged_kv_03_amd import _lib
    from workloads import GQLA_CONFIGS, make_gqla_inputs

    cfg = GQLA_CONFIGS["dsv3"]
    dev = torch.device("cuda:0")
    L = _lib.lib()
    d = make_gqla_inputs(cfg)
    B, T, H, G = cfg.batch, cfg.s_q, cfg.h_q, cfg.h_kv
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
        torch.bfloat16).to(dev)
    q, kv, wk, wv = bf(d["q"]), bf(d["kv"]), bf(d["w_uk"]), bf(d["w_uv"])
    bt = torch.from_numpy(d["block_table"]).to(dev)
    sl = torch.from_numpy(d["cache_seqlens"]).to(dev)
    P = lambda x: ctypes.c_void_p(x.data_ptr()) if x is not None else None
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    NP, maxp = kv.shape[0], bt.shape[1]
    rows = NP * 64
    k_rows = torch.empty(NP, 64, G, 192, dtype=torch.bfloat16, device=dev)
    v_rows = torch.empty(NP, 64, G, 128, dtype=torch.bfloat16, device=dev)
    qa = torch.empty(B, T, H, 576, dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty(B, T, H, 512, dtype=torch.bfloat16, device=dev)
    out_a = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=dev)
    out_g = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=dev)
    plan_a = lib.mla_decode_plan(sl, T, H, 1, 512)
    plan_g = lib.mla_decode_plan(sl, T, H, G, 128)
    ia, ig = plan_a.info, plan_g.info
    wsa, wsba = lib._ws(plan_a)
    wsg, wsbg = lib._ws(plan_g)
    scale = cfg.scale

    def ok(name, rc):
        if rc != 0:
            raise RuntimeError(f"{name} failed with {rc}")

    def expand():
        ok("gqla_expand_kv", L.gqla_expand_kv(P(kv), P(wk), P(wv), P(k_rows), P(v_rows), rows, G,
                                              stream))

    def absorb_q():
        ok("gqla_absorb_query", L.gqla_absorb_query(P(q), P(wk), P(qa), B * T, H, G, stream))

    def absorb_o():
        ok("gqla_absorb_output", L.gqla_absorb_output(P(o_lat), P(wv), P(out_a), B * T, H, G,
                                                      stream))

    def decode_a():
        ok("mla_decode_plan", L.mla_decode_plan(P(sl), B, T, H, 1, 512, P(plan_a.sched_metadata),
                                                P(plan_a.num_splits), ctypes.byref(ia), stream))
        ok("mla_decode", L.mla_decode(P(qa), P(kv), P(bt), P(sl), B, T, H, NP, maxp, scale, 0,
                                      P(plan_a.sched_metadata), P(plan_a.num_splits), wsa, wsba,
                                      P(o_lat), P(lse), stream))

    def decode_g():
        ok("mla_decode_plan", L.mla_decode_plan(P(sl), B, T, H, G, 128, P(plan_g.sched_metadata),
                                                P(plan_g.num_splits), ctypes.byref(ig), stream))
        ok("gqla_decode", L.gqla_decode(P(q), P(k_rows), P(v_rows), P(bt), P(sl), B, T, H, G, NP,
                                        maxp, scale, 0, P(plan_g.sched_metadata),
                                        P(plan_g.num_splits), wsg, wsbg, P(out_g), P(lse),
                                        stream))

    def absorb_step():
        absorb_q()
        decode_a()
        absorb_o()

    hip = ctypes.CDLL("libamdhip64.so")

    def timed(fn, n, events=False):
        """Average us per call over n back-to-back calls; with events, also
        the decode kernel alone (raw HIP events handed to the library's
        hook, which records them on the kernel's stream)."""
        for _ in range(max(1, n // 4)):
            fn()
        torch.cuda.synchronize()
        ev = []
        if events:
            for _ in range(2 * n):
                h = ctypes.c_void_p()
                if hip.hipEventCreate(ctypes.byref(h)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                ev.append(h)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(n):
            if events:
                L.mla_profile_events(ev[2 * i], ev[2 * i + 1])
            fn()
        t1.record()
        torch.cuda.synchronize()
        L.mla_profile_events(None, None)
        us = t0.elapsed_time(t1) / n * 1e3
        kus = None
        if events:
            tot = 0.0
            for i in range(n):
                ms = ctypes.c_float()
                if hip.hipEventElapsedTime(ctypes.byref(ms), ev[2 * i], ev[2 * i + 1]) != 0:
                    raise RuntimeError("hipEventElapsedTime failed")
                tot += ms.value
            for h in ev:
                hip.hipEventDestroy(h)
            kus = tot / n * 1e3
        return us, kus

    expand()
    torch.cuda.synchronize()
    n = args.steps
    t_exp, _ = timed(expand, max(5, n // 20))
    t_aq, _ = timed(absorb_q, n)
    t_ao, _ = timed(absorb_o, n)
    t_a, k_a = timed(absorb_step, n, events=True)
    t_g, k_g = timed(decode_g, n, events=True)
    tokens = B * T
    toks = lambda us: tokens / (us * 1e-6)
    ctx = int(d["cache_seqlens"].astype(np.int64).sum())
    lat_bytes = ctx * 576 * 2 + B * T * H * (576 + 512) * 2 + B * T * H * 4
    gqa_bytes = ctx * G * (192 + 128) * 2 + B * T * H * (192 + 128) * 2 + B * T * H * 4
    lat_flops = 2 * T * H * ctx * (576 + 512)
    gqa_flops = 2 * T * H * ctx * (192 + 128)
    proj_flops = 2 * B * T * H * 128 * 512
    exp_flops = 2 * rows * 512 * (128 + 128) * G
    exp_bytes = rows * 576 * 2 + rows * G * (192 + 128) * 2 + 2 * G * 512 * 128 * 2

    def roof(nbytes, flops, us):
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e6
        t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6
        if t_hbm >= t_mfma:
            ach = nbytes / (us * 1e-6) / 1e9
            return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4)}
        ach = flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}

    print(f"[bench] gqla: absorb step {t_a:.1f} us (decode kernel {k_a:.1f}, absorb q "
          f"{t_aq:.1f}, absorb out {t_ao:.1f}); GQA step {t_g:.1f} us (decode kernel "
          f"{k_g:.1f}); expansion of {rows} rows {t_exp:.1f} us", flush=True)
    best = min(t_a, t_g)
    print(json.dumps({
        "metric": "GQLA decode tokens/s, faster of the MQA-absorb and GQA paths (same weights)",
        "value": round(toks(best), 1), "unit": "tokens/s", "n_gpus": 1, "steps": n,
        "warmup": max(1, n // 4), "ms_per_step": round(best / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random latent cache and random group up-projections)",
        "config": {"workload": cfg.name, "batch": B, "s_q": T, "h_q": H, "h_kv": G,
                   "seqlen_total": ctx},
        "paths": {
            "absorb": {"us_per_step": round(t_a, 2), "tokens_per_s": round(toks(t_a), 1),
                       "decode_kernel_us": round(k_a, 2), "absorb_query_us": round(t_aq, 2),
                       "absorb_output_us": round(t_ao, 2),
                       "decode_roofline": roof(lat_bytes, lat_flops, k_a),
                       "projection_flops_each": proj_flops},
            "gqa": {"us_per_step": round(t_g, 2), "tokens_per_s": round(toks(t_g), 1),
                    "decode_kernel_us": round(k_g, 2),
                    "decode_roofline": roof(gqa_bytes, gqa_flops, k_g)},
            "faster": "absorb" if t_a <= t_g else "gqa"},
        "expansion": {"rows": rows, "us": round(t_exp, 1),
                      "roofline": roof(exp_bytes, exp_flops, t_exp),
                      "tflops": round(exp_flops / (t_exp * 1e-6) / 1e12, 1),
                      "algorithmic_bytes": exp_bytes, "flops": exp_flops}}), flush=True)


def bench_ceilings(args):
    """Practical ceilings measured with the decode's own instructions, next to
    the nominal peaks: bf16 MFMA loops on register operands (16x16x32 and
    32x32x16, one and two waves per SIMD), a non-temporal streaming read of
    4 GiB, and the HBM -> LDS page-copy loop of the decode alone (2 GiB in
    72 KiB blocks, one workgroup per CU), plus torch's bf16 GEMM (hipBLASLt)
    at 8192^3 for reference. Events around back-to-back launches after a
    warm-up; one JSON line per measurement."""
    import torch
    from mla_paged_kv_03_amd import _lib

    L = _lib.lib()
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    n = max(1, args.steps)

    def timed(fn, reps):
        for _ in range(max(2, reps // 4)):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps * 1e-3  # seconds per launch

    def emit(name, achieved, unit, peak, extra):
        rec = {"ceiling": name, "achieved": round(achieved, 1), "unit": unit, "peak": peak,
               "frac_of_peak": round(achieved / peak, 4)}
        rec.update(extra)
        print(json.dumps(rec), flush=True)

    which = args.ceiling
    if which in ("mfma", "all"):
        sink = torch.empty(cus * 2 * 256, dtype=torch.float32, device=dev)
        iters = 4096
        for kind, nacc, name in ((0, 4, "16x16x32"), (0, 8, "16x16x32"), (1, 2, "32x32x16"),
                                 (1, 4, "32x32x16")):
            for wps in (1, 2):
                def call():
                    rc = L.mla_ceiling_mfma(kind, nacc, wps, iters, cus, P(sink), stream)
                    if rc:
                        raise RuntimeError(f"mla_ceiling_mfma failed with {rc}")
                sec = timed(call, n)
                # per wave: iters * nacc MFMAs; 4 waves per workgroup
                flop = (16384 if kind == 0 else 32768) * nacc * iters * cus * wps * 4
                emit(f"mfma_bf16_{name}", flop / sec / 1e12, "TFLOP/s", MFMA_BF16_PEAK_TFLOPS,
                     {"accumulators": nacc, "waves_per_simd": wps, "launch_us": round(sec * 1e6, 1)})
    if which in ("stream", "all"):
        nbytes = 4 << 30
        buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        sink = torch.empty(cus * 8 * 256, dtype=torch.int32, device=dev)
        for per_cu in (4, 8):
            def call():
                rc = L.mla_ceiling_stream_read(P(buf), nbytes, cus * per_cu, P(sink), stream)
                if rc:
                    raise RuntimeError(f"mla_ceiling_stream_read failed with {rc}")
            sec = timed(call, max(3, n // 10))
            emit("hbm_stream_read", nbytes / sec / 1e9, "GB/s", HBM_PEAK_GBS,
                 {"bytes": nbytes, "workgroups_per_cu": per_cu, "launch_us": round(sec * 1e6, 1)})
        del buf
    if which in ("lds", "all"):
        blk = 72 * 1024
        nblocks = (2 << 30) // blk
        nbytes = nblocks * blk
        buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        sink = torch.empty(cus, dtype=torch.int32, device=dev)
        for waves in (4, 8):
            def call():
                rc = L.mla_ceiling_lds_fill(P(buf), nbytes, waves, cus, P(sink), stream)
                if rc:
                    raise RuntimeError(f"mla_ceiling_lds_fill failed with {rc}")
            sec = timed(call, max(3, n // 10))
            emit("hbm_to_lds_page_copies", nbytes / sec / 1e9, "GB/s", HBM_PEAK_GBS,
                 {"bytes": nbytes, "waves": waves, "workgroups": cus,
                  "per_cu_bytes_per_clk_at_2.4GHz": round(nbytes / sec / cus / 2.4e9, 2),
                  "launch_us": round(sec * 1e6, 1)})
        del buf
    if which in ("ldsop", "all"):
        iters = 2048
        sink = torch.empty(cus * 512, dtype=torch.float32, device=dev)
        for mode, name in ((0, "ds_read_b128"), (1, "ds_read_b128+mfma32"),
                           (3, "ds_read_b64_tr_x2"), (2, "ds_read_b64_tr_x2+mfma32"),
                           (4, "ds_read_b128+mfma32_prefetch8"),
                           (5, "ds_read_b64_tr_x2+mfma32_prefetch8")):
            for waves in (4, 8):
                def call():
                    rc = L.mla_ceiling_lds_operand(mode, waves, iters, cus, P(sink), stream)
                    if rc:
                        raise RuntimeError(f"mla_ceiling_lds_operand failed with {rc}")
                sec = timed(call, n)
                steps = iters * 16 * waves * cus          # one KiB and (modes 1, 2) one MFMA each
                extra = {"waves": waves, "lds_bytes_per_clk_per_cu_at_2.4GHz":
                         round(steps * 1024 / sec / cus / 2.4e9, 1), "launch_us": round(sec * 1e6, 1)}
                if mode in (1, 2, 4, 5):
                    emit(f"lds_operand_{name}", steps * 32768 / sec / 1e12, "TFLOP/s",
                         MFMA_BF16_PEAK_TFLOPS, extra)
                else:
                    # nominal: 128 bytes per clock per CU at 2.4 GHz
                    emit(f"lds_operand_{name}", steps * 1024 / sec / 1e9, "GB/s",
                         round(128 * cus * 2.4, 1), extra)
    if which in ("write", "all"):
        # one 256 KiB block per workgroup (a split's fp32 partial rows), one
        # or several workgroups per CU, blocks packed or spaced apart
        blk = 256 << 10
        for per_cu, pad in ((1, 0), (1, 4096), (1, 65536), (4, 0), (4, 4096)):
            grid = cus * per_cu
            stride = blk + pad
            buf = torch.empty(grid * stride // 4 + 64, dtype=torch.int32, device=dev)
            def call():
                rc = L.mla_ceiling_block_write(P(buf), blk, stride, grid, stream)
                if rc:
                    raise RuntimeError(f"mla_ceiling_block_write failed with {rc}")
            sec = timed(call, max(10, n))
            emit("hbm_block_write", grid * blk / sec / 1e9, "GB/s", HBM_PEAK_GBS,
                 {"block_bytes": blk, "stride_bytes": stride, "workgroups": grid,
                  "launch_us": round(sec * 1e6, 1)})
            del buf
    if which in ("gemm", "all"):
        m = 8192
        a = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
        b = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
        c = torch.empty(m, m, dtype=torch.bfloat16, device=dev)
        sec = timed(lambda: torch.matmul(a, b, out=c), max(5, n // 10))
        emit("torch_bf16_gemm_8192", 2 * m ** 3 / sec / 1e12, "TFLOP/s", MFMA_BF16_PEAK_TFLOPS,
             {"launch_us": round(sec * 1e6, 1)})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--op", choices=["decode", "append", "gqla"], default="decode",
                    help="decode (the default step), the paged KV append alone, or GQLA's "
                         "two decode paths")
    ap.add_argument("--kv", choices=["bf16", "fp8"], default="bf16",
                    help="latent cache format for the MLA configs (fp8: E4M3 codes with a "
                         "per-token scale, quantised on the GPU before the timed region)")
    ap.add_argument("--append-tokens", type=int, default=0,
                    help="new tokens per sequence for --op append (default: the config's s_q)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--ceiling", choices=["mfma", "stream", "lds", "ldsop", "write", "gemm", "all"], default=None,
                    help="only measure practical ceilings: bf16 MFMA loops, a streaming HBM "
                         "read, the decode's HBM -> LDS page-copy loop alone, LDS operand reads "
                         "with and without MFMAs, torch's bf16 GEMM")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs the decode on one GPU only; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.ceiling:
        bench_ceilings(args)
        return
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 3}), flush=True)
        return
    import mla_paged_kv_03_amd as lib
    from mla_paged_kv_03_amd import _lib
    from workloads import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    fp8 = args.kv == "fp8"
    if fp8 and cfg.kind != "mla":
        print("bench.py: --kv fp8 applies to the MLA configs (1-4)", file=sys.stderr)
        sys.exit(2)
    if args.op == "gqla":
        bench_gqla(args)
        return
    if args.op == "append":
        bench_append(args, cfg)
        return
    dev = torch.device("cuda:0")
    L = _lib.lib()
    sets = []
    for r in range(args.rotate):
        # rotated sets share the first set's lengths (same work), not its values
        d = make_inputs(cfg, seed=cfg.seed + 1000 * r,
                        seqlens=sets[0][0]["cache_seqlens"] if sets else None)
        t = {"q": torch.from_numpy(d["q"].view(np.int16)).view(torch.bfloat16).to(dev),
             "bt": torch.from_numpy(d["block_table"]).to(dev),
             "sl": torch.from_numpy(d["cache_seqlens"]).to(dev)}
        for k in ("kv", "k", "v"):
            if k in d:
                t[k] = torch.from_numpy(d[k].view(np.int16)).view(torch.bfloat16).to(dev)
        if fp8:
            t["codes"], t["scales"] = lib.mla_kv_quantize_fp8(t.pop("kv"))
        sets.append((d, t))
        if r > 0:
            for k in ("kv", "k", "v"):
                d.pop(k, None)  # the first set's host copy serves the CPU baseline
    d0 = sets[0][0]
    work = algorithmic_work(d0, fp8)
    B, T, H, G = cfg.batch, cfg.s_q, cfg.h_q, cfg.h_kv
    dv = cfg.d_v
    plan = lib.mla_decode_plan(sets[0][1]["sl"], T, H, G, dv, kv_fp8=fp8)
    info = plan.info
    out = torch.empty(B, T, H, dv, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=dev)
    ws, wsb = lib._ws(plan)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    pinfo = ctypes.byref(info)

    def step(i):
        _, t = sets[i % len(sets)]
        if fp8:
            rc = L.mla_decode_plan_fp8(P(t["sl"]), B, T, H, P(plan.sched_metadata),
                                       P(plan.num_splits), pinfo, stream)
        else:
            rc = L.mla_decode_plan(P(t["sl"]), B, T, H, G, dv, P(plan.sched_metadata),
                                   P(plan.num_splits), pinfo, stream)
        if rc:
            raise lib.DecodeError("mla_decode_plan", rc)
        if fp8:
            rc = L.mla_decode_fp8(P(t["q"]), P(t["codes"]), P(t["scales"]), P(t["bt"]), P(t["sl"]),
                                  B, T, H, t["codes"].shape[0], t["bt"].shape[1], cfg.scale,
                                  int(cfg.causal), P(plan.sched_metadata), P(plan.num_splits),
                                  ws, wsb, P(out), P(lse), stream)
        elif cfg.kind == "mla":
            rc = L.mla_decode(P(t["q"]), P(t["kv"]), P(t["bt"]), P(t["sl"]), B, T, H,
                              t["kv"].shape[0], t["bt"].shape[1], cfg.scale, int(cfg.causal),
                              P(plan.sched_metadata), P(plan.num_splits), ws, wsb, P(out),
                              P(lse), stream)
        else:
            rc = L.gqa_decode(P(t["q"]), P(t["k"]), P(t["v"]), P(t["bt"]), P(t["sl"]), B, T,
                              H, G, t["k"].shape[0], t["bt"].shape[1], cfg.scale,
                              int(cfg.causal), P(plan.sched_metadata), P(plan.num_splits), ws,
                              wsb, P(out), P(lse), stream)
        if rc:
            raise lib.DecodeError("decode", rc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # timed region: whole steps, and the decode kernel alone via the
    # library's event hook (HIP events recorded on the kernel's own stream)
    hip = ctypes.CDLL("libamdhip64.so")
    K = args.steps
    ev = []
    for _ in range(2 * K):
        h = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        ev.append(h)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(K):
        L.mla_profile_events(ev[2 * i], ev[2 * i + 1])
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    L.mla_profile_events(None, None)
    ms_step = t_start.elapsed_time(t_end) / K
    kern_ms = []
    for i in range(K):
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), ev[2 * i], ev[2 * i + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        kern_ms.append(ms.value)
    for h in ev:
        hip.hipEventDestroy(h)
    kern_ms = np.array(kern_ms)
    kern_avg = float(kern_ms.mean())

    # same loop without the event hook: the step rate with nothing extra
    torch.cuda.synchronize()
    t_start.record()
    for i in range(K):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    ms_step_plain = t_start.elapsed_time(t_end) / K
    ms_step = min(ms_step, ms_step_plain)
    print(f"[bench] {K} steps: {ms_step * 1e3:.1f} us/step, decode kernel "
          f"{kern_avg * 1e3:.1f} us (median {np.median(kern_ms) * 1e3:.1f})",
          file=sys.stderr, flush=True)

    s = ms_step * 1e-3
    tflops = work["flops"] / s / 1e12
    gbs = work["bytes"] / s / 1e9
    k_gbs = work["bytes"] / (kern_avg * 1e-3) / 1e9
    k_tflops = work["flops"] / (kern_avg * 1e-3) / 1e12
    kname, ksrc = decode_kernel_of(cfg, fp8)
    traffic = None if fp8 else stored_traffic(cfg.name, ksrc)
    bound = "hbm" if work["flops"] / work["bytes"] < MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3 \
        else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(k_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(k_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic}
    roof["kernel"] = kname
    roof["kernel_avg_us"] = round(kern_avg * 1e3, 2)
    roof["kernel_median_us"] = round(float(np.median(kern_ms)) * 1e3, 2)
    roof["algorithmic_bytes_per_launch"] = work["bytes"]
    roof["algorithmic_flops_per_launch"] = work["flops"]

    res = {
        "metric": METRIC,
        "value": round(B * T / s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3 cache, bf16 MFMA" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name + ("_fp8kv" if fp8 else ""), "batch": B, "s_q": T, "h_q": H, "h_kv": G,
                   "d_qk": cfg.d_qk, "d_v": dv, "page": 64, "causal": cfg.causal,
                   "seqlen_total": int(d0["cache_seqlens"].sum()),
                   "workers": info.num_workers, "input_sets_rotated": args.rotate},
        "tflops": round(tflops, 2),
        "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "hbm_gbs": round(gbs, 1),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": roof,
    }
    if not args.no_cpu and not fp8:
        res["cpu_baseline"] = cpu_baseline(d0)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
