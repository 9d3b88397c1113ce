"""Which decode path is faster on this GPU, per model shape.

The GQLA review ("2. Motivation & Problem Statement", "3. Method & Key
Results", Figure 3) argues that MLA's single MQA-absorb decode path suits
GPUs with a high compute-to-bandwidth ratio, and that GPUs with a low one
are better served by a GQA path over a per-group expanded cache. On MI355X
that ratio is 2.5 PFLOP/s dense bf16 over 8 TB/s, about 315 flop/B. This
module times both paths of this library on the same shapes:

  * absorb (mla_decode): every query head attends the shared 576-wide latent
    row (1152 B per cached token), 2 (576 + 512) flop per row and key;
  * GQA (gqa_decode): h_kv groups of 128-wide K and V (512 h_kv B per
    token), 2 (128 + 128) flop per row and key;

for h_q query heads, s_q query tokens (causal when s_q > 1), h_kv groups
and sequence length L, with the batch sized so that it holds about 2^18
cached tokens. Inputs are random bf16 values made on the device (values do
not change the time).

    python -m mla_paged_kv_03_amd.path_study [--quick] [--out FILE]

prints one JSON line per measured point and, with --out, writes a Markdown
table of the step times and the winner per shape. With --long-context it
times small batches of long sequences instead (step, decode kernel and the
rest: plan and split merge).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import sys

import numpy as np

HBM_PEAK = 8.0e12
MFMA_PEAK = 2.5166e15
TOKENS = 1 << 18


def _time(step, K=30, W=8):
    import torch
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(K):
        step()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / K * 1e3  # us per step


def _kernel_time(L, step, K=30):
    """Decode kernel alone: HIP events recorded by the library around it."""
    import torch
    hip = ctypes.CDLL("libamdhip64.so")
    ev = []
    for _ in range(2 * K):
        h = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        ev.append(h)
    for i in range(K):
        L.mla_profile_events(ev[2 * i], ev[2 * i + 1])
        step()
    torch.cuda.synchronize()
    L.mla_profile_events(None, None)
    ms = []
    for i in range(K):
        x = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(x), ev[2 * i], ev[2 * i + 1])
        ms.append(x.value)
    for h in ev:
        hip.hipEventDestroy(h)
    return float(np.mean(ms)) * 1e3


def measure(kind, h_q, s_q, h_kv, seqlen, batch=None):
    """Time one path on one shape (batch: default about 2^18 cached tokens);
    returns a dict of the point."""
    import torch
    import mla_paged_kv_03_amd as lib
    from mla_paged_kv_03_amd import _lib

    L = _lib.lib()
    dev = torch.device("cuda:0")
    B = batch if batch else max(1, TOKENS // seqlen)
    pages = (seqlen + 63) // 64
    P = B * pages
    g = torch.Generator(device=dev)
    g.manual_seed(h_q * 1000 + s_q * 100 + h_kv * 10 + pages)
    bf = lambda *shape: (torch.randn(*shape, generator=g, device=dev) * 0.5).to(torch.bfloat16)
    bt = torch.randperm(P, generator=g, device=dev).to(torch.int32).view(B, pages)
    sl = torch.full((B,), seqlen, dtype=torch.int32, device=dev)
    causal = int(s_q > 1)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if kind == "absorb":
        G, D, DV = 1, 576, 512
        q, kv = bf(B, s_q, h_q, D), bf(P, 64, 1, D)
        scale = 1.0 / math.sqrt(192.0)
    else:
        G, D, DV = h_kv, 128, 128
        q, kc, vc = bf(B, s_q, h_q, D), bf(P, 64, G, D), bf(P, 64, G, D)
        scale = 1.0 / math.sqrt(128.0)
    plan = lib.mla_decode_plan(sl, s_q, h_q, G, DV)
    ws, wsb = lib._ws(plan)
    info = plan.info
    out = torch.empty(B, s_q, h_q, DV, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, s_q, h_q, dtype=torch.float32, device=dev)

    def step():
        rc = L.mla_decode_plan(ptr(sl), B, s_q, h_q, G, DV, ptr(plan.sched_metadata),
                               ptr(plan.num_splits), ctypes.byref(info), stream)
        if rc == 0:
            if kind == "absorb":
                rc = L.mla_decode(ptr(q), ptr(kv), ptr(bt), ptr(sl), B, s_q, h_q, P, pages, scale,
                                  causal, ptr(plan.sched_metadata), ptr(plan.num_splits), ws, wsb,
                                  ptr(out), ptr(lse), stream)
            else:
                rc = L.gqa_decode(ptr(q), ptr(kc), ptr(vc), ptr(bt), ptr(sl), B, s_q, h_q, G, P,
                                  pages, scale, causal, ptr(plan.sched_metadata),
                                  ptr(plan.num_splits), ws, wsb, ptr(out), ptr(lse), stream)
        if rc != 0:
            raise lib.DecodeError(kind, rc)

    step_us = _time(step)
    kernel_us = _kernel_time(L, step)
    tok_bytes = G * (D + (DV if kind == "gqa" else 0)) * 2
    vis = s_q * seqlen - (s_q * (s_q - 1) // 2 if causal else 0)  # key visits per head
    flops = 2 * (D + DV) * h_q * B * vis
    nbytes = B * seqlen * tok_bytes + B * s_q * h_q * (D + DV) * 2
    roof_us = max(nbytes / HBM_PEAK, flops / MFMA_PEAK) * 1e6
    return {"path": kind, "h_q": h_q, "s_q": s_q, "h_kv": G, "L": seqlen, "batch": B,
            "step_us": round(step_us, 2), "kernel_us": round(kernel_us, 2),
            "outside_kernel_us": round(step_us - kernel_us, 2),
            "bytes": nbytes, "flops": flops, "flop_per_byte": round(flops / nbytes, 1),
            "roofline_us": round(roof_us, 2), "frac": round(roof_us / kernel_us, 3)}


# small batches of long sequences: a sequence spreads over many workers and
# its partial results are merged in two launches (path, h_q, s_q, h_kv, L, batch)
LONG_CONTEXT = [("absorb", 128, 1, 1, 65536, 1), ("absorb", 128, 1, 1, 16384, 1),
                ("absorb", 16, 1, 1, 131072, 1), ("absorb", 128, 2, 1, 32768, 2),
                ("gqa", 128, 1, 8, 65536, 1), ("absorb", 128, 1, 1, 4096, 64)]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--quick", action="store_true", help="a small grid")
    ap.add_argument("--long-context", action="store_true",
                    help="time the small-batch long-context shapes instead of the grid")
    ap.add_argument("--out", default=None, help="write a Markdown summary here")
    args = ap.parse_args(argv)
    if args.long_context:
        for kind, h, t, g, seqlen, b in LONG_CONTEXT:
            print(json.dumps(measure(kind, h, t, g, seqlen, batch=b)), flush=True)
        return 0
    heads = (32, 128) if args.quick else (16, 32, 64, 128)
    tokens = (1, 2) if args.quick else (1, 2, 4)
    groups = (8,) if args.quick else (4, 8, 16)
    lengths = (4096,) if args.quick else (1024, 4096, 16384)
    rows = []
    for h in heads:
        for t in tokens:
            for seqlen in lengths:
                a = measure("absorb", h, t, 1, seqlen)
                print(json.dumps(a), flush=True)
                for gk in groups:
                    if gk > h:
                        continue
                    b = measure("gqa", h, t, gk, seqlen)
                    print(json.dumps(b), flush=True)
                    rows.append((a, b))
    if args.out:
        lines = ["| h_q | s_q | h_kv (GQA) | L | absorb step us (kernel, frac) | "
                 "GQA step us (kernel, frac) | flop/B absorb / GQA | faster |",
                 "|---|---|---|---|---|---|---|---|"]
        for a, b in rows:
            win = "absorb" if a["step_us"] <= b["step_us"] else "GQA"
            lines.append(
                f"| {a['h_q']} | {a['s_q']} | {b['h_kv']} | {a['L']} | {a['step_us']} "
                f"({a['kernel_us']}, {a['frac']}) | {b['step_us']} ({b['kernel_us']}, {b['frac']}) "
                f"| {a['flop_per_byte']} / {b['flop_per_byte']} | {win} |")
        with open(args.out, "w") as f:
            f.write("\n".join(lines) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
