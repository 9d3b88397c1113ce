"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
library through its C interface, and run the oracle on the same inputs."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from workloads import make_inputs


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_tensor(arr, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)


def to_device(d, dev):
    import torch
    t = {"q": bf16_tensor(d["q"], dev),
         "block_table": torch.from_numpy(d["block_table"]).to(dev),
         "cache_seqlens": torch.from_numpy(d["cache_seqlens"]).to(dev)}
    for k in ("kv", "k", "v"):
        if k in d:
            t[k] = bf16_tensor(d[k], dev)
    return t


def run_gpu(d, t, plan=None, out=None, lse=None):
    """Decode on the GPU; returns (out fp64 numpy, lse fp64 numpy)."""
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = d["cfg"]
    if cfg.kind == "mla":
        o, l = lib.mla_decode(t["q"], t["kv"], t["block_table"], t["cache_seqlens"], cfg.scale,
                              cfg.causal, plan=plan, out=out, lse=lse)
    else:
        o, l = lib.gqa_decode(t["q"], t["k"], t["v"], t["block_table"], t["cache_seqlens"],
                              cfg.scale, cfg.causal, plan=plan, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), l.cpu().double().numpy()


def run_oracle(d, batch_idx=None, spread=False):
    """Oracle out and lse of the chosen sequences; with spread=True also the
    value spread (oracle.value_spread) that sizes the tighter allowance."""
    cfg = d["cfg"]
    idx = np.arange(cfg.batch) if batch_idx is None else np.asarray(batch_idx)
    q = d["q"][idx]
    bt = d["block_table"][idx]
    L = d["cache_seqlens"][idx]
    if cfg.kind == "mla":
        args = (q, d["kv"], bt, L, cfg.scale, cfg.causal)
        kw = {"d_v": cfg.d_v}
    else:
        args = (q, d["k"], bt, L, cfg.scale, cfg.causal)
        kw = {"v_cache": d["v"]}
    out, lse = oracle.attend_two_pass(*args, **kw)
    if not spread:
        return out, lse
    return out, lse, oracle.value_spread(*args, **kw)


def check(out, lse, ref_out, ref_lse, what, spread=None):
    res = oracle.compare(out, lse, ref_out, ref_lse, spread=spread)
    log(f"[parity] {what}: " + ", ".join(f"{k}={v}" for k, v in res.items()))
    assert res["ok"], f"{what}: {res}"
    return res


def inputs(cfg, seed=None, **kw):
    return make_inputs(cfg, seed=seed, **kw)
