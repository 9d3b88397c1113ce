"""mla_decode_noalloc: the decode for callers that cannot allocate, with the
plan and the split partials in the library's static device scratch. Its
results must equal mla_decode's (same kernels, same plan) bit for bit, on
two calls in a row where the second is smaller than the first and leaves
stale data of the first in the scratch, and match the oracle."""
import ctypes

import numpy as np
import pytest

from gpu_helpers import check, inputs, log, run_gpu, run_oracle, to_device
from test_parity_gpu import _mla

pytestmark = pytest.mark.gpu


def _noalloc(d, t):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = d["cfg"]
    B, T, H = cfg.batch, cfg.s_q, cfg.h_q
    out = torch.empty(B, T, H, 512, dtype=torch.bfloat16, device=t["q"].device)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=t["q"].device)
    o, l = lib.mla_decode_noalloc(t["q"], t["kv"], t["block_table"], t["cache_seqlens"],
                                  cfg.scale, cfg.causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), l.cpu().double().numpy()


def test_noalloc_equals_mla_decode_on_two_calls(dev):
    import mla_paged_kv_03_amd as lib
    big = _mla(16, 2, 128, (9000, 1, 64, 4100, 300, 0, 12000, 65, 2, 7000, 127, 640, 5000, 1000,
                            3, 8192), True)
    small = _mla(3, 1, 16, (700, 64, 1), False)
    for name, cfg, seed in (("big", big, 31), ("small", small, 32)):
        d = inputs(cfg, seed=seed)
        t = to_device(d, dev)
        plan = lib.mla_decode_plan(t["cache_seqlens"], cfg.s_q, cfg.h_q)
        if name == "big":
            assert int(plan.num_splits[-1].item()) > 0, "the large call must split sequences"
        log(f"[case] noalloc {name}: B={cfg.batch} s_q={cfg.s_q} h_q={cfg.h_q}")
        o_ref, l_ref = run_gpu(d, t, plan=plan)
        o, l = _noalloc(d, t)
        assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref), name
        ref_out, ref_lse, spread = run_oracle(d, spread=True)
        check(o, l, ref_out, ref_lse, f"noalloc {name}", spread=spread)


def test_noalloc_rejects_calls_beyond_its_scratch(dev):
    import torch
    from mla_paged_kv_03_amd import _lib
    x = torch.zeros(64, dtype=torch.int32, device=dev)
    p = ctypes.c_void_p(x.data_ptr())
    # 200000 sequences: the plan's metadata would exceed 512 KiB
    rc = _lib.lib().mla_decode_noalloc(p, p, p, p, 200000, 1, 16, 1, 1, 0.1, 0, p, p,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == -6
    torch.cuda.synchronize()
