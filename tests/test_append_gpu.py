"""GPU parity of the paged KV append (bit-exact against the oracle), and an
append followed by a decode that reads the appended rows."""
import numpy as np
import pytest

import oracle
from workloads import CONFIGS, make_inputs, f32_to_bf16_bits
from gpu_helpers import bf16_tensor, check, log, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu


def _new_rows(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _mla(B, T, Ls):
    return CONFIGS[3].with_(batch=B, s_q=T, h_q=16, causal=True, seqlen_rule="fixed",
                            seqlens_fixed=tuple(Ls))


def _gqa(B, T, G, Ls):
    return CONFIGS[5].with_(batch=B, s_q=T, h_q=2 * G, h_kv=G, seqlen_rule="fixed",
                            seqlens_fixed=tuple(Ls))


CASES = {
    # lengths count the new tokens; 0 and short sequences (L < T) included,
    # and runs of new tokens that cross a page boundary
    "mla_t1": _mla(8, 1, (0, 1, 63, 64, 65, 128, 129, 500)),
    "mla_t2": _mla(8, 2, (0, 1, 2, 64, 65, 66, 129, 700)),
    "mla_t4": _mla(6, 4, (3, 4, 62, 66, 130, 257)),
    "mla_t64": _mla(4, 64, (63, 64, 127, 300)),
    "gqa_t1_g8": _gqa(6, 1, 8, (0, 1, 64, 65, 200, 1000)),
    "gqa_t3_g2": _gqa(6, 3, 2, (1, 2, 3, 64, 66, 333)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_append_matches_oracle_bit_for_bit(dev, name):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = CASES[name]
    d = make_inputs(cfg)
    rng = np.random.default_rng(41)
    B, T = cfg.batch, cfg.s_q
    bt = torch.from_numpy(d["block_table"]).to(dev)
    sl = torch.from_numpy(d["cache_seqlens"]).to(dev)
    log(f"[append] {name}")
    if cfg.kind == "mla":
        new = _new_rows(rng, (B, T, 576))
        kv = bf16_tensor(d["kv"], dev)
        lib.mla_kv_append(bf16_tensor(new, dev), kv, bt, sl)
        got = kv.view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle.append_rows(d["kv"], new.reshape(B, T, 1, 576), d["block_table"],
                                 d["cache_seqlens"])
        assert np.array_equal(got, ref)
    else:
        G = cfg.h_kv
        nk, nv = _new_rows(rng, (B, T, G, 128)), _new_rows(rng, (B, T, G, 128))
        k, v = bf16_tensor(d["k"], dev), bf16_tensor(d["v"], dev)
        lib.gqa_kv_append(bf16_tensor(nk, dev), bf16_tensor(nv, dev), k, v, bt, sl)
        for t, new, src in ((k, nk, d["k"]), (v, nv, d["v"])):
            got = t.view(torch.int16).cpu().numpy().view(np.uint16)
            ref = oracle.append_rows(src, new, d["block_table"], d["cache_seqlens"])
            assert np.array_equal(got, ref)


def test_block_table_entries_outside_the_cache_are_skipped(dev):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = _mla(2, 1, (10, 10))
    d = make_inputs(cfg)
    bt_np = d["block_table"].copy()
    bt_np[1, 0] = d["num_pages"]  # one past the last page
    new = _new_rows(np.random.default_rng(3), (2, 1, 576))
    kv = bf16_tensor(d["kv"], dev)
    lib.mla_kv_append(bf16_tensor(new, dev), kv, torch.from_numpy(bt_np).to(dev),
                      torch.from_numpy(d["cache_seqlens"]).to(dev))
    got = kv.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.append_rows(d["kv"], new.reshape(2, 1, 1, 576), bt_np, d["cache_seqlens"])
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("kind", ["mla", "gqa"])
def test_decode_after_append_sees_the_new_rows(dev, kind):
    """Append T new tokens whose rows differ from what the cache held, then
    decode (causal) with the lengths that count them: the GPU result must
    match the oracle's attention over the oracle's appended cache."""
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = (_mla(5, 2, (2, 65, 130, 640, 1000)) if kind == "mla"
           else _gqa(5, 2, 4, (2, 65, 130, 640, 1000)).with_(causal=True))
    d = make_inputs(cfg, seed=9)
    rng = np.random.default_rng(8)
    B, T = cfg.batch, cfg.s_q
    t = to_device(d, dev)
    d2 = dict(d)
    if kind == "mla":
        new = _new_rows(rng, (B, T, 576))
        lib.mla_kv_append(bf16_tensor(new, dev), t["kv"], t["block_table"], t["cache_seqlens"])
        d2["kv"] = oracle.append_rows(d["kv"], new.reshape(B, T, 1, 576), d["block_table"],
                                      d["cache_seqlens"])
    else:
        nk = _new_rows(rng, (B, T, cfg.h_kv, 128))
        nv = _new_rows(rng, (B, T, cfg.h_kv, 128))
        lib.gqa_kv_append(bf16_tensor(nk, dev), bf16_tensor(nv, dev), t["k"], t["v"],
                          t["block_table"], t["cache_seqlens"])
        d2["k"] = oracle.append_rows(d["k"], nk, d["block_table"], d["cache_seqlens"])
        d2["v"] = oracle.append_rows(d["v"], nv, d["block_table"], d["cache_seqlens"])
    out, lse = run_gpu(d2, t)
    ref_out, ref_lse, spread = run_oracle(d2, spread=True)
    check(out, lse, ref_out, ref_lse, f"decode after append ({kind})", spread=spread)
