"""GPU parity of GQLA's two decode paths through the C interface.

  * The up-projection products (expand, absorb query, absorb output): every
    output within one bf16 step of the exact fp64 value plus the fp32
    summation bound K * 2^-24 * sum |a_i w_i|; the copied rope columns
    bit-exact.
  * The decode kernel over expanded 192-wide K and 128-wide V pages: the
    decode bars (max-abs 1e-2 with the one-bf16-step allowance, rel-L2 5e-3,
    LSE 1e-3) against the attention oracle.
  * Both paths end to end: the decode bars against the oracle with the same
    bf16 rounding points, and a looser bar against the exact definition (it
    absorbs the rounding of the bf16 intermediates; derived in the design
    notes).
"""
import numpy as np
import pytest

import oracle
from oracle import gqla
from workloads import CONFIGS, GQLA_CONFIGS, make_gqla_inputs, make_inputs, f32_to_bf16_bits
from gpu_helpers import bf16_tensor, check, log

pytestmark = pytest.mark.gpu

SCALE = 1.0 / np.sqrt(192.0)
# exact-definition bar for the chained bf16 intermediates
CHAIN_MAX_ABS, CHAIN_REL_L2, CHAIN_LSE = 3e-2, 1e-2, 1e-2


def _f64(t):
    return t.float().cpu().double().numpy()


def _bits(t):
    import torch
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _absbits(x):
    return np.asarray(x, dtype=np.uint16) & np.uint16(0x7FFF)


def _product_check(got, ref, absref, K, what):
    err = np.abs(got - ref)
    allowed = oracle.bf16_step(ref) + K * 2.0 ** -24 * absref
    bad = int((err > allowed).sum())
    log(f"[parity] {what}: max_err={float(err.max()):.3e} "
        f"max_rel_step={float((err / oracle.bf16_step(ref)).max()):.3f} bad={bad}")
    assert bad == 0, what


def _dev_inputs(d, dev, names=("q", "kv", "w_uk", "w_uv")):
    import torch
    t = {k: bf16_tensor(d[k], dev) for k in names}
    t["block_table"] = torch.from_numpy(d["block_table"]).to(dev)
    t["cache_seqlens"] = torch.from_numpy(d["cache_seqlens"]).to(dev)
    return t


# ----------------------------------------------------------- the products
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("rows", ["cache", "new_tokens"])
def test_expand_kv_matches_oracle(dev, G, rows):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = GQLA_CONFIGS["small"].with_(h_kv=G, h_q=16 if G <= 4 else 32)
    d = make_gqla_inputs(cfg, seed=21)
    kv = d["kv"] if rows == "cache" else d["kv"][:2, :7]   # 9 pages (576 rows) or 14 rows
    log(f"[case] expand G={G} rows={rows} shape={kv.shape}")
    k, v = lib.gqla_expand_kv(bf16_tensor(kv, dev), bf16_tensor(d["w_uk"], dev),
                              bf16_tensor(d["w_uv"], dev))
    torch.cuda.synchronize()
    assert tuple(k.shape) == kv.shape[:2] + (G, 192) and tuple(v.shape) == kv.shape[:2] + (G, 128)
    K, V = gqla.expand_group_cache(kv, d["w_uk"], d["w_uv"])
    aK, aV = gqla.expand_group_cache(_absbits(kv), _absbits(d["w_uk"]), _absbits(d["w_uv"]))
    _product_check(_f64(k)[..., :128], K[..., :128], aK[..., :128], 512, "expand K")
    _product_check(_f64(v), V, aV, 512, "expand V")
    kb = _bits(k)
    assert np.array_equal(kb[..., 128:], np.repeat(kv[:, :, :, 512:], G, axis=2)), "rope columns"


@pytest.mark.parametrize("shape", [(3, 2, 16, 4), (64, 1, 128, 8), (5, 3, 8, 8), (2, 1, 24, 1)])
def test_absorb_query_matches_oracle(dev, shape):
    import torch
    import mla_paged_kv_03_amd as lib
    B, T, H, G = shape
    cfg = GQLA_CONFIGS["small"].with_(batch=B, s_q=T, h_q=H, h_kv=G, seqlens_fixed=(1,) * B)
    d = make_gqla_inputs(cfg, seed=22)
    log(f"[case] absorb_query B={B} T={T} H={H} G={G}")
    qa = lib.gqla_absorb_query(bf16_tensor(d["q"], dev), bf16_tensor(d["w_uk"], dev))
    torch.cuda.synchronize()
    ref = gqla.absorb_query(d["q"], d["w_uk"])
    aref = gqla.absorb_query(_absbits(d["q"]), _absbits(d["w_uk"]))
    _product_check(_f64(qa)[..., :512], ref[..., :512], aref[..., :512], 128, "absorb query")
    assert np.array_equal(_bits(qa)[..., 512:], d["q"][..., 128:]), "rope columns"


@pytest.mark.parametrize("shape", [(3, 2, 16, 4), (64, 1, 128, 8), (7, 1, 40, 5)])
def test_absorb_output_matches_oracle(dev, shape):
    import torch
    import mla_paged_kv_03_amd as lib
    B, T, H, G = shape
    cfg = GQLA_CONFIGS["small"].with_(batch=B, s_q=T, h_q=H, h_kv=G, seqlens_fixed=(1,) * B)
    d = make_gqla_inputs(cfg, seed=23)
    rng = np.random.default_rng(24)
    o_lat = f32_to_bf16_bits(rng.standard_normal((B, T, H, 512), dtype=np.float32))
    log(f"[case] absorb_output B={B} T={T} H={H} G={G}")
    out = lib.gqla_absorb_output(bf16_tensor(o_lat, dev), bf16_tensor(d["w_uv"], dev))
    torch.cuda.synchronize()
    ref = gqla.absorb_output(oracle.bf16_to_f64(o_lat), d["w_uv"])
    aref = gqla.absorb_output(oracle.bf16_to_f64(_absbits(o_lat)), _absbits(d["w_uv"]))
    _product_check(_f64(out), ref, aref, 512, "absorb output")


# ------------------------------------------- decode over expanded pages
RAGGED = (0, 1, 2, 63, 64, 65, 127, 200, 640, 1000)


def _rope_cfg(B, T, H, G, Ls, causal=False):
    return CONFIGS[5].with_(batch=B, s_q=T, h_q=H, h_kv=G, d_qk=192, d_v=128, causal=causal,
                            seqlen_rule="fixed", seqlens_fixed=tuple(Ls), scale=SCALE)


ROPE = {
    "h128_g8_t1": _rope_cfg(10, 1, 128, 8, RAGGED),
    "h32_g4_t2_causal": _rope_cfg(10, 2, 32, 4, RAGGED, True),
    "h128_g8_t2_causal": _rope_cfg(10, 2, 128, 8, RAGGED, True),
    "h128_g8_t4": _rope_cfg(10, 4, 128, 8, RAGGED),
    "h16_g16_t1": _rope_cfg(10, 1, 16, 16, RAGGED),
}


def _run_rope_decode(d, dev, plan=None):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = d["cfg"]
    t = {k: bf16_tensor(d[k], dev) for k in ("q", "k", "v")}
    bt = torch.from_numpy(d["block_table"]).to(dev)
    L = torch.from_numpy(d["cache_seqlens"]).to(dev)
    out, lse = lib.gqla_decode(t["q"], t["k"], t["v"], bt, L, cfg.scale, cfg.causal, plan=plan)
    torch.cuda.synchronize()
    return _f64(out), lse.cpu().double().numpy()


@pytest.mark.parametrize("name", list(ROPE))
def test_rope_layout_decode_matches_oracle(dev, name):
    d = make_inputs(ROPE[name], seed=31)
    log(f"[case] gqla_decode {name} seqlens={list(d['cache_seqlens'])}")
    out, lse = _run_rope_decode(d, dev)
    ref_out, ref_lse = oracle.attend_two_pass(d["q"], d["k"], d["block_table"],
                                              d["cache_seqlens"], SCALE, d["cfg"].causal,
                                              v_cache=d["v"])
    check(out, lse, ref_out, ref_lse, f"gqla_decode {name}")


def test_rope_layout_decode_reads_no_slot_past_the_end(dev):
    """Page tails and block-table pads filled with NaN leave the result
    unchanged."""
    cfg = _rope_cfg(10, 2, 128, 8, RAGGED, True)
    clean = make_inputs(cfg, seed=5)
    dirty = make_inputs(cfg, seed=5, poison=True)
    log("[case] gqla_decode poisoned tails and pads")
    out, lse = _run_rope_decode(dirty, dev)
    ref_out, ref_lse = oracle.attend_two_pass(clean["q"], clean["k"], clean["block_table"],
                                              clean["cache_seqlens"], SCALE, True,
                                              v_cache=clean["v"])
    check(out, lse, ref_out, ref_lse, "gqla_decode poisoned")


# ------------------------------------------------- both paths end to end
def _both_paths(d, dev):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = d["cfg"]
    t = _dev_inputs(d, dev)
    qa = lib.gqla_absorb_query(t["q"], t["w_uk"])
    o_lat, lse_a = lib.mla_decode(qa, t["kv"], t["block_table"], t["cache_seqlens"], cfg.scale,
                                  cfg.causal)
    out_a = lib.gqla_absorb_output(o_lat, t["w_uv"])
    k, v = lib.gqla_expand_kv(t["kv"], t["w_uk"], t["w_uv"])
    out_g, lse_g = lib.gqla_decode(t["q"], k, v, t["block_table"], t["cache_seqlens"], cfg.scale,
                                   cfg.causal)
    torch.cuda.synchronize()
    return ((_f64(out_a), lse_a.cpu().double().numpy()),
            (_f64(out_g), lse_g.cpu().double().numpy()))


def _chain_check(out, lse, ref_out, ref_lse, what):
    res = oracle.compare(out, lse, ref_out, ref_lse, max_abs=CHAIN_MAX_ABS, rel_l2=CHAIN_REL_L2,
                         lse_abs=CHAIN_LSE)
    log(f"[parity] {what} vs exact definition: " + ", ".join(f"{k}={v}" for k, v in res.items()))
    assert res["ok"], f"{what}: {res}"


def _e2e(d, dev, idx):
    cfg = d["cfg"]
    (out_a, lse_a), (out_g, lse_g) = _both_paths(d, dev)
    sub = dict(q=d["q"][idx], kv=d["kv"], w_uk=d["w_uk"], w_uv=d["w_uv"],
               block_table=d["block_table"][idx], seqlens=d["cache_seqlens"][idx],
               scale=cfg.scale, causal=cfg.causal)
    args = tuple(sub.values())
    bt = sub["block_table"]
    used = [int(p) for p in bt[bt >= 0]]
    log(f"[case] oracle over sequences {list(idx)}")
    ra_out, ra_lse, _ = gqla.attend_absorb(*args, round_bf16=True)
    rg_out, rg_lse = gqla.attend_gqa_path(*args, round_bf16=True, pages=used)
    check(out_a[idx], lse_a[idx], ra_out, ra_lse, "absorb path (bf16 rounding points)")
    check(out_g[idx], lse_g[idx], rg_out, rg_lse, "GQA path (bf16 rounding points)")
    ex_out, ex_lse = gqla.attend_direct(*args)
    _chain_check(out_a[idx], lse_a[idx], ex_out, ex_lse, "absorb path")
    _chain_check(out_g[idx], lse_g[idx], ex_out, ex_lse, "GQA path")


@pytest.mark.parametrize("kw", [{}, dict(causal=False, s_q=1, seqlens_fixed=(700, 64, 1)),
                                dict(h_kv=1, h_q=8), dict(h_kv=8, h_q=128, s_q=1,
                                                          seqlens_fixed=(0, 5, 129))])
def test_both_paths_small(dev, kw):
    cfg = GQLA_CONFIGS["small"].with_(**kw)
    d = make_gqla_inputs(cfg)
    log(f"[case] both paths {cfg.name} {kw}")
    _e2e(d, dev, np.arange(cfg.batch))


def test_both_paths_dsv3_size(dev):
    """64 sequences of 4096 tokens, 128 heads in 8 groups: the GPU runs the
    whole batch, the oracle three sampled sequences."""
    cfg = GQLA_CONFIGS["dsv3"]
    log(f"[case] both paths {cfg.name}: generating inputs")
    d = make_gqla_inputs(cfg)
    _e2e(d, dev, np.array([0, 17, 63]))
