"""GPU parity of the FP8 latent cache through the C interface.

  * Quantisation (whole rows and the paged append): codes and scales
    bit-exact against the oracle's float32 rule.
  * Decode over an FP8 cache made by the oracle's quantiser: the decode bars
    (max-abs 1e-2 with the one-bf16-step allowance, rel-L2 5e-3, LSE 1e-3)
    against the oracle's attention over the dequantised cache, on ragged
    small shapes, NaN-poisoned tails and pads, scores climbing past the fixed
    reference, and full-size workloads (sampled sequences).
  * GPU quantise then GPU decode, end to end, against the oracle.
"""
import numpy as np
import pytest

import oracle
from oracle import fp8
from workloads import CONFIGS, make_inputs, f32_to_bf16_bits
from gpu_helpers import bf16_tensor, check, log
from test_parity_gpu import RAGGED, _climbing_scores, _mla

pytestmark = pytest.mark.gpu


def _dev_fp8(codes, scales, dev):
    import torch
    return (torch.from_numpy(np.ascontiguousarray(codes)).to(dev),
            torch.from_numpy(np.ascontiguousarray(scales)).to(dev))


def _decode(d, codes, scales, dev, plan=None):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = d["cfg"]
    c, s = _dev_fp8(codes, scales, dev)
    q = bf16_tensor(d["q"], dev)
    bt = torch.from_numpy(d["block_table"]).to(dev)
    L = torch.from_numpy(d["cache_seqlens"]).to(dev)
    out, lse = lib.mla_decode_fp8(q, c, s, bt, L, cfg.scale, cfg.causal, plan=plan)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy()


def _oracle(d, codes, scales, idx=None):
    cfg = d["cfg"]
    idx = np.arange(cfg.batch) if idx is None else np.asarray(idx)
    return fp8.attend_fp8(d["q"][idx], codes, scales, d["block_table"][idx],
                          d["cache_seqlens"][idx], cfg.scale, cfg.causal)


# ------------------------------------------------------------ quantisation
def _special_rows():
    rng = np.random.default_rng(3)
    rows = [np.zeros(576, np.float32),                                   # all zero
            rng.standard_normal(576).astype(np.float32) * 1e-3,          # small
            rng.standard_normal(576).astype(np.float32) * 300.0,         # large
            np.where(np.arange(576) == 5, 1e4, 1e-2).astype(np.float32),  # one outlier
            -np.abs(rng.standard_normal(576)).astype(np.float32),         # all negative
            np.linspace(-1, 1, 576).astype(np.float32),
            np.full(576, 1e-38, np.float32),                              # scale at 2^-126
            np.full(576, 56.0, np.float32)]                               # amax / 448 = 1/8
    return f32_to_bf16_bits(np.stack(rows))


@pytest.mark.parametrize("which", ["special", "config1", "config3_part"])
def test_quantize_rows_bit_exact(dev, which):
    import torch
    import mla_paged_kv_03_amd as lib
    if which == "special":
        rows = _special_rows()
    elif which == "config1":
        rows = make_inputs(CONFIGS[1])["kv"][:, :, 0, :].reshape(-1, 576)
    else:
        rows = make_inputs(CONFIGS[3].with_(batch=16))["kv"][:, :, 0, :].reshape(-1, 576)
    log(f"[case] quantize {which}: {rows.shape[0]} rows")
    codes, scales = lib.mla_kv_quantize_fp8(bf16_tensor(rows, dev))
    torch.cuda.synchronize()
    ref_codes, ref_scales = fp8.quantize_rows(rows)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), ref_scales.view(np.uint32)), "scales"
    bad = int((got_c != ref_codes).sum())
    log(f"[parity] quantize {which}: code mismatches {bad} of {got_c.size}")
    assert bad == 0


@pytest.mark.parametrize("T", [1, 3, 64])
def test_append_fp8_bit_exact(dev, T):
    """New tokens quantised into their slots; lengths shorter than s_q and a
    block-table entry outside the cache are skipped; nothing else changes."""
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = CONFIGS[1].with_(batch=4, seqlen_rule="fixed", seqlens_fixed=(1, 64, 65, 200))
    d = make_inputs(cfg, seed=9)
    codes0, scales0 = fp8.quantize_cache(d["kv"])
    bt = d["block_table"].copy()
    if T == 3:
        bt[3, 3] = 10 ** 6          # outside the cache: those slots are skipped
    rng = np.random.default_rng(T)
    new = f32_to_bf16_bits(rng.standard_normal((cfg.batch, T, 576)).astype(np.float32))
    new_c, new_s = fp8.quantize_rows(new)
    ref_codes = oracle.append_rows(codes0, new_c, bt, d["cache_seqlens"])
    ref_scales = oracle.append_rows(scales0, new_s, bt, d["cache_seqlens"])
    c, s = _dev_fp8(codes0, scales0, dev)
    log(f"[case] append fp8 T={T}")
    lib.mla_kv_append_fp8(bf16_tensor(new, dev), c, s, torch.from_numpy(bt).to(dev),
                          torch.from_numpy(d["cache_seqlens"]).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), ref_codes)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_scales.view(np.uint32))


# ------------------------------------------------------------ decode
SMALL = {
    "h8_t1": _mla(10, 1, 8, RAGGED, False),
    "h16_t1": _mla(10, 1, 16, RAGGED, False),
    "h32_t1": _mla(10, 1, 32, RAGGED, False),
    "h64_t1": _mla(10, 1, 64, RAGGED, False),
    "h128_t1": _mla(10, 1, 128, RAGGED, False),
    "h128_t2_causal": _mla(10, 2, 128, RAGGED, True),
    "h16_t3_causal": _mla(10, 3, 16, RAGGED, True),
    "h40_t2_causal": _mla(10, 2, 40, RAGGED, True),
    # dequantising copy waves with one sequence split over every worker
    "h128_t1_one_long": _mla(1, 1, 128, (20000,), False),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_decode_small_shapes(dev, name):
    d = make_inputs(SMALL[name], seed=13)
    codes, scales = fp8.quantize_cache(d["kv"])
    log(f"[case] fp8 decode {name} seqlens={list(d['cache_seqlens'])}")
    out, lse = _decode(d, codes, scales, dev)
    ref_out, ref_lse = _oracle(d, codes, scales)
    check(out, lse, ref_out, ref_lse, f"fp8 decode {name}")


def test_fp8_decode_reads_no_slot_past_the_end(dev):
    """Tail slots and an extra pad page hold NaN codes (0x7F) and NaN scales;
    the result equals the clean cache's."""
    cfg = _mla(10, 2, 128, RAGGED, True)
    d = make_inputs(cfg, seed=5, poison=True)
    clean = make_inputs(cfg, seed=5)
    codes, scales = fp8.quantize_cache(clean["kv"])
    P = d["kv"].shape[0]                       # the poisoned pool has one more page
    pc = np.full((P, 64, 576), 0x7F, np.uint8)
    ps = np.full((P, 64), np.nan, np.float32)
    for b in range(cfg.batch):
        L = int(d["cache_seqlens"][b])
        for j in range((L + 63) // 64):
            page, used = d["block_table"][b, j], min(64, L - 64 * j)
            pc[page, :used] = codes[page, :used]
            ps[page, :used] = scales[page, :used]
    log("[case] fp8 decode with NaN tails and pads")
    out, lse = _decode(d, pc, ps, dev)
    ref_out, ref_lse = _oracle(clean, codes, scales)
    check(out, lse, ref_out, ref_lse, "fp8 decode poisoned")


@pytest.mark.parametrize("period,heads", [(3, 16), (5, 16), (3, 64)])
def test_fp8_scores_climbing_from_page_to_page(dev, period, heads):
    """Both softmax passes (fixed reference, then the rescaling fallback) on an
    FP8 cache, at 16 rows per KV head and at 64 (pages dequantised by the
    copy waves, whose page loop then also runs twice)."""
    import mla_paged_kv_03_amd as lib
    import torch
    Ls = (64 * 300, 64 * 280 + 17, 64 * 300, 64 * 290)
    cfg = _mla(4, 1, heads, Ls, False)
    d = make_inputs(cfg, seed=12)
    _climbing_scores(d, cfg, period=period)
    codes, scales = fp8.quantize_cache(d["kv"])
    log(f"[case] fp8 climbing scores period {period} heads {heads}")
    out, lse = _decode(d, codes, scales, dev)
    ref_out, ref_lse = _oracle(d, codes, scales)
    check(out, lse, ref_out, ref_lse, f"fp8 climbing scores (period {period}, {heads} heads)")


@pytest.mark.parametrize("heads", [16, 64])
def test_fp8_decode_rows_of_every_magnitude(dev, heads):
    """Cache rows scaled by 2^e, e from -40 to 0 (token scales from about
    2^-47 to 2^-7): the dequantised values stay exact on both page paths
    (converted in the compute waves at 16 heads, dequantised by the copy
    waves at 64), so the decode meets the bars against the oracle."""
    cfg = _mla(6, 1, heads, (64, 200, 640, 1000, 65, 3), False)
    d = make_inputs(cfg, seed=21)
    rng = np.random.default_rng(21)
    f = (d["kv"].astype(np.uint32) << 16).view(np.float32)
    e = rng.integers(-40, 1, size=f.shape[:2]).astype(np.float32)
    d["kv"] = f32_to_bf16_bits(f * np.exp2(e)[:, :, None, None])  # exact in bf16
    codes, scales = fp8.quantize_cache(d["kv"])
    log(f"[case] fp8 rows of every magnitude, {heads} heads")
    out, lse = _decode(d, codes, scales, dev)
    ref_out, ref_lse = _oracle(d, codes, scales)
    check(out, lse, ref_out, ref_lse, f"fp8 rows of every magnitude ({heads} heads)")


def _sample(cfg, L, k=4):
    rng = np.random.default_rng(99)
    pick = {int(np.argmin(L)), int(np.argmax(L))}
    pick |= set(int(x) for x in rng.choice(cfg.batch, size=min(k, cfg.batch), replace=False))
    return sorted(pick)


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_fp8_decode_full_size(dev, idx):
    """The GPU quantises the config's cache and decodes the whole batch; the
    oracle quantises the same cache and decodes sampled sequences."""
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = CONFIGS[idx]
    log(f"[case] fp8 config {idx} {cfg.name}: generating inputs")
    d = make_inputs(cfg)
    kv = bf16_tensor(d["kv"], dev)
    c, s = lib.mla_kv_quantize_fp8(kv)
    del kv
    q = bf16_tensor(d["q"], dev)
    bt = torch.from_numpy(d["block_table"]).to(dev)
    L = torch.from_numpy(d["cache_seqlens"]).to(dev)
    out, lse = lib.mla_decode_fp8(q, c, s, bt, L, cfg.scale, cfg.causal)
    torch.cuda.synchronize()
    out = out.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    assert np.isfinite(out).all()
    idx_s = _sample(cfg, d["cache_seqlens"])
    log(f"[case] oracle over sequences {idx_s}")
    pages = sorted(set(int(p) for b in idx_s
                       for p in d["block_table"][b, :(int(d["cache_seqlens"][b]) + 63) // 64]))
    codes = np.zeros((d["kv"].shape[0], 64, 576), np.uint8)
    scales = np.ones((d["kv"].shape[0], 64), np.float32)
    codes[pages], scales[pages] = fp8.quantize_rows(d["kv"][pages][:, :, 0, :])
    ref_out, ref_lse = _oracle(d, codes, scales, idx_s)
    check(out[idx_s], lse[idx_s], ref_out, ref_lse, f"fp8 config {idx} (sampled)")
    # the GPU's codes of those pages are the oracle's
    assert np.array_equal(c.cpu().numpy()[pages], codes[pages])


# ------------------------------------------------------------ scale check
def _scale_status(scales, dev):
    import torch
    import mla_paged_kv_03_amd as lib
    st = lib.mla_check_fp8_scales(torch.from_numpy(np.ascontiguousarray(scales)).to(dev))
    torch.cuda.synchronize()
    s = st.cpu().numpy().astype(np.int64)
    first = (s[1] & 0xffffffff) | (s[2] << 32)
    return int(s[0]), int(first), int(s[3]) & 0xffffffff


@pytest.mark.parametrize("which", ["config1", "config3_part"])
def test_scale_check_passes_quantised_caches(dev, which):
    """Scales the oracle's quantiser writes are powers of two: none flagged."""
    cfg = CONFIGS[1] if which == "config1" else CONFIGS[3].with_(batch=16)
    kv = make_inputs(cfg)["kv"][:, :, 0, :]
    _, scales = fp8.quantize_rows(kv.reshape(-1, 576))
    log(f"[case] scale check {which}: {scales.size} scales")
    assert _scale_status(scales.reshape(kv.shape[0], -1), dev) == (0, -1, 0)


def test_scale_check_counts_planted_scales(dev):
    """Planted scales that are not positive normal powers of two are counted,
    and the first of them is named with its bits: 3.0 (mantissa set), -0.5
    (sign), a subnormal, 0, +inf and NaN (exponent field 0 or 255); the
    largest and smallest normal powers of two pass."""
    n = 64 * 1000 + 37                       # several passes of the workgroup, ragged tail
    scales = np.exp2(np.random.default_rng(11).integers(-20, 20, n)).astype(np.float32)
    scales[5] = np.float32(2.0 ** 127)
    scales[6] = np.float32(2.0 ** -126)
    assert _scale_status(scales, dev) == (0, -1, 0)
    planted = {777: 3.0, 1024: -0.5, 4097: np.float32(2.0 ** -130), 40000: 0.0,
               50001: np.inf, n - 1: np.nan}
    for i, v in planted.items():
        scales[i] = v
    log(f"[case] scale check: {n} scales, {len(planted)} planted")
    assert _scale_status(scales, dev) == (len(planted), 777, int(np.float32(3.0).view(np.uint32)))
    scales[777] = 1.0
    assert _scale_status(scales, dev) == (len(planted) - 1, 1024,
                                         int(np.float32(-0.5).view(np.uint32)))
    empty = np.zeros(0, np.float32)
    assert _scale_status(empty, dev) == (0, -1, 0)
