"""Pins of the FP8 cache oracle (CPU).

The E4M3 table and rounding are pinned by the format's defining values and
by torch's float8_e4m3fn (an independent library implementation); the
quantiser by its error bound, exact power-of-two cases and the scale rule;
FP8 decode by caches whose dequantised values are bf16-exact, which reduce
it to the already pinned attention oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from workloads import CONFIGS, make_inputs, f32_to_bf16_bits


def test_defining_codes():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0,
             0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for c, v in cases.items():
        assert fp8.e4m3_value(c) == v, hex(c)
    assert np.isnan(fp8.e4m3_value(0x7F)) and np.isnan(fp8.e4m3_value(0xFF))
    assert fp8.e4m3_value(0x80) == 0.0 and np.signbit(fp8.e4m3_value(0x80))


def test_table_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_rounding_matches_torch_on_random_and_midpoint_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.6, 20000)).astype(np.float32)
    x = x[np.abs(x) <= 448]
    vals = fp8.e4m3_value(np.arange(0x7F))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)        # exact in float32
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1000))])
    ours = fp8.e4m3_round(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_every_finite_value_rounds_to_its_own_code_and_ties_go_even():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_round(fp8.e4m3_value(codes)), codes)
    assert fp8.e4m3_round(1.0625) == 0x38        # between 1 (0x38) and 1.125: even
    assert fp8.e4m3_round(1.1875) == 0x3A        # between 1.125 and 1.25 (0x3A): even
    assert fp8.e4m3_round(2.0 ** -10) == 0x00    # half the smallest subnormal
    assert fp8.e4m3_round(1.5 * 2.0 ** -9) == 0x02
    assert fp8.e4m3_round(7.5 * 2.0 ** -9) == 0x08   # subnormal 7 / normal 8: even
    assert fp8.e4m3_round(440.0) == 0x7E and fp8.e4m3_round(-420.0) == 0xFD
    with pytest.raises(ValueError):
        fp8.e4m3_round(449.0)


def test_quantiser_scale_rule_and_error_bound():
    d = make_inputs(CONFIGS[1])
    rows = d["kv"][:, :, 0, :].reshape(-1, 576)
    rows = np.concatenate([rows, _special_rows()])
    codes, scales = fp8.quantize_rows(rows)
    x = oracle.bf16_to_f64(rows)
    amax = np.abs(x).max(axis=1)
    live = amax > 0
    # a power of two, the smallest one not below the float32 quotient amax / 448
    m, _ = np.frexp(scales.astype(np.float64))
    assert np.all(m == 0.5)
    r = (amax.astype(np.float32) / np.float32(448)).astype(np.float64)
    assert np.all(scales[live] >= r[live]) and np.all(scales[live] / 2 < np.maximum(r[live], 2.0 ** -125))
    # the largest element lands in [224, 448] (225 rounds down to 224) unless
    # the scale sits at its 2^-126 floor
    i = np.abs(x).argmax(axis=1)
    top = np.abs(fp8.e4m3_value(codes[np.arange(len(i)), i]))
    unclamped = live & (r >= 2.0 ** -126)
    assert unclamped.sum() < len(unclamped)  # the floor case is in the sample
    assert scales[-1] == 2.0 ** -126           # the 1e-38 row: quotient below 2^-126
    assert np.all((top[unclamped] >= 224) & (top[unclamped] <= 448))
    # half a step of the E4M3 grid (2^-4 relative for normals, 2^-10 absolute
    # below 2^-6), times the scale; x / scale itself is exact
    deq = fp8.dequantize(codes, scales)
    y = np.abs(x) / scales[:, None]
    bound = scales[:, None] * np.maximum(y * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(deq - x) <= bound)


def _special_rows():
    rng = np.random.default_rng(3)
    rows = [rng.standard_normal(576) * 1e-3, rng.standard_normal(576) * 300.0,
            np.where(np.arange(576) == 5, 1e4, 1e-2), -np.abs(rng.standard_normal(576)),
            np.full(576, 448.0 * 2.0 ** -3), np.full(576, 1e-38)]
    return f32_to_bf16_bits(np.stack(rows).astype(np.float32))


def test_quantiser_zero_row_and_exact_power_of_two_rows():
    z = np.zeros((1, 576), np.uint16)
    codes, scales = fp8.quantize_rows(z)
    assert scales[0] == 1.0 and not codes.any()
    # values taken from the E4M3 grid times 2^-3 with the maximum 448 * 2^-3
    rng = np.random.default_rng(1)
    grid = fp8.e4m3_value(rng.integers(0, 0x7E, 576))
    grid[17] = 448.0
    x = (grid * 0.125).astype(np.float32)
    rows = f32_to_bf16_bits(x)[None]
    codes, scales = fp8.quantize_rows(rows)
    assert scales[0] == 0.125
    assert np.array_equal(fp8.dequantize(codes, scales)[0], x.astype(np.float64))


def _exact_fp8_cache(P, seed):
    """Codes anywhere on the grid (no NaN) with power-of-two scales: every
    dequantised value is a bf16 value."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (P, 64, 576)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C
    scales = (2.0 ** rng.integers(-9, -4, (P, 64))).astype(np.float32)
    return codes, scales


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_decode_with_bf16_exact_values_equals_attention_oracle(causal):
    cfg = CONFIGS[1].with_(s_q=2, causal=causal, seqlen_rule="fixed", batch=3,
                           seqlens_fixed=(1, 64, 200))
    d = make_inputs(cfg, seed=4)
    P = d["kv"].shape[0]
    codes, scales = _exact_fp8_cache(P, 5)
    vals = fp8.dequantize(codes, scales).astype(np.float32)
    bf = f32_to_bf16_bits(vals)
    assert np.array_equal(oracle.bf16_to_f64(bf), vals.astype(np.float64))
    ref_out, ref_lse = oracle.attend_two_pass(d["q"], bf[:, :, None, :], d["block_table"],
                                              d["cache_seqlens"], cfg.scale, causal, d_v=512)
    out, lse = fp8.attend_fp8(d["q"], codes, scales, d["block_table"], d["cache_seqlens"],
                              cfg.scale, causal)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(out - ref_out).max() <= 1e-12 * max(1.0, np.abs(ref_out).max())
    assert np.abs(lse[fin] - ref_lse[fin]).max() <= 1e-12 * max(1.0, np.abs(ref_lse[fin]).max())
