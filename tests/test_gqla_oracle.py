"""Pins of the GQLA oracle (CPU, fp64).

The absorb path, the GQA path and the direct definition are three separate
routes that agree in exact arithmetic. They are pinned against things
outside themselves: weights that select latent columns reduce the model to
plain attention over bf16 caches (the already pinned attention oracle),
power-of-two group weights expose the head -> group map, a single key gives
the closed form, and the expansion matches a brute-force sum.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import gqla
from workloads import GQLA_CONFIGS, make_gqla_inputs, f32_to_bf16_bits

ONE = np.uint16(0x3F80)  # bf16 1.0


def _small(**kw):
    return make_gqla_inputs(GQLA_CONFIGS["small"].with_(**kw) if kw else GQLA_CONFIGS["small"])


def _run(fn, d):
    c = d["cfg"]
    return fn(d["q"], d["kv"], d["w_uk"], d["w_uv"], d["block_table"], d["cache_seqlens"],
              c.scale, c.causal)


def _close(a, b, rel=1e-11):
    a, b = np.asarray(a), np.asarray(b)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.array_equal(a[~fin], b[~fin])
    scale = max(1.0, float(np.abs(b[fin]).max())) if fin.any() else 1.0
    assert float(np.abs(a[fin] - b[fin]).max(initial=0.0)) <= rel * scale


@pytest.mark.parametrize("kw", [{}, dict(causal=False, s_q=1),
                                dict(h_kv=1), dict(h_kv=16, seqlens_fixed=(64, 65, 5))])
def test_absorb_path_and_gqa_path_equal_the_definition(kw):
    d = _small(**kw)
    out, lse = _run(gqla.attend_direct, d)
    a_out, a_lse, _ = _run(gqla.attend_absorb, d)
    g_out, g_lse = _run(gqla.attend_gqa_path, d)
    _close(a_out, out)
    _close(a_lse, lse)
    _close(g_out, out)
    _close(g_lse, lse)
    assert np.isfinite(lse).any()


def _selection(G, width, starts):
    """bf16 weights W^g[c, i] = 1 where c = starts[g] + i."""
    w = np.zeros((G, 512, width), np.uint16)
    for g, a in enumerate(starts):
        w[g, a + np.arange(width), np.arange(width)] = ONE
    return w


@pytest.mark.parametrize("causal", [False, True])
def test_column_selecting_weights_reduce_to_plain_attention(causal):
    """With W_UK^g selecting latent columns a_g .. a_g+127 and W_UV^g
    columns b_g .. b_g+127, group g's keys are exactly [c[a_g:], rope] and its
    values c[b_g:], both bf16 values of the cache; the pinned attention
    oracle over caches sliced that way must give the same result."""
    d = _small(causal=causal)
    G = d["cfg"].h_kv
    a = [0, 96, 200, 384][:G]
    b = [384, 7, 130, 256][:G]
    d["w_uk"] = _selection(G, 128, a)
    d["w_uv"] = _selection(G, 128, b)
    kv = d["kv"][:, :, 0, :]
    k_cache = np.stack([np.concatenate([kv[..., s:s + 128], kv[..., 512:]], axis=-1) for s in a],
                       axis=2)
    v_cache = np.stack([kv[..., s:s + 128] for s in b], axis=2)
    ref_out, ref_lse = oracle.attend_two_pass(d["q"], k_cache, d["block_table"],
                                              d["cache_seqlens"], d["cfg"].scale, causal,
                                              v_cache=v_cache)
    for fn in (gqla.attend_direct, gqla.attend_gqa_path):
        out, lse = _run(fn, d)
        _close(out, ref_out)
        _close(lse, ref_lse)
    out, lse, _ = _run(gqla.attend_absorb, d)
    _close(out, ref_out)
    _close(lse, ref_lse)


def test_group_weights_scaled_by_powers_of_two_expose_the_head_to_group_map():
    """Same W_UK for every group and W_UV^g = 2^g W_UV^0: head h's output is
    2^(h // (h_q / h_kv)) times that of the one-group model, its lse equal."""
    d = _small()
    G, H = d["cfg"].h_kv, d["cfg"].h_q
    wk0, wv0 = d["w_uk"][:1], d["w_uv"][:1]
    d["w_uk"] = np.repeat(wk0, G, axis=0)
    wv = oracle.bf16_to_f64(wv0[0]).astype(np.float32)
    d["w_uv"] = np.stack([f32_to_bf16_bits(wv * np.float32(2.0 ** g)) for g in range(G)])
    one = dict(d, w_uk=wk0, w_uv=wv0)
    ref_out, ref_lse = _run(gqla.attend_direct, one)
    mult = np.array([2.0 ** (h // (H // G)) for h in range(H)])[None, None, :, None]
    for fn in (gqla.attend_direct, gqla.attend_gqa_path):
        out, lse = _run(fn, d)
        _close(out, ref_out * mult)
        _close(lse, ref_lse)
    out, lse, _ = _run(gqla.attend_absorb, d)
    _close(out, ref_out * mult)


def test_a_single_key_gives_its_value_and_score():
    """L = 1: the softmax weight is 1, so o_h = c W_UV^g and
    lse_h = scale * (q_nope . c W_UK^g + q_rope . k_rope), written out as sums."""
    d = _small(batch=1, s_q=1, causal=False, seqlens_fixed=(1,))
    out, lse = _run(gqla.attend_direct, d)
    a_out, a_lse, _ = _run(gqla.attend_absorb, d)
    row = oracle.bf16_to_f64(d["kv"][d["block_table"][0, 0], 0, 0])
    q = oracle.bf16_to_f64(d["q"][0, 0])
    Wk, Wv = oracle.bf16_to_f64(d["w_uk"]), oracle.bf16_to_f64(d["w_uv"])
    H, G = d["cfg"].h_q, d["cfg"].h_kv
    sigma = float(np.float32(d["cfg"].scale))
    for h in range(0, H, 5):
        g = h // (H // G)
        for j in (0, 77, 127):
            v = math.fsum(row[c] * Wv[g, c, j] for c in range(512))
            assert abs(out[0, 0, h, j] - v) <= 1e-12 * max(1.0, abs(v))
            assert abs(a_out[0, 0, h, j] - v) <= 1e-12 * max(1.0, abs(v))
        k = [math.fsum(row[c] * Wk[g, c, i] for c in range(512)) for i in range(128)]
        s = sigma * math.fsum([q[h, i] * k[i] for i in range(128)] +
                              [q[h, 128 + r] * row[512 + r] for r in range(64)])
        assert abs(lse[0, 0, h] - s) <= 1e-12 * max(1.0, abs(s))
        assert abs(a_lse[0, 0, h] - s) <= 1e-12 * max(1.0, abs(s))


def test_expansion_matches_a_brute_force_sum_and_copies_the_rope():
    d = _small()
    K, V = gqla.expand_group_cache(d["kv"], d["w_uk"], d["w_uv"])
    P, G = d["kv"].shape[0], d["cfg"].h_kv
    assert K.shape == (P, 64, G, 192) and V.shape == (P, 64, G, 128)
    lat = oracle.bf16_to_f64(d["kv"][:, :, 0])
    Wk, Wv = oracle.bf16_to_f64(d["w_uk"]), oracle.bf16_to_f64(d["w_uv"])
    rng = np.random.default_rng(0)
    for _ in range(40):
        p, s, g, i = (int(rng.integers(n)) for n in (P, 64, G, 128))
        k = math.fsum(lat[p, s, c] * Wk[g, c, i] for c in range(512))
        v = math.fsum(lat[p, s, c] * Wv[g, c, i] for c in range(512))
        assert abs(K[p, s, g, i] - k) <= 1e-12 * max(1.0, abs(k))
        assert abs(V[p, s, g, i] - v) <= 1e-12 * max(1.0, abs(v))
    assert np.array_equal(K[..., 128:], np.repeat(lat[:, :, None, 512:], G, axis=2))


def test_absorbed_query_keeps_the_rope_and_folds_w_uk():
    d = _small()
    qa = gqla.absorb_query(d["q"], d["w_uk"])
    q = oracle.bf16_to_f64(d["q"])
    Wk = oracle.bf16_to_f64(d["w_uk"])
    H, G = d["cfg"].h_q, d["cfg"].h_kv
    assert np.array_equal(qa[..., 512:], q[..., 128:])
    for (b, t, h, c) in [(0, 0, 0, 0), (1, 1, 5, 511), (2, 0, 15, 300), (2, 1, 8, 3)]:
        g = h // (H // G)
        x = math.fsum(q[b, t, h, i] * Wk[g, c, i] for i in range(128))
        assert abs(qa[b, t, h, c] - x) <= 1e-12 * max(1.0, abs(x))


def test_rows_without_keys_are_zero_with_minus_infinite_lse():
    d = _small(seqlens_fixed=(0, 1, 300))
    for fn in (gqla.attend_direct, gqla.attend_gqa_path):
        out, lse = _run(fn, d)
        assert np.all(out[0] == 0.0) and np.all(lse[0] == -np.inf)
        # causal, s_q = 2: the first query token of the 1-token sequence sees nothing
        assert np.all(out[1, 0] == 0.0) and np.all(lse[1, 0] == -np.inf)
        assert np.isfinite(lse[1, 1]).all()


def test_bf16_rounding_is_nearest_even():
    one = 1.0
    x = np.array([one, one + 2.0 ** -8, one + 3 * 2.0 ** -8, one + 2.0 ** -8 + 2.0 ** -20,
                  -2.5, 3.0e38, 2.0 ** -130, 2.0 ** -140, one + 2.0 ** -8 + 2.0 ** -30])
    r = gqla.round_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                       # tie -> even (significand ...0)
    assert r[2] == 1.0 + 2.0 ** -6           # tie -> even (significand ...10)
    assert r[3] == 1.0 + 2.0 ** -7           # above the tie -> up
    assert r[4] == -2.5
    assert r[5] == 2.0 ** 127 * 226 / 128   # 3e38 / 2^127 = 1.7632 -> 226 / 128
    assert r[6] == 2.0 ** -130               # a bf16 subnormal, exact
    assert r[7] == 0.0                       # below half the smallest bf16 subnormal (2^-133)
    assert r[8] == 1.0                       # float32 first: the 2^-30 is lost, then a tie
    rng = np.random.default_rng(3)
    y = rng.standard_normal(1000) * 10.0 ** rng.uniform(-5, 5, 1000)
    ry = gqla.round_bf16(y)
    assert np.all(np.abs(ry - y) <= oracle.bf16_step(y) / 2 * (1 + 1e-12))


def test_rounding_points_change_nothing_for_exact_bf16_intermediates():
    """With column-selecting weights every intermediate of both paths is a
    bf16 value already, except the latent attention output; with a single key
    that output is a latent row itself."""
    d = _small(seqlens_fixed=(1, 1, 1), causal=False, s_q=1)
    G = d["cfg"].h_kv
    d["w_uk"] = _selection(G, 128, [0, 128, 256, 384])
    d["w_uv"] = _selection(G, 128, [384, 0, 64, 200])
    ex = _run(gqla.attend_direct, d)
    c = d["cfg"]
    args = (d["q"], d["kv"], d["w_uk"], d["w_uv"], d["block_table"], d["cache_seqlens"],
            c.scale, c.causal)
    a_out, a_lse, _ = gqla.attend_absorb(*args, round_bf16=True)
    g_out, g_lse = gqla.attend_gqa_path(*args, round_bf16=True)
    for o, l in ((a_out, a_lse), (g_out, g_lse)):
        _close(o, ex[0])
        _close(l, ex[1])


def test_gqa_path_restricted_to_used_pages_is_unchanged():
    d = _small()
    c = d["cfg"]
    args = (d["q"], d["kv"], d["w_uk"], d["w_uv"], d["block_table"], d["cache_seqlens"],
            c.scale, c.causal)
    full = gqla.attend_gqa_path(*args)
    bt = d["block_table"]
    used = [int(p) for p in bt[bt >= 0]]
    part = gqla.attend_gqa_path(*args, pages=used)
    _close(part[0], full[0], rel=0)
    _close(part[1], full[1], rel=0)
