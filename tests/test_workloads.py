"""The seeded input generator: bf16 rounding, determinism, page placement."""
import numpy as np
import pytest

from workloads import CONFIGS, config_inputs, f32_to_bf16_bits, make_inputs, draw_seqlens
from workloads.gen import _normal_bf16


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, -2.0, 3.140625,
                  1.0 + 2.0 ** -8,          # halfway, even neighbour is 1.0
                  1.0 + 3 * 2.0 ** -8,      # halfway, even neighbour is 1 + 2^-6
                  1.0 + 2.0 ** -8 + 2.0 ** -20,  # just above halfway: rounds up
                  -(1.0 + 2.0 ** -8)], dtype=np.float32)
    got = f32_to_bf16_bits(x)
    assert list(got) == [0x3F80, 0xC000, 0x4049, 0x3F80, 0x3F82, 0x3F81, 0xBF80]


def test_generation_is_deterministic_and_chunk_free():
    a = make_inputs(CONFIGS[3].with_(batch=6), seed=11)
    b = make_inputs(CONFIGS[3].with_(batch=6), seed=11)
    for k in ("q", "kv", "block_table", "cache_seqlens"):
        assert np.array_equal(a[k], b[k])
    r1, r2 = np.random.default_rng(5), np.random.default_rng(5)
    x1 = _normal_bf16(r1, (40, 64, 1, 8), 1.0, chunk=1)
    x2 = _normal_bf16(r2, (40, 64, 1, 8), 1.0, chunk=7)
    assert np.array_equal(x1, x2)


def test_length_rules():
    rng = np.random.default_rng(0)
    L3 = draw_seqlens(CONFIGS[3].with_(batch=5000), rng)
    assert L3.min() >= 1 and L3.max() <= 16384
    # log-uniform: about half the mass below sqrt(16385)
    assert 0.4 < np.mean(L3 < 128) < 0.6
    L5 = draw_seqlens(CONFIGS[5].with_(batch=5000), rng)
    assert L5.min() >= 8192 and L5.max() <= 32768


def test_seeded_lengths_of_the_variable_length_configs():
    d3 = np.random.default_rng(3)
    L3 = draw_seqlens(CONFIGS[3], d3)
    assert int(L3.sum()) == 184920 and int(((L3 + 63) // 64).sum()) == 2966
    assert int((L3 == 1).sum()) == 5
    L5 = draw_seqlens(CONFIGS[5], np.random.default_rng(5))
    assert int(L5.sum()) == 624765 and int(((L5 + 63) // 64).sum()) == 9782


@pytest.mark.parametrize("poison", [False, True])
def test_block_table_is_a_permutation(poison):
    cfg = CONFIGS[3].with_(batch=16)
    d = make_inputs(cfg, seed=3, poison=poison)
    L, bt = d["cache_seqlens"], d["block_table"]
    n = (L + 63) // 64
    used = np.concatenate([bt[b, :n[b]] for b in range(cfg.batch)])
    assert sorted(used.tolist()) == list(range(int(n.sum())))
    pads = np.concatenate([bt[b, n[b]:] for b in range(cfg.batch)])
    if poison:
        assert (pads == int(n.sum())).all()
        kv = d["kv"]
        assert (kv[int(n.sum())] == 0x7FC0).all()
        for b in range(cfg.batch):
            r = int(L[b]) % 64
            if r:
                assert (kv[bt[b, n[b] - 1], r:] == 0x7FC0).all()
                assert not (kv[bt[b, n[b] - 1], :r] == 0x7FC0).any()
    else:
        assert (pads == -1).all()


def test_config_shapes():
    d = config_inputs(1)
    assert d["q"].shape == (2, 1, 8, 576) and d["kv"].shape == (5, 64, 1, 576)
    assert list(d["cache_seqlens"]) == [64, 200]
    g = make_inputs(CONFIGS[5].with_(batch=2, seqlen_lo=70, seqlen_hi=130), seed=1)
    assert g["k"].shape[1:] == (64, 8, 128) and g["v"].shape[1:] == (64, 8, 128)
    assert "kv" not in g
