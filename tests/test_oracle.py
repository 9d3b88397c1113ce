"""Pins for the fp64 oracle, each against something other than the oracle:
hand-worked closed forms, brute force, a library routine, and invariants
that the definition of attention fixes."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import (attend_bruteforce, attend_online, attend_two_pass, bf16_to_f64,
                    combine, softmax_weights)
from workloads import CONFIGS, f32_to_bf16_bits, make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def run(fn, d, **kw):
    cfg = d["cfg"]
    if cfg.kind == "mla":
        return fn(d["q"], d["kv"], d["block_table"], d["cache_seqlens"], cfg.scale,
                  cfg.causal, d_v=cfg.d_v, **kw)
    return fn(d["q"], d["k"], d["block_table"], d["cache_seqlens"], cfg.scale,
              cfg.causal, v_cache=d["v"], **kw)


def assert_close(a, b, rtol=1e-12, atol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb), "non-finite pattern differs"
    assert np.array_equal(a[~fa], b[~fb])
    np.testing.assert_allclose(a[fa], b[fb], rtol=rtol, atol=atol)


# small shapes that still cross page boundaries and cover empty/one-key rows
TINY = {
    "mla": CONFIGS[1].with_(batch=4, h_q=4, d_qk=40, d_v=32, seqlen_rule="fixed",
                            seqlens_fixed=(0, 1, 130, 64)),
    "mla_causal2": CONFIGS[3].with_(batch=5, h_q=4, d_qk=40, d_v=32, seqlen_rule="fixed",
                                    seqlens_fixed=(1, 2, 65, 64, 129)),
    "mla_causal3": CONFIGS[3].with_(batch=3, s_q=3, h_q=2, d_qk=24, d_v=16,
                                    seqlen_rule="fixed", seqlens_fixed=(2, 66, 3)),
    "gqa": CONFIGS[5].with_(batch=3, h_q=6, h_kv=3, d_qk=16, d_v=12, seqlen_rule="fixed",
                            seqlens_fixed=(70, 1, 128)),
    "gqa_causal": CONFIGS[5].with_(batch=2, s_q=2, causal=True, h_q=4, h_kv=2, d_qk=16,
                                   d_v=16, seqlen_rule="fixed", seqlens_fixed=(65, 3)),
    "c1": CONFIGS[1],
}


def tiny(name, seed=7, **kw):
    return make_inputs(TINY[name], seed=seed, **kw)


# ---------------------------------------------------------------- bf16 decode
def test_bf16_decode_exact_values():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F80, 0xFF80, 0x0000, 0x3F81],
                    dtype=np.uint16)
    v = bf16_to_f64(bits)
    assert list(v[:3]) == [1.0, -1.0, 3.140625]
    assert v[3] == 2.0 ** -133           # smallest subnormal bf16
    assert v[4] == np.inf and v[5] == -np.inf and v[6] == 0.0
    assert v[7] == 1.0 + 2.0 ** -7


# ---------------------------------------------------------- worked examples
def _golden_inputs(case):
    q = np.array(case["q"], dtype=np.float32)[None]            # [1, T, 1, 4]
    keys = np.array(case["keys"], dtype=np.float32)
    for arr in (q, keys):
        assert np.array_equal(bf16_to_f64(f32_to_bf16_bits(arr)), arr.astype(np.float64))
    kv = np.zeros((1, 64, 1, 4), dtype=np.uint16)
    kv[0, :len(keys), 0] = f32_to_bf16_bits(keys)
    bt = np.zeros((1, 1), dtype=np.int32)
    L = np.array([len(keys)], dtype=np.int32)
    return f32_to_bf16_bits(q), kv, bt, L


@pytest.mark.parametrize("fn", [attend_two_pass, attend_online, attend_bruteforce])
def test_worked_examples(fn):
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        q, kv, bt, L = _golden_inputs(case)
        out, lse = fn(q, kv, bt, L, case["scale"], case["causal"], d_v=2)
        np.testing.assert_allclose(out[0], np.array(case["out"]), rtol=1e-14, atol=1e-14,
                                   err_msg=case["name"])
        np.testing.assert_allclose(lse[0], np.array(case["lse"]), rtol=1e-14, atol=1e-14,
                                   err_msg=case["name"])


# ------------------------------------------------------------- brute force
@pytest.mark.parametrize("name", list(TINY))
def test_two_pass_matches_bruteforce(name):
    d = tiny(name)
    o1, l1 = run(attend_two_pass, d)
    o2, l2 = run(attend_bruteforce, d)
    assert_close(o1, o2)
    assert_close(l1, l2)


@pytest.mark.parametrize("seed", range(6))
def test_random_tiny_shapes_match_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    G = int(rng.integers(1, 4))
    H = G * int(rng.integers(1, 4))
    T = int(rng.integers(1, 4))
    kind = "mla" if seed % 2 == 0 else "gqa"
    d_qk = int(rng.integers(4, 33))
    d_v = int(rng.integers(1, d_qk + 1)) if kind == "mla" else int(rng.integers(1, 20))
    B = int(rng.integers(1, 5))
    Ls = tuple(int(x) for x in rng.integers(0, 200, size=B))
    cfg = CONFIGS[5 if kind == "gqa" else 3].with_(
        kind=kind, batch=B, s_q=T, h_q=H, h_kv=G, d_qk=d_qk, d_v=d_v,
        causal=bool(seed % 3), seqlen_rule="fixed", seqlens_fixed=Ls,
        scale=float(rng.uniform(0.05, 0.5)))
    d = make_inputs(cfg, seed=seed)
    o1, l1 = run(attend_two_pass, d)
    o2, l2 = run(attend_bruteforce, d)
    assert_close(o1, o2)
    assert_close(l1, l2)


# ------------------------------------------------- library routine (SDPA)
@pytest.mark.parametrize("name", ["mla", "mla_causal2", "gqa", "gqa_causal", "c1"])
def test_two_pass_matches_torch_sdpa_fp64(name):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    d = tiny(name)
    cfg = d["cfg"]
    out, lse = run(attend_two_pass, d)
    sigma = float(np.float32(cfg.scale))
    q_t = torch.from_numpy(d["q"].view(np.int16)).view(torch.bfloat16).double()
    kname = "kv" if cfg.kind == "mla" else "k"
    k_all = torch.from_numpy(d[kname].view(np.int16)).view(torch.bfloat16).double()
    v_all = (k_all[..., :cfg.d_v] if cfg.kind == "mla" else
             torch.from_numpy(d["v"].view(np.int16)).view(torch.bfloat16).double())
    hpg = cfg.h_q // cfg.h_kv
    checked = 0
    for b in range(cfg.batch):
        L = int(d["cache_seqlens"][b])
        if L == 0:
            continue
        n = (L + 63) // 64
        idx = torch.from_numpy(d["block_table"][b, :n].astype(np.int64))
        K = k_all[idx].reshape(n * 64, cfg.h_kv, -1)[:L]           # [L, G, D]
        V = v_all[idx].reshape(n * 64, cfg.h_kv, -1)[:L]
        K = K.repeat_interleave(hpg, dim=1).permute(1, 0, 2)       # [H, L, D]
        V = V.repeat_interleave(hpg, dim=1).permute(1, 0, 2)
        qb = q_t[b].permute(1, 0, 2)                                # [H, T, D]
        T = cfg.s_q
        j = torch.arange(L)[None, :]
        t = torch.arange(T)[:, None]
        mask = (j <= L - T + t) if cfg.causal else torch.ones(T, L, dtype=torch.bool)
        ref = F.scaled_dot_product_attention(qb, K, V, attn_mask=mask, scale=sigma)
        rows = mask.any(dim=1)
        got = torch.from_numpy(out[b]).permute(1, 0, 2)              # [H, T, Dv]
        np.testing.assert_allclose(got[:, rows].numpy(), ref[:, rows].numpy(),
                                   rtol=1e-10, atol=1e-12)
        s = torch.einsum("htd,hld->htl", qb, K) * sigma
        s = s.masked_fill(~mask[None], float("-inf"))
        ref_lse = torch.logsumexp(s, dim=-1)                          # [H, T]
        np.testing.assert_allclose(lse[b].T[:, rows.numpy()], ref_lse[:, rows].numpy(),
                                   rtol=1e-12, atol=1e-12)
        checked += int(rows.sum())
    assert checked > 0


# --------------------------------------------------------- online == 2-pass
@pytest.mark.parametrize("name", list(TINY))
def test_online_equals_two_pass(name):
    d = tiny(name)
    o1, l1 = run(attend_two_pass, d)
    o2, l2 = run(attend_online, d)
    assert_close(o1, o2)
    assert_close(l1, l2)


@pytest.mark.parametrize("block", [1, 7, 64, 1000])
def test_online_block_size_does_not_matter(block):
    d = tiny("mla_causal2")
    o1, l1 = run(attend_two_pass, d)
    o2, l2 = run(attend_online, d, block=block)
    assert_close(o1, o2)
    assert_close(l1, l2)


# ------------------------------------------------------ normalisation
def test_softmax_rows_sum_to_one():
    d = tiny("mla_causal2")
    cfg = d["cfg"]
    for b in range(cfg.batch):
        for t in range(cfg.s_q):
            w = softmax_weights(d["q"], d["kv"], d["block_table"], d["cache_seqlens"],
                                cfg.scale, cfg.causal, b, t)
            if w.shape[1]:
                np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-13)
                assert (w >= 0).all()


def test_softmax_weights_match_worked_examples():
    # hand-worked weights: equal scores, one key, scores 0 and 1, and the
    # bottom-right causal case (token 0 of two sees only key 0)
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        q, kv, bt, L = _golden_inputs(case)
        for t, per_head in enumerate(case["weights"]):
            w = softmax_weights(q, kv, bt, L, case["scale"], case["causal"], 0, t)
            np.testing.assert_allclose(w, np.array(per_head), rtol=1e-14, atol=1e-15,
                                       err_msg=f"{case['name']} token {t}")


@pytest.mark.parametrize("name", ["mla_causal2", "mla_causal3", "gqa", "gqa_causal"])
def test_softmax_weights_reproduce_bruteforce(name):
    """The weights of every (b, t, h) times the V rows of the visible keys
    give the dense brute-force output, and a row with no visible key has no
    weights exactly where brute force gives lse = -inf. A wrong scale, head
    to group map or visible count in the weights moves the product."""
    d = tiny(name)
    cfg = d["cfg"]
    ob, lb = run(attend_bruteforce, d)
    hpg = cfg.h_q // cfg.h_kv
    vcache = d["kv"] if cfg.kind == "mla" else d["v"]
    for b in range(cfg.batch):
        for t in range(cfg.s_q):
            w = softmax_weights(d["q"], d["kv" if cfg.kind == "mla" else "k"],
                                d["block_table"], d["cache_seqlens"], cfg.scale, cfg.causal,
                                b, t)
            vis = w.shape[1]
            if vis == 0:
                assert (lb[b, t] == -np.inf).all()
                continue
            # V rows of keys 0 .. vis-1, slot by slot (no page walk)
            V = np.stack([bf16_to_f64(vcache[d["block_table"][b, j // 64], j % 64])
                          for j in range(vis)])[..., :cfg.d_v]        # [vis, G, dv]
            for h in range(cfg.h_q):
                np.testing.assert_allclose(w[h] @ V[:, h // hpg], ob[b, t, h], rtol=1e-12,
                                           atol=1e-12, err_msg=f"{name} b={b} t={t} h={h}")


def _weights_pins_hold():
    """True when the two pins above hold for the current softmax_weights."""
    try:
        test_softmax_weights_match_worked_examples()
        for name in ("mla_causal2", "gqa", "gqa_causal"):
            test_softmax_weights_reproduce_bruteforce(name)
    except (AssertionError, IndexError, ValueError):
        return False
    return True


@pytest.mark.parametrize("plant", ["scale dropped", "strided group map", "top-left causal",
                                   "one key short"])
def test_softmax_weights_pins_catch_planted_mistakes(monkeypatch, plant):
    """Each plausible mistake in the weights fails one of the pins above."""
    import oracle.attention as A
    assert _weights_pins_hold()
    if plant == "scale dropped":
        monkeypatch.setattr(A, "scale_as_received", lambda s: 1.0)
    elif plant == "strided group map":
        monkeypatch.setattr(A, "_heads_per_group", lambda H, G: 1)
    elif plant == "top-left causal":
        monkeypatch.setattr(A, "visible_keys",
                            lambda L, s_q, t, causal: min(t + 1, L) if causal else L)
    else:
        monkeypatch.setattr(A, "visible_keys", lambda L, s_q, t, causal: max(
            (min(L - s_q + 1 + t, L) if causal else L) - 1, 0))
    held = _weights_pins_hold()
    monkeypatch.undo()
    assert not held, f"planted mistake not caught: {plant}"


def test_constant_v_gives_that_constant():
    # with every V entry equal to c, out = c * (sum of weights) = c
    d = tiny("gqa")
    d["v"][:] = f32_to_bf16_bits(np.full(d["v"].shape, 2.5, dtype=np.float32))
    out, lse = run(attend_two_pass, d)
    L = d["cache_seqlens"]
    for b in range(d["cfg"].batch):
        if L[b]:
            np.testing.assert_allclose(out[b], 2.5, rtol=1e-14)


# ---------------------------------------------------- closed forms
@pytest.mark.parametrize("name", ["mla", "gqa"])
def test_single_key_returns_its_v_row(name):
    cfg = TINY[name].with_(seqlens_fixed=(1,) * TINY[name].batch, s_q=1, causal=False)
    d = make_inputs(cfg, seed=3)
    out, lse = run(attend_two_pass, d)
    hpg = cfg.h_q // cfg.h_kv
    for b in range(cfg.batch):
        page = d["block_table"][b, 0]
        krow = bf16_to_f64(d["kv" if cfg.kind == "mla" else "k"][page, 0])    # [G, D]
        vrow = krow[:, :cfg.d_v] if cfg.kind == "mla" else bf16_to_f64(d["v"][page, 0])
        qb = bf16_to_f64(d["q"][b, 0])
        for h in range(cfg.h_q):
            assert np.array_equal(out[b, 0, h], vrow[h // hpg])
            s = float(np.float32(cfg.scale)) * float(qb[h] @ krow[h // hpg])
            assert abs(lse[b, 0, h] - s) <= 1e-15 * max(1.0, abs(s))


def test_identical_keys_give_mean_of_v_gqa():
    cfg = TINY["gqa"].with_(seqlens_fixed=(70, 1, 128))
    d = make_inputs(cfg, seed=4)
    d["k"][:] = d["k"][0, 0]             # every cached K row equal (per KV head)
    out, lse = run(attend_two_pass, d)
    hpg = cfg.h_q // cfg.h_kv
    sigma = float(np.float32(cfg.scale))
    for b in range(cfg.batch):
        L = int(d["cache_seqlens"][b])
        n = (L + 63) // 64
        V = np.concatenate([bf16_to_f64(d["v"][p]) for p in d["block_table"][b, :n]])[:L]
        qb = bf16_to_f64(d["q"][b, 0])
        krow = bf16_to_f64(d["k"][0, 0])
        for h in range(cfg.h_q):
            g = h // hpg
            np.testing.assert_allclose(out[b, 0, h], V[:, g].mean(axis=0), rtol=1e-12, atol=1e-13)
            s = sigma * float(qb[h] @ krow[g])
            assert abs(lse[b, 0, h] - (s + math.log(L))) < 1e-12


def test_identical_scores_give_mean_of_v_mla():
    # V is a slice of K on the latent path, so equal keys would mean equal V;
    # equal *scores* come from a q that is zero on the latent part and keys
    # whose rope part is the same in every row.
    cfg = TINY["mla"].with_(seqlens_fixed=(3, 130, 64, 1))
    d = make_inputs(cfg, seed=5)
    d["q"][..., :cfg.d_v] = 0
    d["kv"][..., cfg.d_v:] = d["kv"][0, 0, 0, cfg.d_v:]
    out, lse = run(attend_two_pass, d)
    for b in range(cfg.batch):
        L = int(d["cache_seqlens"][b])
        n = (L + 63) // 64
        V = np.concatenate([bf16_to_f64(d["kv"][p]) for p in d["block_table"][b, :n]])[:L]
        np.testing.assert_allclose(out[b, 0], np.broadcast_to(V[:, 0, :cfg.d_v].mean(0),
                                                              out[b, 0].shape),
                                   rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- gather
@pytest.mark.parametrize("name", ["mla_causal2", "gqa"])
def test_page_permutation_leaves_results_bitwise_equal(name):
    d = tiny(name)
    o1, l1 = run(attend_two_pass, d)
    rng = np.random.default_rng(9)
    P = d["num_pages"]
    perm = rng.permutation(P)             # physical page p moves to slot perm[p]
    bt = d["block_table"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    d2 = dict(d, block_table=bt)
    for key in ("kv", "k", "v"):
        if key in d:
            moved = np.empty_like(d[key])
            moved[perm] = d[key]
            d2[key] = moved
    o2, l2 = run(attend_two_pass, d2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------- causal
def test_causal_tokens_reduce_to_single_token_decode():
    cfg = TINY["mla_causal2"]
    d = tiny("mla_causal2")
    out, lse = run(attend_two_pass, d)
    L = d["cache_seqlens"]
    one = cfg.with_(s_q=1, causal=False)
    for shift, t in ((0, 1), (1, 0)):
        d1 = dict(d, cfg=one, q=np.ascontiguousarray(d["q"][:, t:t + 1]),
                  cache_seqlens=np.maximum(L - shift, 0).astype(np.int32))
        o1, l1 = run(attend_two_pass, d1)
        assert_close(out[:, t], o1[:, 0])
        assert_close(lse[:, t], l1[:, 0])


def test_empty_rows_are_zero_and_minus_inf():
    d = tiny("mla_causal2")                    # L=1, s_q=2: token 0 sees nothing
    out, lse = run(attend_two_pass, d)
    assert (out[0, 0] == 0).all() and (lse[0, 0] == -np.inf).all()
    assert np.isfinite(lse[0, 1]).all()
    d = tiny("mla")                            # L=0: nothing at all
    out, lse = run(attend_two_pass, d)
    assert (out[0] == 0).all() and (lse[0] == -np.inf).all()


# ------------------------------------------------------------- combine
@pytest.mark.parametrize("cuts", [(64,), (1, 2, 3), (0, 64, 128), (17, 100, 129, 500)])
def test_combine_of_key_partition_equals_whole(cuts):
    d = tiny("mla_causal2")
    full = run(attend_two_pass, d)
    edges = [0] + list(cuts) + [10 ** 6]
    parts = [run(attend_two_pass, d, key_range=(lo, hi)) for lo, hi in zip(edges, edges[1:])]
    o, l = combine(parts)
    assert_close(o, full[0])
    assert_close(l, full[1])


def test_combine_of_one_part_is_identity_and_empty_parts_vanish():
    d = tiny("gqa")
    o, l = run(attend_two_pass, d)
    empty = (np.zeros_like(o), np.full_like(l, -np.inf))
    o2, l2 = combine([empty, (o, l), empty])
    assert_close(o2, o)
    assert_close(l2, l)


# ------------------------------------------------------------- poison
@pytest.mark.parametrize("name", ["mla_causal2", "gqa", "c1"])
def test_nan_in_page_tails_and_pads_is_never_read(name):
    clean = tiny(name)
    dirty = tiny(name, poison=True)
    assert np.array_equal(clean["q"], dirty["q"])
    o1, l1 = run(attend_two_pass, clean)
    o2, l2 = run(attend_two_pass, dirty)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.isfinite(o2).all()
    o3, l3 = run(attend_online, dirty)
    assert_close(o3, o1)


# ------------------------------------------------- planted mistakes are caught
def test_pins_catch_planted_mistakes(monkeypatch):
    """Each pin above must fail for a plausible oracle bug; plant a few in a
    copy of the oracle's helpers on the CPU and check one pin catches each."""
    import oracle.attention as A
    d = tiny("mla_causal2")
    good = run(A.attend_two_pass, d)
    brute = run(A.attend_bruteforce, d)
    assert np.allclose(good[0], brute[0])
    # wrong causal alignment (top-left instead of bottom-right)
    monkeypatch.setattr(A, "visible_keys", lambda L, T, t, c: min(t + 1, L) if c else L)
    bad = run(A.attend_two_pass, d)
    assert not np.allclose(bad[0], brute[0])
    monkeypatch.undo()
    # scale ignored
    monkeypatch.setattr(A, "scale_as_received", lambda s: 1.0)
    bad = run(A.attend_two_pass, d)
    assert not np.allclose(bad[1], brute[1])


# ------------------------------------------------------------- tolerance
def test_tolerance_checker():
    from oracle import compare, bf16_step
    assert bf16_step(np.array([1.0]))[0] == 2.0 ** -7
    assert bf16_step(np.array([5.0]))[0] == 2.0 ** -5
    ref = np.zeros((2, 101))
    ref[0, :100], ref[0, 100] = 1.0, 5.0
    lse_ref = np.array([0.5, -np.inf])
    got = ref.copy()
    got[0, 100] = 5.03125                      # one bf16 step above 5: allowed
    ok = compare(got, np.array([0.5004, -np.inf]), ref, lse_ref)
    assert ok["ok"] and ok["ulp_exceptions"] == 1
    got = ref.copy()
    got[0, 0] = 1.02                           # 0.02 off at 1.0: more than a bf16 step
    assert not compare(got, np.array([0.5, -np.inf]), ref, lse_ref)["ok"]
    got = ref.copy()
    got[1, 3] = 1e-3                           # an empty row must be exactly zero
    bad = compare(got, np.array([0.5, -np.inf]), ref, lse_ref)
    assert not bad["ok"] and not bad["empty_ok"]
    assert not compare(ref, np.array([0.502, -np.inf]), ref, lse_ref)["ok"]
    got = ref.copy()
    got[0, :100] = 1.0078125                   # every element one step off: rel-L2 fails
    assert not compare(got, np.array([0.5, -np.inf]), ref, lse_ref)["ok"]


def test_tolerance_with_the_arithmetic_bound():
    """With the value spread given, an element passes within half a bf16 step
    of the exact value plus the bound of the decode's arithmetic, which is
    tighter than one whole step where the values are concentrated."""
    from oracle import compare, rounding_allowance
    ref = np.zeros((1, 101))
    ref[0, :100], ref[0, 100] = 1.0, 5.0
    lse_ref = np.array([0.5])
    sd = np.zeros_like(ref)                     # every weight on one value
    mean_abs = np.abs(ref)
    nkeys = np.array([1])
    spread = (sd, mean_abs, nkeys)
    half = 2.0 ** -6                            # half a bf16 step at 5
    allow = rounding_allowance(ref, spread)
    assert allow[0, 100] == half + 17 * 2.0 ** -24 * 5.0
    got = ref.copy()
    got[0, 100] = 5.0 + 0.9 * half              # within half a step: passes
    assert compare(got, lse_ref, ref, lse_ref, spread=spread)["ok"]
    got[0, 100] = 5.03125                       # a whole step: only the loose rule passes it
    assert not compare(got, lse_ref, ref, lse_ref, spread=spread)["ok"]
    assert compare(got, lse_ref, ref, lse_ref)["ok"]
    # a wide spread of values widens the bound by 2^-7 of its deviation
    wide = (np.full_like(ref, 2.0), mean_abs, nkeys)
    assert rounding_allowance(ref, wide)[0, 100] == half + 2.0 ** -6 + 17 * 2.0 ** -24 * 5.0


# ------------------------------------------------------------ value spread
def test_value_spread_single_key_and_identical_keys():
    """One visible key: the weight is 1, so the deviation is 0 and the mean
    |v| is |v| of that key. Identical keys: equal weights, so the deviation
    is the population standard deviation of V over the keys and the mean
    |v| their plain mean (numpy's std and mean, not the oracle)."""
    from oracle import gather_pages, value_spread
    d = tiny("mla")
    cfg = d["cfg"]
    sd, ma, nk = run(value_spread, d)
    b = 1                                        # length 1
    v = bf16_to_f64(d["kv"][d["block_table"][b, 0], 0, 0, :cfg.d_v])
    assert np.all(sd[b] == 0.0) and np.allclose(ma[b], np.abs(v)[None, None, :], rtol=0, atol=0)
    assert np.all(nk[b] == 1) and np.all(nk[0] == 0)
    # identical scores: the columns past d_v (the part of the key row that is
    # not V) are made equal on every row of sequence 2, and the query is
    # zero on the first d_v columns, so every key scores the same while V
    # still differs from row to row
    kv = d["kv"].copy()
    L = int(d["cache_seqlens"][2])
    pages = d["block_table"][2, :(L + 63) // 64]
    for p in pages:
        kv[p, :, 0, cfg.d_v:] = kv[pages[0], 0, 0, cfg.d_v:]
    q = d["q"].copy()
    q[2, :, :, :cfg.d_v] = 0
    sd2, ma2, _ = value_spread(q, kv, d["block_table"], d["cache_seqlens"], cfg.scale,
                               cfg.causal, d_v=cfg.d_v)
    V = gather_pages(kv, d["block_table"][2], L)[:, 0, :cfg.d_v]
    np.testing.assert_allclose(sd2[2, 0, 0], V.std(axis=0), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(ma2[2, 0, 0], np.abs(V).mean(axis=0), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("name", ["mla_causal2", "gqa_causal"])
def test_value_spread_brute_force(name):
    """Against explicit loops over rows, keys and columns on tiny inputs,
    with the softmax written out per row."""
    from oracle import value_spread
    d = tiny(name)
    cfg = d["cfg"]
    sd, ma, nk = run(value_spread, d)
    B, T, H, _ = d["q"].shape
    G = cfg.h_kv
    for b in range(B):
        L = int(d["cache_seqlens"][b])
        for t in range(T):
            vis = min(max(L - T + 1 + t, 0), L) if cfg.causal else L
            for h in range(H):
                g = h // (H // G)
                qv = bf16_to_f64(d["q"][b, t, h])
                s, vals = [], []
                for j in range(vis):
                    page = int(d["block_table"][b, j // 64])
                    if cfg.kind == "mla":
                        row = bf16_to_f64(d["kv"][page, j % 64, g])
                        k, v = row, row[:cfg.d_v]
                    else:
                        k = bf16_to_f64(d["k"][page, j % 64, g])
                        v = bf16_to_f64(d["v"][page, j % 64, g])
                    s.append(float(np.float32(cfg.scale)) * float(k @ qv))
                    vals.append(v)
                assert nk[b, t, h] == vis
                if vis == 0:
                    continue
                s = np.array(s)
                w = np.exp(s - s.max())
                w /= w.sum()
                vals = np.array(vals)
                mean = (w[:, None] * vals).sum(axis=0)
                var = (w[:, None] * (vals - mean) ** 2).sum(axis=0)
                np.testing.assert_allclose(sd[b, t, h], np.sqrt(var), rtol=1e-7, atol=1e-9)
                np.testing.assert_allclose(ma[b, t, h], (w[:, None] * np.abs(vals)).sum(axis=0),
                                           rtol=1e-12, atol=1e-15)
