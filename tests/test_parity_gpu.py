"""GPU parity: the HIP path through the C interface against the fp64 oracle
on the same seeded inputs (max-abs 1e-2 with a one-bf16-step allowance,
rel-L2 5e-3, LSE 1e-3), plus properties that hold at any size."""
import numpy as np
import pytest

from workloads import CONFIGS
from gpu_helpers import check, inputs, log, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------ small shapes
def _mla(B, T, H, Ls, causal, **kw):
    return CONFIGS[3].with_(batch=B, s_q=T, h_q=H, causal=causal, seqlen_rule="fixed",
                            seqlens_fixed=tuple(Ls), **kw)


def _gqa(B, T, H, G, Ls, causal=False):
    return CONFIGS[5].with_(batch=B, s_q=T, h_q=H, h_kv=G, causal=causal, seqlen_rule="fixed",
                            seqlens_fixed=tuple(Ls))


RAGGED = (0, 1, 2, 63, 64, 65, 127, 200, 640, 1000)
SMALL = {
    "mla_h8_t1": _mla(10, 1, 8, RAGGED, False),
    "mla_h16_t1": _mla(10, 1, 16, RAGGED, False),
    "mla_h32_t1": _mla(10, 1, 32, RAGGED, False),
    "mla_h64_t1": _mla(10, 1, 64, RAGGED, False),
    "mla_h128_t1": _mla(10, 1, 128, RAGGED, False),
    "mla_h128_t2_causal": _mla(10, 2, 128, RAGGED, True),
    "mla_h16_t3_causal": _mla(10, 3, 16, RAGGED, True),
    # 40 and 8 heads per token: one wave's 16 rows mix query tokens, so under
    # causal masking some rows of a wave see a key while others see none yet
    "mla_h40_t2_causal": _mla(10, 2, 40, RAGGED, True),
    "mla_h128_t1_kvhalf": _mla(4, 1, 128, (4096, 100, 3000, 1), False, kv_std=0.5),
    # many short sequences at 64-row blocks: a worker's range crosses many
    # sequences, empty ones included, and the copy waves' and compute waves'
    # sequence loops must stay in step through all of them
    "mla_h128_t1_many_short": _mla(300, 1, 128, (RAGGED[:8] * 38)[:300], False),
    "mla_h64_t2_many_short_causal": _mla(300, 2, 64, (RAGGED[1:9] * 38)[:300], True),
    # one sequence over every worker: 128 partial results per row to merge
    "mla_h16_t1_one_long": _mla(1, 1, 16, (16384,), False),
    "mla_h128_t2_causal_long": _mla(3, 2, 128, (20000, 3, 700), True),
    "gqa_h16_g2_one_long": _gqa(1, 1, 16, 2, (30000,)),
    # 4 query tokens at 128 heads: 512 rows in four 128-row blocks
    "mla_h128_t4_causal": _mla(6, 4, 128, (1, 64, 65, 200, 1000, 3000), True),
    # 150 rows: the second 128-row block ends inside a wave's 32 rows, whose
    # output then leaves without the staged row stores
    "mla_h50_t3_causal": _mla(10, 3, 50, RAGGED, True),
    # 16 KV heads of 8 query heads each
    "gqa_h128_g16": _gqa(10, 1, 128, 16, RAGGED),
    "gqa_h128_g8": _gqa(10, 1, 128, 8, RAGGED),
    "gqa_h16_g2": _gqa(10, 1, 16, 2, RAGGED),
    "gqa_h8_g8": _gqa(10, 1, 8, 8, RAGGED),
    "gqa_h32_g4_t2_causal": _gqa(10, 2, 32, 4, RAGGED, True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_shapes_match_oracle(dev, name):
    cfg = SMALL[name]
    d = inputs(cfg, seed=11)
    log(f"[case] {name} seqlens={list(d['cache_seqlens'])}")
    out, lse = run_gpu(d, to_device(d, dev))
    ref_out, ref_lse, spread = run_oracle(d, spread=True)
    check(out, lse, ref_out, ref_lse, name, spread=spread)


# ------------------------------------------------------- the five configs
@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_config_matches_oracle(dev, idx):
    """Every sequence of each configuration at full size, in the launch
    configuration bench.py times, against the oracle."""
    import torch
    cfg = CONFIGS[idx]
    log(f"[case] config {idx} {cfg.name}: generating inputs")
    d = inputs(cfg)
    t = to_device(d, dev)
    out, lse = run_gpu(d, t)
    assert np.isfinite(out).all(), "non-finite output"
    L = d["cache_seqlens"]
    empty_rows = ~np.isfinite(lse)
    # at any size: rows with keys have finite lse; rows without are exactly empty
    if not cfg.causal:
        assert np.array_equal(empty_rows.any(axis=(1, 2)), L == 0)
    log(f"[case] config {idx}: oracle on all {cfg.batch} sequences")
    ref_out, ref_lse, spread = run_oracle(d, spread=True)
    check(out, lse, ref_out, ref_lse, f"config {idx} ({cfg.name})", spread=spread)
    del t
    torch.cuda.empty_cache()


# ------------------------------------------------------------- properties
@pytest.mark.parametrize("name", ["mla_h128_t2_causal", "mla_h16_t1", "gqa_h128_g8"])
def test_nan_in_page_tails_and_pads_is_never_read(dev, name):
    cfg = SMALL[name]
    clean = inputs(cfg, seed=5)
    dirty = inputs(cfg, seed=5, poison=True)
    o1, l1 = run_gpu(clean, to_device(clean, dev))
    o2, l2 = run_gpu(dirty, to_device(dirty, dev))
    assert np.isfinite(o2).all()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name", ["mla_h128_t2_causal", "gqa_h32_g4_t2_causal",
                                  "mla_h16_t1_one_long"])
def test_page_permutation_and_rerun_are_bitwise_equal(dev, name):
    cfg = SMALL[name]
    d = inputs(cfg, seed=6)
    o1, l1 = run_gpu(d, to_device(d, dev))
    o1b, l1b = run_gpu(d, to_device(d, dev))
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b), "not deterministic"
    rng = np.random.default_rng(2)
    perm = rng.permutation(d["num_pages"])
    bt = d["block_table"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    d2 = dict(d, block_table=bt)
    for key in ("kv", "k", "v"):
        if key in d:
            moved = np.empty_like(d[key])
            moved[perm] = d[key]
            d2[key] = moved
    o2, l2 = run_gpu(d2, to_device(d2, dev))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_split_count_does_not_change_the_result(dev):
    # one long sequence alone is cut over every worker; in a crowded batch
    # it is cut fewer times
    cfg_alone = _mla(1, 2, 128, (5000,), True)
    cfg_batch = _mla(40, 2, 128, (5000,) + (4000,) * 39, True)
    alone = inputs(cfg_alone, seed=8)
    crowd = inputs(cfg_batch, seed=8)
    # put the same sequence (q and pages) in slot 0 of the crowded batch
    n0 = (5000 + 63) // 64
    crowd["q"][0] = alone["q"][0]
    crowd["kv"][crowd["block_table"][0, :n0]] = alone["kv"][alone["block_table"][0, :n0]]
    o1, l1 = run_gpu(alone, to_device(alone, dev))
    o2, l2 = run_gpu(crowd, to_device(crowd, dev))
    ref_out, ref_lse = run_oracle(alone)
    check(o1, l1, ref_out, ref_lse, "alone")
    check(o2[:1], l2[:1], ref_out, ref_lse, "in a batch")


def test_causal_tokens_reduce_to_single_token_decode(dev):
    cfg = SMALL["mla_h128_t2_causal"]
    d = inputs(cfg, seed=9)
    out, lse = run_gpu(d, to_device(d, dev))
    L = d["cache_seqlens"]
    one = cfg.with_(s_q=1, causal=False)
    for shift, tok in ((0, 1), (1, 0)):
        d1 = dict(d, cfg=one, q=np.ascontiguousarray(d["q"][:, tok:tok + 1]),
                  cache_seqlens=np.maximum(L - shift, 0).astype(np.int32))
        o1, l1 = run_gpu(d1, to_device(d1, dev))
        check(out[:, tok:tok + 1], lse[:, tok:tok + 1], o1, l1, f"token {tok} vs single")


def test_empty_batch_is_a_no_op(dev):
    import torch
    import mla_paged_kv_03_amd as lib
    q = torch.zeros(0, 1, 16, 576, dtype=torch.bfloat16, device=dev)
    kv = torch.zeros(1, 64, 1, 576, dtype=torch.bfloat16, device=dev)
    bt = torch.zeros(0, 1, dtype=torch.int32, device=dev)
    sl = torch.zeros(0, dtype=torch.int32, device=dev)
    out, lse = lib.mla_decode(q, kv, bt, sl, 0.1, False)
    torch.cuda.synchronize()
    assert out.shape == (0, 1, 16, 512)


def test_workspace_too_small_is_reported(dev):
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = SMALL["mla_h16_t1"]
    d = inputs(cfg, seed=1)
    t = to_device(d, dev)
    plan = lib.mla_decode_plan(t["cache_seqlens"], 1, 16)
    plan.workspace = plan.workspace[:16]
    with pytest.raises(lib.DecodeError) as e:
        lib.mla_decode(t["q"], t["kv"], t["block_table"], t["cache_seqlens"], cfg.scale, False,
                       plan=plan)
    assert e.value.code == -4


def test_device_plan_equals_host_plan(dev):
    import torch
    import mla_paged_kv_03_amd as lib
    for Ls, T, H, G, dv in [((64, 200), 1, 8, 1, 512),
                            (tuple(np.random.default_rng(3).integers(0, 16385, 128)), 2, 128, 1, 512),
                            ((8192,) * 256, 1, 16, 1, 512), ((100, 0, 70000), 1, 128, 8, 128),
                            # more sequences than the plan kernel's 1024 threads: the scans
                            # carry across blocks of the batch
                            (tuple(np.random.default_rng(5).integers(0, 3000, 2500)), 1, 16, 1, 512),
                            (tuple([0] * 1500 + [1] * 700 + [64] * 30), 2, 128, 1, 512),
                            # equal lengths (pieces on block boundaries) and one sequence
                            # spread over every worker
                            ((4096,) * 64, 1, 128, 1, 512), ((1 << 20,), 1, 16, 1, 512)]:
        sl = torch.tensor(Ls, dtype=torch.int32, device=dev)
        plan = lib.mla_decode_plan(sl, T, H, G, dv)
        torch.cuda.synchronize()
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        meta, splits, info = lib.mla_decode_plan_host(Ls, T, H, G, dv, num_cus=cus)
        assert np.array_equal(plan.sched_metadata.cpu().numpy(), meta)
        assert np.array_equal(plan.num_splits.cpu().numpy(), splits)


@pytest.mark.parametrize("name", ["mla_h128_t2_causal_long", "gqa_h16_g2_one_long"])
def test_plan_reuse_is_exact(dev, name):
    """One plan serves several decode calls (the layers of a step): every
    call gives the same bits and leaves the plan as the plan kernel wrote
    it."""
    import torch
    import mla_paged_kv_03_amd as lib
    cfg = SMALL[name]
    d = inputs(cfg, seed=7)
    t = to_device(d, dev)
    G = cfg.h_kv if cfg.kind == "gqa" else 1
    dv = 512 if cfg.kind == "mla" else 128
    plan = lib.mla_decode_plan(t["cache_seqlens"], cfg.s_q, cfg.h_q, G, dv)
    runs = [run_gpu(d, t, plan=plan) for _ in range(3)]
    for o, l in runs[1:]:
        assert np.array_equal(o, runs[0][0]) and np.array_equal(l, runs[0][1])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    meta, splits, info = lib.mla_decode_plan_host(list(d["cache_seqlens"]), cfg.s_q, cfg.h_q, G,
                                                  dv, num_cus=cus)
    assert np.array_equal(plan.sched_metadata.cpu().numpy(), meta)
    ref_out, ref_lse = run_oracle(d)
    check(runs[0][0], runs[0][1], ref_out, ref_lse, name)


def test_attn_combine_matches_oracle_combine(dev):
    import torch
    import oracle
    import mla_paged_kv_03_amd as lib
    rng = np.random.default_rng(4)
    B, R, dv = 3, 5, 64
    counts = [3, 0, 2]
    slots = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    S = int(slots[-1])
    po = rng.standard_normal((S, R, dv)).astype(np.float32)
    pl = (rng.standard_normal((S, R)) * 3).astype(np.float32)
    pl[1, 2] = -np.inf                       # a part that saw no key
    pl[3:5, 4] = -np.inf                     # a row with no key at all
    po[3:5, 4] = 0.0
    out, lse = lib.attn_combine(torch.from_numpy(po).to(dev), torch.from_numpy(pl).to(dev),
                                torch.from_numpy(slots).to(dev))
    torch.cuda.synchronize()
    out = out.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    for b in range(B):
        if counts[b] == 0:
            assert (out[b] == 0).all() and (lse[b] == -np.inf).all()  # untouched
            continue
        parts = [(po[s].astype(np.float64), pl[s].astype(np.float64))
                 for s in range(slots[b], slots[b + 1])]
        ro, rl = oracle.combine(parts)
        check(out[b], lse[b], ro, rl, f"combine b={b}")



def test_attn_combine_many_partials(dev):
    """More partials per row than a wave has lanes (100 and 70): the weights
    of partials 64 and up are recomputed rather than shuffled; some parts see
    no key, and one row sees none in any part."""
    import torch
    import oracle
    import mla_paged_kv_03_amd as lib
    rng = np.random.default_rng(8)
    B, R, dv = 2, 3, 512
    counts = [100, 70]
    slots = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    S = int(slots[-1])
    po = rng.standard_normal((S, R, dv)).astype(np.float32)
    pl = (rng.standard_normal((S, R)) * 4).astype(np.float32)
    pl[[5, 64, 99], 1] = -np.inf
    pl[100:, 2] = -np.inf
    po[100:, 2] = 0.0
    out, lse = lib.attn_combine(torch.from_numpy(po).to(dev), torch.from_numpy(pl).to(dev),
                                torch.from_numpy(slots).to(dev))
    torch.cuda.synchronize()
    out = out.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    for b in range(B):
        parts = [(po[s].astype(np.float64), pl[s].astype(np.float64))
                 for s in range(slots[b], slots[b + 1])]
        ro, rl = oracle.combine(parts)
        check(out[b], lse[b], ro, rl, f"combine many b={b}")
    assert (out[1, 2] == 0).all() and lse[1, 2] == -np.inf

def _climbing_scores(d, cfg, period=5, step=18.0, seed=7):
    """Give every query head the same q, and page j keys close to
    alpha_j * q with alpha_j chosen so the log2-domain score of page j is
    about step * (j mod period): within each run of `period` pages every
    row's scores climb past the previous page's by `step`."""
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    q0 = rng.standard_normal(cfg.d_qk).astype(np.float32)
    d["q"][:] = f32_to_bf16_bits(np.broadcast_to(q0, d["q"].shape))
    kname = "kv" if cfg.kind == "mla" else "k"
    sigma = float(np.float32(cfg.scale)) * 1.4426950408889634
    per_unit = float(q0 @ q0) * sigma
    for b in range(cfg.batch):
        n = (int(d["cache_seqlens"][b]) + 63) // 64
        for j in range(n):
            alpha = step * (j % period) / per_unit
            noise = 0.05 * rng.standard_normal((64,) + d[kname].shape[2:]).astype(np.float32)
            d[kname][d["block_table"][b, j]] = f32_to_bf16_bits(alpha * q0 + noise)


@pytest.mark.parametrize("period", [3, 5])
@pytest.mark.parametrize("kind", ["mla", "mla_h128", "mla_h128_short", "gqa"])
def test_scores_climbing_from_page_to_page(dev, kind, period):
    """Scores rise by 18 (log2 units) from page to page within runs of
    `period` pages, far more than the rescale slack. With period 3 a row's
    scores end up to 36 above the first page's, which the fixed-reference
    pass absorbs (weights up to 2^36); with period 5 the rise reaches 72,
    past the fixed pass's limit, and ranges that start at the bottom of a
    run fall back to the rescaling pass. Each worker owns several
    consecutive pages (the batch has far more pages than workers)."""
    import mla_paged_kv_03_amd as lib
    Ls = (64 * 300, 64 * 280 + 17, 64 * 300, 64 * 290)
    # 300 sequences of 3 to 8 pages at 128 heads: most workers take one or
    # two whole sequences, a sequence of five or more pages climbs past the
    # fixed reference and falls back to the second pass, and the worker then
    # goes on to its next sequence, whose first page went out before the
    # epilogue
    short = tuple(64 * (5, 6, 7, 3, 8)[i % 5] - 7 * (i % 3) for i in range(300))
    # 128 heads: the 128-row latent kernel
    cfg = {"mla": lambda: _mla(4, 1, 16, Ls, False),
           "mla_h128": lambda: _mla(4, 1, 128, Ls, False),
           "mla_h128_short": lambda: _mla(300, 1, 128, short, False),
           "gqa": lambda: _gqa(4, 1, 16, 2, Ls)}[kind]()
    d = inputs(cfg, seed=12)
    _climbing_scores(d, cfg, period=period)
    t = to_device(d, dev)
    plan = lib.mla_decode_plan(t["cache_seqlens"], cfg.s_q, cfg.h_q, cfg.h_kv, cfg.d_v)
    pages = int(((d["cache_seqlens"] + 63) // 64).sum())
    assert pages > 2 * plan.info.num_workers  # several pages per worker
    out, lse = run_gpu(d, t, plan=plan)
    ref_out, ref_lse, spread = run_oracle(d, spread=True)
    check(out, lse, ref_out, ref_lse, f"climbing scores ({kind}, period {period})", spread=spread)
