"""Comparison of a GPU result with the oracle, to the stated tolerances.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark).

Bars: max-abs error 1e-2 on the bf16 output, relative L2 error 5e-3 over
non-empty rows, and 1e-3 absolute on the LSE. The output is compared with
the unrounded fp64 oracle. Where 1e-2 is below what a bf16 output can reach
(a correctly rounded bf16 value can be half a bf16 step from the exact one:
0.0156 for |x| in [4, 8)), an element also passes within

  half a bf16 step of the exact value
  + 2^-7 * sd      (the decode rounds its softmax weights to bf16, relative
                    error <= 2^-9 each, and normalises by their sum; the
                    output then moves by at most 2^-8 * sum_j w_j |v_j - out|
                    <= 2^-8 * sd, and once more where split results are
                    merged with weights from the unrounded sums)
  + (n + 16) * 2^-24 * mean|v|   (fp32 accumulation over the row's n keys,
                    and the fp32 exponential)

with sd and mean|v| the attention-weighted deviation and magnitude of the
row's values (attention.value_spread). Without those (a comparison of two
GPU results, or a path whose inputs the oracle does not see bit for bit)
the allowance is one bf16 step. The number of elements that pass only by
the allowance is reported. Rows with no visible key must be exactly out = 0
and lse = -inf.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = 1e-2
REL_L2 = 5e-3
LSE_ABS = 1e-3


def bf16_step(x: np.ndarray) -> np.ndarray:
    """Distance between consecutive bf16 values around |x| (8 significand bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.maximum(2.0 ** (e - 7), 2.0 ** -133)


def rounding_allowance(out_ref, spread=None):
    """Per-element allowance beyond the max-abs bar (see the module text):
    one bf16 step without `spread`, else half a step plus the bound of the
    decode's own arithmetic. spread = (sd, mean_abs, nkeys) of value_spread,
    shaped like out_ref (nkeys without the last axis)."""
    r = np.asarray(out_ref, dtype=np.float64)
    if spread is None:
        return bf16_step(r)
    sd, mean_abs, nkeys = (np.asarray(x, dtype=np.float64) for x in spread)
    return (0.5 * bf16_step(r) + 2.0 ** -7 * sd
            + (nkeys[..., None] + 16.0) * 2.0 ** -24 * mean_abs)


def compare(out, lse, out_ref, lse_ref, max_abs=MAX_ABS, rel_l2=REL_L2, lse_abs=LSE_ABS,
            spread=None):
    """out/out_ref [..., Dv], lse/lse_ref [...]; returns a dict with the
    metrics and 'ok'. spread: value_spread of the same rows, for the
    tighter allowance."""
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    out_ref = np.asarray(out_ref, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    assert out.shape == out_ref.shape and lse.shape == lse_ref.shape
    empty = ~np.isfinite(lse_ref)
    res = {"rows": int(lse_ref.size), "empty_rows": int(empty.sum())}
    empty_ok = bool(np.all(out[empty] == 0.0) and np.all(lse[empty] == -np.inf))
    full = ~empty
    o, r = out[full], out_ref[full]
    err = np.abs(o - r)
    finite = bool(np.isfinite(o).all() and np.isfinite(lse[full]).all())
    allow = rounding_allowance(out_ref, spread)
    allowed = np.maximum(max_abs, allow[full])
    res["max_abs"] = float(err.max()) if err.size else 0.0
    res["ulp_exceptions"] = int(((err > max_abs) & (err <= allowed)).sum())
    res["elem_fail"] = int((err > allowed).sum())
    den = float(np.sqrt((r ** 2).sum()))
    res["rel_l2"] = float(np.sqrt((err ** 2).sum()) / den) if den > 0 else 0.0
    lerr = np.abs(lse[full] - lse_ref[full])
    res["lse_max_abs"] = float(lerr.max()) if lerr.size else 0.0
    res["allowance"] = "one bf16 step" if spread is None else "half step + arithmetic bound"
    res["ok"] = bool(empty_ok and finite and res["elem_fail"] == 0 and res["rel_l2"] <= rel_l2
                     and res["lse_max_abs"] <= lse_abs)
    res["empty_ok"] = empty_ok
    res["finite"] = finite
    return res
