"""FP8 (e4m3) latent cache: quantiser, dequantiser and decode, fp64 on the CPU.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library neither
imports nor calls it, and it shares no code with the GPU path.

The pages name FP8 only as FlashAttention-3's low-precision mode
(FlashAttention (KO), "FlashAttention-3 (2024)"), so the cache format is a
reading, listed in the design notes:
  * codes are OCP FP8 E4M3: sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no
    infinities; the largest finite value is 448;
  * one float32 scale per cached token (the whole 576-wide latent row):
    value = e4m3(code) * scale;
  * quantisation of a bf16 row x: amax = max |x|; the scale is the
    smallest power of two not below the float32 quotient amax / 448, at
    least 2^-126 (1 when amax = 0) — a power-of-two (E8M0-like) scale, as
    the OCP microscaling formats use; code = the E4M3 value nearest to
    clamp(x / scale, -448, 448), ties to the even mantissa. x / scale is
    exact; the quotient amax / 448 is rounded as float32 rounds it.
Decode with such a cache is the attention definition (as in
oracle.attention) over the dequantised rows, in float64.
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_to_f64, scale_as_received, visible_keys, PAGE

E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Value of E4M3 codes (uint8), float64; NaN for the two NaN codes."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


# the 127 finite non-negative values and their codes, ascending
_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.int64)
_POS_VALUES = e4m3_value(_POS_CODES)


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 code to each finite value with |x| <= 448, ties to the
    code with an even mantissa (the even code), as uint8. Zero keeps its sign
    bit."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) > E4M3_MAX).any():
        raise ValueError("e4m3_round takes finite values within +-448")
    a = np.abs(x)
    hi = np.searchsorted(_POS_VALUES, a, side="left")       # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    vlo, vhi = _POS_VALUES[lo], _POS_VALUES[hi]
    dlo, dhi = a - vlo, vhi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    pick_hi |= (vhi == a)
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    neg = np.signbit(x)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows(rows_bf16):
    """bf16 rows (uint16 patterns, [..., D]) -> (codes uint8 [..., D],
    scales float32 [...]). amax, the scale and x / scale are float32
    operations, rounded as float32 rounds them."""
    x = bf16_to_f64(rows_bf16).astype(np.float32)            # exact
    amax = np.max(np.abs(x), axis=-1)
    r = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    # the smallest power of two >= r, from r's float32 exponent and mantissa
    mant, ex = np.frexp(r.astype(np.float64))                # r = mant * 2^ex, mant in [0.5, 1)
    pow2 = np.where(mant == 0.5, np.ldexp(1.0, ex - 1), np.ldexp(1.0, ex))
    pow2 = np.maximum(pow2, 2.0 ** -126)
    scale = np.where(amax > 0, pow2, 1.0).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)            # exact: a power of two
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_round(y.astype(np.float64)), scale


def dequantize(codes, scales) -> np.ndarray:
    """float64 values e4m3(code) * scale, scales broadcast over the last axis."""
    return e4m3_value(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def attend_fp8(q, codes, scales, block_table, seqlens, scale, causal, d_v=512):
    """Attention decode over an FP8 latent cache. q bf16 patterns
    [B, T, H, 576]; codes uint8 [P, 64, 576]; scales float32 [P, 64]. V is
    the first d_v dequantised columns. Returns out float64 [B, T, H, d_v] and
    lse [B, T, H] (natural log); a row with no visible key gets 0 and -inf."""
    B, T, H, D = q.shape
    sigma = scale_as_received(scale)
    qf = bf16_to_f64(q)
    out = np.zeros((B, T, H, d_v))
    lse = np.full((B, T, H), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        if L <= 0:
            continue
        n = (L + PAGE - 1) // PAGE
        rows = np.concatenate([dequantize(codes[int(p)], scales[int(p)])
                               for p in block_table[b, :n]], axis=0)[:L]   # [L, 576]
        s = sigma * np.einsum("thd,ld->thl", qf[b], rows)
        for t in range(T):
            vis = visible_keys(L, T, t, causal)
            if vis <= 0:
                continue
            st = s[t, :, :vis]
            m = st.max(axis=1, keepdims=True)
            e = np.exp(st - m)
            l = e.sum(axis=1)
            out[b, t] = (e @ rows[:vis, :d_v]) / l[:, None]
            lse[b, t] = m[:, 0] + np.log(l)
    return out, lse


def quantize_cache(kv_bf16):
    """A whole bf16 latent cache [P, 64, 1, D] -> codes [P, 64, D], scales
    [P, 64]."""
    return quantize_rows(kv_bf16[:, :, 0, :])
