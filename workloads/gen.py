"""Seeded synthetic inputs for paged attention decode.

Both the CPU oracle's tests and the GPU path draw their inputs here, so this
module holds no attention arithmetic: it draws sequence lengths, a random
placement of pages in a page pool, and bf16 q / cache values.

Draw order from ``numpy.random.default_rng(seed)`` (fixed, so a seed names
one input set):
  1. cache_seqlens (only for the log-uniform and uniform length rules),
  2. the permutation that places logical pages on physical pages,
  3. q,
  4. the cache: the latent cache for MLA; K then V for GQA. Every slot of
     every page is drawn, page tails included, in chunks of whole pages.

Values are float32 standard normals times a factor, rounded to bf16 with
round-to-nearest-even and returned as uint16 bit patterns.

Page placement follows PagedAttention's block table (FlashAttention (KO),
"참고 문헌": Kwon et al. 2023): sequence b's logical page j lives at
physical page ``block_table[b, j]``; pads are -1.
"""
from __future__ import annotations

import numpy as np

from .configs import CONFIGS, DecodeConfig, GqlaConfig, PAGE

BF16_NAN = np.uint16(0x7FC0)
_CHUNK_PAGES = 256


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the 16-bit patterns. Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def draw_seqlens(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    if cfg.seqlen_rule == "fixed":
        L = np.array(cfg.seqlens_fixed, dtype=np.int64)
        assert L.shape == (cfg.batch,)
    elif cfg.seqlen_rule == "loguniform":
        # L = floor(exp(U[ln lo, ln(hi + 1)))) lies in [lo, hi]
        u = rng.uniform(np.log(cfg.seqlen_lo), np.log(cfg.seqlen_hi + 1), size=cfg.batch)
        L = np.minimum(np.floor(np.exp(u)).astype(np.int64), cfg.seqlen_hi)
    elif cfg.seqlen_rule == "uniform":
        L = rng.integers(cfg.seqlen_lo, cfg.seqlen_hi, size=cfg.batch, endpoint=True)
    else:
        raise ValueError(cfg.seqlen_rule)
    return L.astype(np.int32)


def _normal_bf16(rng, shape_pages, std, chunk=_CHUNK_PAGES):
    """Draw a [num_pages, ...] bf16 array page-chunk by page-chunk."""
    out = np.empty(shape_pages, dtype=np.uint16)
    n = shape_pages[0]
    for p0 in range(0, n, chunk):
        p1 = min(n, p0 + chunk)
        x = rng.standard_normal((p1 - p0,) + tuple(shape_pages[1:]), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[p0:p1] = f32_to_bf16_bits(x)
    return out


def make_inputs(cfg: DecodeConfig, seed: int | None = None, seqlens=None,
                poison: bool = False) -> dict:
    """Draw one input set for ``cfg``.

    ``seqlens`` overrides the length draw (step 1 is then skipped).
    ``poison`` fills every page tail slot (token >= L_b in a sequence's last
    page) with bf16 NaN, appends one all-NaN page to the pool and points every
    block-table pad at it, so that a read of an invalid slot shows up in the
    result.

    Returns a dict with uint16 bf16 patterns ``q`` [B, s_q, h_q, d_qk] and
    ``kv`` [P, 64, h_kv, d_qk] (MLA) or ``k``/``v`` [P, 64, h_kv, d] (GQA),
    int32 ``block_table`` [B, max_pages] and ``cache_seqlens`` [B], and the
    config fields needed to interpret them.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    if seqlens is None:
        L = draw_seqlens(cfg, rng)
    else:
        L = np.asarray(seqlens, dtype=np.int32)
        assert L.shape == (cfg.batch,)
    pages = (L.astype(np.int64) + PAGE - 1) // PAGE
    num_pages = int(pages.sum())
    max_pages = max(1, int(pages.max()) if len(pages) else 1)
    perm = rng.permutation(num_pages).astype(np.int32)
    pool = num_pages + (1 if poison else 0)
    pad = num_pages if poison else -1
    bt = np.full((cfg.batch, max_pages), pad, dtype=np.int32)
    off = 0
    for b in range(cfg.batch):
        n = int(pages[b])
        bt[b, :n] = perm[off:off + n]
        off += n

    q = _normal_bf16(rng, (cfg.batch, cfg.s_q, cfg.h_q, cfg.d_qk), cfg.q_std, chunk=1 << 30)
    out = dict(cfg=cfg, q=q, block_table=bt, cache_seqlens=L, num_pages=pool)
    shape = (pool, PAGE, cfg.h_kv, cfg.d_qk)
    if cfg.kind == "mla":
        caches = {"kv": shape}
    else:
        caches = {"k": shape, "v": (pool, PAGE, cfg.h_kv, cfg.d_v)}
    for name, shp in caches.items():
        arr = np.empty(shp, dtype=np.uint16)
        arr[:num_pages] = _normal_bf16(rng, (num_pages,) + shp[1:], cfg.kv_std)
        if poison:
            arr[num_pages:] = BF16_NAN
            for b in range(cfg.batch):
                n, rem = int(pages[b]), int(L[b]) % PAGE
                if n and rem:
                    arr[bt[b, n - 1], rem:] = BF16_NAN
        out[name] = arr
    return out


def config_inputs(idx: int, **kw) -> dict:
    return make_inputs(CONFIGS[idx], **kw)


def make_gqla_inputs(cfg: GqlaConfig, seed: int | None = None, seqlens=None) -> dict:
    """Draw one GQLA input set: the latent cache, queries and the per-group
    up-projection weights (synthetic: there are no trained weights).

    Draw order from ``default_rng(seed)``: cache_seqlens (unless fixed or
    given), the page permutation, q [B, s_q, h_q, d_h + d_r], the latent cache
    [P, 64, 1, d_c + d_r] (whole pages, tails included), then w_uk and w_uv
    [h_kv, d_c, d_h | d_v]. All bf16 patterns (uint16), RNE from float32
    normals times the config's std.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    if seqlens is None:
        L = draw_seqlens(cfg, rng)
    else:
        L = np.asarray(seqlens, dtype=np.int32)
        assert L.shape == (cfg.batch,)
    pages = (L.astype(np.int64) + PAGE - 1) // PAGE
    num_pages = int(pages.sum())
    max_pages = max(1, int(pages.max()) if len(pages) else 1)
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((cfg.batch, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(cfg.batch):
        n = int(pages[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    q = _normal_bf16(rng, (cfg.batch, cfg.s_q, cfg.h_q, cfg.d_q), cfg.q_std, chunk=1 << 30)
    kv = _normal_bf16(rng, (num_pages, PAGE, 1, cfg.d_c + cfg.d_r), cfg.kv_std)
    w_uk = _normal_bf16(rng, (cfg.h_kv, cfg.d_c, cfg.d_h), cfg.w_std, chunk=1 << 30)
    w_uv = _normal_bf16(rng, (cfg.h_kv, cfg.d_c, cfg.d_v), cfg.w_std, chunk=1 << 30)
    return dict(cfg=cfg, q=q, kv=kv, w_uk=w_uk, w_uv=w_uv, block_table=bt,
                cache_seqlens=L, num_pages=num_pages)
