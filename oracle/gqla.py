"""GQLA decode in fp64 on the CPU: the direct definition and its two paths.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library neither
imports nor calls it, and it shares no code with the GPU path.

What it computes. GQLA keeps MLA's latent cache but indexes the
up-projections by KV group instead of by query head (GQLA review, "2.
Motivation & Problem Statement"), so one set of weights exposes two decode
paths (same review, "1. Key Terms & Definitions"): the MQA-absorb path folds
the key up-projection into the query and the value up-projection into the
output and attends the shared latent rows; the GQA path expands the cache
into per-group K and V and runs ordinary grouped attention.

Readings where the pages give no formulas (each listed in the design notes):
  * A cached token is one latent row [c (d_c = 512), k_rope (d_r = 64)], the
    MLA cache row. Group g has W_UK^g [d_c, d_h = 128] and W_UV^g [d_c,
    d_v = 128]; its key for a token is [c W_UK^g, k_rope] (the rope part is
    shared by all groups, as in MLA's decoupled rope), its value c W_UV^g.
  * A query row is [q_nope (d_h), q_rope (d_r)]; query head h belongs to
    group h // (h_q / h_kv); the softmax scale multiplies the full
    (d_h + d_r)-wide dot product.
  * The absorb path's query is [q_nope W_UK^g^T, q_rope] (576 wide) and its
    attention output over the latent values c is multiplied by W_UV^g.
  * The output projection after attention is not part of this step.
In exact arithmetic both paths equal the direct definition; here all three
are evaluated in float64 from the bf16 inputs, with no rounding in between.
With ``round_bf16=True`` a path instead rounds its stored intermediates to
bf16 (nearest-even, by way of float32) where a bf16 implementation stores
them: the absorbed query and the latent attention output (absorb path), the
expanded K and V rows (GQA path); everything else stays float64.

Inputs: bf16 bit patterns as uint16 numpy arrays — q [B, T, H, d_h + d_r],
kv [P, 64, 1, d_c + d_r], w_uk [G, d_c, d_h], w_uv [G, d_c, d_v] — plus int32
block_table [B, max_pages] and seqlens [B].
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_to_f64, gather_pages, scale_as_received, visible_keys

D_C, D_R = 512, 64


def round_bf16(x):
    """float64 values rounded to float32 (nearest-even) and then to bf16
    (nearest-even on the top 16 bits of the float32 pattern), returned as
    float64. Finite inputs only."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _groups(H, G):
    if G <= 0 or H % G:
        raise ValueError(f"h_q={H} is not a multiple of h_kv={G}")
    return H // G


def expand_group_cache(kv, w_uk, w_uv):
    """The GQA path's cache: for every token row and group g,
    K[..., g, :] = [c W_UK^g, k_rope] and V[..., g, :] = c W_UV^g, in float64.
    kv [P, 64, 1, d_c + d_r] -> K [P, 64, G, d_h + d_r], V [P, 64, G, d_v]."""
    lat = bf16_to_f64(kv[:, :, 0, :])              # [P, 64, 576]
    c, rope = lat[..., :D_C], lat[..., D_C:]
    Wk, Wv = bf16_to_f64(w_uk), bf16_to_f64(w_uv)  # [G, 512, d]
    G = Wk.shape[0]
    K = np.empty(lat.shape[:2] + (G, Wk.shape[2] + D_R))
    V = np.empty(lat.shape[:2] + (G, Wv.shape[2]))
    for g in range(G):
        K[:, :, g, :Wk.shape[2]] = c @ Wk[g]
        K[:, :, g, Wk.shape[2]:] = rope
        V[:, :, g, :] = c @ Wv[g]
    return K, V


def absorb_query(q, w_uk):
    """The absorb path's query: [q_nope W_UK^g^T, q_rope] per head, float64.
    q [B, T, H, d_h + d_r] -> [B, T, H, d_c + d_r]."""
    qf = bf16_to_f64(q)
    Wk = bf16_to_f64(w_uk)
    G, _, d_h = Wk.shape
    hpg = _groups(q.shape[2], G)
    out = np.empty(q.shape[:3] + (D_C + D_R,))
    for g in range(G):
        hs = slice(g * hpg, (g + 1) * hpg)
        out[:, :, hs, :D_C] = qf[:, :, hs, :d_h] @ Wk[g].T
        out[:, :, hs, D_C:] = qf[:, :, hs, d_h:]
    return out


def absorb_output(o_lat, w_uv):
    """The absorb path's output: o_latent W_UV^g per head, float64.
    o_lat [B, T, H, d_c] (float) -> [B, T, H, d_v]."""
    Wv = bf16_to_f64(w_uv)
    G = Wv.shape[0]
    hpg = _groups(o_lat.shape[2], G)
    out = np.empty(o_lat.shape[:3] + (Wv.shape[2],))
    for g in range(G):
        hs = slice(g * hpg, (g + 1) * hpg)
        out[:, :, hs, :] = np.asarray(o_lat[:, :, hs, :], dtype=np.float64) @ Wv[g]
    return out


def _attend(qrows, K, V, sigma, vis):
    """softmax(sigma q K^T) V for each query row over its first vis[r] keys
    (max first, then exponentials and their sum). qrows [R, D], K [L, D],
    V [L, Dv] float64. Returns out [R, Dv], lse [R]; a row with no key gets
    out = 0, lse = -inf."""
    out = np.zeros((qrows.shape[0], V.shape[1]))
    lse = np.full(qrows.shape[0], -np.inf)
    for r in range(qrows.shape[0]):
        n = int(vis[r])
        if n <= 0:
            continue
        s = sigma * (K[:n] @ qrows[r])
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        out[r] = (e @ V[:n]) / l
        lse[r] = m + np.log(l)
    return out, lse


def _latent_rows(kv, bt_row, L):
    return gather_pages(kv, bt_row, L)[:, 0, :]  # [L, 576] float64


def attend_direct(q, kv, w_uk, w_uv, block_table, seqlens, scale, causal):
    """The definition: each group's keys and values are formed from the
    latent rows, then o_h = softmax(scale q_h K^g^T) V^g. Returns out
    [B, T, H, d_v] and lse [B, T, H] (natural log), float64."""
    B, T, H, _ = q.shape
    Wk, Wv = bf16_to_f64(w_uk), bf16_to_f64(w_uv)
    G, _, d_h = Wk.shape
    hpg = _groups(H, G)
    sigma = scale_as_received(scale)
    qf = bf16_to_f64(q)
    out = np.zeros((B, T, H, Wv.shape[2]))
    lse = np.full((B, T, H), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        if L <= 0:
            continue
        lat = _latent_rows(kv, block_table[b], L)
        c, rope = lat[:, :D_C], lat[:, D_C:]
        for g in range(G):
            K = np.concatenate([c @ Wk[g], rope], axis=1)   # [L, d_h + d_r]
            V = c @ Wv[g]                                   # [L, d_v]
            for t in range(T):
                hs = slice(g * hpg, (g + 1) * hpg)
                vis = [visible_keys(L, T, t, causal)] * hpg
                out[b, t, hs], lse[b, t, hs] = _attend(qf[b, t, hs], K, V, sigma, vis)
    return out, lse


def attend_absorb(q, kv, w_uk, w_uv, block_table, seqlens, scale, causal, round_bf16=False):
    """The MQA-absorb path: absorbed queries attend the 576-wide latent rows
    with the latent c as values, and the result is multiplied by W_UV^g.
    Returns (out [B, T, H, d_v], lse [B, T, H], o_latent [B, T, H, d_c])."""
    rnd = globals()["round_bf16"] if round_bf16 else (lambda x: x)
    B, T, H, _ = q.shape
    sigma = scale_as_received(scale)
    qa = rnd(absorb_query(q, w_uk))
    o_lat = np.zeros((B, T, H, D_C))
    lse = np.full((B, T, H), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        if L <= 0:
            continue
        lat = _latent_rows(kv, block_table[b], L)
        for t in range(T):
            vis = [visible_keys(L, T, t, causal)] * H
            o_lat[b, t], lse[b, t] = _attend(qa[b, t], lat, lat[:, :D_C], sigma, vis)
    o_lat = rnd(o_lat)
    return absorb_output(o_lat, w_uv), lse, o_lat


def attend_gqa_path(q, kv, w_uk, w_uv, block_table, seqlens, scale, causal, round_bf16=False,
                    pages=None):
    """The GQA path: expand the cache per group, then grouped attention of
    the unchanged queries over the expanded pages. ``pages`` limits the
    expansion to the physical pages the given sequences use (the rest of the
    pool is never read). Returns out, lse."""
    idx = (np.arange(kv.shape[0]) if pages is None
           else np.asarray(sorted(set(int(p) for p in pages)), dtype=np.int64))
    K, V = expand_group_cache(kv[idx], w_uk, w_uv)   # rows of the listed pages only
    at = {int(p): i for i, p in enumerate(idx)}
    if round_bf16:
        K, V = globals()["round_bf16"](K), globals()["round_bf16"](V)
    B, T, H, _ = q.shape
    G = K.shape[2]
    hpg = _groups(H, G)
    sigma = scale_as_received(scale)
    qf = bf16_to_f64(q)
    out = np.zeros((B, T, H, V.shape[3]))
    lse = np.full((B, T, H), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        if L <= 0:
            continue
        n = (L + 63) // 64
        rows = [at[int(p)] for p in block_table[b, :n]]
        Kb = np.concatenate([K[i] for i in rows], axis=0)[:L]   # [L, G, D]
        Vb = np.concatenate([V[i] for i in rows], axis=0)[:L]
        for g in range(G):
            hs = slice(g * hpg, (g + 1) * hpg)
            for t in range(T):
                vis = [visible_keys(L, T, t, causal)] * hpg
                out[b, t, hs], lse[b, t, hs] = _attend(qf[b, t, hs], Kb[:, g], Vb[:, g], sigma, vis)
    return out, lse
