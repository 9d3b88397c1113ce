"""Plain fp64 CPU attention decode over a paged KV cache: the oracle.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library neither
imports nor calls it, and it shares no code with the GPU path.

What it computes. The method is exact attention reached faster, not an
approximation: FlashAttention (KO) says the speed-up keeps full computational
accuracy (opening paragraph) and that the online softmax gives the exact
result (section "온라인 Softmax 계산"). So the oracle is the definition itself,
softmax(Q K^T * scale) V (section "표준 Attention의 문제점"), evaluated in
float64 on the bf16 inputs, over the keys that the block table gathers
(PagedAttention, cited in "참고 문헌"; 64-token pages per the FlashMLA blog,
"기술 기반").

The two decode shapes come from the GQLA review, "1. Key Terms &
Definitions": on the MQA-absorb path every query head attends the same
latent cache row; on the GQA path each group of heads attends its own
expanded K and V rows.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * V of the latent cache is the first ``d_v`` (512) columns of the K row.
  * Query head h uses KV head g = h // (h_q / h_kv).
  * Causal decode with s_q > 1 query tokens aligns bottom-right: query token
    t is the (L - s_q + t)-th token of the sequence and sees keys
    0 .. L - s_q + t.
  * A row that sees no key returns out = 0 and lse = -inf.
  * lse = m + ln(sum_j exp(s_j - m)), natural log, in units of the scaled
    scores s_j = scale * q . k_j.
  * ``scale`` is used as the float32 value the GPU receives.

Inputs are numpy arrays: bf16 bit patterns as uint16 (q [B, T, H, D];
cache [P, 64, G, D]), int32 block_table [B, max_pages], int32 seqlens [B].
"""
from __future__ import annotations

import numpy as np

PAGE = 64


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the pattern is the top half of an
    IEEE float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def scale_as_received(scale: float) -> float:
    """The softmax scale is handed to the GPU as a float32; the oracle uses
    that exact value."""
    return float(np.float32(scale))


def visible_keys(L: int, s_q: int, t: int, causal: bool) -> int:
    """Number of cached keys query token t may attend (bottom-right causal
    alignment), clamped to [0, L]."""
    if not causal:
        return int(L)
    return int(min(max(L - s_q + 1 + t, 0), L))


def gather_pages(cache: np.ndarray, block_table_row: np.ndarray, L: int) -> np.ndarray:
    """Rows 0..L-1 of one sequence, page by page through its block table,
    decoded to float64: [L, G, D]. Page slots at or past L are never read,
    and neither are block-table entries past the last needed page."""
    n = (L + PAGE - 1) // PAGE
    G, D = cache.shape[2], cache.shape[3]
    out = np.empty((n * PAGE, G, D), dtype=np.float64)
    for j in range(n):
        used = min(PAGE, L - j * PAGE)
        out[j * PAGE:j * PAGE + used] = bf16_to_f64(cache[int(block_table_row[j]), :used])
    return out[:L]


def _sequence_kv(k_cache, v_cache, d_v, bt_row, L):
    K = gather_pages(k_cache, bt_row, L)
    V = K[:, :, :d_v] if v_cache is None else gather_pages(v_cache, bt_row, L)
    return K, V


def _heads_per_group(H, G):
    if G <= 0 or H % G:
        raise ValueError(f"h_q={H} is not a multiple of h_kv={G}")
    return H // G


def attend_two_pass(q, k_cache, block_table, seqlens, scale, causal,
                    v_cache=None, d_v=None, key_range=None):
    """softmax(q K^T * scale) V per query row, by the textbook two passes
    (row max, then exponentials and their sum).

    ``v_cache=None`` is the latent cache: V = K[..., :d_v].
    ``key_range=(lo, hi)`` restricts every row to keys lo <= j < hi (still
    intersected with what the row may see); used to build split results.
    Returns out float64 [B, T, H, Dv] and lse float64 [B, T, H].
    """
    B, T, H, D = q.shape
    G = k_cache.shape[2]
    hpg = _heads_per_group(H, G)
    if d_v is None:
        d_v = D if v_cache is None else v_cache.shape[3]
    sigma = scale_as_received(scale)
    out = np.zeros((B, T, H, d_v))
    lse = np.full((B, T, H), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        if L <= 0:
            continue
        K, V = _sequence_kv(k_cache, v_cache, d_v, block_table[b], L)
        qb = bf16_to_f64(q[b])                                  # [T, H, D]
        for g in range(G):
            hs = slice(g * hpg, (g + 1) * hpg)
            s = sigma * np.matmul(qb[:, hs, :], K[:, g, :].T)   # [T, hpg, L]
            for t in range(T):
                hi = visible_keys(L, T, t, causal)
                lo = 0
                if key_range is not None:
                    lo, hi = max(lo, key_range[0]), min(hi, key_range[1])
                if hi <= lo:
                    continue
                st = s[t, :, lo:hi]
                m = st.max(axis=1, keepdims=True)
                e = np.exp(st - m)
                l = e.sum(axis=1)
                out[b, t, hs] = np.matmul(e, V[lo:hi, g, :]) / l[:, None]
                lse[b, t, hs] = m[:, 0] + np.log(l)
    return out, lse


def value_spread(q, k_cache, block_table, seqlens, scale, causal, v_cache=None, d_v=None):
    """Per output element, how far the values it averages lie from the
    output: the attention-weighted standard deviation of V,
    sqrt(sum_j w_j v_j^2 - (sum_j w_j v_j)^2), and the weighted mean of |V|,
    sum_j w_j |v_j|, with w the softmax weights of that row (the same weights
    as attend_two_pass); plus the number of keys the row sees. They size the
    error of a decode whose products round their weights: an output
    sum_j w_j v_j moves by sum_j dw_j (v_j - out) when the weights move by dw
    with sum_j dw_j = 0. Returns sd [B, T, H, Dv], mean_abs [B, T, H, Dv] and
    nkeys [B, T, H] (0 where the row sees nothing)."""
    B, T, H, D = q.shape
    G = k_cache.shape[2]
    hpg = _heads_per_group(H, G)
    if d_v is None:
        d_v = D if v_cache is None else v_cache.shape[3]
    sigma = scale_as_received(scale)
    sd = np.zeros((B, T, H, d_v))
    mean_abs = np.zeros((B, T, H, d_v))
    nkeys = np.zeros((B, T, H), dtype=np.int64)
    for b in range(B):
        L = int(seqlens[b])
        if L <= 0:
            continue
        K, V = _sequence_kv(k_cache, v_cache, d_v, block_table[b], L)
        qb = bf16_to_f64(q[b])
        for g in range(G):
            hs = slice(g * hpg, (g + 1) * hpg)
            s = sigma * np.matmul(qb[:, hs, :], K[:, g, :].T)   # [T, hpg, L]
            Vg = V[:, g, :]
            for t in range(T):
                hi = visible_keys(L, T, t, causal)
                if hi <= 0:
                    continue
                st = s[t, :, :hi]
                e = np.exp(st - st.max(axis=1, keepdims=True))
                w = e / e.sum(axis=1, keepdims=True)            # [hpg, hi]
                mean = w @ Vg[:hi]
                second = w @ (Vg[:hi] ** 2)
                sd[b, t, hs] = np.sqrt(np.maximum(second - mean ** 2, 0.0))
                mean_abs[b, t, hs] = w @ np.abs(Vg[:hi])
                nkeys[b, t, hs] = hi
    return sd, mean_abs, nkeys


def softmax_weights(q, k_cache, block_table, seqlens, scale, causal, b, t):
    """The attention weights of every head of query (b, t) over the keys it
    sees: [H, visible]. Used to check that each row sums to one."""
    B, T, H, D = q.shape
    G = k_cache.shape[2]
    hpg = _heads_per_group(H, G)
    L = int(seqlens[b])
    vis = visible_keys(L, T, t, causal)
    K = gather_pages(k_cache, block_table[b], L)[:vis]
    qb = bf16_to_f64(q[b, t])
    w = np.empty((H, vis))
    if vis == 0:
        return w
    for h in range(H):
        s = scale_as_received(scale) * (K[:, h // hpg, :] @ qb[h])
        e = np.exp(s - s.max())
        w[h] = e / e.sum()
    return w


def attend_online(q, k_cache, block_table, seqlens, scale, causal,
                  v_cache=None, d_v=None, block=PAGE):
    """The same result by the online softmax of FlashAttention (KO), section
    "온라인 Softmax 계산": keys are visited in blocks of ``block`` in page
    order, keeping per row a running maximum m, a running sum l of
    exponentials and an unnormalised accumulator; when a block raises the
    maximum, l and the accumulator are rescaled by exp(m_old - m_new).
    The result is normalised once at the end."""
    B, T, H, D = q.shape
    G = k_cache.shape[2]
    hpg = _heads_per_group(H, G)
    if d_v is None:
        d_v = D if v_cache is None else v_cache.shape[3]
    sigma = scale_as_received(scale)
    out = np.zeros((B, T, H, d_v))
    lse = np.full((B, T, H), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        if L <= 0:
            continue
        K, V = _sequence_kv(k_cache, v_cache, d_v, block_table[b], L)
        qb = bf16_to_f64(q[b])
        for t in range(T):
            vis = visible_keys(L, T, t, causal)
            for h in range(H):
                g = h // hpg
                m, l = -np.inf, 0.0
                acc = np.zeros(d_v)
                for j0 in range(0, vis, block):
                    j1 = min(vis, j0 + block)
                    s = sigma * (K[j0:j1, g, :] @ qb[t, h])
                    m_new = max(m, s.max())
                    alpha = np.exp(m - m_new) if m > -np.inf else 0.0
                    p = np.exp(s - m_new)
                    l = alpha * l + p.sum()
                    acc = alpha * acc + p @ V[j0:j1, g, :]
                    m = m_new
                if l > 0.0:
                    out[b, t, h] = acc / l
                    lse[b, t, h] = m + np.log(l)
    return out, lse


def combine(parts):
    """Merge results computed over disjoint key subsets of the same rows.

    ``parts`` is a list of (out_i, lse_i) pairs of equal shapes. Each part is
    a softmax-normalised result over its own keys with lse_i its log-sum-exp,
    so exp(lse_i) is its share of the full normaliser: the merged lse is the
    log of the summed exp(lse_i) and the merged out weights each part by
    exp(lse_i - lse). A part that saw no key (lse_i = -inf) adds nothing; a
    row with no key in any part gives out = 0, lse = -inf. This follows from
    the running-statistics update of the online softmax (FlashAttention (KO),
    "온라인 Softmax 계산") applied once per part."""
    lses = np.stack([p[1] for p in parts])                 # [n, ...]
    outs = np.stack([p[0] for p in parts])                 # [n, ..., Dv]
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - m_safe), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    wn = np.where(finite, w / np.where(finite, tot, 1.0), 0.0)
    out = (wn[..., None] * outs).sum(axis=0)
    return out, lse


def attend_bruteforce(q, k_cache, block_table, seqlens, scale, causal,
                      v_cache=None, d_v=None):
    """Dense attention for tiny inputs: every query row of the batch against
    every key slot of every sequence, one score matrix, with an explicit
    boolean mask (same sequence, same KV head, key visible), then a row
    softmax and a product with V. Written without the page walk above: a key
    slot (b, j) is read as cache[block_table[b, j // 64], j % 64]."""
    B, T, H, D = q.shape
    G = k_cache.shape[2]
    hpg = H // G
    if d_v is None:
        d_v = D if v_cache is None else v_cache.shape[3]
    Lmax = int(max(seqlens)) if B else 0
    sigma = float(np.float32(scale))
    # key slots: index (b, j, g)
    keys = np.zeros((B, Lmax, G, D))
    vals = np.zeros((B, Lmax, G, d_v))
    for b in range(B):
        for j in range(int(seqlens[b])):
            page = int(block_table[b, j // 64])
            row = bf16_to_f64(k_cache[page, j % 64])
            keys[b, j] = row
            vals[b, j] = row[:, :d_v] if v_cache is None else bf16_to_f64(v_cache[page, j % 64])
    Q = bf16_to_f64(q).reshape(B * T * H, D)
    Kf = keys.reshape(B * Lmax * G, D)
    Vf = vals.reshape(B * Lmax * G, d_v)
    S = sigma * (Q @ Kf.T)                                   # [BTH, B*Lmax*G]
    qb, qt, qh = np.meshgrid(np.arange(B), np.arange(T), np.arange(H), indexing="ij")
    kb, kj, kg = np.meshgrid(np.arange(B), np.arange(Lmax), np.arange(G), indexing="ij")
    qb, qt, qh = qb.ravel(), qt.ravel(), qh.ravel()
    kb, kj, kg = kb.ravel(), kj.ravel(), kg.ravel()
    Lq = np.asarray(seqlens)[qb]
    limit = np.where(causal, Lq - T + 1 + qt, Lq)
    mask = ((qb[:, None] == kb[None, :]) & (qh[:, None] // hpg == kg[None, :])
            & (kj[None, :] < limit[:, None]) & (kj[None, :] < Lq[:, None]))
    S = np.where(mask, S, -np.inf)
    rowmax = S.max(axis=1)
    has = np.isfinite(rowmax)
    E = np.where(mask, np.exp(S - np.where(has, rowmax, 0.0)[:, None]), 0.0)
    den = E.sum(axis=1)
    out = np.where(has[:, None], (E @ Vf) / np.where(has, den, 1.0)[:, None], 0.0)
    lse = np.where(has, rowmax + np.log(np.where(has, den, 1.0)), -np.inf)
    return out.reshape(B, T, H, d_v), lse.reshape(B, T, H)
