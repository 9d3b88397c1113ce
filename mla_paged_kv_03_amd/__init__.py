"""Paged MLA / GQA attention decode on MI355X (gfx950).

Thin Python binding over the C interface in include/mla_decode.h: the
functions below only check and marshal torch tensors (device pointers and
the current HIP stream); every step of the decode runs in the library's HIP
kernels. There is no CPU fallback: without the built library the import of
the native code fails loudly.

    plan = mla_decode_plan(cache_seqlens, s_q, h_q, h_kv=1, head_dim_v=512)
    out, lse = mla_decode(q, kv_cache, block_table, cache_seqlens, scale, causal, plan)
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import DecodeError, PlanInfo

__all__ = ["Plan", "PlanInfo", "DecodeError", "plan_info", "mla_decode_plan", "mla_decode",
           "mla_decode_noalloc",
           "gqa_decode", "attn_combine", "mla_kv_append", "gqa_kv_append",
           "mla_decode_fp8", "mla_kv_append_fp8", "mla_kv_quantize_fp8", "gqla_expand_kv", "gqla_absorb_query", "gqla_absorb_output", "gqla_decode",
           "mla_decode_plan_host", "mla_check_pages", "mla_check_fp8_scales", "profile_events"]

MLA_D, MLA_DV = 576, 512
GQA_D = 128
GQLA_DC, GQLA_DR, GQLA_DH, GQLA_DV = 512, 64, 128, 128
GQLA_DQ = GQLA_DH + GQLA_DR


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


@dataclass
class Plan:
    """A split-KV schedule for one decode step (reusable across layers)."""
    sched_metadata: torch.Tensor
    num_splits: torch.Tensor
    info: PlanInfo
    workspace: torch.Tensor | None
    shape: tuple  # (batch, s_q, h_q, h_kv, head_dim_v, kv_fp8)


def _plan_call(fp8, seqlens, batch, s_q, h_q, h_kv, head_dim_v, meta, splits, info, stream):
    if fp8:
        if h_kv != 1 or head_dim_v != MLA_DV:
            raise ValueError("an FP8 cache plan is for h_kv = 1 and head_dim_v = 512")
        return "mla_decode_plan_fp8", _lib.lib().mla_decode_plan_fp8(
            seqlens, batch, s_q, h_q, meta, splits, ctypes.byref(info), stream)
    return "mla_decode_plan", _lib.lib().mla_decode_plan(
        seqlens, batch, s_q, h_q, h_kv, head_dim_v, meta, splits, ctypes.byref(info), stream)


def plan_info(batch, s_q, h_q, h_kv=1, head_dim_v=MLA_DV, kv_fp8=False) -> PlanInfo:
    """Buffer sizes of a plan on the current device (no device work)."""
    info = PlanInfo()
    _lib.check(*_plan_call(kv_fp8, None, batch, s_q, h_q, h_kv, head_dim_v, None, None, info,
                           None))
    return info


def mla_decode_plan(cache_seqlens, s_q, h_q, h_kv=1, head_dim_v=MLA_DV, kv_fp8=False) -> Plan:
    """Allocate the plan's buffers (metadata, num_splits, workspace) and
    enqueue the plan kernel on the current stream. kv_fp8: the plan of
    mla_decode_fp8 (C: mla_decode_plan_fp8)."""
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    batch = cache_seqlens.shape[0]
    info = plan_info(batch, s_q, h_q, h_kv, head_dim_v, kv_fp8)
    dev = cache_seqlens.device
    meta = torch.empty(info.metadata_bytes // 4, dtype=torch.int32, device=dev)
    splits = torch.empty(batch + 1, dtype=torch.int32, device=dev)
    ws = (torch.empty(info.workspace_bytes // 4 + 64, dtype=torch.float32, device=dev)
          if info.workspace_bytes else None)
    _lib.check(*_plan_call(kv_fp8, _ptr(cache_seqlens), batch, s_q, h_q, h_kv, head_dim_v,
                           _ptr(meta), _ptr(splits), info, _stream()))
    return Plan(meta, splits, info, ws, (batch, s_q, h_q, h_kv, head_dim_v, bool(kv_fp8)))


def _ws(plan):
    if plan.workspace is None:
        return None, 0
    # 256-byte aligned start inside the allocation
    p = plan.workspace.data_ptr()
    off = (-p) % 256
    return ctypes.c_void_p(p + off), plan.workspace.numel() * 4 - off


def mla_decode(q, kv_cache, block_table, cache_seqlens, softmax_scale, causal=False,
               plan: Plan | None = None, out=None, lse=None):
    """MQA-absorb MLA decode. q bf16 [B, s_q, h_q, 576]; kv_cache bf16
    [num_pages, 64, 1, 576]; block_table int32 [B, max_pages]; cache_seqlens
    int32 [B]. Returns (out bf16 [B, s_q, h_q, 512], lse fp32 [B, s_q, h_q])."""
    _need(q, "q", torch.bfloat16, 4)
    _need(kv_cache, "kv_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, T, H, D = q.shape
    if D != MLA_D or tuple(kv_cache.shape[1:]) != (64, 1, MLA_D):
        raise ValueError("mla_decode expects q [..., 576] and kv_cache [P, 64, 1, 576]")
    if block_table.shape[0] != B or cache_seqlens.shape[0] != B:
        raise ValueError("batch mismatch")
    if plan is None:
        plan = mla_decode_plan(cache_seqlens, T, H, 1, MLA_DV)
    if plan.shape != (B, T, H, 1, MLA_DV, False):
        raise ValueError(f"plan was made for {plan.shape}")
    if out is None:
        out = torch.empty(B, T, H, MLA_DV, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16)
    _need(lse, "lse", torch.float32)
    ws, wsb = _ws(plan)
    _lib.check("mla_decode", _lib.lib().mla_decode(
        _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(cache_seqlens), B, T, H,
        kv_cache.shape[0], block_table.shape[1], float(softmax_scale), int(bool(causal)),
        _ptr(plan.sched_metadata), _ptr(plan.num_splits), ws, wsb, _ptr(out), _ptr(lse),
        _stream()))
    return out, lse


def mla_decode_noalloc(q, kv_cache, block_table, cache_seqlens, softmax_scale, causal=False,
                       out=None, lse=None):
    """mla_decode without plan or workspace buffers: the library plans into
    its own static device scratch (see include/mla_decode.h). Calls on one
    GPU share that scratch, so they must not overlap in time. With out and
    lse given, nothing is allocated on the way."""
    _need(q, "q", torch.bfloat16, 4)
    _need(kv_cache, "kv_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, T, H, D = q.shape
    if D != MLA_D or tuple(kv_cache.shape[1:]) != (64, 1, MLA_D):
        raise ValueError("mla_decode_noalloc expects q [..., 576] and kv_cache [P, 64, 1, 576]")
    if block_table.shape[0] != B or cache_seqlens.shape[0] != B:
        raise ValueError("batch mismatch")
    if out is None:
        out = torch.empty(B, T, H, MLA_DV, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16)
    _need(lse, "lse", torch.float32)
    if tuple(out.shape) != (B, T, H, MLA_DV) or tuple(lse.shape) != (B, T, H):
        raise ValueError("out must be [B, s_q, h_q, 512] and lse [B, s_q, h_q]")
    _lib.check("mla_decode_noalloc", _lib.lib().mla_decode_noalloc(
        _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(cache_seqlens), B, T, H,
        kv_cache.shape[0], block_table.shape[1], float(softmax_scale), int(bool(causal)),
        _ptr(out), _ptr(lse), _stream()))
    return out, lse


def gqa_decode(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale, causal=False,
               plan: Plan | None = None, out=None, lse=None):
    """GQA decode with a per-group expanded cache. q bf16 [B, s_q, h_q, 128];
    k_cache, v_cache bf16 [num_pages, 64, h_kv, 128]."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, T, H, D = q.shape
    P, page, G, Dk = k_cache.shape
    if D != GQA_D or Dk != GQA_D or page != 64 or tuple(v_cache.shape) != (P, 64, G, GQA_D):
        raise ValueError("gqa_decode expects q [..., 128] and k/v caches [P, 64, h_kv, 128]")
    if plan is None:
        plan = mla_decode_plan(cache_seqlens, T, H, G, GQA_D)
    if plan.shape != (B, T, H, G, GQA_D, False):
        raise ValueError(f"plan was made for {plan.shape}")
    if out is None:
        out = torch.empty(B, T, H, GQA_D, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    ws, wsb = _ws(plan)
    _lib.check("gqa_decode", _lib.lib().gqa_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(cache_seqlens), B, T, H,
        G, P, block_table.shape[1], float(softmax_scale), int(bool(causal)),
        _ptr(plan.sched_metadata), _ptr(plan.num_splits), ws, wsb, _ptr(out), _ptr(lse),
        _stream()))
    return out, lse


def mla_kv_append(new_kv, kv_cache, block_table, cache_seqlens):
    """Write the s_q new tokens' latent rows into the paged cache in place.
    new_kv bf16 [B, s_q, 576]; kv_cache bf16 [num_pages, 64, 1, 576];
    cache_seqlens counts the new tokens (token t of sequence b is position
    cache_seqlens[b] - s_q + t)."""
    _need(new_kv, "new_kv", torch.bfloat16, 3)
    _need(kv_cache, "kv_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, T, D = new_kv.shape
    P, page, one, Dk = kv_cache.shape
    if D != MLA_D or Dk != MLA_D or page != 64 or one != 1:
        raise ValueError("mla_kv_append expects new_kv [B, s_q, 576], kv_cache [P, 64, 1, 576]")
    _lib.check("mla_kv_append", _lib.lib().mla_kv_append(
        _ptr(new_kv), _ptr(kv_cache), _ptr(block_table), _ptr(cache_seqlens), B, T, P,
        block_table.shape[1], _stream()))
    return kv_cache


def gqa_kv_append(new_k, new_v, k_cache, v_cache, block_table, cache_seqlens):
    """The same for the GQA caches: new_k, new_v bf16 [B, s_q, h_kv, 128];
    k_cache, v_cache bf16 [num_pages, 64, h_kv, 128]."""
    for t, n in ((new_k, "new_k"), (new_v, "new_v")):
        _need(t, n, torch.bfloat16, 4)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, T, G, D = new_k.shape
    P, page, Gc, Dk = k_cache.shape
    if (D != GQA_D or Dk != GQA_D or page != 64 or Gc != G or tuple(new_v.shape) != (B, T, G, D)
            or tuple(v_cache.shape) != (P, 64, G, GQA_D)):
        raise ValueError("gqa_kv_append expects new k/v [B, s_q, h_kv, 128] and "
                         "k/v caches [P, 64, h_kv, 128]")
    _lib.check("gqa_kv_append", _lib.lib().gqa_kv_append(
        _ptr(new_k), _ptr(new_v), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(cache_seqlens), B, T, G, P, block_table.shape[1], _stream()))
    return k_cache, v_cache


def mla_kv_quantize_fp8(kv_rows, codes=None, scales=None):
    """Quantise bf16 latent rows (kv_rows [..., 576], e.g. a cache
    [P, 64, 1, 576]) to E4M3 codes uint8 [..., 576] and one fp32 scale per
    row [...] (a trailing 1 of the leading dims dropped)."""
    _need(kv_rows, "kv_rows", torch.bfloat16)
    if kv_rows.shape[-1] != MLA_D:
        raise ValueError("kv_rows must end in 576 columns")
    lead = tuple(kv_rows.shape[:-1])
    if len(lead) >= 2 and lead[-1] == 1:
        lead = lead[:-1]
    n = kv_rows.numel() // MLA_D
    if codes is None:
        codes = torch.empty(lead + (MLA_D,), dtype=torch.uint8, device=kv_rows.device)
    if scales is None:
        scales = torch.empty(lead, dtype=torch.float32, device=kv_rows.device)
    _need(codes, "codes", torch.uint8)
    _need(scales, "scales", torch.float32)
    if codes.numel() != n * MLA_D or scales.numel() != n:
        raise ValueError("codes / scales do not match kv_rows")
    _lib.check("mla_kv_quantize_fp8", _lib.lib().mla_kv_quantize_fp8(
        _ptr(kv_rows), _ptr(codes), _ptr(scales), n, _stream()))
    return codes, scales


def _fp8_cache(kv_codes, kv_scales):
    _need(kv_codes, "kv_codes", torch.uint8, 3)
    _need(kv_scales, "kv_scales", torch.float32, 2)
    P = kv_codes.shape[0]
    if tuple(kv_codes.shape) != (P, 64, MLA_D) or tuple(kv_scales.shape) != (P, 64):
        raise ValueError("an FP8 cache is kv_codes uint8 [P, 64, 576] and kv_scales fp32 [P, 64]")
    return P


def mla_kv_append_fp8(new_kv, kv_codes, kv_scales, block_table, cache_seqlens):
    """Quantise the s_q new tokens' rows (new_kv bf16 [B, s_q, 576]) into
    their slots of an FP8 cache, in place (slot rule of mla_kv_append)."""
    _need(new_kv, "new_kv", torch.bfloat16, 3)
    P = _fp8_cache(kv_codes, kv_scales)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, T, D = new_kv.shape
    if D != MLA_D or block_table.shape[0] != B or cache_seqlens.shape[0] != B:
        raise ValueError("mla_kv_append_fp8 expects new_kv [B, s_q, 576] and B block-table rows")
    _lib.check("mla_kv_append_fp8", _lib.lib().mla_kv_append_fp8(
        _ptr(new_kv), _ptr(kv_codes), _ptr(kv_scales), _ptr(block_table), _ptr(cache_seqlens),
        B, T, P, block_table.shape[1], _stream()))
    return kv_codes, kv_scales


def mla_decode_fp8(q, kv_codes, kv_scales, block_table, cache_seqlens, softmax_scale,
                   causal=False, plan: Plan | None = None, out=None, lse=None):
    """MLA decode over an FP8 latent cache (kv_codes uint8 [P, 64, 576],
    kv_scales fp32 [P, 64]); otherwise as mla_decode."""
    _need(q, "q", torch.bfloat16, 4)
    P = _fp8_cache(kv_codes, kv_scales)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, T, H, D = q.shape
    if D != MLA_D:
        raise ValueError("mla_decode_fp8 expects q [..., 576]")
    if block_table.shape[0] != B or cache_seqlens.shape[0] != B:
        raise ValueError("batch mismatch")
    if plan is None:
        plan = mla_decode_plan(cache_seqlens, T, H, 1, MLA_DV, kv_fp8=True)
    if plan.shape != (B, T, H, 1, MLA_DV, True):
        raise ValueError(f"plan was made for {plan.shape}")
    if out is None:
        out = torch.empty(B, T, H, MLA_DV, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16)
    _need(lse, "lse", torch.float32)
    ws, wsb = _ws(plan)
    _lib.check("mla_decode_fp8", _lib.lib().mla_decode_fp8(
        _ptr(q), _ptr(kv_codes), _ptr(kv_scales), _ptr(block_table), _ptr(cache_seqlens), B, T,
        H, P, block_table.shape[1], float(softmax_scale), int(bool(causal)),
        _ptr(plan.sched_metadata), _ptr(plan.num_splits), ws, wsb, _ptr(out), _ptr(lse),
        _stream()))
    return out, lse


def _gqla_weights(w_uk, w_uv=None):
    _need(w_uk, "w_uk", torch.bfloat16, 3)
    G = w_uk.shape[0]
    if tuple(w_uk.shape) != (G, GQLA_DC, GQLA_DH):
        raise ValueError("w_uk must be [h_kv, 512, 128]")
    if w_uv is not None:
        _need(w_uv, "w_uv", torch.bfloat16, 3)
        if tuple(w_uv.shape) != (G, GQLA_DC, GQLA_DV):
            raise ValueError("w_uv must be [h_kv, 512, 128] with the same h_kv as w_uk")
    return G


def gqla_expand_kv(kv_rows, w_uk, w_uv, k_rows=None, v_rows=None):
    """GQLA's GQA-path cache: per group g, K = [c W_UK^g, k_rope] and
    V = c W_UV^g of every latent row. kv_rows bf16 [..., 576] (e.g. a cache
    [P, 64, 1, 576]); returns k_rows [..., h_kv, 192] and v_rows
    [..., h_kv, 128] (the leading dims of kv_rows, a trailing 1 dropped)."""
    _need(kv_rows, "kv_rows", torch.bfloat16)
    G = _gqla_weights(w_uk, w_uv)
    if kv_rows.shape[-1] != GQLA_DC + GQLA_DR:
        raise ValueError("kv_rows must end in 576 columns")
    lead = tuple(kv_rows.shape[:-1])
    if len(lead) >= 2 and lead[-1] == 1:
        lead = lead[:-1]
    n = kv_rows.numel() // (GQLA_DC + GQLA_DR)
    if k_rows is None:
        k_rows = torch.empty(lead + (G, GQLA_DQ), dtype=torch.bfloat16, device=kv_rows.device)
    if v_rows is None:
        v_rows = torch.empty(lead + (G, GQLA_DV), dtype=torch.bfloat16, device=kv_rows.device)
    _need(k_rows, "k_rows", torch.bfloat16)
    _need(v_rows, "v_rows", torch.bfloat16)
    if k_rows.numel() != n * G * GQLA_DQ or v_rows.numel() != n * G * GQLA_DV:
        raise ValueError("k_rows / v_rows do not match kv_rows and h_kv")
    _lib.check("gqla_expand_kv", _lib.lib().gqla_expand_kv(
        _ptr(kv_rows), _ptr(w_uk), _ptr(w_uv), _ptr(k_rows), _ptr(v_rows), n, G, _stream()))
    return k_rows, v_rows


def gqla_absorb_query(q, w_uk, out=None):
    """The MQA-absorb path's queries: [q_nope W_UK^g^T, q_rope] per head.
    q bf16 [B, s_q, h_q, 192] -> bf16 [B, s_q, h_q, 576] (mla_decode's q)."""
    _need(q, "q", torch.bfloat16, 4)
    G = _gqla_weights(w_uk)
    B, T, H, D = q.shape
    if D != GQLA_DQ:
        raise ValueError("q must be [B, s_q, h_q, 192]")
    if out is None:
        out = torch.empty(B, T, H, GQLA_DC + GQLA_DR, dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 4)
    if tuple(out.shape) != (B, T, H, GQLA_DC + GQLA_DR):
        raise ValueError("out must be [B, s_q, h_q, 576]")
    _lib.check("gqla_absorb_query", _lib.lib().gqla_absorb_query(
        _ptr(q), _ptr(w_uk), _ptr(out), B * T, H, G, _stream()))
    return out


def gqla_absorb_output(o_latent, w_uv, out=None):
    """The MQA-absorb path's output: o_latent W_UV^g per head.
    o_latent bf16 [B, s_q, h_q, 512] -> bf16 [B, s_q, h_q, 128]."""
    _need(o_latent, "o_latent", torch.bfloat16, 4)
    _need(w_uv, "w_uv", torch.bfloat16, 3)
    G = w_uv.shape[0]
    if tuple(w_uv.shape) != (G, GQLA_DC, GQLA_DV):
        raise ValueError("w_uv must be [h_kv, 512, 128]")
    B, T, H, D = o_latent.shape
    if D != GQLA_DC:
        raise ValueError("o_latent must be [B, s_q, h_q, 512]")
    if out is None:
        out = torch.empty(B, T, H, GQLA_DV, dtype=torch.bfloat16, device=o_latent.device)
    _need(out, "out", torch.bfloat16, 4)
    if tuple(out.shape) != (B, T, H, GQLA_DV):
        raise ValueError("out must be [B, s_q, h_q, 128]")
    _lib.check("gqla_absorb_output", _lib.lib().gqla_absorb_output(
        _ptr(o_latent), _ptr(w_uv), _ptr(out), B * T, H, G, _stream()))
    return out


def gqla_decode(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale, causal=False,
                plan: Plan | None = None, out=None, lse=None):
    """GQLA's GQA path: q bf16 [B, s_q, h_q, 192] over the expanded caches
    k_cache bf16 [P, 64, h_kv, 192], v_cache bf16 [P, 64, h_kv, 128]. The
    plan is the GQA one (h_kv, head_dim_v = 128)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, T, H, D = q.shape
    P, page, G, Dk = k_cache.shape
    if (D != GQLA_DQ or Dk != GQLA_DQ or page != 64
            or tuple(v_cache.shape) != (P, 64, G, GQLA_DV)):
        raise ValueError("gqla_decode expects q [..., 192], k_cache [P, 64, h_kv, 192] and "
                         "v_cache [P, 64, h_kv, 128]")
    if plan is None:
        plan = mla_decode_plan(cache_seqlens, T, H, G, GQLA_DV)
    if plan.shape != (B, T, H, G, GQLA_DV, False):
        raise ValueError(f"plan was made for {plan.shape}")
    if out is None:
        out = torch.empty(B, T, H, GQLA_DV, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    ws, wsb = _ws(plan)
    _lib.check("gqla_decode", _lib.lib().gqla_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(cache_seqlens), B, T, H,
        G, P, block_table.shape[1], float(softmax_scale), int(bool(causal)),
        _ptr(plan.sched_metadata), _ptr(plan.num_splits), ws, wsb, _ptr(out), _ptr(lse),
        _stream()))
    return out, lse


def attn_combine(o_partial, lse_partial, num_splits, out=None, lse=None):
    """Log-sum-exp merge of partials. o_partial fp32 [slots, R, dv],
    lse_partial fp32 [slots, R], num_splits int32 [B + 1] (slot prefix).
    Returns out bf16 [B, R, dv], lse fp32 [B, R] (rows of sequences without
    slots are left as given)."""
    _need(o_partial, "o_partial", torch.float32, 3)
    _need(lse_partial, "lse_partial", torch.float32, 2)
    _need(num_splits, "num_splits", torch.int32, 1)
    _, R, dv = o_partial.shape
    B = num_splits.shape[0] - 1
    if out is None:
        out = torch.zeros(B, R, dv, dtype=torch.bfloat16, device=o_partial.device)
    if lse is None:
        lse = torch.full((B, R), float("-inf"), dtype=torch.float32, device=o_partial.device)
    _lib.check("attn_combine", _lib.lib().attn_combine(
        _ptr(o_partial), _ptr(lse_partial), _ptr(num_splits), B, R, dv, _ptr(out), _ptr(lse),
        _stream()))
    return out, lse


def mla_check_pages(block_table, cache_seqlens, num_pages, status=None):
    """Check the decode calls' device-side preconditions: every length in
    [0, 64 * max_pages] and every used block-table entry in [0, num_pages).
    block_table int32 [B, max_pages], cache_seqlens int32 [B]. Returns status
    int32 [4] on the device, filled asynchronously: [violations, first
    sequence or -1, its page index (-1: the length), offending value]."""
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, max_pages = block_table.shape
    if cache_seqlens.shape[0] != B:
        raise ValueError("cache_seqlens must have one entry per block-table row")
    if status is None:
        status = torch.empty(4, dtype=torch.int32, device=block_table.device)
    _lib.check("mla_check_pages", _lib.lib().mla_check_pages(
        _ptr(block_table), _ptr(cache_seqlens), B, int(num_pages), max_pages, _ptr(status),
        _stream()))
    return status


def mla_check_fp8_scales(kv_scales, status=None):
    """Check that every per-token scale of an FP8 cache is a positive
    normal power of two (what mla_decode_fp8 dequantises exactly).
    kv_scales fp32 [num_pages, 64]. Returns status int32 [4] on the device,
    filled asynchronously: [violations, first index low word, high word,
    its fp32 bits]."""
    _need(kv_scales, "kv_scales", torch.float32)
    if status is None:
        status = torch.empty(4, dtype=torch.int32, device=kv_scales.device)
    _lib.check("mla_check_fp8_scales", _lib.lib().mla_check_fp8_scales(
        _ptr(kv_scales), kv_scales.numel(), _ptr(status), _stream()))
    return status


def mla_decode_plan_host(seqlens, s_q, h_q, h_kv=1, head_dim_v=MLA_DV, num_cus=256):
    """The plan computed on the host (for checking the schedule without a
    GPU). seqlens: sequence of ints. Returns (metadata, num_splits, info) as
    Python lists and a PlanInfo."""
    import numpy as np
    L = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    info = PlanInfo()
    lib = _lib.lib()
    _lib.check("mla_decode_plan_host", lib.mla_decode_plan_host(
        L.ctypes.data_as(ctypes.c_void_p), len(L), s_q, h_q, h_kv, head_dim_v, num_cus, None,
        None, ctypes.byref(info)))
    meta = np.zeros(info.metadata_bytes // 4, dtype=np.int32)
    splits = np.zeros(len(L) + 1, dtype=np.int32)
    _lib.check("mla_decode_plan_host", lib.mla_decode_plan_host(
        L.ctypes.data_as(ctypes.c_void_p), len(L), s_q, h_q, h_kv, head_dim_v, num_cus,
        meta.ctypes.data_as(ctypes.c_void_p), splits.ctypes.data_as(ctypes.c_void_p),
        ctypes.byref(info)))
    return meta, splits, info


def profile_events(start=None, stop=None):
    """Record the HIP events `start` / `stop` (raw hipEvent_t handles, as
    ints or ctypes.c_void_p) around the main decode kernel of every following
    decode call on its stream; None clears."""
    conv = lambda e: None if e is None else (e if isinstance(e, ctypes.c_void_p)
                                             else ctypes.c_void_p(int(e)))
    _lib.lib().mla_profile_events(conv(start), conv(stop))
