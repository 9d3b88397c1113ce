"""The five decode workloads: shapes, length mixes and value distributions.

These are synthetic stand-ins for the workloads the pages describe without
giving their sizes: bf16 decode over a KV cache cut into 64-token pages, with
variable sequence lengths (FlashMLA blog, "기술 기반" list), on the two decode
shapes of the GQLA review ("1. Key Terms & Definitions": the MQA-absorb path,
where every query head reads one shared latent row, and the GQA path with a
per-group expanded cache).

This module holds no attention arithmetic; it only names sizes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

PAGE = 64  # tokens per KV page (FlashMLA blog, "기술 기반": 64-token paged KV cache)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    seed: int
    kind: str            # "mla" (one shared latent row per token) or "gqa"
    batch: int
    s_q: int             # query tokens per sequence in this decode step
    h_q: int             # query heads
    h_kv: int            # KV heads (1 for the latent cache)
    d_qk: int            # width of q and of a K row
    d_v: int             # width of a V row
    causal: bool
    seqlen_rule: str     # "fixed", "loguniform" or "uniform"
    seqlens_fixed: tuple = ()
    seqlen_lo: int = 0
    seqlen_hi: int = 0
    q_std: float = 1.0
    kv_std: float = 1.0
    scale: float = 1.0
    page: int = PAGE

    @property
    def rows(self) -> int:
        """Query rows that share one KV head: s_q * h_q / h_kv."""
        return self.s_q * self.h_q // self.h_kv

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


MLA_SCALE = 1.0 / math.sqrt(192.0)
GQA_SCALE = 1.0 / math.sqrt(128.0)

CONFIGS = {
    1: DecodeConfig("tiny_mla_b2_h8", 1, "mla", batch=2, s_q=1, h_q=8, h_kv=1,
                    d_qk=576, d_v=512, causal=False, seqlen_rule="fixed",
                    seqlens_fixed=(64, 200), scale=MLA_SCALE),
    2: DecodeConfig("dsv3_mla_b64_h128_L4096", 2, "mla", batch=64, s_q=1, h_q=128,
                    h_kv=1, d_qk=576, d_v=512, causal=False, seqlen_rule="fixed",
                    seqlens_fixed=(4096,) * 64, kv_std=0.5, scale=MLA_SCALE),
    3: DecodeConfig("mtp2_varlen_mla_b128_h128", 3, "mla", batch=128, s_q=2,
                    h_q=128, h_kv=1, d_qk=576, d_v=512, causal=True,
                    seqlen_rule="loguniform", seqlen_lo=1, seqlen_hi=16384,
                    scale=MLA_SCALE),
    4: DecodeConfig("headshare_mla_b256_h16_L8192", 4, "mla", batch=256, s_q=1,
                    h_q=16, h_kv=1, d_qk=576, d_v=512, causal=False,
                    seqlen_rule="fixed", seqlens_fixed=(8192,) * 256,
                    scale=MLA_SCALE),
    5: DecodeConfig("gqa_b32_h128_g8_L8k-32k", 5, "gqa", batch=32, s_q=1, h_q=128,
                    h_kv=8, d_qk=128, d_v=128, causal=False, seqlen_rule="uniform",
                    seqlen_lo=8192, seqlen_hi=32768, scale=GQA_SCALE),
}


@dataclass(frozen=True)
class GqlaConfig:
    """A GQLA decode step: a latent cache plus per-group up-projections
    (GQLA review, "2. Motivation & Problem Statement": the up-projections are
    indexed by KV group, not by query head, so the same weights serve the
    MQA-absorb path and the GQA path). Widths follow the DeepSeek-V3 shapes
    of the latent row: d_c latent + d_r rope; each group's keys are d_h wide
    plus the shared rope, its values d_v wide."""
    name: str
    seed: int
    batch: int
    s_q: int
    h_q: int
    h_kv: int            # KV groups; query head h uses group h // (h_q / h_kv)
    causal: bool
    seqlen_rule: str
    seqlens_fixed: tuple = ()
    seqlen_lo: int = 0
    seqlen_hi: int = 0
    q_std: float = 1.0
    kv_std: float = 1.0
    w_std: float = 1.0 / math.sqrt(512.0)
    scale: float = 1.0 / math.sqrt(192.0)
    d_c: int = 512
    d_r: int = 64
    d_h: int = 128
    d_v: int = 128
    page: int = PAGE

    @property
    def d_q(self) -> int:
        """Width of a query row: d_h (no-rope part) + d_r (rope part)."""
        return self.d_h + self.d_r

    def with_(self, **kw) -> "GqlaConfig":
        return replace(self, **kw)


# With w_std = 1/sqrt(d_c) the expanded keys and values have unit variance,
# so the scaled scores have about unit variance, as in the other workloads.
GQLA_CONFIGS = {
    "small": GqlaConfig("gqla_small_b3_h16_g4", 11, batch=3, s_q=2, h_q=16, h_kv=4,
                        causal=True, seqlen_rule="fixed", seqlens_fixed=(1, 130, 300)),
    "dsv3": GqlaConfig("gqla_dsv3_b64_h128_g8_L4096", 12, batch=64, s_q=1, h_q=128, h_kv=8,
                       causal=False, seqlen_rule="fixed", seqlens_fixed=(4096,) * 64),
}


def bytes_per_token(cfg: DecodeConfig) -> int:
    """HBM bytes of one cached token for one sequence: the latent row for MLA,
    K and V rows of every KV head for GQA (bf16)."""
    if cfg.kind == "mla":
        return cfg.h_kv * cfg.d_qk * 2
    return cfg.h_kv * (cfg.d_qk + cfg.d_v) * 2
