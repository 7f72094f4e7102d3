"""Workload registry for the index-selection sparse attention layer.

Each entry describes one synthetic workload: query rows, cached context
lengths, the indexer and MLA shapes, precisions, cache layout and seed.
The shapes follow the problem statement of the lightning indexer (LI) and
sparse flash attention (SFA) described on "Large Language Model Inference
Acceleration in Practice" (section 1.2, DSA) and the paged-cache / quantized
variants on "Kimi New Model Open Source: Day0 Inference Adaptation ..."
(sections 3 and 4).  Value distributions are synthetic stand-ins: the pages
measure only on private or external evaluation suites, none of which is used.

This module holds no arithmetic of the method; it only names sizes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    # query rows
    mode: str                   # "decode": one row per sequence at its last position
                                # "prefill": q_rows rows at the tail of sequence 0
    num_seqs: int
    seq_len: Optional[int]      # fixed length of every sequence, or None when drawn
    len_range: Optional[Tuple[int, int]] = None   # inclusive uniform range when drawn
    q_rows: int = 0             # prefill: number of query rows at the tail
    # indexer
    H_I: int = 64
    D_I: int = 128
    K: int = 2048
    # MLA
    H: int = 128
    D_latent: int = 512
    D_rope: int = 64
    softmax_scale: float = 1.0 / math.sqrt(576.0)
    # storage
    indexer_dtype: str = "bf16"     # "bf16" | "fp8" | "mxfp8" (e4m3 + E8M0 scale per 32 elements)
    kv_dtype: str = "bf16"          # "bf16" | "fp8" | "fp8_tile128"
    paged: bool = False
    block_size: int = 64
    kv_scale_group: int = 64        # tokens per fp32 latent-cache scale (fp8 only)
    # value distribution
    dist: str = "gauss"             # "gauss" | "int8range" (integers in [-8, 8])
    q_mla_std: float = 1.0          # std of the MLA queries ("sharp" variants raise it)

    @property
    def D_qk(self) -> int:
        return self.D_latent + self.D_rope

    @property
    def D_v(self) -> int:
        return self.D_latent

    @property
    def rows(self) -> int:
        return self.num_seqs if self.mode == "decode" else self.q_rows

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the problem statement (numbered 0..4) plus the
# headline point of the throughput metric (every sequence at L = 32768).
TINY = Workload(
    name="tiny_l256", seed=0, mode="decode", num_seqs=1, seq_len=256,
    H_I=4, D_I=32, K=32, H=8, D_latent=64, D_rope=16,
    softmax_scale=1.0 / math.sqrt(80.0), dist="int8range")

DECODE_8K = Workload(
    name="decode_l8192", seed=1, mode="decode", num_seqs=1, seq_len=8192)

BATCHED_PAGED = Workload(
    name="batched_paged_64x4k_32k", seed=2, mode="decode", num_seqs=64, seq_len=None,
    len_range=(4096, 32768), paged=True)

PREFILL_64K = Workload(
    name="prefill_4096q_l65536", seed=3, mode="prefill", num_seqs=1, seq_len=65536,
    q_rows=4096)

FP8_LONG = Workload(
    name="fp8_decode_16x131072", seed=4, mode="decode", num_seqs=16, seq_len=131072,
    indexer_dtype="fp8", kv_dtype="fp8")

M32K_B64 = Workload(
    name="decode_paged_64x32768", seed=5, mode="decode", num_seqs=64, seq_len=32768,
    paged=True)

M32K_B1 = Workload(
    name="decode_paged_1x32768", seed=6, mode="decode", num_seqs=1, seq_len=32768,
    paged=True)

# The headline point with the pages' MXFP8 indexer (queries and keys e4m3 with
# one E8M0 scale per 32 elements; "Day0 ... for Kimi K3.1 Pro", section 4).
M32K_B64_MX = Workload(
    name="decode_paged_64x32768_mxfp8", seed=7, mode="decode", num_seqs=64, seq_len=32768,
    paged=True, indexer_dtype="mxfp8")

CONFIGS = [TINY, DECODE_8K, BATCHED_PAGED, PREFILL_64K, FP8_LONG]
# the same with the attention's latent cache in fp8 with one scale per
# 128-element tile of each row
M32K_B64_FP8KV = Workload(
    name="decode_paged_64x32768_fp8tilekv", seed=8, mode="decode", num_seqs=64, seq_len=32768,
    paged=True, kv_dtype="fp8_tile128")

BENCH = {w.name: w for w in CONFIGS + [M32K_B64, M32K_B1, M32K_B64_MX, M32K_B64_FP8KV]}


def get(name: str) -> Workload:
    if name in BENCH:
        return BENCH[name]
    aliases = {f"cfg{i}": w for i, w in enumerate(CONFIGS)}
    aliases.update({"m32k_b64": M32K_B64, "m32k_b1": M32K_B1})
    return aliases[name]
