"""Seeded synthetic inputs for the index-selection sparse attention layer.

This module is shared by the HIP path's tests/benchmark and by the CPU
oracle's tests: it only draws random numbers, rounds them to the stored
precisions and lays them out in the cache formats.  It contains none of the
layer's arithmetic (no scoring, selection or attention).

Recipe (fixed draw order): sequence lengths and block permutation (CPU
generator, so shapes never depend on the device), then on the target
device's generator: indexer keys, latent cache rows, indexer queries, head
weight logits, MLA queries.

* "int8range": every q/k/latent value is an integer drawn uniformly from
  [-8, 8] and stored as bf16 (exact); head weights are k/16 for k drawn
  uniformly from {0..16}.
* "gauss": indexer q/k ~ N(0,1); head weights = softmax over heads of N(0,1)
  logits (computed in float64, stored float32); latent rows
  ~ N(0,1)/sqrt(D_latent + D_rope); MLA queries ~ N(0, q_mla_std^2).

fp8 storage (OCP e4m3, max 448) uses amax/448 scales (1 when amax is 0):
indexer keys one scale per token, indexer queries one scale per query token
(over all heads), latent rows one scale per group of kv_scale_group
consecutive physical slots, or (kv_dtype "fp8_tile128") one scale per tile of
128 elements of each row (integer inputs: the power-of-two scales 1/2, 1, 2
in turn over the tiles, so every value stays exact).  The quantisation is part of input preparation:
both the kernels and the oracle consume the stored codes and scales.

Paged layout: blocks of block_size tokens; the physical block ids are a
random permutation of all blocks, dealt to the sequences in order; unused
slots of the last block of each sequence hold NaN so that any read of them
poisons a result.  Contiguous layout: sequence b starts at seq_base[b]
(multiples of block_size); the gaps hold NaN as well.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

from .configs import Workload

BF16_NAN_BITS = 0x7FC0
E4M3_NAN_BITS = 0x7F
E4M3_MAX = 448.0


@dataclasses.dataclass
class Batch:
    wl: Workload
    device: torch.device
    seq_lens: List[int]
    # query side
    q_idx: torch.Tensor                 # [R, H_I, D_I] bf16, or uint8 e4m3 codes
    q_scale: Optional[torch.Tensor]     # [R] fp32 (fp8 indexer only)
    w: torch.Tensor                     # [R, H_I] fp32
    q: torch.Tensor                     # [R, H, D_qk] bf16
    row_seq: torch.Tensor               # [R] int32
    row_pos: torch.Tensor               # [R] int32
    # caches (shared slot space for the indexer keys and the latent rows)
    num_slots: int
    k_data: torch.Tensor                # [num_slots, D_I] bf16 / uint8
    k_scale: Optional[torch.Tensor]     # [num_slots] fp32
    kv_data: torch.Tensor               # [num_slots, D_qk] bf16 / uint8
    kv_scale: Optional[torch.Tensor]    # [num_slots // kv_scale_group] fp32, or [num_slots, ceil(D_qk / 128)]
                                        # for fp8_tile128
    block_table: Optional[torch.Tensor]  # [num_seqs, bt_stride] int32 (paged)
    seq_base: Optional[torch.Tensor]    # [num_seqs] int64 (contiguous)

    @property
    def R(self) -> int:
        return int(self.row_pos.shape[0])

    @property
    def max_visible(self) -> int:
        return max(self.seq_lens)


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def quantize_e4m3(x: torch.Tensor, dim) -> (torch.Tensor, torch.Tensor):
    """Per-group amax/448 scaling, then round-to-nearest-even e4m3 codes."""
    amax = x.abs().amax(dim=dim, keepdim=True).to(torch.float32)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x.to(torch.float32) / scale).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


KV_TILE = 128   # elements per scale tile of the tile-scaled fp8 latent cache


def quantize_tiles(x: torch.Tensor, tile: int, exact_pow2: bool = False) -> (torch.Tensor, torch.Tensor):
    """Rows x [n, W] -> e4m3 codes [n, W] and fp32 scales [n, ceil(W / tile)],
    one per tile of `tile` columns: amax/448 (1 for an all-zero tile), or with
    exact_pow2 the scales 1/2, 1, 2 in turn over the tiles (for integer-valued
    rows, whose quotients stay exact in e4m3)."""
    n, W = x.shape
    nt = (W + tile - 1) // tile
    xf = x.to(torch.float32)
    pad = nt * tile - W
    xp = torch.cat([xf, torch.zeros(n, pad, device=x.device)], dim=1) if pad else xf
    g = xp.view(n, nt, tile)
    if exact_pow2:
        sc = torch.tensor([0.5, 1.0, 2.0], device=x.device)[torch.arange(nt, device=x.device) % 3]
        sc = sc.view(1, nt, 1).expand(n, nt, 1).contiguous()
    else:
        amax = g.abs().amax(dim=2, keepdim=True)
        sc = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (g / sc).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).view(n, nt * tile)[:, :W].contiguous()
    return codes, sc.view(n, nt)


def quantize_mx(x: torch.Tensor, block: int = 32) -> (torch.Tensor, torch.Tensor):
    """MXFP8 (OCP MX): per block of 32 consecutive elements of the last dim,
    shared exponent floor(log2(amax)) - 8 clamped to [-127, 127] (0 for an
    all-zero block); elements x / 2^shared saturated to +-448 and rounded to
    e4m3 (nearest even).  Returns (e4m3 codes, E8M0 scale bytes)."""
    shape = x.shape
    g = x.to(torch.float32).reshape(*shape[:-1], shape[-1] // block, block)
    amax = g.abs().amax(dim=-1)
    _, e = torch.frexp(amax)
    shared = torch.where(amax > 0, e - 9, torch.zeros_like(e)).clamp(-127, 127)
    y = (g / torch.ldexp(torch.ones_like(amax), shared)[..., None]).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(shape)
    return codes, (shared + 127).to(torch.uint8)


def _values(wl: Workload, shape, gen, device, std=1.0) -> torch.Tensor:
    if wl.dist == "int8range":
        return torch.randint(-8, 9, shape, generator=gen, device=device).to(torch.float32)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x * std if std != 1.0 else x


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    raise ValueError(dtype)


def make_batch(wl: Workload, device="cpu", chunk_tokens: int = 1 << 16) -> Batch:
    device = torch.device(device)
    cpu_gen = torch.Generator(device="cpu").manual_seed(wl.seed)
    dev_gen = torch.Generator(device=device).manual_seed(wl.seed + 1000003)

    # 1. lengths
    if wl.seq_len is not None:
        seq_lens = [wl.seq_len] * wl.num_seqs
    else:
        lo, hi = wl.len_range
        seq_lens = torch.randint(lo, hi + 1, (wl.num_seqs,), generator=cpu_gen).tolist()

    bs = wl.block_size
    nblk = [_round_up(L, bs) // bs for L in seq_lens]
    total_blocks = sum(nblk)
    num_slots = total_blocks * bs

    # 2. layout: slot of every (sequence, position)
    block_table = seq_base = None
    if wl.paged:
        perm = torch.randperm(total_blocks, generator=cpu_gen).to(torch.int32)
        bt_stride = max(nblk)
        bt = torch.full((wl.num_seqs, bt_stride), -1, dtype=torch.int32)
        off = 0
        for b, n in enumerate(nblk):
            bt[b, :n] = perm[off:off + n]
            off += n
        block_table = bt
    else:
        bases, off = [], 0
        for n in nblk:
            bases.append(off * bs)
            off += n
        seq_base = torch.tensor(bases, dtype=torch.int64)

    def slots_of(b: int, p0: int, p1: int) -> torch.Tensor:
        pos = torch.arange(p0, p1, dtype=torch.int64)
        if wl.paged:
            return block_table[b, pos // bs].to(torch.int64) * bs + pos % bs
        return seq_base[b] + pos

    fp8_idx = wl.indexer_dtype == "fp8"
    mx_idx = wl.indexer_dtype == "mxfp8"
    fp8_kv = wl.kv_dtype == "fp8"
    tile_kv = wl.kv_dtype == "fp8_tile128"

    # 3. indexer keys
    if mx_idx:
        k_data = torch.full((num_slots, wl.D_I), E4M3_NAN_BITS, dtype=torch.uint8, device=device)
        k_scale = torch.full((num_slots, wl.D_I // 32), 255, dtype=torch.uint8, device=device)
    elif fp8_idx:
        k_data = torch.full((num_slots, wl.D_I), E4M3_NAN_BITS, dtype=torch.uint8, device=device)
        k_scale = torch.full((num_slots,), float("nan"), dtype=torch.float32, device=device)
    else:
        k_data = torch.full((num_slots, wl.D_I), BF16_NAN_BITS, dtype=torch.int16,
                            device=device).view(torch.bfloat16)
        k_scale = None
    for b, L in enumerate(seq_lens):
        for p0 in range(0, L, chunk_tokens):
            p1 = min(L, p0 + chunk_tokens)
            sl = slots_of(b, p0, p1).to(device)
            x = _values(wl, (p1 - p0, wl.D_I), dev_gen, device)
            if mx_idx:
                codes, sc = quantize_mx(x)
                k_data[sl] = codes
                k_scale[sl] = sc
            elif fp8_idx:
                if wl.dist == "int8range":
                    codes = x.to(torch.float8_e4m3fn).view(torch.uint8)
                    sc = torch.ones(p1 - p0, 1, device=device)
                else:
                    codes, sc = quantize_e4m3(x, dim=1)
                k_data[sl] = codes
                k_scale[sl] = sc[:, 0]
            else:
                k_data[sl] = _store(x, "bf16")

    # 4. latent cache rows
    D_qk = wl.D_qk
    kv_std = 1.0 / math.sqrt(D_qk)
    g = wl.kv_scale_group
    if fp8_kv:
        if wl.paged:
            assert bs % g == 0
        kv_data = torch.full((num_slots, D_qk), E4M3_NAN_BITS, dtype=torch.uint8, device=device)
        kv_scale = torch.full((num_slots // g,), float("nan"), dtype=torch.float32, device=device)
    elif tile_kv:
        n_tiles = (D_qk + KV_TILE - 1) // KV_TILE
        kv_data = torch.full((num_slots, D_qk), E4M3_NAN_BITS, dtype=torch.uint8, device=device)
        kv_scale = torch.full((num_slots, n_tiles), float("nan"), dtype=torch.float32, device=device)
    else:
        kv_data = torch.full((num_slots, D_qk), BF16_NAN_BITS, dtype=torch.int16,
                             device=device).view(torch.bfloat16)
        kv_scale = None
    kv_chunk = _round_up(max(g, chunk_tokens // 4), bs)
    for b, L in enumerate(seq_lens):
        for p0 in range(0, L, kv_chunk):
            p1 = min(L, p0 + kv_chunk)
            sl = slots_of(b, p0, p1).to(device)
            x = _values(wl, (p1 - p0, D_qk), dev_gen, device,
                        std=kv_std if wl.dist == "gauss" else 1.0)
            if fp8_kv:
                # one scale per group of g consecutive positions (groups never
                # straddle sequences because sequence starts are block aligned)
                n = p1 - p0
                ng = (n + g - 1) // g
                pad = ng * g - n
                xp = torch.cat([x, torch.zeros(pad, D_qk, device=device)]) if pad else x
                xg = xp.view(ng, g, D_qk)
                if wl.dist == "int8range":
                    codes = xg.to(torch.float8_e4m3fn).view(torch.uint8)
                    sc = torch.ones(ng, 1, 1, device=device)
                else:
                    codes, sc = quantize_e4m3(xg, dim=(1, 2))
                kv_data[sl] = codes.view(ng * g, D_qk)[:n]
                kv_scale[(sl[::g] // g)] = sc.view(ng)
            elif tile_kv:
                codes, sc = quantize_tiles(x, KV_TILE, wl.dist == "int8range")
                kv_data[sl] = codes
                kv_scale[sl] = sc
            else:
                kv_data[sl] = _store(x, "bf16")

    # 5. query rows
    if wl.mode == "decode":
        row_seq = torch.arange(wl.num_seqs, dtype=torch.int32)
        row_pos = torch.tensor([L - 1 for L in seq_lens], dtype=torch.int32)
    else:
        L = seq_lens[0]
        row_seq = torch.zeros(wl.q_rows, dtype=torch.int32)
        row_pos = torch.arange(L - wl.q_rows, L, dtype=torch.int32)
    R = int(row_pos.shape[0])

    xq = _values(wl, (R, wl.H_I, wl.D_I), dev_gen, device)
    if mx_idx:
        q_idx, q_scale = quantize_mx(xq)
    elif fp8_idx:
        if wl.dist == "int8range":
            q_idx = xq.to(torch.float8_e4m3fn).view(torch.uint8)
            q_scale = torch.ones(R, dtype=torch.float32, device=device)
        else:
            q_idx, sc = quantize_e4m3(xq, dim=(1, 2))
            q_scale = sc.view(R)
    else:
        q_idx = _store(xq, "bf16")
        q_scale = None

    # 6. head weights
    if wl.dist == "int8range":
        w = torch.randint(0, 17, (R, wl.H_I), generator=dev_gen, device=device).to(torch.float32) / 16.0
    else:
        logits = torch.randn((R, wl.H_I), generator=dev_gen, device=device, dtype=torch.float32)
        w = torch.softmax(logits.to(torch.float64), dim=1).to(torch.float32)

    # 7. MLA queries (in row chunks to bound the float32 temporary)
    q = torch.empty((R, wl.H, D_qk), dtype=torch.bfloat16, device=device)
    rchunk = max(1, (1 << 24) // (wl.H * D_qk))
    for r0 in range(0, R, rchunk):
        r1 = min(R, r0 + rchunk)
        q[r0:r1] = _store(_values(wl, (r1 - r0, wl.H, D_qk), dev_gen, device,
                                  std=wl.q_mla_std), "bf16")

    to = lambda t: None if t is None else t.to(device)
    return Batch(wl=wl, device=device, seq_lens=seq_lens,
                 q_idx=q_idx, q_scale=q_scale, w=w, q=q,
                 row_seq=row_seq.to(device), row_pos=row_pos.to(device),
                 num_slots=num_slots, k_data=k_data, k_scale=k_scale,
                 kv_data=kv_data, kv_scale=kv_scale,
                 block_table=to(block_table), seq_base=to(seq_base))


def make_scores(rows: int, cols: int, kind: str, seed: int, device="cpu") -> torch.Tensor:
    """Synthetic fp32 score matrices for testing the selector on its own.

    kinds: "gauss" (continuous), "ties" (a handful of distinct values),
    "signed_zero" (+0.0 / -0.0 / small integers), "const" (all equal),
    "int" (integers in [-1000, 1000]), "extreme" (mix of +-inf, huge and tiny
    magnitudes, denormals).
    """
    gen = torch.Generator(device="cpu").manual_seed(seed)
    if kind == "gauss":
        x = torch.randn(rows, cols, generator=gen)
    elif kind == "ties":
        x = torch.randint(0, 5, (rows, cols), generator=gen).to(torch.float32) * 0.25
    elif kind == "signed_zero":
        v = torch.randint(-2, 3, (rows, cols), generator=gen).to(torch.float32)
        neg = torch.randint(0, 2, (rows, cols), generator=gen).bool()
        x = torch.where((v == 0) & neg, torch.full_like(v, -0.0), v)
    elif kind == "const":
        x = torch.full((rows, cols), 0.5)
    elif kind == "int":
        x = torch.randint(-1000, 1001, (rows, cols), generator=gen).to(torch.float32)
    elif kind == "extreme":
        pool = torch.tensor([float("inf"), float("-inf"), 3.0e38, -3.0e38, 1e-45, -1e-45,
                             1e-40, 0.0, -0.0, 1.0, -1.0, 2.0], dtype=torch.float32)
        x = pool[torch.randint(0, len(pool), (rows, cols), generator=gen)]
        x = x + torch.where(torch.rand(rows, cols, generator=gen) < 0.5,
                            torch.randn(rows, cols, generator=gen), torch.zeros(rows, cols))
    else:
        raise ValueError(kind)
    return x.to(torch.float32).contiguous().to(device)


def to_numpy(batch: Batch) -> Dict[str, object]:
    """Raw stored values as numpy arrays (bf16 as uint16 bit patterns,
    e4m3 as uint8 codes) plus the layout and scalars: the oracle's input."""
    def bits(t):
        if t is None:
            return None
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    wl = batch.wl
    return dict(
        H_I=wl.H_I, D_I=wl.D_I, K=wl.K, H=wl.H, D_latent=wl.D_latent, D_rope=wl.D_rope,
        softmax_scale=wl.softmax_scale, indexer_dtype=wl.indexer_dtype, kv_dtype=wl.kv_dtype,
        block_size=wl.block_size, kv_scale_group=wl.kv_scale_group,
        q_idx=bits(batch.q_idx), q_scale=bits(batch.q_scale), w=bits(batch.w), q=bits(batch.q),
        row_seq=bits(batch.row_seq), row_pos=bits(batch.row_pos),
        k_data=bits(batch.k_data), k_scale=bits(batch.k_scale),
        kv_data=bits(batch.kv_data), kv_scale=bits(batch.kv_scale),
        block_table=bits(batch.block_table), seq_base=bits(batch.seq_base),
        seq_lens=list(batch.seq_lens),
    )
