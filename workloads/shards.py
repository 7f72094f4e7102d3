"""Input layouts of a context-parallel split (no arithmetic of the method).

With context parallelism every GPU holds a contiguous range of each
sequence's cached positions.  On one GPU the shards are views of the same
cache pools: shard g of sequence b covers logical positions [lo, hi), a
whole number of 64-token blocks, and its own cache addresses them as local
positions 0..hi-lo-1 (a paged cache through a block table shifted by lo/64
blocks, a contiguous one through seq_base + lo).  This module only builds
those index arrays; the kernels never see anything but a cache and rows.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np
import torch

from .generate import Batch


def context_shards(b: Batch, G: int, align: int = 64) -> List[Dict[str, object]]:
    """Split every sequence of the batch into G contiguous shards of
    ceil(L / (G * align)) * align positions (the last ones may be short or
    empty).  Per shard: block_table or seq_base of its local caches, and per
    query row its range [lo, hi), local visible count and local row_pos."""
    L = [int(x) for x in b.seq_lens]
    S = [-(-Lb // (G * align)) * align for Lb in L]
    rs = b.row_seq.cpu().numpy().astype(np.int64)
    rp = b.row_pos.cpu().numpy().astype(np.int64)
    dev = b.row_pos.device
    out = []
    for g in range(G):
        lo = [min(g * Sb, Lb) for Sb, Lb in zip(S, L)]
        hi = [min((g + 1) * Sb, Lb) for Sb, Lb in zip(S, L)]
        block_table = seq_base = None
        if b.block_table is not None:
            bt = b.block_table.cpu()
            btl = torch.zeros_like(bt)
            for s in range(len(L)):
                nb = -(-(hi[s] - lo[s]) // align)
                btl[s, :nb] = bt[s, lo[s] // align: lo[s] // align + nb]
            block_table = btl.to(dev)
        else:
            seq_base = b.seq_base + torch.tensor(lo, dtype=torch.int64, device=b.seq_base.device)
        lo_r = np.array([lo[s] for s in rs], dtype=np.int64)
        hi_r = np.array([hi[s] for s in rs], dtype=np.int64)
        vis = np.clip(rp + 1 - lo_r, 0, hi_r - lo_r)
        out.append(dict(
            block_table=block_table, seq_base=seq_base, lo=lo_r, hi=hi_r,
            row_pos=torch.tensor(vis - 1, dtype=torch.int32, device=dev),
            pos_offset=torch.tensor(lo_r, dtype=torch.int32, device=dev),
            range=torch.tensor(np.stack([lo_r, hi_r], 1), dtype=torch.int32, device=dev),
            max_vis=int(vis.max()) if vis.size else 0))
    return out
