"""CPU oracle of the context-parallel pieces of the sparse attention layer.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it.  Plain NumPy
in float64; shares nothing with the HIP library.

Context parallelism splits the cached positions of a sequence over several
GPUs ("Day0 Inference Adaptation and Performance Optimization for Kimi K3.1
Pro", section 5; the Kimi K3 decode article in Japanese, part 1 item 1: with
decode context parallelism every GPU holds a region of the KV cache,
attends over its own region, and a fused kernel merges the partial results).
For the index-selection layer this makes three steps per shard plus one
merge, each written here in its plainest form:

1. shard_candidates: the shard scores its own positions and keeps its local
   Top-K, as (global position, score) pairs.  Every globally selected
   position is among its own shard's local Top-K, because a position's rank
   inside its shard can only be lower than its rank in the whole row.
2. merge_candidates: the K best of the gathered candidates under the same
   order as the single-GPU selection (larger score first, equal scores to the
   lower position).
3. attention of the shard's selected rows: ordinary sparse attention over the
   selected positions that the shard holds (the oracle's sparse_mla on that
   subset), giving a normalised output and its log-sum-exp.
4. combine_partials: softmax attention over a union of disjoint row sets is
   the log-sum-exp weighted mean of the per-set results:
       M = max_g lse_g,  a_g = exp(lse_g - M),
       out = sum_g a_g out_g / sum_g a_g,  lse = M + log(sum_g a_g).

Prefill uses the Zigzag partition ("Day0 Inference Adaptation and
Performance Optimization for a New Model", section 5.2, and the Kimi K3.1
Pro page, section 5): the sequence is cut into 2G equal segments and GPU g
takes segment g and segment 2G-1-g, pairing a short-history segment with a
long-history one; after the computation the rows are put back in their
original order.  The pages show only the 8-segment, 2-GPU example; segment
boundaries for lengths not divisible by 2G are taken here as
floor(i * n / (2G)) (a reading: the pages say nothing about ragged lengths).
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from .lisfa_oracle import select_topk


def shard_candidates(local_scores: np.ndarray, K: int, pos_offset: int) -> Tuple[np.ndarray, np.ndarray]:
    """Local Top-K of one shard: local_scores[t] is the score of global
    position pos_offset + t.  Returns (positions, scores), K entries each,
    positions ascending, padded with (-1, -inf)."""
    local = select_topk(np.asarray(local_scores, dtype=np.float64), K)
    pos = np.full(K, -1, dtype=np.int64)
    sc = np.full(K, -np.inf)
    m = local >= 0
    pos[m] = local[m] + int(pos_offset)
    sc[m] = np.asarray(local_scores, dtype=np.float64)[local[m]]
    return pos, sc


def merge_candidates(cand_scores: np.ndarray, cand_pos: np.ndarray, K: int) -> np.ndarray:
    """The K best candidates (position < 0 = no candidate), larger score
    first and equal scores toward the lower position; ascending positions,
    -1 padded to K.  The candidates may come in any order."""
    s = np.asarray(cand_scores, dtype=np.float64).ravel()
    p = np.asarray(cand_pos, dtype=np.int64).ravel()
    m = p >= 0
    s, p = s[m], p[m]
    # primary key: larger score (-s ascending; -0.0 == +0.0), secondary: lower position
    order = np.lexsort((p, -s))
    take = np.sort(p[order[:K]])
    out = np.full(K, -1, dtype=np.int64)
    out[:take.shape[0]] = take
    return out


def combine_partials(outs: np.ndarray, lses: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """outs [G, H, D] normalised partial outputs, lses [G, H] natural-log
    normalisers (-inf = the part had no row).  Returns (out [H, D], lse [H]);
    a head with no row in any part gets out = 0 and lse = -inf."""
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    G, H, D = outs.shape
    out = np.zeros((H, D))
    lse = np.full(H, -np.inf)
    for h in range(H):
        M = lses[:, h].max()
        if M == -np.inf:
            continue
        a = np.exp(lses[:, h] - M)
        out[h] = (a[:, None] * outs[:, h, :]).sum(axis=0) / a.sum()
        lse[h] = M + np.log(a.sum())
    return out, lse


def zigzag_segments(n: int, G: int) -> List[Tuple[int, int]]:
    """The 2G segments [start, end) of a length-n sequence."""
    return [(i * n // (2 * G), (i + 1) * n // (2 * G)) for i in range(2 * G)]


def zigzag_share(n: int, G: int, g: int) -> List[Tuple[int, int]]:
    """The two segments GPU g of G takes: segment g, then segment 2G-1-g."""
    seg = zigzag_segments(n, G)
    return [seg[g], seg[2 * G - 1 - g]]


def zigzag_order(n: int, G: int) -> np.ndarray:
    """Original positions in gathered order: GPU 0's two segments, then GPU
    1's, ... (what an all-gather of the shares holds)."""
    parts = []
    for g in range(G):
        for a, b in zigzag_share(n, G, g):
            parts.append(np.arange(a, b, dtype=np.int64))
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def zigzag_restore(gathered: np.ndarray, G: int) -> np.ndarray:
    """Rows in gathered order -> rows in original order."""
    gathered = np.asarray(gathered)
    n = gathered.shape[0]
    out = np.empty_like(gathered)
    out[zigzag_order(n, G)] = gathered
    return out
