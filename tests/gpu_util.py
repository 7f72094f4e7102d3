"""Glue for the GPU parity tests: run the HIP path through the binding on a
seeded batch, and compare with the oracle under the stated rules."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import indexer_selected_sparse_li_amd as lisfa
import oracle as O
import workloads as W

BF16_ATOL, BF16_RTOL, BF16_NORM = 2e-2, 1e-2, 1e-2
FP8_ATOL, FP8_RTOL, FP8_NORM = 5e-2, 1e-2, 5e-2
BAND_REL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def batch_on_gpu(wl: W.Workload, gen_device: str = "cpu") -> W.Batch:
    b = W.make_batch(wl, device=gen_device)
    if gen_device == "cpu":
        for f in ("q_idx", "q_scale", "w", "q", "row_seq", "row_pos", "k_data", "k_scale", "kv_data",
                  "kv_scale", "block_table", "seq_base"):
            t = getattr(b, f)
            if t is not None:
                setattr(b, f, t.cuda())
        b.device = torch.device("cuda")
    return b


def caches(b: W.Batch):
    wl = b.wl
    kc = lisfa.KVCache(data=b.k_data, scale=b.k_scale, scale_group=1, block_table=b.block_table,
                       block_size=wl.block_size, seq_base=b.seq_base)
    vc = lisfa.KVCache(data=b.kv_data, scale=b.kv_scale, scale_group=wl.kv_scale_group,
                       block_table=b.block_table, block_size=wl.block_size, seq_base=b.seq_base)
    return kc, vc


def rows_per_group(b: W.Batch) -> int:
    if b.wl.mode != "prefill":
        return 1
    return 16 if b.R % 16 == 0 else 8 if b.R % 8 == 0 else 1


def gpu_scores(b: W.Batch, ld: int = None) -> torch.Tensor:
    kc, _ = caches(b)
    ld = ld or (b.max_visible + 63) // 64 * 64
    scores = torch.full((b.R, ld), float("nan"), dtype=torch.float32, device="cuda")
    lisfa.li_score(b.q_idx, b.w, kc, b.row_seq, b.row_pos, scores, b.max_visible, q_scale=b.q_scale,
                   rows_per_group=rows_per_group(b))
    torch.cuda.synchronize()
    return scores


def gpu_topk(scores: torch.Tensor, row_pos: torch.Tensor, K: int) -> torch.Tensor:
    idx = torch.full((scores.shape[0], K), -7, dtype=torch.int32, device="cuda")
    lisfa.topk_select(scores, row_pos, K, idx)
    torch.cuda.synchronize()
    return idx


def gpu_sfa(b: W.Batch, idx: torch.Tensor):
    _, vc = caches(b)
    wl = b.wl
    out = torch.full((b.R, wl.H, wl.D_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((b.R, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    lisfa.sparse_mla_attn(b.q, vc, b.row_seq, idx, out, lse, softmax_scale=wl.softmax_scale)
    torch.cuda.synchronize()
    return out, lse


def gpu_fused(b: W.Batch, K: int = None):
    kc, vc = caches(b)
    wl = b.wl
    K = K or wl.K
    out = torch.full((b.R, wl.H, wl.D_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((b.R, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((b.R, K), -7, dtype=torch.int32, device="cuda")
    lisfa.li_topk_sfa(b.q_idx, b.w, kc, b.q, vc, b.row_seq, b.row_pos, K, b.max_visible, out, lse,
                      idx_out=idx, q_scale=b.q_scale, rows_per_group=rows_per_group(b),
                      softmax_scale=wl.softmax_scale)
    torch.cuda.synchronize()
    return idx, out, lse


def score_bound(inp, r: int) -> np.ndarray:
    """Forward error bound of an fp32 evaluation of the score with exact
    products: gamma_n * sum_j |w_j| sum_d |q_jd k_d|, n = D_I + H_I + 4, unit
    roundoff 2^-23 (covers any rounding mode), times 2 for safety."""
    seq = int(inp["row_seq"][r])
    n = int(inp["row_pos"][r]) + 1
    q = np.abs(O.indexer_query(inp, r))
    k = np.abs(O.indexer_keys(inp, seq, n))
    w = np.abs(inp["w"][r].astype(np.float64))
    nn = inp["D_I"] + inp["H_I"] + 4
    u = 2.0 ** -23
    gamma = nn * u / (1 - nn * u)
    return 2.0 * gamma * ((k @ q.T) @ w) + 1e-30


def check_index_set(gpu_idx: np.ndarray, oracle_scores: np.ndarray, oracle_idx: np.ndarray, K: int):
    """Equal except for positions whose oracle scores lie within BAND_REL
    (relative) of the oracle's K-th largest score."""
    g = [int(x) for x in gpu_idx if x >= 0]
    o = [int(x) for x in oracle_idx if x >= 0]
    assert len(g) == len(o), (len(g), len(o))
    assert g == sorted(g) and len(set(g)) == len(g), "not ascending/unique"
    assert all(x == -1 for x in gpu_idx[len(g):]), "bad -1 padding"
    if len(o) < K:  # everything visible is kept
        assert g == o
        return 0
    sstar = np.sort(oracle_scores)[::-1][K - 1]
    diff = set(g) ^ set(o)
    band = abs(sstar) * BAND_REL
    bad = [p for p in diff if abs(oracle_scores[p] - sstar) > band]
    assert not bad, f"{len(bad)} positions outside the tie band, e.g. {bad[:5]}"
    return len(diff)


def check_out(gpu_out: np.ndarray, ref: np.ndarray, fp8: bool, label: str = ""):
    atol, rtol, norm = (FP8_ATOL, FP8_RTOL, FP8_NORM) if fp8 else (BF16_ATOL, BF16_RTOL, BF16_NORM)
    err = np.abs(gpu_out - ref)
    assert np.isfinite(gpu_out).all(), f"{label}: non-finite output"
    assert (err <= atol + rtol * np.abs(ref)).all(), f"{label}: max abs err {err.max()}"
    scale = np.abs(ref).max()
    if scale > 0:
        assert err.max() / scale <= norm, f"{label}: normalised err {err.max() / scale}"
    return float(err.max()), float(err.max() / scale if scale > 0 else 0.0)


def check_lse(gpu_lse: np.ndarray, ref: np.ndarray, label: str = ""):
    fin = np.isfinite(ref)
    assert (np.isfinite(gpu_lse) == fin).all(), f"{label}: lse finiteness differs"
    err = np.abs(gpu_lse[fin] - ref[fin])
    assert (err <= 1e-3 + 1e-3 * np.abs(ref[fin])).all(), f"{label}: lse err {err.max()}"
    assert (gpu_lse[~fin] == ref[~fin]).all()
