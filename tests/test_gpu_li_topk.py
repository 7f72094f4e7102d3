"""li_topk: the fused score + Top-K step (decode rows scored and selected in
one launch, the scores kept on chip) against li_score followed by topk_select,
bit for bit, and against the oracle.

The fused kernel splits a row over up to 64 workgroups that select together:
the row's key range, up to three histogram levels, then either the whole
boundary bin, the tie rule (equal scores toward the lower position) or a
ranked list of the boundary bin's keys.  The cases reach each of these:

* Gaussian inputs (the boundary bin is ranked as a list);
* crafted scores: the queries and head weights are one-hot, so a row's score
  at a position is ReLU of one chosen key element (exact in fp32), and the
  cases put whole classes of equal or nearly equal scores across the K-th
  place: one value everywhere, three values, 128 values in one octave, the
  same with huge and tiny outliers that widen the key range, sums that need
  fp32's full mantissa, signed scores with +0.0 / -0.0;
* rows shorter than K, an empty row, rows of different lengths, holes in the
  block table (NaN scores), one row of 131072 positions over 64 workgroups,
  64 rows of 32768 (256 workgroups), many rows of one workgroup each, a shape
  that the fused launch does not take, and the bf16, per-token fp8 and MXFP8
  key formats.
"""
import numpy as np
import pytest
import torch

import indexer_selected_sparse_li_amd as lisfa
import oracle as O
import workloads as W
from gpu_util import batch_on_gpu, caches, check_index_set, gpu_scores, gpu_topk, say

pytestmark = pytest.mark.gpu


def both(b, K):
    """(li_topk result, li_score + topk_select result, inputs as numpy)."""
    kc, _ = caches(b)
    idx = torch.full((b.R, K), -7, dtype=torch.int32, device="cuda")
    lisfa.li_topk(b.q_idx, b.w, kc, b.row_seq, b.row_pos, K, idx, b.max_visible, q_scale=b.q_scale)
    torch.cuda.synchronize()
    ref = gpu_topk(gpu_scores(b), b.row_pos, K)
    return idx.cpu().numpy(), ref.cpu().numpy()


def decode_wl(B, L, K, H_I=64, D_I=128, dtype="bf16", paged=True, block_size=64, len_range=None, seed=11,
              dist="gauss"):
    return W.CONFIGS[1].with_(num_seqs=B, seq_len=None if len_range else L, len_range=len_range, K=K, H_I=H_I,
                              D_I=D_I, indexer_dtype=dtype, H=8, D_latent=64, D_rope=16, paged=paged,
                              block_size=block_size, seed=seed, dist=dist,
                              name=f"lt_{B}x{L}_{dtype}_{D_I}_{H_I}")


@pytest.mark.parametrize("B,L,K,H_I,D_I,dtype,paged,bs,lr", [
    (1, 32768, 2048, 64, 128, "bf16", True, 64, None),      # 32 workgroups on one row
    (64, 32768, 2048, 64, 128, "bf16", True, 64, None),     # 4 per row, 256 in all
    (2, 131072, 2048, 64, 128, "bf16", True, 64, None),     # 64 per row
    (3, 9000, 512, 24, 32, "bf16", False, 64, None),        # ragged last chunk, contiguous cache
    (5, None, 1024, 9, 128, "bf16", True, 16, (100, 20000)),  # mixed lengths, some shorter than K
    (300, 3000, 128, 64, 128, "bf16", True, 64, None),      # one workgroup per row, no exchange
    (200, 4000, 256, 64, 128, "bf16", True, 64, None),      # 400 workgroups: separate kernels
    (16, 32768, 2048, 64, 128, "mxfp8", True, 64, None),
    (16, 65536, 2048, 64, 128, "fp8", True, 64, None),
    (4, 20000, 2048, 32, 128, "mxfp8", False, 64, None),
])
def test_li_topk_matches_score_then_select(lib, B, L, K, H_I, D_I, dtype, paged, bs, lr):
    say(f"[case] li_topk B={B} L={L} K={K} H_I={H_I} D_I={D_I} {dtype} paged={paged} bs={bs} lens={lr}")
    b = batch_on_gpu(decode_wl(B, L, K, H_I, D_I, dtype, paged, bs, lr))
    got, ref = both(b, K)
    assert np.array_equal(got, ref)
    # the oracle on a few rows (fp32 scores: equal except within the band at the K-th place)
    inp = W.to_numpy(b)
    for r in sorted({0, b.R // 2, b.R - 1}):
        sc = O.scores_row(inp, r)
        check_index_set(got[r], sc, O.select_topk(sc, K), K)


def test_li_topk_short_and_empty_rows(lib):
    wl = decode_wl(6, 5000, 1024, 16, 128)
    b = batch_on_gpu(wl)
    b.row_pos = torch.tensor([4999, 1023, 1022, 0, -1, 3000], dtype=torch.int32, device="cuda")
    say("[case] li_topk rows of 5000, 1024, 1023, 1, 0 and 3001 positions, K 1024")
    got, ref = both(b, 1024)
    assert np.array_equal(got, ref)
    assert (got[4] == -1).all()
    assert np.array_equal(got[1], np.arange(1024))
    assert np.array_equal(got[2][:1023], np.arange(1023)) and got[2][1023] == -1
    assert got[3][0] == 0 and (got[3][1:] == -1).all()


def test_li_topk_block_table_holes(lib):
    """Positions whose block is unmapped score NaN (above +inf) in both paths."""
    b = batch_on_gpu(decode_wl(2, 32768, 2048, 64, 128))
    bt = b.block_table.clone()
    bt[0, 17] = -1
    bt[1, 3] = -1
    bt[1, 200] = -1
    b.block_table = bt
    say("[case] li_topk with unmapped blocks")
    got, ref = both(b, 2048)
    assert np.array_equal(got, ref)
    for r, blk in ((0, 17), (1, 3), (1, 200)):
        assert set(range(blk * 64, blk * 64 + 64)) <= set(got[r].tolist())


def crafted(B, L, K, kind, seed, D_I=32, block_size=64):
    """Scores = ReLU(k[s, 0]) (+ ReLU(k[s, 1]) for "fine", - for "signed"):
    one-hot queries and head weights, chosen key elements."""
    wl = decode_wl(B, L, K, H_I=4, D_I=D_I, block_size=block_size, seed=seed, dist="int8range")
    b = batch_on_gpu(wl)
    g = torch.Generator(device="cpu").manual_seed(seed + 5)
    R = b.R
    q = torch.zeros(R, 4, D_I)
    q[:, 0, 0] = 1.0
    q[:, 1, 1] = 1.0
    w = torch.zeros(R, 4)
    w[:, 0] = 1.0
    n = b.k_data.shape[0]
    v1 = torch.zeros(n)
    if kind == "const":
        v0 = torch.ones(n)
    elif kind == "ties3":
        u = torch.rand(n, generator=g)
        v0 = torch.where(u < 0.1, 4.0, torch.where(u < 0.4, 2.0, 1.0))
    elif kind in ("dense", "wide", "fine"):
        v0 = 1.0 + torch.randint(0, 128, (n,), generator=g).float() / 128
        if kind == "wide":
            u = torch.rand(n, generator=g)
            v0 = torch.where(u < 0.004, 2.0 ** 100, torch.where(u > 0.996, 2.0 ** -100, v0))
        if kind == "fine":
            v1 = torch.randint(0, 256, (n,), generator=g).float() * 2.0 ** -17
            w[:, 1] = 1.0
    elif kind == "signed":
        v0 = torch.randn(n, generator=g)
        v1 = torch.randn(n, generator=g)
        w[:, 1] = -1.0
    else:
        raise ValueError(kind)
    k = b.k_data.cpu().clone()
    k[:, 0] = v0.to(torch.bfloat16)
    k[:, 1] = v1.to(torch.bfloat16)
    b.k_data = k.cuda()
    b.q_idx = q.to(torch.bfloat16).cuda()
    b.w = w.cuda()
    return b


@pytest.mark.parametrize("kind", ["const", "ties3", "dense", "wide", "fine", "signed"])
@pytest.mark.parametrize("B,L,K", [(1, 32768, 2048), (4, 8192, 2048), (260, 2000, 256)])
def test_li_topk_crafted_scores(lib, kind, B, L, K):
    say(f"[case] li_topk crafted {kind} B={B} L={L} K={K}")
    b = crafted(B, L, K, kind, seed=B * 7 + L)
    got, ref = both(b, K)
    assert np.array_equal(got, ref)
    inp = W.to_numpy(b)
    for r in sorted({0, b.R - 1}):
        sc = O.scores_row(inp, r)
        want = O.select_topk(sc, K)
        if kind == "signed":   # differences of bf16 values round in fp32
            check_index_set(got[r], sc, want, K)
        else:                  # exact in fp32: the same set, ties included
            assert np.array_equal(got[r], want), f"row {r}"


@pytest.mark.parametrize("K", [1, 7, 300, 32000, 32767])
def test_li_topk_boundary_outside_the_first_range(lib, K):
    """The first histogram of a row split over workgroups bins a sample of the
    scores; with K this small or this large the K-th place lies above or below
    the sample's range, in a clamped edge bin, and the levels that follow
    refine it from there."""
    say(f"[case] li_topk 2 x 32768, K={K}")
    b = batch_on_gpu(decode_wl(2, 32768, K, 64, 128, seed=5))
    got, ref = both(b, K)
    assert np.array_equal(got, ref)
    inp = W.to_numpy(b)
    sc = O.scores_row(inp, 1)
    check_index_set(got[1], sc, O.select_topk(sc, K), K)


@pytest.mark.parametrize("K", [8, 130, 2048])
def test_li_topk_outliers_outside_the_sample(lib, K):
    """Huge and tiny outlier scores that a sample of each workgroup's first
    keys may miss (the first level's edge bins then hold them)."""
    say(f"[case] li_topk crafted wide, 2 x 32768, K={K}")
    b = crafted(2, 32768, K, "wide", seed=3)
    got, ref = both(b, K)
    assert np.array_equal(got, ref)
    inp = W.to_numpy(b)
    for r in range(2):
        assert np.array_equal(got[r], O.select_topk(O.scores_row(inp, r), K)), f"row {r}"
