"""Every kernel variant the C ABI can reach, each against the oracle.

The entry points pick a kernel from the shapes and formats of their arguments
(indexer dtype x head dim x head count x row grouping; attention latent shape
x cache format x head count x index entries per workgroup).  These cases walk
that whole table at small sizes, so no variant ships without a parity check:

* li_score on integer-valued inputs: scores bit-exact against the oracle for
  bf16 / per-token fp8 / MXFP8 keys, D_I 32 and 128, 9 / 24 / 64 heads (the
  three head-tile counts) and row groups of 1, 8 and 16;
* sparse_mla_attn on given index lists (random subsets with -1 padding, a row
  with no entry): 512+64 and 64+16 rows in bf16, per-64-token fp8 and
  tile-scaled fp8, head counts on both sides of the 32- and 64-head block
  sizes, with few rows (split index lists and the LSE combine) and with many
  rows (one workgroup per 2048 entries);
* li_topk_sfa on a prefill batch of two sequences that the fused call must cut
  into row chunks, with 16-row groups.
"""
import math

import numpy as np
import pytest
import torch

import indexer_selected_sparse_li_amd as lisfa
import oracle as O
import workloads as W
from gpu_util import batch_on_gpu, caches, check_index_set, check_lse, check_out, say

pytestmark = pytest.mark.gpu


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


# ------------------------------------------------------------- li_score ---

@pytest.mark.parametrize("rpg", [1, 8, 16])
@pytest.mark.parametrize("H_I", [9, 24, 64])
# MXFP8 keys are defined for D_I = 128 only (the ABI refuses other widths)
@pytest.mark.parametrize("dtype,D_I", [("bf16", 32), ("bf16", 128), ("fp8", 32), ("fp8", 128), ("mxfp8", 128)])
def test_li_score_variants_bit_exact(lib, dtype, D_I, H_I, rpg):
    wl = W.CONFIGS[3].with_(seq_len=1100, q_rows=48, H_I=H_I, D_I=D_I, indexer_dtype=dtype, H=8, D_latent=64,
                            D_rope=16, K=64, dist="int8range", paged=True, block_size=32,
                            name=f"li_{dtype}_{D_I}_{H_I}_{rpg}")
    say(f"[case] li_score {dtype} D_I={D_I} H_I={H_I} rows_per_group={rpg}")
    b = batch_on_gpu(wl)
    kc, _ = caches(b)
    ld = (b.max_visible + 63) // 64 * 64 + 64
    sc = torch.full((b.R, ld), float("nan"), dtype=torch.float32, device="cuda")
    lisfa.li_score(b.q_idx, b.w, kc, b.row_seq, b.row_pos, sc, b.max_visible, q_scale=b.q_scale,
                   rows_per_group=rpg)
    torch.cuda.synchronize()
    got = _np(sc)
    inp = W.to_numpy(b)
    for r in range(b.R):
        n = int(inp["row_pos"][r]) + 1
        ref = O.scores_row(inp, r)
        assert np.array_equal(got[r, :n].astype(np.float64), ref), f"row {r}"
        assert np.isnan(got[r, n:]).all(), f"row {r}: entries past the row's position were written"


# ------------------------------------------------------ sparse_mla_attn ---

def _mla_batch(D_latent, D_rope, kv, H, R, L, nseq, seed, paged=True):
    """A cache of nseq sequences of length L and R query rows over them, with
    sharp MLA queries (logit std about 3) so the softmax is far from uniform."""
    D_qk = D_latent + D_rope
    wl = W.CONFIGS[1].with_(num_seqs=nseq, seq_len=L, H=H, D_latent=D_latent, D_rope=D_rope, kv_dtype=kv,
                            softmax_scale=1.0 / math.sqrt(D_qk), H_I=4, D_I=32, paged=paged, seed=seed,
                            name=f"mla_{D_latent}_{kv}_{H}")
    b = batch_on_gpu(wl)
    g = torch.Generator(device="cpu").manual_seed(seed + 17)
    std = 3.0 * math.sqrt(D_qk)
    b.q = (torch.randn(R, H, D_qk, generator=g) * std).to(torch.bfloat16).cuda()
    b.row_seq = (torch.arange(R, dtype=torch.int32) % nseq).cuda()
    b.row_pos = torch.full((R,), L - 1, dtype=torch.int32).cuda()
    return b


def _index_lists(R, K, L, seed):
    """Row r: a random sorted subset of [0, L) of size K - (r % 3) * 37 (at
    least 1), -1 padded; row 1 (when R > 1) selects nothing."""
    g = np.random.default_rng(seed)
    idx = np.full((R, K), -1, dtype=np.int32)
    for r in range(R):
        n = max(1, min(L, K - (r % 3) * 37))
        if R > 1 and r == 1:
            continue
        idx[r, :n] = np.sort(g.choice(L, size=n, replace=False))
    return idx


def _check_mla(b, idx_np, rows, fp8, label):
    idx = torch.from_numpy(idx_np).cuda()
    _, vc = caches(b)
    R, H, _ = b.q.shape
    D_v = b.wl.D_v
    out = torch.full((R, H, D_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda")
    lisfa.sparse_mla_attn(b.q, vc, b.row_seq, idx, out, lse, softmax_scale=b.wl.softmax_scale)
    torch.cuda.synchronize()
    out, lse = _np(out), _np(lse)
    inp = W.to_numpy(b)
    worst = 0.0
    for r in rows:
        ref_out, ref_lse = O.attend_row(inp, r, idx_np[r])
        e = check_out(out[r], ref_out, fp8, f"{label} row {r}")
        check_lse(lse[r], ref_lse, f"{label} row {r}")
        worst = max(worst, e[1])
    say(f"  {label}: rows checked {len(rows)}, worst normalised error {worst:.3g}")


MLA_SHAPES = [(512, 64), (64, 16)]
MLA_HEADS = {(512, 64): [16, 32, 40, 128], (64, 16): [8, 40]}


@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp8_tile128"])
@pytest.mark.parametrize("shape", MLA_SHAPES, ids=["512+64", "64+16"])
def test_sparse_mla_few_rows_split_lists(lib, shape, kv):
    """Few rows: each row's list is split over several workgroups and merged."""
    D_latent, D_rope = shape
    for H in MLA_HEADS[shape]:
        say(f"[case] sparse MLA {D_latent}+{D_rope} {kv} H={H}, 3 rows, split lists")
        b = _mla_batch(D_latent, D_rope, kv, H, R=3, L=2600, nseq=2, seed=40 + H)
        idx = _index_lists(3, 2048, 2600, seed=H)
        _check_mla(b, idx, range(3), kv != "bf16", f"{kv} H={H}")
        del b
        torch.cuda.empty_cache()


@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp8_tile128"])
@pytest.mark.parametrize("shape", MLA_SHAPES, ids=["512+64", "64+16"])
def test_sparse_mla_many_rows_whole_lists(lib, shape, kv):
    """Many rows: one workgroup per row and head block takes all 2048 entries
    (no split); sampled rows are checked."""
    D_latent, D_rope = shape
    for H in MLA_HEADS[shape]:
        say(f"[case] sparse MLA {D_latent}+{D_rope} {kv} H={H}, 256 rows, whole lists")
        b = _mla_batch(D_latent, D_rope, kv, H, R=256, L=2300, nseq=8, seed=80 + H)
        idx = _index_lists(256, 2048, 2300, seed=H + 1)
        _check_mla(b, idx, [0, 1, 2, 5, 63, 100, 127, 128, 200, 255], kv != "bf16", f"{kv} H={H}")
        del b
        torch.cuda.empty_cache()


def test_sparse_mla_single_split_rows(lib):
    """K < 32 and K not a multiple of the 32-row tile."""
    for K in (1, 31, 33):
        say(f"[case] sparse MLA K={K}")
        b = _mla_batch(512, 64, "bf16", 128, R=5, L=300, nseq=1, seed=5 + K)
        idx = _index_lists(5, K, 300, seed=K)
        _check_mla(b, idx, range(5), False, f"K={K}")


@pytest.mark.parametrize("L", [2300, 2600], ids=["table-row-staged", "direct-lookups"])
def test_sparse_mla_unaddressable_positions_skipped(lib, L):
    """Index entries the paged cache cannot address (a position past the
    sequence's block-table row, any negative value) are skipped, i.e. the
    result is the attention over the addressable entries.  L = 2300 gives a
    36-entry table row (staged in LDS by the kernel), L = 2600 a 41-entry row
    (looked up entry by entry)."""
    R, K = 4, 2048
    b = _mla_batch(512, 64, "bf16", 128, R=R, L=L, nseq=2, seed=L)
    bt_stride = int(b.block_table.shape[1])
    far = bt_stride * b.wl.block_size
    idx = _index_lists(R, K, L, seed=L + 1)
    g = np.random.default_rng(L + 2)
    valid = idx.copy()
    for r in range(R):
        n = int((idx[r] >= 0).sum())
        if n < 8:
            continue
        pick = g.choice(n, size=n // 4, replace=False)
        bad = np.where(g.random(pick.size) < 0.5, far + g.integers(0, 1 << 20, pick.size),
                       -g.integers(2, 1 << 30, pick.size))
        idx[r, pick] = bad.astype(np.int32)
        valid[r, pick] = -1
    say(f"[case] sparse MLA unaddressable entries, L={L}, table row {bt_stride}")
    idx_t = torch.from_numpy(idx).cuda()
    _, vc = caches(b)
    out = torch.full((R, 128, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, 128), float("nan"), dtype=torch.float32, device="cuda")
    lisfa.sparse_mla_attn(b.q, vc, b.row_seq, idx_t, out, lse, softmax_scale=b.wl.softmax_scale)
    torch.cuda.synchronize()
    out, lse = _np(out), _np(lse)
    inp = W.to_numpy(b)
    for r in range(R):
        ref_out, ref_lse = O.attend_row(inp, r, valid[r])
        check_out(out[r], ref_out, False, f"L={L} row {r}")
        check_lse(lse[r], ref_lse, f"L={L} row {r}")


# ------------------------------------------------------------ fused call ---

def test_fused_prefill_two_sequences_row_chunks(lib):
    """Rows of two sequences in one prefill batch, 16-row groups, more rows
    than one chunk of the fused call's score scratch holds: the chunk cut
    falls inside the first sequence's rows, the sequence change on a 16-row
    boundary after it.  Rows on both sides of both boundaries are checked."""
    L = 36864
    n0, n1 = 1824, 24
    R = n0 + n1
    wl = W.CONFIGS[1].with_(num_seqs=2, seq_len=L, H=8, D_latent=64, D_rope=16, K=2048,
                            softmax_scale=1.0 / math.sqrt(80.0), seed=91, name="prefill_two_seqs")
    say(f"[case] fused prefill, two sequences, R={R}, L={L}")
    b = batch_on_gpu(wl)
    g = torch.Generator(device="cpu").manual_seed(92)
    b.q_idx = torch.randn(R, wl.H_I, wl.D_I, generator=g).to(torch.bfloat16).cuda()
    b.w = torch.softmax(torch.randn(R, wl.H_I, generator=g, dtype=torch.float64), dim=1).float().cuda()
    b.q = (torch.randn(R, wl.H, wl.D_qk, generator=g) * 27.0).to(torch.bfloat16).cuda()
    b.row_seq = torch.cat([torch.zeros(n0, dtype=torch.int32), torch.ones(n1, dtype=torch.int32)]).cuda()
    b.row_pos = torch.cat([torch.arange(L - n0, L, dtype=torch.int32),
                           torch.arange(L - n1, L, dtype=torch.int32)]).cuda()
    kc, vc = caches(b)
    # the fused call keeps at most 256 MB of scores at a time
    assert (256 << 20) // (((L + 63) // 64 * 64) * 4) < R, "the rows must not fit one chunk"
    out = torch.full((R, wl.H, wl.D_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((R, wl.K), -7, dtype=torch.int32, device="cuda")
    lisfa.li_topk_sfa(b.q_idx, b.w, kc, b.q, vc, b.row_seq, b.row_pos, wl.K, L, out, lse, idx_out=idx,
                      rows_per_group=16, softmax_scale=wl.softmax_scale)
    torch.cuda.synchronize()
    idx, out, lse = _np(idx), _np(out), _np(lse)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    inp = W.to_numpy(b)
    for r in [0, 1790, 1807, 1808, 1809, 1823, 1824, 1825, 1839, 1840, R - 1]:
        o = O.layer_row(inp, r)
        check_index_set(idx[r], o["scores"], o["idx"], wl.K)
        g_out, g_lse = O.attend_row(inp, r, idx[r])
        check_out(out[r], g_out, False, f"row {r}")
        check_lse(lse[r], g_lse, f"row {r}")
