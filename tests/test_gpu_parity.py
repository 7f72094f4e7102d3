"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Integer-valued inputs: scores and index lists bit-exact.  Gaussian inputs:
scores within the fp32 forward error bound, index sets equal except inside
the 1e-3 relative tie band around the K-th score, attention outputs within
2e-2 abs / 1e-2 rel (bf16; 5e-2 abs for fp8) plus a normalised check."""
import numpy as np
import pytest
import torch

import indexer_selected_sparse_li_amd as lisfa
import oracle as O
import workloads as W
from gpu_util import (batch_on_gpu, caches, check_index_set, check_lse, check_out, gpu_fused, gpu_scores,
                      gpu_sfa, gpu_topk, say, score_bound)

pytestmark = pytest.mark.gpu

TINY = W.CONFIGS[0]
D8K = W.CONFIGS[1]


def _oracle_rows(inp, rows, K=None):
    return [O.layer_row(inp, r, K=K) for r in rows]


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


# --------------------------------------------------------------- integer ---

@pytest.mark.parametrize("wl", [TINY, D8K.with_(dist="int8range", name="int_decode_l8192")],
                         ids=["tiny", "int_8k"])
def test_integer_inputs_bit_exact(lib, wl):
    say(f"[case] integer bit-exact {wl.name}")
    b = batch_on_gpu(wl)
    inp = W.to_numpy(b)
    ref = _oracle_rows(inp, range(b.R))
    sc = _np(gpu_scores(b))
    for r, o in enumerate(ref):
        n = int(inp["row_pos"][r]) + 1
        assert np.array_equal(sc[r, :n].astype(np.float64), o["scores"]), "scores differ"
    idx = _np(gpu_topk(gpu_scores(b), b.row_pos, wl.K))
    for r, o in enumerate(ref):
        assert np.array_equal(idx[r], o["idx"]), "idx differ"
    fidx, out, lse = gpu_fused(b)
    fidx, out, lse = _np(fidx), _np(out), _np(lse)
    for r, o in enumerate(ref):
        assert np.array_equal(fidx[r], o["idx"])
        check_out(out[r], o["out"], False, "fused")
        check_lse(lse[r], o["lse"], "fused")


# -------------------------------------------------------------- gaussian ---

@pytest.mark.parametrize("wl", [D8K, D8K.with_(q_mla_std=72.0, name="sharp_8k")], ids=["gauss", "sharp"])
def test_decode_8k_gaussian(lib, wl):
    say(f"[case] gaussian decode {wl.name}")
    b = batch_on_gpu(wl)
    inp = W.to_numpy(b)
    o = O.layer_row(inp, 0)
    sc = _np(gpu_scores(b))[0, : b.max_visible].astype(np.float64)
    bound = score_bound(inp, 0)
    assert (np.abs(sc - o["scores"]) <= bound).all(), np.max(np.abs(sc - o["scores"]) / bound)
    idx, out, lse = gpu_fused(b)
    nd = check_index_set(_np(idx)[0], o["scores"], o["idx"], wl.K)
    say(f"  index-set differences inside the band: {nd}")
    # attention on the oracle's own index set
    oidx = torch.from_numpy(o["idx"].astype(np.int32))[None].cuda()
    out2, lse2 = gpu_sfa(b, oidx)
    e = check_out(_np(out2)[0], o["out"], False, "sfa")
    check_lse(_np(lse2)[0], o["lse"], "sfa")
    say(f"  sfa max abs err {e[0]:.3g}, normalised {e[1]:.3g}")
    # fused output against the oracle over the GPU's index set
    g_out, g_lse = O.attend_row(inp, 0, _np(idx)[0])
    check_out(_np(out)[0], g_out, False, "fused")
    check_lse(_np(lse)[0], g_lse, "fused")


# ------------------------------------------------------------ selection ---

@pytest.mark.parametrize("kind", ["gauss", "ties", "signed_zero", "const", "int", "extreme"])
def test_topk_isolated_bit_exact(lib, kind):
    say(f"[case] topk isolated {kind}")
    rows, cols = 24, 5000
    seeds = {"gauss": 1, "ties": 2, "signed_zero": 3, "const": 4, "int": 5, "extreme": 6}
    s = W.make_scores(rows, cols, kind, seed=seeds[kind])
    pos = torch.tensor([-1, 0, 1, 31, 32, 33, 63, 64, 100, 127, 128, 129, 1000, 1023, 1024, 1025,
                        2047, 2048, 2049, 3000, 4095, 4096, 4999, 7000], dtype=torch.int32)
    for K in (1, 32, 128, 2048):
        idx = _np(gpu_topk(s.cuda(), pos.cuda(), K))
        for r in range(rows):
            n = max(0, min(int(pos[r]) + 1, cols))
            ref = O.select_topk(s[r, :n].numpy().astype(np.float64), K)
            assert np.array_equal(idx[r], ref), (kind, K, r)


def test_topk_many_candidates_general_path(lib):
    """Rows whose first-digit bin at the K-th value holds more candidates than
    the LDS list keeps (three distinct values over 30000 positions): the
    general selection takes over; still bit-exact."""
    say("[case] topk many candidates")
    g = torch.Generator().manual_seed(7)
    for ld in (20000, 40000):
        s = torch.randint(0, 3, (4, ld), generator=g).to(torch.float32) * 0.5
        pos = torch.tensor([ld - 1, ld // 2, 9000, 12345], dtype=torch.int32)
        for K in (2048, 9000):
            idx = _np(gpu_topk(s.cuda(), pos.cuda(), K))
            for r in range(4):
                n = int(pos[r]) + 1
                ref = O.select_topk(s[r, :n].numpy().astype(np.float64), K)
                assert np.array_equal(idx[r], ref), (ld, K, r)


def test_topk_long_rows(lib):
    say("[case] topk long rows")
    for kind in ("gauss", "ties"):
        s = W.make_scores(3, 131072, kind, seed=11)
        pos = torch.tensor([131071, 70000, 65536], dtype=torch.int32)
        idx = _np(gpu_topk(s.cuda(), pos.cuda(), 2048))
        for r in range(3):
            ref = O.select_topk(s[r, : int(pos[r]) + 1].numpy().astype(np.float64), 2048)
            assert np.array_equal(idx[r], ref)


# --------------------------------------------------------- cache layouts ---

def _check_all_rows(b, label, fp8=False):
    inp = W.to_numpy(b)
    idx, out, lse = gpu_fused(b)
    idx, out, lse = _np(idx), _np(out), _np(lse)
    for r in range(b.R):
        o = O.layer_row(inp, r)
        check_index_set(idx[r], o["scores"], o["idx"], b.wl.K)
        g_out, g_lse = O.attend_row(inp, r, idx[r])
        check_out(out[r], g_out, fp8, f"{label} row {r}")
        check_lse(lse[r], g_lse, f"{label} row {r}")


def test_paged_batched_reduced(lib):
    wl = W.CONFIGS[2].with_(num_seqs=6, len_range=(100, 3000), name="paged_small")
    say(f"[case] paged batched reduced {wl.name}")
    b = batch_on_gpu(wl)
    _check_all_rows(b, "paged")


def test_prefill_reduced_with_short_rows(lib):
    wl = W.CONFIGS[3].with_(seq_len=2100, q_rows=64, name="prefill_small")
    say(f"[case] prefill reduced {wl.name}")
    b = batch_on_gpu(wl)
    _check_all_rows(b, "prefill")


def test_fp8_reduced(lib):
    wl = W.CONFIGS[4].with_(num_seqs=3, seq_len=5000, name="fp8_small")
    say(f"[case] fp8 reduced {wl.name}")
    b = batch_on_gpu(wl)
    _check_all_rows(b, "fp8", fp8=True)


def test_fp8_integer_bit_exact(lib):
    wl = W.CONFIGS[4].with_(num_seqs=2, seq_len=3000, dist="int8range", name="fp8_int")
    say(f"[case] fp8 integer {wl.name}")
    b = batch_on_gpu(wl)
    inp = W.to_numpy(b)
    sc = _np(gpu_scores(b))
    idx, out, lse = gpu_fused(b)
    idx, out = _np(idx), _np(out)
    for r in range(b.R):
        o = O.layer_row(inp, r)
        n = int(inp["row_pos"][r]) + 1
        assert np.array_equal(sc[r, :n].astype(np.float64), o["scores"])
        assert np.array_equal(idx[r], o["idx"])
        check_out(out[r], o["out"], True, "fp8 int")


def test_fp8_per_head_query_scales(lib):
    """Per-(row, head) query scales: multiplying head h's scale by 2^e_h must give
    the same fp32 scores, bit for bit, as multiplying its weight by 2^e_h instead
    (both are exact power-of-two rescalings of the same products)."""
    wl = W.CONFIGS[4].with_(num_seqs=2, seq_len=3000, name="fp8_head_scales")
    say(f"[case] fp8 per-head query scales {wl.name}")
    b = batch_on_gpu(wl)
    assert b.q_scale is not None and b.q_scale.dim() == 1
    kc, _ = caches(b)
    e = torch.tensor([2.0 ** ((h % 3) - 1) for h in range(wl.H_I)], dtype=torch.float32, device="cuda")
    ld = (b.max_visible + 63) // 64 * 64
    by_w = torch.full((b.R, ld), float("nan"), dtype=torch.float32, device="cuda")
    by_s = torch.full((b.R, ld), float("nan"), dtype=torch.float32, device="cuda")
    lisfa.li_score(b.q_idx, (b.w * e[None, :]).contiguous(), kc, b.row_seq, b.row_pos, by_w, b.max_visible,
                   q_scale=b.q_scale)
    lisfa.li_score(b.q_idx, b.w, kc, b.row_seq, b.row_pos, by_s, b.max_visible,
                   q_scale=(b.q_scale[:, None] * e[None, :]).contiguous())
    torch.cuda.synchronize()
    for r in range(b.R):
        n = int(b.row_pos[r]) + 1
        assert torch.equal(by_w[r, :n], by_s[r, :n]), f"row {r}"
        assert torch.isfinite(by_s[r, :n]).all()


# ----------------------------------------------------------------- edges ---

@pytest.mark.parametrize("L,K", [(1, 1), (1, 2048), (63, 64), (65, 64), (200, 2048), (2049, 2048)])
def test_edge_lengths(lib, L, K):
    wl = D8K.with_(seq_len=L, K=K, name=f"edge_{L}_{K}")
    say(f"[case] edge L={L} K={K}")
    b = batch_on_gpu(wl)
    _check_all_rows(b, f"edge L={L} K={K}")


def test_zero_weights_pick_first_positions(lib):
    say("[case] zero weights")
    b = batch_on_gpu(D8K.with_(seq_len=3000))
    b.w.zero_()
    idx, out, _ = gpu_fused(b)
    assert np.array_equal(_np(idx)[0], np.arange(2048))


def test_dense_equivalence_when_K_covers_context(lib):
    """K >= visible: the sparse layer equals dense causal attention."""
    say("[case] K >= L dense equivalence")
    wl = D8K.with_(seq_len=1500, K=2048, q_mla_std=72.0)
    b = batch_on_gpu(wl)
    inp = W.to_numpy(b)
    idx, out, lse = gpu_fused(b)
    assert np.array_equal(_np(idx)[0], np.r_[np.arange(1500), -np.ones(548, dtype=np.int64)])
    rows = O.latent_rows(inp, 0, np.arange(1500))
    z = wl.softmax_scale * O.mla_query(inp, 0) @ rows.T
    p = np.exp(z - z.max(1, keepdims=True))
    dense = (p / p.sum(1, keepdims=True)) @ rows[:, :512]
    check_out(_np(out)[0], dense, False, "dense")


def test_tiny_heads_and_dims(lib):
    """H=8 heads with a 64+16 latent/rope split and a 4x32 indexer (the
    smallest supported shapes) on Gaussian values."""
    wl = TINY.with_(dist="gauss", seq_len=700, K=32, name="tiny_gauss")
    say("[case] tiny gaussian")
    b = batch_on_gpu(wl)
    _check_all_rows(b, "tiny gauss")


def test_determinism(lib):
    say("[case] determinism")
    b = batch_on_gpu(W.CONFIGS[2].with_(num_seqs=4, len_range=(3000, 9000)))
    first = [_np(t) for t in gpu_fused(b)]
    for _ in range(3):
        again = [_np(t) for t in gpu_fused(b)]
        for x, y in zip(first, again):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_rows_per_group_16_matches_8(lib):
    """Groups of 16 rows (two rows per wave, each key operand read feeding
    both) give the same fp32 scores, bit for bit, as groups of 8 and as one row
    at a time would for the same rows: every row's products and sums are
    evaluated in the same order."""
    wl = W.CONFIGS[3].with_(seq_len=3000, q_rows=48, name="prefill_groups")
    say(f"[case] 16- vs 8-row groups {wl.name}")
    b = batch_on_gpu(wl)
    kc, _ = caches(b)
    ld = (b.max_visible + 63) // 64 * 64
    out = {}
    for g in (16, 8):
        sc = torch.full((b.R, ld), float("nan"), dtype=torch.float32, device="cuda")
        lisfa.li_score(b.q_idx, b.w, kc, b.row_seq, b.row_pos, sc, b.max_visible, q_scale=b.q_scale,
                       rows_per_group=g)
        out[g] = sc
    torch.cuda.synchronize()
    inp = W.to_numpy(b)
    for r in range(b.R):
        n = int(b.row_pos[r]) + 1
        assert torch.equal(out[16][r, :n], out[8][r, :n]), f"row {r}"
    for r in (0, 17, 47):
        n = int(b.row_pos[r]) + 1
        ref = O.scores_row(inp, r)
        got = out[16][r, :n].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ref) <= score_bound(inp, r) + 0.0), f"row {r}"


def test_rows_per_group_mismatch_poisons_scores(lib):
    """A row whose sequence differs from its group's first row gets NaN
    scores instead of silently reading another sequence's keys."""
    say("[case] group mismatch")
    wl = W.CONFIGS[3].with_(seq_len=600, q_rows=16)
    b = batch_on_gpu(wl)
    b.row_seq[3] = 1  # out of range sequence in a group of 8
    sc = _np(gpu_scores(b))
    assert np.isnan(sc[3, : int(b.row_pos[3]) + 1]).all()
    assert np.isfinite(sc[2, : int(b.row_pos[2]) + 1]).all()
