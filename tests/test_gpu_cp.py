"""GPU parity of one GPU's share of a context-parallel split, through the C
ABI: local Top-K candidates, the candidate merge, fp32 partial attention,
the LSE combine and the Zigzag restore, checked against the oracle.  Every
rank of a split is run in turn on the one GPU; the gathers between GPUs
become concatenations.  Also the two-pass Top-K of rows longer than 64K
positions, which uses the same candidate and merge kernels."""
import ctypes

import numpy as np
import pytest
import torch

import indexer_selected_sparse_li_amd as lisfa
import oracle as O
import workloads as W
from gpu_util import batch_on_gpu, caches, check_index_set, check_lse, check_out, gpu_fused, say

pytestmark = pytest.mark.gpu


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


# ------------------------------------------------------------------ Top-K ---

@pytest.mark.parametrize("kind,ld", [("gauss", 131072), ("ties", 131072), ("int", 100003),
                                     ("signed_zero", 131072), ("extreme", 70000)])
def test_topk_long_rows_two_pass(lib, kind, ld):
    """Rows longer than one workgroup holds: slices keep their Top-K, an
    ordered merge selects; bit-exact with the oracle, and with the
    single-workgroup path taken when no workspace is given."""
    K = 2048
    say(f"[case] two-pass top-k {kind} ld={ld}")
    sc = W.make_scores(4, ld, kind, seed=ld % 97).cuda()
    row_pos = torch.tensor([ld - 1, ld // 2 + 7, K - 1, 66000 % ld], dtype=torch.int32, device="cuda")
    idx = torch.full((4, K), -7, dtype=torch.int32, device="cuda")
    lisfa.topk_select(sc, row_pos, K, idx)             # binding supplies the workspace
    idx1 = torch.full((4, K), -7, dtype=torch.int32, device="cuda")
    rc = lisfa.load().topk_select(sc.data_ptr(), ld, row_pos.data_ptr(), 4, K, idx1.data_ptr(), None, 0,
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    s = _np(sc).astype(np.float64)
    rp = _np(row_pos)
    g, g1 = _np(idx), _np(idx1)
    for r in range(4):
        want = O.select_topk(s[r, :int(rp[r]) + 1], K)
        assert g[r].tolist() == want.tolist(), f"row {r}"
        assert g1[r].tolist() == want.tolist(), f"row {r} (single pass)"


@pytest.mark.parametrize("ld,K", [(3000, 64), (40000, 2048), (131072, 2048)])
def test_topk_candidates_match_oracle(lib, ld, K):
    say(f"[case] topk_candidates ld={ld} K={K}")
    R = 5
    sc = W.make_scores(R, ld, "ties", seed=ld + K).cuda()
    row_pos = torch.tensor([ld - 1, -1, K - 2, ld // 3, 5], dtype=torch.int32, device="cuda")
    off = torch.tensor([0, 77, 1000, 123456, 9], dtype=torch.int32, device="cuda")
    cp = torch.full((R, K), -7, dtype=torch.int32, device="cuda")
    cs = torch.full((R, K), 7.0, dtype=torch.float32, device="cuda")
    lisfa.topk_candidates(sc, row_pos, K, cp, cs, pos_offset=off)
    torch.cuda.synchronize()
    s = _np(sc).astype(np.float64)
    rp, of = _np(row_pos), _np(off)
    gp, gs = _np(cp), _np(cs)
    for r in range(R):
        pos, scr = O.shard_candidates(s[r, :max(int(rp[r]) + 1, 0)], K, int(of[r]))
        assert gp[r].tolist() == pos.tolist(), f"row {r}"
        assert np.array_equal(gs[r].astype(np.float64), scr), f"row {r} scores"


@pytest.mark.parametrize("G,K,kind", [(8, 2048, "ties"), (3, 100, "int"), (4, 512, "gauss"), (2, 7, "const")])
def test_topk_merge_matches_oracle(lib, G, K, kind):
    """Candidates of a contiguous split (from the oracle) merged on the GPU,
    in rank order (ordered) and shuffled (unordered)."""
    say(f"[case] topk_merge G={G} K={K} {kind}")
    R, L = 6, G * K + 5000
    rng = np.random.default_rng(G * 1000 + K)
    s = W.make_scores(R, L, kind, seed=G + K).numpy().astype(np.float64)
    cps, css, want = [], [], []
    for r in range(R):
        n = int(rng.integers(1, L + 1))
        cuts = [0] + sorted(rng.integers(0, n + 1, size=G - 1).tolist()) + [n]
        parts = [O.shard_candidates(s[r, cuts[g]:cuts[g + 1]], K, cuts[g]) for g in range(G)]
        cps.append(np.concatenate([p[0] for p in parts]))
        css.append(np.concatenate([p[1] for p in parts]))
        want.append(O.merge_candidates(css[-1], cps[-1], K))
        assert want[-1].tolist() == O.select_topk(s[r, :n], K).tolist()
    cp = torch.tensor(np.stack(cps), dtype=torch.int32, device="cuda")
    cs = torch.tensor(np.stack(css), dtype=torch.float32, device="cuda")
    for ordered in (True, False):
        if not ordered:
            perm = torch.stack([torch.randperm(cp.shape[1], generator=torch.Generator().manual_seed(r))
                                for r in range(R)]).cuda()
            cp_in, cs_in = torch.gather(cp, 1, perm), torch.gather(cs, 1, perm)
        else:
            cp_in, cs_in = cp, cs
        idx = torch.full((R, K), -7, dtype=torch.int32, device="cuda")
        isc = torch.full((R, K), 7.0, dtype=torch.float32, device="cuda")
        lisfa.topk_merge(cs_in.contiguous(), cp_in.contiguous(), K, idx, idx_score=isc, ordered=ordered)
        torch.cuda.synchronize()
        gi, gs = _np(idx), _np(isc)
        for r in range(R):
            assert gi[r].tolist() == want[r].tolist(), f"row {r} ordered={ordered}"
            m = want[r] >= 0
            assert np.array_equal(gs[r][m].astype(np.float64), s[r, want[r][m]])
            assert np.all(gs[r][~m] == -np.inf)


# ------------------------------------------------------ the share pipeline ---

def _shards(b, G):
    """Shard layouts (workloads.context_shards) with the binding's caches."""
    kc, vc = caches(b)
    out = []
    for s in W.context_shards(b, G):
        s = dict(s)
        s["kc"] = lisfa.KVCache(data=kc.data, scale=kc.scale, scale_group=kc.scale_group,
                                block_table=s["block_table"], block_size=kc.block_size, seq_base=s["seq_base"])
        s["vc"] = lisfa.KVCache(data=vc.data, scale=vc.scale, scale_group=vc.scale_group,
                                block_table=s["block_table"], block_size=vc.block_size, seq_base=s["seq_base"])
        out.append(s)
    return out


def _dcp_layer(b, G, K):
    """Every rank's share in turn: local scores, local candidates; the
    gather; the merge; every rank's partial attention; the combine."""
    wl = b.wl
    R = b.R
    sh = _shards(b, G)
    cps, css = [], []
    for s in sh:
        ld = max(64, -(-s["max_vis"] // 64) * 64)
        scores = torch.full((R, ld), float("nan"), dtype=torch.float32, device="cuda")
        lisfa.li_score(b.q_idx, b.w, s["kc"], b.row_seq, s["row_pos"], scores, s["max_vis"], q_scale=b.q_scale)
        cp = torch.empty((R, K), dtype=torch.int32, device="cuda")
        cs = torch.empty((R, K), dtype=torch.float32, device="cuda")
        lisfa.topk_candidates(scores, s["row_pos"], K, cp, cs, pos_offset=s["pos_offset"])
        cps.append(cp)
        css.append(cs)
    cand_pos, cand_score = torch.cat(cps, 1).contiguous(), torch.cat(css, 1).contiguous()
    idx = torch.full((R, K), -7, dtype=torch.int32, device="cuda")
    lisfa.topk_merge(cand_score, cand_pos, K, idx, ordered=True)
    idx_u = torch.full((R, K), -7, dtype=torch.int32, device="cuda")
    lisfa.topk_merge(cand_score, cand_pos, K, idx_u, ordered=False)
    pouts, plses = [], []
    for s in sh:
        po = torch.full((R, wl.H, wl.D_v), float("nan"), dtype=torch.float32, device="cuda")
        pl = torch.full((R, wl.H), float("nan"), dtype=torch.float32, device="cuda")
        lisfa.sparse_mla_attn_partial(b.q, s["vc"], b.row_seq, idx, po, pl, shard_range=s["range"],
                                      softmax_scale=wl.softmax_scale)
        pouts.append(po)
        plses.append(pl)
    out = torch.full((R, wl.H, wl.D_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    lisfa.lse_combine(torch.stack(pouts).contiguous(), torch.stack(plses).contiguous(), out, lse)
    torch.cuda.synchronize()
    return sh, idx, idx_u, pouts, plses, out, lse


def _check_pipeline(wl, G, rows, exact):
    say(f"[case] DCP share pipeline {wl.name} G={G}")
    b = batch_on_gpu(wl, gen_device="cuda")
    inp = W.to_numpy(b)
    fp8 = wl.kv_dtype == "fp8"
    sh, idx, idx_u, pouts, plses, out, lse = _dcp_layer(b, G, wl.K)
    idx1, out1, _ = gpu_fused(b)
    gi, gu, g1 = _np(idx), _np(idx_u), _np(idx1)
    # same scores per key on every path, so the same selection as one GPU
    assert np.array_equal(gi, g1)
    assert np.array_equal(gu, g1)
    o_np, l_np = _np(out), _np(lse)
    for r in rows:
        say(f"  oracle row {r}")
        o = O.layer_row(inp, r)
        if exact:
            assert gi[r].tolist() == o["idx"].tolist()
        else:
            check_index_set(gi[r], o["scores"], o["idx"], wl.K)
        ref_out, ref_lse = O.attend_row(inp, r, gi[r])
        check_out(o_np[r], ref_out, fp8, f"combined row {r}")
        check_lse(l_np[r], ref_lse, f"combined row {r}")
        for g, s in enumerate(sh):
            sel = gi[r][(gi[r] >= s["lo"][r]) & (gi[r] < s["hi"][r])]
            p_out, p_lse = O.attend_row(inp, r, sel)
            po, pl = _np(pouts[g][r]), _np(plses[g][r])
            if sel.size == 0:
                assert np.all(po == 0) and np.all(pl == -np.inf)
            else:
                check_out(po, p_out, fp8, f"shard {g} row {r}")
                check_lse(pl, p_lse, f"shard {g} row {r}")


def test_dcp_share_integer_inputs(lib):
    wl = W.CONFIGS[0].with_(name="tiny_4x3000", num_seqs=4, seq_len=3000, seed=41)
    _check_pipeline(wl, 4, range(4), exact=True)


def test_dcp_share_paged_gaussian(lib):
    wl = W.CONFIGS[2].with_(name="paged_8x4k_20k", num_seqs=8, len_range=(4096, 20000), seed=42)
    _check_pipeline(wl, 4, [0, 5], exact=False)


def test_dcp_share_fp8(lib):
    wl = W.CONFIGS[4].with_(name="fp8_4x24576", num_seqs=4, seq_len=24576, seed=43)
    _check_pipeline(wl, 4, [1], exact=False)


def test_dcp_share_more_ranks_than_blocks(lib):
    """Short sequences split 8 ways: some shards hold nothing for some rows."""
    wl = W.CONFIGS[2].with_(name="paged_6x100_900", num_seqs=6, len_range=(100, 900), seed=44, K=64)
    _check_pipeline(wl, 8, [0, 3], exact=False)


# ------------------------------------------------------------------ zigzag ---

@pytest.mark.parametrize("n,G,width", [(4099, 8, 16), (1000, 3, 12), (77, 2, 3), (8, 2, 1024), (5, 4, 16)])
def test_zigzag_restore_matches_oracle(lib, n, G, width):
    say(f"[case] zigzag restore n={n} G={G} width={width}")
    rows = torch.randint(0, 256, (n, width), dtype=torch.uint8, generator=torch.Generator().manual_seed(n))
    gathered = np.concatenate([rows.numpy()[a:b] for g in range(G) for a, b in O.zigzag_share(n, G, g)])
    src = torch.tensor(gathered).cuda()
    dst = torch.zeros_like(src)
    lisfa.zigzag_restore(src, dst, G)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), O.zigzag_restore(gathered, G))
    assert np.array_equal(dst.cpu().numpy(), rows.numpy())


def test_zigzag_prefill_shares_restore_the_full_result(lib):
    """Chunked prefill rows split over G ranks by the Zigzag partition: every
    rank runs the fused layer on its two segments; gathered and restored,
    the index lists equal the unsplit run's and the outputs the oracle's."""
    wl = W.CONFIGS[3].with_(name="prefill_512q_l8192", seq_len=8192, q_rows=512, seed=45)
    G = 4
    say(f"[case] zigzag prefill shares {wl.name} G={G}")
    b = batch_on_gpu(wl, gen_device="cuda")
    idx_full, out_full, _ = gpu_fused(b)
    kc, vc = caches(b)
    n = b.R
    idx_parts, out_parts = [], []
    for g in range(G):
        rows = torch.cat([torch.arange(a, c) for a, c in lisfa.zigzag_share(n, G, g)]).cuda()
        m = rows.numel()
        q_scale = b.q_scale[rows].contiguous() if b.q_scale is not None else None
        out = torch.full((m, wl.H, wl.D_v), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((m, wl.H), dtype=torch.float32, device="cuda")
        idx = torch.full((m, wl.K), -7, dtype=torch.int32, device="cuda")
        lisfa.li_topk_sfa(b.q_idx[rows].contiguous(), b.w[rows].contiguous(), kc, b.q[rows].contiguous(), vc,
                          b.row_seq[rows].contiguous(), b.row_pos[rows].contiguous(), wl.K, b.max_visible, out,
                          lse, idx_out=idx, q_scale=q_scale, rows_per_group=8, softmax_scale=wl.softmax_scale)
        idx_parts.append(idx)
        out_parts.append(out)
    gi = torch.cat(idx_parts).contiguous()
    go = torch.cat(out_parts).contiguous()
    ri, ro = torch.empty_like(gi), torch.empty_like(go)
    lisfa.zigzag_restore(gi, ri, G)
    lisfa.zigzag_restore(go, ro, G)
    torch.cuda.synchronize()
    assert torch.equal(ri, idx_full)
    inp = W.to_numpy(b)
    ro_np, rf_np = _np(ro), _np(out_full)
    for r in (0, 130, 511):
        ref_out, _ = O.attend_row(inp, r, _np(ri)[r])
        check_out(ro_np[r], ref_out, False, f"restored row {r}")
        check_out(ro_np[r], rf_np[r].astype(np.float64), False, f"restored row {r} vs unsplit")
