"""The allocation-free fused entry point (li_topk_sfa_noalloc) against the
fused entry with a caller workspace, through the C ABI: the same kernels on
the same inputs, so index lists, outputs and lse must agree bit for bit; a
few rows are also checked against the oracle.  Two calls in a row, the second
smaller, then one whose rows must be cut into more chunks to fit the static
scratch array."""
import numpy as np
import pytest
import torch

import indexer_selected_sparse_li_amd as lisfa
import oracle as O
import workloads as W
from gpu_util import batch_on_gpu, caches, check_index_set, check_lse, check_out, gpu_fused, rows_per_group, say

pytestmark = pytest.mark.gpu


def _noalloc(b):
    kc, vc = caches(b)
    wl = b.wl
    out = torch.full((b.R, wl.H, wl.D_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((b.R, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((b.R, wl.K), -7, dtype=torch.int32, device="cuda")
    lisfa.li_topk_sfa_noalloc(b.q_idx, b.w, kc, b.q, vc, b.row_seq, b.row_pos, wl.K, b.max_visible, out, lse,
                              idx_out=idx, q_scale=b.q_scale, rows_per_group=rows_per_group(b),
                              softmax_scale=wl.softmax_scale)
    torch.cuda.synchronize()
    return idx, out, lse


def _same(b, rows, label):
    ref = gpu_fused(b)
    got = _noalloc(b)
    for x, y, name in zip(ref, got, ("idx", "out", "lse")):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y), f"{label}: {name} differs"
    inp = W.to_numpy(b)
    idx, out, lse = (t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy() for t in got)
    for r in rows:
        o = O.layer_row(inp, r)
        check_index_set(idx[r], o["scores"], o["idx"], b.wl.K)
        g_out, g_lse = O.attend_row(inp, r, idx[r])
        check_out(out[r], g_out, b.wl.kv_dtype != "bf16", f"{label} row {r}")
        check_lse(lse[r], g_lse, f"{label} row {r}")
    say(f"  {label}: identical to the workspace entry; oracle rows {list(rows)} within the bar")


def test_noalloc_matches_workspace_entry_two_calls(lib):
    say("[case] no-alloc: paged batch, then a smaller tiny batch")
    b1 = batch_on_gpu(W.CONFIGS[2].with_(num_seqs=6, len_range=(100, 3000), name="noalloc_paged"))
    _same(b1, [0, 3, 5], "paged 6 rows")
    b2 = batch_on_gpu(W.CONFIGS[0])
    _same(b2, [0], "tiny 1 row")


def test_noalloc_cuts_rows_to_fit_the_scratch(lib):
    say("[case] no-alloc: prefill rows that need smaller chunks than the workspace entry")
    wl = W.CONFIGS[3].with_(seq_len=16384, q_rows=2048, H=8, D_latent=64, D_rope=16,
                            softmax_scale=1.0 / 80 ** 0.5, name="noalloc_prefill")
    b = batch_on_gpu(wl)
    ld = (b.max_visible + 63) // 64 * 64
    assert b.R * ld * 4 > lisfa._c.LISFA_NOALLOC_SCRATCH_BYTES, "the scores alone must exceed the scratch"
    _same(b, [0, 1023, 2047], "prefill 2048 rows")


def test_noalloc_fused_index_step(lib):
    """Rows whose index step is the fused scoring + Top-K launch: its exchange
    area and control words live in the static scratch too, and are cleared
    anew on every call (two calls in a row, the second smaller)."""
    say("[case] no-alloc: 64 rows x 8192 (fused index step), then 64 rows x 4096")
    b1 = batch_on_gpu(W.BENCH["decode_paged_64x32768"].with_(seq_len=8192, name="noalloc_fused", seed=71))
    kc, _ = caches(b1)
    assert lisfa.li_topk_plan(b1.q_idx, b1.w, kc, b1.row_seq, b1.row_pos, b1.wl.K, b1.max_visible, layer=True) == 4
    _same(b1, [0, 63], "fused 64 x 8192")
    b2 = batch_on_gpu(W.BENCH["decode_paged_64x32768"].with_(seq_len=4096, name="noalloc_fused2", seed=72))
    _same(b2, [5], "fused 64 x 4096")
