"""GPU parity of the attention over a tile-scaled fp8 latent cache (e4m3
codes, one fp32 scale per 128-element tile of each row) against the oracle,
through the C ABI: integer inputs exact up to the output tolerance, Gaussian
inputs on every row, the narrow shape whose rows are one tile, fewer heads, and
the partial output of a context shard."""
import numpy as np
import pytest
import torch

import indexer_selected_sparse_li_amd as lisfa
import oracle as O
import workloads as W
from gpu_util import batch_on_gpu, caches, check_index_set, check_lse, check_out, gpu_fused, gpu_sfa, say

pytestmark = pytest.mark.gpu


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def _all_rows(b, label):
    inp = W.to_numpy(b)
    idx, out, lse = gpu_fused(b)
    idx, out, lse = _np(idx), _np(out), _np(lse)
    for r in range(b.R):
        o = O.layer_row(inp, r)
        check_index_set(idx[r], o["scores"], o["idx"], b.wl.K)
        g_out, g_lse = O.attend_row(inp, r, idx[r])
        check_out(out[r], g_out, True, f"{label} row {r}")
        check_lse(lse[r], g_lse, f"{label} row {r}")


def test_integer_rows(lib):
    wl = W.CONFIGS[2].with_(num_seqs=3, len_range=(200, 2600), dist="int8range", kv_dtype="fp8_tile128",
                            name="tile_int", seed=31)
    say(f"[case] tile-scaled fp8 KV, integer {wl.name}")
    b = batch_on_gpu(wl)
    inp = W.to_numpy(b)
    idx, out, lse = gpu_fused(b)
    idx, out = _np(idx), _np(out)
    for r in range(b.R):
        o = O.layer_row(inp, r)
        assert np.array_equal(idx[r], o["idx"])
        check_out(out[r], o["out"], True, f"int row {r}")


def test_gaussian_paged_rows(lib):
    wl = W.CONFIGS[2].with_(num_seqs=6, len_range=(100, 3000), kv_dtype="fp8_tile128", name="tile_paged",
                            seed=32)
    say(f"[case] tile-scaled fp8 KV, paged {wl.name}")
    _all_rows(batch_on_gpu(wl), "paged")


def test_one_tile_rows(lib):
    wl = W.CONFIGS[0].with_(kv_dtype="fp8_tile128", dist="gauss", name="tile_tiny", seed=33)
    say(f"[case] tile-scaled fp8 KV, rows of one tile {wl.name}")
    _all_rows(batch_on_gpu(wl), "tiny")


@pytest.mark.parametrize("H", [32, 96])
def test_fewer_heads(lib, H):
    wl = W.CONFIGS[2].with_(num_seqs=4, len_range=(1000, 5000), H=H, kv_dtype="fp8_tile128",
                            name=f"tile_h{H}", seed=34 + H)
    say(f"[case] tile-scaled fp8 KV, {H} heads")
    _all_rows(batch_on_gpu(wl), f"H={H}")


def test_partial_output(lib):
    wl = W.CONFIGS[2].with_(num_seqs=5, len_range=(3000, 7000), kv_dtype="fp8_tile128", name="tile_partial",
                            seed=35)
    say(f"[case] tile-scaled fp8 KV, partial output {wl.name}")
    b = batch_on_gpu(wl)
    _, vc = caches(b)
    g = np.random.default_rng(2)
    pos = b.row_pos.cpu().numpy()
    idx = np.full((b.R, wl.K), -1, dtype=np.int32)
    for r in range(b.R):
        sel = np.sort(g.choice(int(pos[r]) + 1, size=min(wl.K, int(pos[r]) + 1), replace=False))
        idx[r, :len(sel)] = sel
    out = torch.full((b.R, wl.H, wl.D_v), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((b.R, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    lisfa.sparse_mla_attn_partial(b.q, vc, b.row_seq, torch.from_numpy(idx).cuda(), out, lse,
                                  softmax_scale=wl.softmax_scale)
    torch.cuda.synchronize()
    inp = W.to_numpy(b)
    for r in range(b.R):
        g_out, g_lse = O.attend_row(inp, r, idx[r])
        check_out(out[r].cpu().numpy(), g_out, True, f"partial row {r}")
        check_lse(lse[r].cpu().numpy(), g_lse, f"partial row {r}")
