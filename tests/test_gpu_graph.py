"""The fused decode call captured once in a HIP graph and replayed: every
replay, with the program's own eager work and synchronisations between
replays, equals the eager call bit for bit (the kernels are deterministic and
the library issues no memset or allocation inside the call)."""
import numpy as np
import pytest
import torch

import indexer_selected_sparse_li_amd as lisfa
import workloads as W
from gpu_util import batch_on_gpu, caches, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", [
    W.CONFIGS[2].with_(num_seqs=8, len_range=(3000, 9000), name="paged_8_graph", seed=61),
    W.CONFIGS[4].with_(num_seqs=2, seq_len=70000, name="fp8_long_graph", seed=62),
    W.BENCH["decode_paged_64x32768_mxfp8"].with_(num_seqs=4, seq_len=5000, name="mx_graph", seed=63),
    # 64 rows of 8192 positions: the layer's index step is the fused launch
    # (4 workgroups per row, a clear of their control words before it)
    W.BENCH["decode_paged_64x32768"].with_(seq_len=8192, name="fused_index_graph", seed=64),
], ids=["paged", "fp8_long", "mxfp8", "fused_index"])
def test_fused_call_replays_in_a_graph(lib, wl):
    say(f"[case] graph replay {wl.name}")
    b = batch_on_gpu(wl, gen_device="cuda")
    kc, vc = caches(b)
    R = b.R
    out = torch.empty(R, wl.H, wl.D_v, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(R, wl.H, dtype=torch.float32, device="cuda")
    idx = torch.empty(R, wl.K, dtype=torch.int32, device="cuda")
    ws = torch.empty(lisfa.workspace_size(2, R, b.max_visible, wl.K, wl.H, wl.D_v), dtype=torch.uint8,
                     device="cuda")

    def call(stream):
        lisfa.li_topk_sfa(b.q_idx, b.w, kc, b.q, vc, b.row_seq, b.row_pos, wl.K, b.max_visible, out, lse,
                          idx_out=idx, q_scale=b.q_scale, softmax_scale=wl.softmax_scale, workspace=ws,
                          stream=stream)

    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = (idx.clone(), out.view(torch.int16).clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        idx.fill_(-9)
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]), f"replay {rep}: idx"
        assert torch.equal(out.view(torch.int16), ref[1]), f"replay {rep}: out"
        assert torch.equal(lse, ref[2]), f"replay {rep}: lse"
        call(torch.cuda.current_stream())          # eager work between replays
        torch.cuda.synchronize()
    del g


def test_li_topk_replays_in_a_graph(lib):
    """li_topk with rows split over 32 workgroups each (the exchange through
    the workspace, its control words cleared by a kernel in the same capture)."""
    wl = W.BENCH["decode_paged_64x32768"].with_(num_seqs=2, name="li_topk_graph", seed=65)
    say(f"[case] graph replay {wl.name}")
    b = batch_on_gpu(wl, gen_device="cuda")
    kc, _ = caches(b)
    assert lisfa.li_topk_plan(b.q_idx, b.w, kc, b.row_seq, b.row_pos, wl.K, b.max_visible) == 32
    idx = torch.empty(b.R, wl.K, dtype=torch.int32, device="cuda")
    ws = torch.empty(lisfa.workspace_size(5, b.R, b.max_visible, wl.K, 0, 0), dtype=torch.uint8, device="cuda")

    def call(stream):
        lisfa.li_topk(b.q_idx, b.w, kc, b.row_seq, b.row_pos, wl.K, idx, b.max_visible, workspace=ws,
                      stream=stream)

    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = idx.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        idx.fill_(-9)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref), f"replay {rep}"
        call(torch.cuda.current_stream())          # eager work between replays
        torch.cuda.synchronize()
