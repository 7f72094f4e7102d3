"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (one li_topk_sfa call over the whole batch): the oracle
recomputes query rows one by one, every row of the decode batches and
spread rows of the 4096-row prefill chunk.  Inputs are generated on the GPU
(seeded) and copied to the host for the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import check_index_set, check_lse, check_out, gpu_fused, say

pytestmark = pytest.mark.gpu


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def _run(wl, rows):
    say(f"[case] full size {wl.name}: generating")
    b = W.make_batch(wl, device="cuda")
    torch.cuda.synchronize()
    say(f"[case] full size {wl.name}: running the fused layer (R={b.R}, max L={b.max_visible})")
    idx, out, lse = gpu_fused(b)
    idx, out, lse = _np(idx), _np(out), _np(lse)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    inp = W.to_numpy(b)
    fp8 = wl.kv_dtype in ("fp8", "fp8_tile128")
    rows = list(rows)
    say(f"  oracle over {len(rows)} rows")
    for r in rows:
        r = r % b.R
        o = O.layer_row(inp, r)
        nd = check_index_set(idx[r], o["scores"], o["idx"], wl.K)
        g_out, g_lse = O.attend_row(inp, r, idx[r])
        e = check_out(out[r], g_out, fp8, f"{wl.name} row {r}")
        check_lse(lse[r], g_lse, f"{wl.name} row {r}")
        say(f"    band differences {nd}, max abs err {e[0]:.3g}, normalised {e[1]:.3g}")
    del b
    torch.cuda.empty_cache()


def test_decode_l8192_full(lib):
    _run(W.CONFIGS[1], [0])


def test_batched_paged_full(lib):
    _run(W.CONFIGS[2], range(64))


def test_prefill_4096q_l65536_full(lib):
    _run(W.CONFIGS[3], [0, 1, 15, 16, 1023, 1024, 2047, 2048, 3071, 3072, 4094, 4095])


def test_fp8_decode_16x131072_full(lib):
    _run(W.CONFIGS[4], range(16))


def test_bench_workload_64x32768_full(lib):
    _run(W.BENCH["decode_paged_64x32768"], range(64))


def test_bench_workload_1x32768_full(lib):
    _run(W.BENCH["decode_paged_1x32768"], [0])


def test_bench_workload_mxfp8_full(lib):
    _run(W.BENCH["decode_paged_64x32768_mxfp8"], range(64))


def test_bench_workload_fp8_tile_kv_full(lib):
    _run(W.BENCH["decode_paged_64x32768_fp8tilekv"], range(64))
