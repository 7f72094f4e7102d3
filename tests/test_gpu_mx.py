"""GPU parity of the MXFP8 indexer (e4m3 queries and keys, one E8M0 scale
per 32 elements, on gfx950's block-scaled MFMA) against the oracle, through
the C ABI: bit-exact scores and index lists on integer inputs, the fp32
error bound and the index-set rule on Gaussian inputs, and the whole layer
(MXFP8 indexer, bf16 latent cache) on decode, paged and prefill rows."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import (batch_on_gpu, check_index_set, check_lse, check_out, gpu_fused, gpu_scores, gpu_topk,
                      say, score_bound)

pytestmark = pytest.mark.gpu


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def _mx(wl, **kw):
    return wl.with_(indexer_dtype="mxfp8", **kw)


@pytest.mark.parametrize("wl", [
    _mx(W.CONFIGS[1], dist="int8range", seq_len=3000, name="mx_int_decode_3000", seed=51),
    _mx(W.CONFIGS[2], dist="int8range", num_seqs=5, len_range=(70, 2500), name="mx_int_paged", seed=52),
    _mx(W.CONFIGS[1], dist="int8range", seq_len=1000, H_I=20, name="mx_int_20heads", seed=53),
], ids=["decode", "paged", "20heads"])
def test_mx_integer_inputs_bit_exact(lib, wl):
    say(f"[case] mxfp8 integer bit-exact {wl.name}")
    b = batch_on_gpu(wl)
    inp = W.to_numpy(b)
    sc = _np(gpu_scores(b))
    idx, out, lse = gpu_fused(b)
    idx, out, lse = _np(idx), _np(out), _np(lse)
    for r in range(b.R):
        o = O.layer_row(inp, r)
        n = int(inp["row_pos"][r]) + 1
        assert np.array_equal(sc[r, :n].astype(np.float64), o["scores"]), f"row {r} scores"
        assert np.array_equal(idx[r], o["idx"]), f"row {r} idx"
        check_out(out[r], o["out"], False, f"mx int row {r}")
        check_lse(lse[r], o["lse"], f"mx int row {r}")


@pytest.mark.parametrize("wl", [
    _mx(W.CONFIGS[1], name="mx_decode_8192", seed=54),
    _mx(W.CONFIGS[2], num_seqs=6, len_range=(100, 5000), name="mx_paged_small", seed=55),
], ids=["decode", "paged"])
def test_mx_gaussian(lib, wl):
    say(f"[case] mxfp8 gaussian {wl.name}")
    b = batch_on_gpu(wl)
    inp = W.to_numpy(b)
    sc = _np(gpu_scores(b))
    idx, out, lse = gpu_fused(b)
    idx, out, lse = _np(idx), _np(out), _np(lse)
    for r in range(b.R):
        o = O.layer_row(inp, r)
        n = int(inp["row_pos"][r]) + 1
        bound = score_bound(inp, r)
        err = np.abs(sc[r, :n].astype(np.float64) - o["scores"])
        assert (err <= bound).all(), f"row {r}: {np.max(err / bound)} of the bound"
        check_index_set(idx[r], o["scores"], o["idx"], wl.K)
        g_out, g_lse = O.attend_row(inp, r, idx[r])
        check_out(out[r], g_out, False, f"mx row {r}")
        check_lse(lse[r], g_lse, f"mx row {r}")


def test_mx_prefill_rows(lib):
    """Prefill rows with the grouping hint: MXFP8 scores each row on its own,
    same values as the oracle."""
    wl = _mx(W.CONFIGS[3], seq_len=2100, q_rows=64, name="mx_prefill_small", seed=56)
    say(f"[case] mxfp8 prefill {wl.name}")
    b = batch_on_gpu(wl)
    inp = W.to_numpy(b)
    sc = _np(gpu_scores(b))
    idx = _np(gpu_topk(gpu_scores(b), b.row_pos, wl.K))
    for r in (0, 17, 63):
        o = O.layer_row(inp, r)
        n = int(inp["row_pos"][r]) + 1
        assert (np.abs(sc[r, :n].astype(np.float64) - o["scores"]) <= score_bound(inp, r)).all()
        check_index_set(idx[r], o["scores"], o["idx"], wl.K)


def test_mx_topk_matches_bf16_path_on_exact_inputs(lib):
    """Integer-valued keys stored both ways give identical scores: the MXFP8
    kernel and the bf16 kernel agree bit for bit."""
    base = W.CONFIGS[1].with_(dist="int8range", seq_len=2000, seed=57)
    b16 = batch_on_gpu(base.with_(name="int_bf16"))
    bmx = batch_on_gpu(base.with_(name="int_mx", indexer_dtype="mxfp8"))
    s16, smx = _np(gpu_scores(b16)), _np(gpu_scores(bmx))
    assert np.array_equal(s16[:, :2000], smx[:, :2000])
