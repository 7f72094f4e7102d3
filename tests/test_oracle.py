"""Pins of the CPU oracle against things other than itself: the hand-derived
golden example, exact rational arithmetic, brute-force ranking, closed forms
of softmax attention, a dense causal formulation via SciPy, and the storage
formats' definitions checked against PyTorch's conversions."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- formats ---

def test_e4m3_table_matches_format_definition():
    t = O.e4m3_table()
    assert t.shape == (256,)
    nan_codes = [c for c in range(256) if np.isnan(t[c])]
    assert nan_codes == [0x7F, 0xFF]
    finite = t[~np.isnan(t)]
    assert finite.max() == 448.0 and finite.min() == -448.0
    assert np.min(finite[finite > 0]) == 2.0 ** -9
    # every integer in [-16, 16] is exactly representable
    for v in range(-16, 17):
        assert v in set(finite.tolist())
    # sign symmetry
    for c in range(128):
        if not np.isnan(t[c]):
            assert t[c | 0x80] == -t[c] or (t[c] == 0 and t[c | 0x80] == 0)


def test_e4m3_table_matches_torch_conversion():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = O.e4m3_table()
    same = (t == ref) | (np.isnan(t) & np.isnan(ref))
    assert same.all()


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(7)
    bits = torch.randint(0, 1 << 16, (5000,), generator=g, dtype=torch.int32)
    # drop NaN patterns (exponent all ones with nonzero mantissa)
    b = bits.numpy().astype(np.uint16)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.decode_bf16(b)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_fp8_quantiser_codes_roundtrip():
    """The generator's e4m3 codes, decoded by the oracle and re-encoded by
    torch, give back the same codes (idempotent round trip)."""
    wl = W.CONFIGS[4].with_(num_seqs=1, seq_len=300)
    b = W.make_batch(wl)
    inp = W.to_numpy(b)
    codes = inp["k_data"][:300]
    vals = O.decode_e4m3(codes)
    assert not np.isnan(vals).any()
    again = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (again == codes).all()
    # dequantised keys stay within the per-token amax used for the scale
    k = O.indexer_keys(inp, 0, 300)
    assert np.all(np.abs(k).max(axis=1) <= inp["k_scale"][:300] * 448.0 * (1 + 1e-6))


# ----------------------------------------------------------- golden case ---

def test_golden_handworked():
    g = json.load(open(os.path.join(GOLDEN, "handworked_small.json")))
    q = np.array(g["q_idx"])
    w = np.array(g["w"])
    keys = np.array(g["keys"])
    sc = O.indexer_scores(q, w, keys)
    assert sc.tolist() == g["scores"]
    for K, want in g["topk_pos3"].items():
        assert O.select_topk(sc, int(K)).tolist() == want
    for K, want in g["topk_pos2"].items():
        assert O.select_topk(sc[:3], int(K)).tolist() == want
    out, lse = O.sparse_mla(np.array(g["attn_q"]), np.array(g["attn_rows"]),
                            g["attn_D_v"], g["attn_scale"])
    np.testing.assert_allclose(out, np.array(g["attn_out"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, np.array(g["attn_lse"]), rtol=0, atol=1e-15)


# -------------------------------------------------------------- indexer ---

def _frac_scores(q_rows, w_row, key_rows):
    """Exact rational evaluation of sum_j w_j * max(0, q_j . k)."""
    out = []
    for k in key_rows:
        s = Fraction(0)
        for qj, wj in zip(q_rows, w_row):
            d = sum(Fraction(int(a)) * Fraction(int(b)) for a, b in zip(qj, k))
            s += Fraction(wj) * max(d, Fraction(0))
        out.append(s)
    return out


def test_scores_exact_on_integer_inputs():
    b = W.make_batch(W.CONFIGS[0])
    inp = W.to_numpy(b)
    sc = O.scores_row(inp, 0)
    q = O.indexer_query(inp, 0)
    keys = O.indexer_keys(inp, 0, 256)
    w = inp["w"][0]
    exact = _frac_scores(q.astype(int).tolist(), [Fraction(float(x)) for x in w],
                         keys.astype(int).tolist())
    assert len(exact) == 256
    assert all(Fraction(float(a)) == e for a, e in zip(sc, exact))
    # every score is a multiple of 1/16 and fits float32 exactly
    assert np.all((sc * 16) == np.round(sc * 16))
    assert np.all(sc.astype(np.float32).astype(np.float64) == sc)


def test_scores_exact_integer_variant_large_shape():
    """64 heads x 128 dims, integer inputs: every score is still exact."""
    wl = W.CONFIGS[1].with_(dist="int8range", seq_len=96)
    inp = W.to_numpy(W.make_batch(wl))
    sc = O.scores_row(inp, 0)
    q = O.indexer_query(inp, 0).astype(int).tolist()
    keys = O.indexer_keys(inp, 0, 96).astype(int).tolist()
    exact = _frac_scores(q, [Fraction(float(x)) for x in inp["w"][0]], keys[:12])
    assert all(Fraction(float(a)) == e for a, e in zip(sc[:12], exact))


def test_scores_fp8_dequantised_exact_fraction():
    """fp8 codes times fp32 scales: scores equal the rational evaluation
    on the dequantised values (float64 holds every product exactly)."""
    wl = W.CONFIGS[4].with_(num_seqs=1, seq_len=40, H_I=4, D_I=32)
    inp = W.to_numpy(W.make_batch(wl))
    sc = O.scores_row(inp, 0)
    q = O.indexer_query(inp, 0)
    keys = O.indexer_keys(inp, 0, 40)
    for s in range(0, 40, 7):
        tot = Fraction(0)
        for j in range(4):
            d = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q[j], keys[s]))
            tot += Fraction(float(inp["w"][0][j])) * max(d, Fraction(0))
        assert abs(float(tot) - sc[s]) <= 1e-12 * max(1.0, abs(float(tot)))


def test_scores_negative_dots_are_clipped():
    q = np.array([[1.0, 0.0]])
    keys = np.array([[-3.0, 0.0], [2.0, 5.0]])
    assert O.indexer_scores(q, np.array([1.0]), keys).tolist() == [0.0, 2.0]


# --------------------------------------------------------------- top-K ---

def _brute_topk(scores, K):
    n = len(scores)
    sel = []
    for p in range(n):
        rank = sum(1 for q in range(n)
                   if scores[q] > scores[p] or (scores[q] == scores[p] and q < p))
        if rank < K:
            sel.append(p)
    return sel + [-1] * (K - len(sel))


@pytest.mark.parametrize("kind", ["ties", "signed_zero", "int", "gauss", "const"])
def test_topk_matches_bruteforce(kind):
    for seed in range(12):
        sc = W.make_scores(1, 1 + (seed * 37) % 300, kind, seed).numpy()[0].astype(np.float64)
        for K in (1, 2, 5, 17, 64, 400):
            assert O.select_topk(sc, K).tolist() == _brute_topk(sc.tolist(), K)


def test_topk_special_cases():
    sc = np.zeros(50)
    assert O.select_topk(sc, 8).tolist() == list(range(8))
    assert O.select_topk(np.arange(5.0), 9).tolist() == [0, 1, 2, 3, 4, -1, -1, -1, -1]
    assert O.select_topk(np.array([3.0]), 1).tolist() == [0]
    # -0.0 and +0.0 are the same value: lower position wins
    assert O.select_topk(np.array([-0.0, 0.0, -1.0]), 1).tolist() == [0]
    assert O.select_topk(np.array([0.0, -0.0, -1.0]), 1).tolist() == [0]


def test_zero_weights_select_first_positions():
    wl = W.CONFIGS[0]
    inp = W.to_numpy(W.make_batch(wl))
    inp["w"] = np.zeros_like(inp["w"])
    res = O.layer_row(inp, 0)
    assert res["idx"].tolist() == list(range(wl.K))


def test_causal_visibility_counts_own_position():
    wl = W.CONFIGS[0].with_(seq_len=40)
    inp = W.to_numpy(W.make_batch(wl))
    res = O.layer_row(inp, 0, K=64)
    assert res["idx"].tolist() == list(range(40)) + [-1] * 24
    assert res["scores"].shape == (40,)


# ------------------------------------------------------------ attention ---

def _dense_causal(q, seq_rows, p, D_v, scale):
    """Dense causal MLA over a whole sequence via SciPy: logits of every
    cached position, positions after p masked to -inf."""
    L = seq_rows.shape[0]
    z = scale * np.einsum("hd,sd->hs", q, seq_rows)
    z[:, p + 1:] = -np.inf
    return softmax(z, axis=1) @ seq_rows[:, :D_v], logsumexp(z, axis=1)


@pytest.mark.parametrize("p", [0, 1, 37, 95])
def test_sparse_equals_dense_when_K_covers_context(p):
    wl = W.CONFIGS[1].with_(seq_len=96, H=8, D_latent=64, D_rope=16, H_I=4, D_I=32,
                            q_mla_std=8.0)
    inp = W.to_numpy(W.make_batch(wl))
    inp["row_pos"] = np.array([p], dtype=np.int32)
    res = O.layer_row(inp, 0, K=128)
    assert res["idx"][: p + 1].tolist() == list(range(p + 1))
    all_rows = O.latent_rows(inp, 0, np.arange(96))
    out_d, lse_d = _dense_causal(O.mla_query(inp, 0), all_rows, p, 64, wl.softmax_scale)
    np.testing.assert_allclose(res["out"], out_d, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"], lse_d, rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(16, 80)) * 5
    rows = rng.normal(size=(200, 80))
    _, _, p = O.sparse_mla(q, rows, 64, 0.3, return_probs=True)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (p >= 0).all()


def test_attention_closed_forms():
    rng = np.random.default_rng(5)
    H, D_lat, D_rope, scale = 4, 6, 3, 0.7
    q = rng.normal(size=(H, D_lat + D_rope))
    # all selected rows equal: output is that row's value part for any q
    row = rng.normal(size=(D_lat + D_rope,))
    rows = np.tile(row, (9, 1))
    out, lse = O.sparse_mla(q, rows, D_lat, scale)
    np.testing.assert_allclose(out, np.tile(row[:D_lat], (H, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, scale * q @ row + math.log(9), atol=1e-13)
    # q = 0: uniform weights, output is the mean of the value parts
    rows = rng.normal(size=(11, D_lat + D_rope))
    out, lse = O.sparse_mla(np.zeros((H, D_lat + D_rope)), rows, D_lat, scale)
    np.testing.assert_allclose(out, np.tile(rows[:, :D_lat].mean(0), (H, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(11), atol=1e-14)
    # one selected row: output is its value part, lse is its logit
    out, lse = O.sparse_mla(q, rows[:1], D_lat, scale)
    np.testing.assert_allclose(out, np.tile(rows[0, :D_lat], (H, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, scale * q @ rows[0], atol=1e-14)
    # no selected row
    out, lse = O.sparse_mla(q, rows[:0], D_lat, scale)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_value_is_latent_part_only():
    """Changing only the rope columns of the rows changes the weights but
    never enters the output as a value."""
    H, D_lat, D_rope = 2, 4, 2
    q = np.zeros((H, D_lat + D_rope))
    rows = np.zeros((3, D_lat + D_rope))
    rows[:, D_lat:] = [[100.0, 1.0], [5.0, 5.0], [7.0, 0.0]]
    rows[:, :D_lat] = np.eye(3, D_lat)
    out, _ = O.sparse_mla(q, rows, D_lat, 1.0)
    np.testing.assert_allclose(out[0], [1 / 3, 1 / 3, 1 / 3, 0.0], atol=1e-15)


# --------------------------------------------------------------- layout ---

def test_paged_slots_are_a_bijection_onto_non_poisoned_slots():
    wl = W.CONFIGS[2].with_(num_seqs=5, len_range=(70, 300), H_I=4, D_I=32,
                            H=8, D_latent=64, D_rope=16)
    b = W.make_batch(wl)
    inp = W.to_numpy(b)
    used = []
    for s, L in enumerate(b.seq_lens):
        sl = O.slots(inp, s, np.arange(L))
        used.extend(sl.tolist())
        k = O.indexer_keys(inp, s, L)
        assert not np.isnan(k).any()
    assert len(set(used)) == len(used)
    unused = sorted(set(range(b.num_slots)) - set(used))
    assert np.isnan(O.decode_bf16(inp["k_data"][unused])).all()


def test_paged_slots_read_back_the_positions_of_a_contiguous_layout():
    """Position-tagged read-back of the paged slot map.  The generator draws a
    sequence's values in position order whatever the layout, so the same
    workload laid out contiguously (slot = base + position, no table) holds the
    same value at every (sequence, position).  Reading every position back
    through the paged map must give those values, row for row, for the key
    cache and the latent cache (a wrong block index, offset or block size
    would read another position's row)."""
    base = W.CONFIGS[2].with_(num_seqs=6, len_range=(1, 400), H_I=4, D_I=32, H=8, D_latent=64, D_rope=16,
                              dist="int8range", block_size=16)
    paged = W.to_numpy(W.make_batch(base))
    contig = W.to_numpy(W.make_batch(base.with_(paged=False)))
    assert paged["seq_lens"] == contig["seq_lens"]
    assert paged["block_table"] is not None and contig["block_table"] is None
    for s, L in enumerate(paged["seq_lens"]):
        pos = np.arange(L)
        # integer tags: position p of sequence s must hold the row the contiguous
        # layout keeps at base[s] + p (values are integers, so equality is exact)
        np.testing.assert_array_equal(O.indexer_keys(paged, s, L), O.indexer_keys(contig, s, L))
        np.testing.assert_array_equal(O.latent_rows(paged, s, pos), O.latent_rows(contig, s, pos))
        # and the rows of distinct positions are not all the same (the check has teeth)
        if L > 1:
            assert not np.array_equal(O.latent_rows(paged, s, pos[:1]), O.latent_rows(paged, s, pos[1:2]))


def test_contiguous_fp8_scale_groups_follow_slots():
    wl = W.CONFIGS[4].with_(num_seqs=2, seq_len=150, H_I=4, D_I=32, H=8,
                            D_latent=64, D_rope=16)
    b = W.make_batch(wl)
    inp = W.to_numpy(b)
    for s in range(2):
        rows = O.latent_rows(inp, s, np.arange(150))
        assert not np.isnan(rows).any()
        # each group of 64 positions is scaled by one amax/448 factor
        for g0 in range(0, 150, 64):
            blk = rows[g0:g0 + 64]
            sc = inp["kv_scale"][(int(inp["seq_base"][s]) + g0) // 64]
            assert np.abs(blk).max() <= 448.0 * sc * (1 + 1e-6)
            assert np.abs(blk).max() >= 0.9 * 448.0 * sc
