"""Pins of the context-parallel oracle (oracle/cp_oracle.py) against things
other than itself: the pages' Zigzag example, brute-force ranking of the
whole row, exact partition and balance identities, and softmax attention over
the union of the parts."""
import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_topk(scores, K):
    """p is selected iff fewer than K positions beat it (higher score, or
    equal score at a lower position); ascending, -1 padded."""
    n = len(scores)
    sel = [p for p in range(n)
           if sum(1 for q in range(n)
                  if scores[q] > scores[p] or (scores[q] == scores[p] and q < p)) < K]
    return sel + [-1] * (K - len(sel))


def _positions(ranges):
    return [p for a, b in ranges for p in range(a, b)]


# ------------------------------------------------------------------ zigzag ---

def test_zigzag_matches_page_example():
    g = json.load(open(os.path.join(GOLDEN, "zigzag_page5.json")))
    n, G = g["n"], g["G"]
    for rank in range(G):
        assert _positions(O.zigzag_share(n, G, rank)) == g["zigzag"][rank]
    # the in-order split of the same example, for contrast
    seg = n // G
    assert [list(range(r * seg, (r + 1) * seg)) for r in range(G)] == g["simple_split"]


@pytest.mark.parametrize("n", [0, 1, 2, 7, 8, 100, 4096, 4099])
def test_zigzag_shares_partition_the_sequence(n):
    for G in range(1, 9):
        got = sorted(p for g in range(G) for p in _positions(O.zigzag_share(n, G, g)))
        assert got == list(range(n))
        sizes = [b - a for a, b in O.zigzag_segments(n, G)]
        assert len(sizes) == 2 * G and max(sizes) - min(sizes) <= 1
        assert sorted(O.zigzag_order(n, G).tolist()) == list(range(n))


@pytest.mark.parametrize("G", [2, 4, 8])
def test_zigzag_balances_causal_work(G):
    """With 2G | n every GPU's causal work sum(p + 1) is the same closed form
    c^2 (2G - 1) + c (c + 1) (c = n / 2G), while the in-order split grows with
    the rank."""
    c = 1000
    n = 2 * G * c
    closed = c * c * (2 * G - 1) + c * (c + 1)
    works = [sum(p + 1 for p in _positions(O.zigzag_share(n, G, g))) for g in range(G)]
    assert works == [closed] * G
    inorder = [sum(p + 1 for p in range(g * n // G, (g + 1) * n // G)) for g in range(G)]
    assert inorder[-1] > inorder[0] * (2 * G - 1) * 0.99


def test_zigzag_restore_inverts_the_gather():
    rng = np.random.default_rng(3)
    for n in (1, 9, 64, 1000):
        for G in (1, 2, 3, 8):
            rows = rng.standard_normal((n, 5))
            gathered = np.concatenate([rows[a:b] for g in range(G) for a, b in O.zigzag_share(n, G, g)])
            assert np.array_equal(O.zigzag_restore(gathered, G), rows)


# --------------------------------------------------------------- selection ---

@pytest.mark.parametrize("kind", ["ties", "int", "gauss", "signed_zero", "const"])
def test_merge_of_shard_candidates_is_the_global_topk(kind):
    rng = np.random.default_rng(11)
    for seed in range(10):
        n = 1 + (seed * 53) % 260
        sc = W.make_scores(1, n, kind, seed).numpy()[0].astype(np.float64)
        for G in (1, 2, 3, 6):
            cuts = np.sort(rng.integers(0, n + 1, size=G - 1))
            bounds = [0] + cuts.tolist() + [n]
            for K in (1, 3, 17, 64, 400):
                cands = [O.shard_candidates(sc[bounds[g]:bounds[g + 1]], K, bounds[g]) for g in range(G)]
                order = rng.permutation(G)        # gathered in any order
                cp = np.concatenate([cands[g][0] for g in order])
                cs = np.concatenate([cands[g][1] for g in order])
                assert O.merge_candidates(cs, cp, K).tolist() == _brute_topk(sc.tolist(), K)


def test_shard_candidates_carry_global_positions_and_scores():
    sc = np.array([1.0, 5.0, 5.0, -2.0, 7.0])
    pos, s = O.shard_candidates(sc, 3, 100)
    assert pos.tolist() == [101, 102, 104] and s.tolist() == [5.0, 5.0, 7.0]
    pos, s = O.shard_candidates(sc[:2], 3, 7)
    assert pos.tolist() == [7, 8, -1] and s[:2].tolist() == [1.0, 5.0] and s[2] == -np.inf
    pos, s = O.shard_candidates(sc[:0], 2, 7)
    assert pos.tolist() == [-1, -1]


def test_merge_candidates_matches_bruteforce_on_unordered_lists():
    rng = np.random.default_rng(5)
    for trial in range(40):
        m = int(rng.integers(1, 120))
        pos = rng.permutation(1000)[:m]
        sc = rng.integers(0, 6, size=m).astype(np.float64)      # many ties
        invalid = rng.random(m) < 0.2
        p_in = np.where(invalid, -1, pos)
        for K in (1, 4, 30, 200):
            valid = sorted(zip(pos[~invalid].tolist(), sc[~invalid].tolist()))
            ranked = _brute_topk([s for _, s in valid], K)
            want = sorted(valid[i][0] for i in ranked if i >= 0)
            want = want + [-1] * (K - len(want))
            assert O.merge_candidates(sc, p_in, K).tolist() == want


# -------------------------------------------------------------- attention ---

def test_combine_of_disjoint_parts_is_attention_over_the_union():
    rng = np.random.default_rng(7)
    for trial in range(20):
        H, D_v, D_qk = 3, 6, 8
        m = int(rng.integers(1, 40))
        q = rng.standard_normal((H, D_qk)) * 2.0
        rows = rng.standard_normal((m, D_qk))
        G = int(rng.integers(1, 6))
        part = rng.integers(0, G, size=m)            # some parts may be empty
        outs, lses = [], []
        for g in range(G):
            o, l = O.sparse_mla(q, rows[part == g], D_v, 0.7)
            outs.append(o)
            lses.append(l)
        out, lse = O.combine_partials(np.stack(outs), np.stack(lses))
        ref_out, ref_lse = O.sparse_mla(q, rows, D_v, 0.7)
        assert np.allclose(out, ref_out, atol=1e-12, rtol=1e-12)
        assert np.allclose(lse, ref_lse, atol=1e-12, rtol=1e-12)


def test_combine_edge_cases():
    o = np.arange(12.0).reshape(1, 2, 6)
    l = np.array([[0.3, -1.0]])
    out, lse = O.combine_partials(o, l)              # one part: identity
    assert np.array_equal(out, o[0]) and np.array_equal(lse, l[0])
    out, lse = O.combine_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.array_equal(out, np.zeros((2, 4))) and np.all(lse == -np.inf)
    # equal normalisers: plain mean
    out, lse = O.combine_partials(np.stack([np.ones((1, 2)), 3 * np.ones((1, 2))]), np.zeros((2, 1)))
    assert np.allclose(out, 2.0) and np.allclose(lse, np.log(2.0))
