"""Pins of the oracle's MXFP8 pieces (E8M0 scale decoding, MX block
dequantisation, the OCP MX quantiser) against the format definitions, an
independent conversion through PyTorch's e4m3 type, exact rational scores and
the MX error bound."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def test_e8m0_decode_matches_definition():
    e = np.arange(256)
    v = O.decode_e8m0(e)
    for code in range(255):
        assert v[code] == math.ldexp(1.0, code - 127)
    assert np.isnan(v[255])
    assert v[127] == 1.0 and v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127


def test_mx_dequant_matches_torch_conversion():
    """decode_mx (table x 2^(e-127)) against torch's e4m3 decoder times the
    scale computed with ldexp, on every code and a range of scales."""
    codes = np.tile(np.arange(256, dtype=np.uint8), 4).reshape(32, 32)
    scales = np.array([100, 120, 127, 140] * 8, dtype=np.uint8).reshape(32, 1)
    got = O.decode_mx(codes, scales)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = t * np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert ((got == ref) | (np.isnan(got) & np.isnan(ref))).all()


@pytest.mark.parametrize("mag", [1e-3, 0.1, 1.0, 37.0, 1e4])
def test_mx_quantize_follows_the_definition(mag):
    rng = np.random.default_rng(int(mag * 1000) % 9973)
    x = rng.standard_normal((64, 128)) * mag
    x[3, 32:64] = 0.0                                   # an all-zero block
    codes, sc = O.mx_quantize(x)
    assert codes.shape == x.shape and sc.shape == (64, 4)
    X = O.decode_e8m0(sc)
    P = O.decode_e4m3(codes).reshape(64, 4, 32)
    g = x.reshape(64, 4, 32)
    amax = np.abs(g).max(-1)
    nz = amax > 0
    # the shared scale puts the block maximum in [2^8, 2^9): |P| max in [256, 448]
    assert np.all(np.abs(P).max(-1)[nz] >= 256) and np.all(np.abs(P).max(-1) <= 448)
    assert np.all(amax[nz] / X[nz] >= 256) and np.all(amax[nz] / X[nz] < 512)
    assert sc[3, 1] == 127 and np.all(codes[3, 32:64] == 0)
    # error: half a unit in the last place of e4m3 (3 mantissa bits), except saturation
    dq = P * X[..., None]
    sat = np.abs(g / X[..., None]) > 448
    err = np.abs(dq - g)
    bound = np.maximum(np.abs(g) * 2.0 ** -4, X[..., None] * 2.0 ** -10)
    assert np.all(err[~sat] <= bound[~sat])
    assert np.all(np.abs(P[sat]) == 448)


def test_mx_quantize_agrees_with_an_independent_conversion():
    """The generator's MX quantiser (PyTorch's e4m3 conversion) and the
    oracle's (table search) give the same codes and scales."""
    for seed in range(6):
        x = torch.randn(200, 128, generator=torch.Generator().manual_seed(seed)) * 10.0 ** (seed - 3)
        c, s = W.quantize_mx(x)
        oc, os_ = O.mx_quantize(x.numpy().astype(np.float64))
        assert np.array_equal(c.numpy(), oc) and np.array_equal(s.numpy(), os_)


def test_mx_integers_round_trip_exactly():
    x = np.arange(-8, 9, dtype=np.float64)
    x = np.concatenate([x, x[::-1], np.zeros(2)])[:32]
    rows = np.stack([x, x * 0.5 * 2, np.roll(x, 5), np.where(x > 0, x, 0.0)])
    codes, sc = O.mx_quantize(rows)
    assert np.array_equal(O.decode_mx(codes, sc), rows)


def test_mx_scores_exact_fraction():
    """MXFP8 integer inputs: every score equals the rational evaluation of
    the definition on the original integers."""
    wl = W.CONFIGS[1].with_(dist="int8range", seq_len=48, H_I=8, indexer_dtype="mxfp8")
    b = W.make_batch(wl)
    inp = W.to_numpy(b)
    sc = O.scores_row(inp, 0)
    q = O.indexer_query(inp, 0)
    keys = O.indexer_keys(inp, 0, 48)
    assert np.array_equal(q, np.round(q)) and np.abs(q).max() <= 8
    for s in range(0, 48, 5):
        tot = Fraction(0)
        for j in range(8):
            d = sum(Fraction(int(a)) * Fraction(int(c)) for a, c in zip(q[j], keys[s]))
            tot += Fraction(float(inp["w"][0][j])) * max(d, Fraction(0))
        assert Fraction(float(sc[s])) == tot
