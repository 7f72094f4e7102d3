"""Pins of the oracle's tile-scaled fp8 latent cache (e4m3 codes, one fp32
scale per 128-element tile of each row; "Day0 Inference Adaptation and
Performance Optimization for Kimi K3.1 Pro", section 4, and "Large Language
Model Inference Acceleration in Practice", section 4)."""
import numpy as np
import torch

import oracle as O
import workloads as W


def _e4m3_value(code: int) -> float:
    """The OCP e4m3 definition written out: sign, 4-bit exponent (bias 7),
    3-bit mantissa, subnormals at exponent 0, S.1111.111 = NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_tile_boundaries_and_the_short_last_tile():
    codes = np.full((1, 576), 0x38, dtype=np.uint8)          # every element 1.0
    scales = np.array([[1.0, 2.0, 4.0, 8.0, 16.0]], dtype=np.float32)
    rows = O.decode_tile_scaled(codes, scales)
    expect = np.repeat([1.0, 2.0, 4.0, 8.0, 16.0], [128, 128, 128, 128, 64])
    assert np.array_equal(rows[0], expect)
    assert rows[0, 127] == 1.0 and rows[0, 128] == 2.0 and rows[0, 511] == 8.0 and rows[0, 512] == 16.0


def test_decode_matches_the_format_definition():
    g = np.random.default_rng(3)
    codes = g.integers(0, 256, size=(7, 576)).astype(np.uint8)
    codes[codes & 0x7F == 0x7F] = 0x00                        # no NaN codes
    scales = g.uniform(0.01, 3.0, size=(7, 5)).astype(np.float32)
    rows = O.decode_tile_scaled(codes, scales)
    for i in range(7):
        for c in range(0, 576, 7):
            assert rows[i, c] == _e4m3_value(int(codes[i, c])) * float(scales[i, c // 128])


def test_equal_tile_scales_reduce_to_a_per_row_scale():
    """A row whose five tile scales are all s is the per-token fp8 row with
    factor s: the attention of both caches is the same number."""
    wl = W.CONFIGS[1].with_(seq_len=700, K=64, name="tile_reduce", seed=5)
    b = W.make_batch(wl.with_(kv_dtype="fp8_tile128"), device="cpu")
    inp = W.to_numpy(b)
    sl = O.slots(inp, 0, np.arange(700))
    s = inp["kv_scale"][sl].astype(np.float64)
    const = inp.copy()
    const["kv_scale"] = np.repeat(s[:, :1], 5, axis=1).astype(np.float32)   # tile scales all = tile 0's
    per_row = inp.copy()
    per_row.update(kv_dtype="fp8", kv_scale_group=1,
                   kv_scale=np.zeros(inp["kv_data"].shape[0], dtype=np.float32))
    per_row["kv_scale"][sl] = s[:, 0]
    idx = np.arange(0, 700, 11)
    o1, l1 = O.attend_row(const, 0, idx)
    o2, l2 = O.attend_row(per_row, 0, idx)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_generated_tiles_round_trip():
    """The generator's tiles decode to the original values within e4m3's
    half-ulp (2^-4 relative below the tile maximum, subnormals absolute)."""
    x = torch.randn(33, 576, dtype=torch.float64) * torch.logspace(-3, 2, 576, dtype=torch.float64)
    codes, sc = W.generate.quantize_tiles(x.to(torch.float32), 128)
    rows = O.decode_tile_scaled(codes.numpy(), sc.numpy())
    xs = x.to(torch.float32).double().numpy()
    s = np.repeat(sc.numpy().astype(np.float64), [128, 128, 128, 128, 64], axis=1)
    err = np.abs(rows - xs)
    assert (err <= np.abs(xs) * 2.0 ** -4 + s * 2.0 ** -10 * 1.0001).all()
    amax = np.abs(xs).reshape(33, -1)[:, :128].max(axis=1)
    assert np.allclose(sc.numpy()[:, 0], amax / 448.0, rtol=1e-6)


def test_integer_rows_are_exact():
    wl = W.CONFIGS[0].with_(kv_dtype="fp8_tile128", D_latent=512, D_rope=64, name="tile_int", seed=9)
    b = W.make_batch(wl, device="cpu")
    assert set(np.unique(b.kv_scale.numpy()[~np.isnan(b.kv_scale.numpy())])) <= {0.5, 1.0, 2.0}
    inp = W.to_numpy(b)
    bf = W.to_numpy(W.make_batch(wl.with_(kv_dtype="bf16"), device="cpu"))
    sl = O.slots(inp, 0, np.arange(256))
    assert np.array_equal(O.latent_rows(inp, 0, np.arange(256)), O.latent_rows(bf, 0, np.arange(256))), sl[:3]
