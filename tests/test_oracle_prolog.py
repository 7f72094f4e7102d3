"""Pins of the prolog oracle (oracle/prolog_oracle.py): LayerNorm against
PyTorch's independent implementation and its defining invariants, the fp32
per-token fp8 rule against the input generator's PyTorch quantiser, and bf16
rounding against PyTorch's conversion."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def test_layer_norm_matches_torch_and_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 128)) * 3 + 1.5
    g = rng.standard_normal(128)
    b = rng.standard_normal(128)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (128,), torch.from_numpy(g), torch.from_numpy(b),
                                         eps=1e-6).numpy()
    assert np.allclose(O.layer_norm(x, g, b, 1e-6), ref, atol=1e-12, rtol=1e-12)
    y = O.layer_norm(x, eps=0.0)
    assert np.allclose(y.mean(-1), 0, atol=1e-12) and np.allclose((y ** 2).mean(-1), 1, atol=1e-12)
    # rows of +-a: mean 0, variance a^2, output +-1 exactly
    row = np.array([4.0, -4.0] * 64)
    assert np.array_equal(O.layer_norm(row[None], eps=0.0)[0], row / 4.0)


def test_fp8_token_rule_matches_the_generator():
    for seed in range(4):
        x = torch.randn(30, 8192, generator=torch.Generator().manual_seed(seed)) * 10.0 ** (seed - 1)
        x[3] = 0.0
        codes, scale = W.quantize_e4m3(x, dim=1)
        oc, os_ = O.fp8_token_quantize(x.numpy())
        assert np.array_equal(codes.numpy(), oc) and np.array_equal(scale[:, 0].numpy(), os_)


def test_quantize_q_formats():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 64, 128)).astype(np.float32)
    c, s = O.quantize_q(q, "mxfp8")
    assert c.shape == q.shape and s.shape == (3, 64, 4)
    X = np.repeat(O.decode_e8m0(s), 32, axis=-1)
    sat = np.abs(q / X) > 448
    err = np.abs(O.decode_mx(c, s) - q)
    assert np.all((err <= np.maximum(np.abs(q) * 2 ** -4, X * 2 ** -10))[~sat])
    c, s = O.quantize_q(q, "fp8")
    assert c.shape == q.shape and s.shape == (3,)
    dq = O.decode_e4m3(c) * s[:, None, None]
    assert np.all(np.abs(dq - q) <= np.abs(q) * 2 ** -4 + s[:, None, None] * 2 ** -10)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-5, 5, 5000), [0.0, -0.0, 1.0]])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_round(x32), ref)
