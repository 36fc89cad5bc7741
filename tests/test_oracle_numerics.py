"""Pins for the oracle's building blocks: closed forms, invariants and library routines."""
import numpy as np
import pytest
import torch

from oracle.numerics import (apply_rope, bf16_bits_to_float, l2_normalize, rmsnorm,
                             round_to_bf16, silu, softmax)


def test_bf16_round_to_nearest_even_closed_forms():
    one = 1.0
    ulp = 2.0 ** -7                                   # bf16 spacing in [1, 2)
    cases = {
        one: one,
        one + ulp / 2: one,                           # tie, 1.0 has even mantissa
        one + 3 * ulp / 2: one + 2 * ulp,             # tie, goes to the even neighbour
        one + ulp / 2 + 2.0 ** -20: one + ulp,        # just above the tie
        one + ulp / 2 - 2.0 ** -20: one,              # just below the tie
        -(one + 3 * ulp / 2): -(one + 2 * ulp),
        0.0: 0.0,
    }
    for x, want in cases.items():
        assert round_to_bf16(np.array([x]))[0] == want, x


def test_bf16_round_matches_torch_library():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        rng.standard_normal(1000)]).astype(np.float32)
    ours = round_to_bf16(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, lib)


def test_bf16_bits_decode():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x3F81], dtype=np.uint16)
    np.testing.assert_array_equal(bf16_bits_to_float(bits), [1.0, -1.0, 2.0, 0.0, 1.0 + 2 ** -7])


def test_rmsnorm_constant_vector_and_library():
    c, eps = 3.0, 1e-6
    x = np.full(64, c)
    g = np.linspace(0.5, 1.5, 64)
    np.testing.assert_allclose(rmsnorm(x, g, eps), c / np.sqrt(c * c + eps) * g, rtol=1e-15)
    rng = np.random.default_rng(0)
    X = rng.standard_normal((5, 96))
    G = rng.standard_normal(96)
    lib = torch.nn.functional.rms_norm(torch.from_numpy(X), (96,), torch.from_numpy(G), eps).numpy()
    np.testing.assert_allclose(rmsnorm(X, G, eps), lib, rtol=1e-12, atol=1e-14)


def _rope_complex(x, pos, theta):
    """Textbook complex form: pair (x_i, x_{i+hd/2}) as x_i + i*x_{i+hd/2}, times e^{i pos w_i}."""
    hd = x.shape[-1]
    half = hd // 2
    w = theta ** (-2.0 * np.arange(half) / hd)
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * pos * w)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_identity_norm_and_complex_form():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 80))
    np.testing.assert_array_equal(apply_rope(x, 0, 10000.0), x)
    for pos in (1, 17, 2047, 8191):
        y = apply_rope(x, pos, 10000.0)
        np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
        np.testing.assert_allclose(y, _rope_complex(x, pos, 10000.0), rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_only_on_offset():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    s = [apply_rope(q[None], m + 5, 1e4)[0] @ apply_rope(k[None], m, 1e4)[0] for m in (0, 11, 300)]
    np.testing.assert_allclose(s, s[0], rtol=1e-11)


def test_rope_batched_positions_match_scalar():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 3, 16))
    pos = np.arange(6) * 7
    y = apply_rope(x, pos, 500.0)
    for r in range(6):
        np.testing.assert_array_equal(y[r], apply_rope(x[r], pos[r], 500.0))


def test_silu_softmax_l2():
    x = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-13)
    assert silu(np.array([0.0]))[0] == 0.0
    s = softmax(np.array([1.0, 1.0, 1.0, 1.0]))
    np.testing.assert_allclose(s, 0.25)
    np.testing.assert_allclose(softmax(x), torch.softmax(torch.from_numpy(x), 0).numpy(), rtol=1e-12)
    v = np.random.default_rng(4).standard_normal((3, 80))
    np.testing.assert_allclose(np.linalg.norm(l2_normalize(v, 0.0), axis=-1), 1.0, rtol=1e-14)
