"""Pins of the oracle's scalar pieces against library routines, closed forms and
independent formulations (CPU only)."""
import cmath
import math

import numpy as np
import pytest
import torch

from oracle import bf16_round, rope, rmsnorm, silu, logsumexp, log_softmax, split_hilo


def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 20, 200_000))).astype(np.float32)
    # add exact halfway cases: bf16 value + half an ulp, both parities
    base = torch.from_numpy(x[:1000]).to(torch.bfloat16).float().numpy().astype(np.float64)
    m, e = np.frexp(base)
    half = np.ldexp(np.ones_like(base), e - 9)
    ties = (base + np.sign(base) * half).astype(np.float32)
    assert np.all(ties.astype(np.float64) == base + np.sign(base) * half)  # exact in fp32
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_is_idempotent_and_monotone():
    rng = np.random.default_rng(1)
    x = np.sort(rng.standard_normal(100_000) * 10)
    r = bf16_round(x)
    assert np.array_equal(bf16_round(r), r)
    assert np.all(np.diff(r) >= 0)
    assert np.max(np.abs(r - x) / np.abs(x)) <= 2.0 ** -8   # half an ulp of an 8-bit significand


def test_hilo_split_error_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(100_000)
    hi, lo = split_hilo(x)
    assert np.max(np.abs(hi + lo - x) / np.abs(x)) <= 2.0 ** -16


def _rope_complex(x, p, base):
    """Independent formulation: pair (x_j, x_{j+d/2}) as a complex number times e^{i p w_j}."""
    d = len(x)
    out = np.empty(d)
    for j in range(d // 2):
        w = base ** (-2.0 * j / d)
        z = complex(x[j], x[j + d // 2]) * cmath.exp(1j * p * w)
        out[j], out[j + d // 2] = z.real, z.imag
    return out


@pytest.mark.parametrize("d,base", [(8, 1e4), (64, 1e4), (128, 1e6)])
def test_rope_against_complex_rotation(d, base):
    rng = np.random.default_rng(d)
    for p in [0, 1, 7, 4095, 32767]:
        x = rng.standard_normal(d)
        # the angle p*w carries a relative rounding of ~1e-16, i.e. ~1e-16*p absolute
        assert np.allclose(rope(x, p, base), _rope_complex(x, p, base), rtol=0, atol=1e-15 * (10 + p))


def test_rope_invariants():
    rng = np.random.default_rng(3)
    d, base = 128, 1e6
    x = rng.standard_normal((5, d))
    assert np.array_equal(rope(x, np.zeros(5), base), x)                       # position 0: identity
    y = rope(x, np.array([3, 100, 2048, 9000, 32000]), base)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n, c in [(5, 2, 100), (4100, 17, 3000), (0, 31000, 1234)]:
        a = rope(q, m, base) @ rope(k, n, base)
        b = rope(q, m + c, base) @ rope(k, n + c, base)
        assert abs(a - b) <= 1e-9 * (np.linalg.norm(q) * np.linalg.norm(k))  # relative position only


def test_rmsnorm_closed_form():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 256)) * 5 + 1
    u = rmsnorm(x, np.ones(256), 0.0)
    assert np.allclose(np.sqrt(np.mean(u * u, axis=-1)), 1.0, rtol=1e-14)
    assert np.allclose(rmsnorm(3.5 * x, np.ones(256), 0.0), u, rtol=1e-14)   # scale invariance
    g = rng.standard_normal(256)
    assert np.allclose(rmsnorm(x, g, 0.0), u * g, rtol=1e-14)
    # eps enters under the root: one-element row x -> x / sqrt(x^2 + eps)
    assert np.isclose(rmsnorm(np.array([[2.0]]), [1.0], 1e-6)[0, 0], 2.0 / math.sqrt(4.0 + 1e-6))


def test_activation_and_softmax_pieces_match_libraries():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(1000) * 8
    assert np.allclose(silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-15)
    z = rng.standard_normal((4, 3000)) * 30
    from scipy.special import logsumexp as sp_lse
    assert np.allclose(logsumexp(z), sp_lse(z, axis=-1), rtol=1e-14)
    assert np.allclose(np.exp(log_softmax(z)).sum(-1), 1.0, rtol=1e-13)
