"""Pins of the oracle's verification and counter-based sampling (CPU only)."""
import itertools
import os

import numpy as np
import pytest

import oracle
import brute


def test_greedy_one_hot_target_accepts_whole_block():
    rng = np.random.default_rng(0)
    bt, B, V = 5, 8, 50
    d = rng.integers(0, V, (bt, B))
    z = rng.standard_normal((bt, B + 1, V))
    for b in range(bt):
        for i in range(B):
            z[b, i] = 0.0
            z[b, i, d[b, i]] = 1.0
    acc, out = oracle.verify_greedy(z, d)
    assert np.all(acc == B)
    assert np.array_equal(out[:, :B], d) and np.array_equal(out[:, B], np.argmax(z[:, B], -1))


def test_greedy_all_mismatched_gives_zero_and_target_token():
    rng = np.random.default_rng(1)
    bt, B, V = 4, 6, 30
    z = rng.standard_normal((bt, B + 1, V))
    d = (np.argmax(z[:, :B], -1) + 1) % V
    acc, out = oracle.verify_greedy(z, d)
    assert np.all(acc == 0)
    assert np.array_equal(out[:, 0], np.argmax(z[:, 0], -1)) and np.all(out[:, 1:] == -1)


def test_greedy_matches_brute_by_enumeration():
    """Every draft block over a 3-token vocabulary with B = 3, against rows with ties."""
    z = np.array([[[0.1, 0.7, 0.7], [2.0, -1.0, 0.0], [0.0, 0.0, 0.0], [1.0, 3.0, 2.0]]])
    for d in itertools.product(range(3), repeat=3):
        d = np.array([d])
        acc, out = oracle.verify_greedy(z, d)
        ab, ob = brute.greedy_verify(z.tolist(), d.tolist())
        assert acc.tolist() == ab and out.tolist() == ob
        assert 0 <= acc[0] <= 3


def test_greedy_acceptance_range_property():
    rng = np.random.default_rng(2)
    for B in (1, 4, 8, 16):
        z = rng.standard_normal((20, B + 1, 7))
        d = rng.integers(0, 7, (20, B))
        acc, out = oracle.verify_greedy(z, d)
        assert np.all((acc >= 0) & (acc <= B))
        for b in range(20):
            a = acc[b]
            assert np.array_equal(out[b, :a], d[b, :a]) and out[b, a] >= 0 and np.all(out[b, a + 1:] == -1)


def test_inverse_cdf_brute():
    rng = np.random.default_rng(3)
    for _ in range(200):
        w = rng.random(9) * (rng.random(9) > 0.3)
        if w.sum() == 0:
            continue
        u = rng.random()
        k, _ = oracle.inverse_cdf(w, u)
        run = 0.0
        for j, x in enumerate(w):
            run += x
            if run > u * w.sum():
                break
        assert k == j and w[k] > 0


def test_sampled_equal_distributions_accept_everything():
    rng = np.random.default_rng(4)
    bt, B, V = 6, 8, 40
    zd = rng.standard_normal((bt, B, V))
    zt = np.concatenate([zd, rng.standard_normal((bt, 1, V))], axis=1)
    d = rng.integers(0, V, (bt, B))
    U = rng.random((bt, B + 1, 2))
    acc, out, _ = oracle.verify_sampled(zt, zd, d, U, 1.0)
    assert np.all(acc == B)


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


@pytest.mark.parametrize("T", [1.0, 0.5])
def test_sampled_output_law_is_target_distribution(T):
    """Integrate over the draft token (drawn from q) and a midpoint grid of both
    uniforms: the first output token must be distributed exactly as p."""
    rng = np.random.default_rng(5)
    V, B = 4, 1
    zd = rng.standard_normal((1, B, V)) * 1.5
    zt = rng.standard_normal((1, B + 1, V)) * 1.5
    p, q = _softmax(zt[0, 0] / T), _softmax(zd[0, 0] / T)
    n = 200
    grid = (np.arange(n) + 0.5) / n
    law = np.zeros(V)
    for dtok in range(V):
        for u0 in grid:
            for u1 in grid[::4]:
                U = np.array([[[u0, u1], [0.5, 0.5]]])
                acc, out, _ = oracle.verify_sampled(zt, zd, np.array([[dtok]]), U, T)
                law[out[0, 0]] += q[dtok] / (n * len(grid[::4]))
    assert np.allclose(law, p, atol=3.0 / n * 4)
    # closed form of the same law: q*min(1,p/q) + (1 - sum min(p,q)) * residual
    res = np.maximum(p - q, 0)
    closed = np.minimum(p, q) + (1 - np.minimum(p, q).sum()) * res / res.sum()
    assert np.allclose(closed, p, rtol=1e-12)


def test_sampled_low_temperature_reduces_to_greedy():
    rng = np.random.default_rng(6)
    bt, B, V = 8, 6, 25
    zt = rng.standard_normal((bt, B + 1, V)) * 3
    d = np.argmax(zt[:, :B], -1)
    flip = rng.random((bt, B)) < 0.3
    d = np.where(flip, (d + 1) % V, d)
    zd = np.zeros((bt, B, V))
    zd[np.arange(bt)[:, None], np.arange(B)[None, :], d] = 3.0        # draft one-hot-ish on d
    U = rng.random((bt, B + 1, 2)) * 0.98 + 0.01
    acc, out, _ = oracle.verify_sampled(zt, zd, d, U, 1e-3)
    acc_g, out_g = oracle.verify_greedy(zt, d)
    assert np.array_equal(acc, acc_g) and np.array_equal(out, out_g)


def test_philox_known_answer_vectors():
    """Known-answer vectors published with the Random123 library (Salmon et al., SC'11),
    stored in tests/golden/philox4x32_10_kat.txt."""
    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        w = [int(x, 16) for x in r]
        assert oracle.philox4x32_10(w[0:4], w[4:6]).tolist() == w[6:10]


def test_uniform_map_stays_inside_unit_interval():
    x = np.array([0, 255, 256, 0xFFFFFFFF], dtype=np.uint32)
    u = oracle.uniform24(x)
    assert np.all((u > 0) & (u < 1))
    assert u[0] == u[1] == 0.5 * 2.0 ** -24 and u[3] == 1 - 0.5 * 2.0 ** -24


def test_gumbel_max_frequencies_follow_softmax():
    """Chi-square test: argmax(z + G) over many independent counters ~ softmax(z)."""
    z = np.array([0.0, 1.0, -0.5, 2.0, 0.3])
    p = _softmax(z)
    n = 20000
    counts = np.zeros(len(z))
    for b in range(n):
        counts[np.argmax(z + oracle.gumbel_noise(77, b, 0, 0, len(z)))] += 1
    chi2 = ((counts - n * p) ** 2 / (n * p)).sum()
    assert chi2 < 20.5        # 4 degrees of freedom, p-value ~ 4e-4
