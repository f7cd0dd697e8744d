"""Host logic of the adaptive block size (dflash_adaptive_block_size, CPU only):
the match-probability estimate against draws from the acceptance law it
assumes, and the choice against brute-force expectations over that law."""
import numpy as np
import pytest

from block_diffusion_drafter_injection_amd import binding as B


@pytest.fixture(scope="module")
def L():
    return B.lib()


def draw_acceptance(p, blocks, rng):
    """Leading matches of independent Bernoulli(p) positions, capped at the block."""
    out = []
    for b in blocks:
        match = rng.random(b) < p
        out.append(int(np.argmin(match)) if not match.all() else b)
    return out


def expected_commit_brute(p, b):
    """E[a + 1] by summing over the acceptance law P(a = k) = p^k (1 - p) (k < b), p^b (k = b)."""
    pmf = [p ** k * (1 - p) for k in range(b)] + [p ** b]
    assert abs(sum(pmf) - 1.0) < 1e-12
    return sum((k + 1) * q for k, q in enumerate(pmf))


@pytest.mark.parametrize("p", [0.3, 0.75, 0.92])
def test_estimate_recovers_match_probability(L, p):
    rng = np.random.default_rng(int(p * 100))
    blocks = rng.choice([4, 8, 16], size=20000).tolist()
    acc = draw_acceptance(p, blocks, rng)
    _, est = B.dflash_adaptive_block_size(acc, blocks, [8], [1.0], prior_a=0.0, prior_b=0.0)
    # binomial-type error of the ratio estimate: well under 0.01 at 20000 steps
    assert abs(est - p) < 0.01, (est, p)


def test_choice_maximises_expected_tokens_per_time(L):
    rng = np.random.default_rng(5)
    cands = [4, 8, 16]
    for trial in range(200):
        p = float(rng.uniform(0.05, 0.98))
        times = rng.uniform(1.0, 3.0, size=3).tolist()
        # observations that put the estimate exactly at p: n steps at block 1 with a = 1 or 0
        n = 1000
        ones = int(round(p * n))
        pe = ones / n
        choice, est = B.dflash_adaptive_block_size([1] * ones + [0] * (n - ones), [1] * n, cands, times,
                                                   prior_a=0.0, prior_b=0.0)
        assert abs(est - pe) < 1e-6
        rates = [expected_commit_brute(pe, b) / t for b, t in zip(cands, times)]
        best = cands[int(np.argmax(rates))]
        if sorted(rates)[-1] - sorted(rates)[-2] > 1e-9 * max(rates):
            assert choice == best, (trial, pe, times, rates, choice)


def test_special_cases(L):
    # no observations, no prior: p = 1/2
    c, p = B.dflash_adaptive_block_size([], [], [4, 8], [1.0, 1.0], prior_a=0.0, prior_b=0.0)
    assert p == 0.5 and c == 8
    # every block fully accepted and no prior: p = 1, E[a+1] = B+1; equal times favour the largest block
    c, p = B.dflash_adaptive_block_size([8, 8, 8], [8, 8, 8], [4, 8, 16], [1.0, 1.0, 1.0], prior_a=0.0,
                                        prior_b=0.0)
    assert p == 1.0 and c == 16
    # nothing ever accepted: p = 0, every block commits one token; the fastest wins
    c, p = B.dflash_adaptive_block_size([0, 0], [16, 16], [4, 8, 16], [3.0, 2.0, 2.5], prior_a=0.0, prior_b=0.0)
    assert p == 0.0 and c == 8
    # equal rates: the smaller block
    c, _ = B.dflash_adaptive_block_size([0], [4], [16, 4], [1.0, 1.0], prior_a=0.0, prior_b=0.0)
    assert c == 4
    # the prior alone sets the estimate
    _, p = B.dflash_adaptive_block_size([], [], [4], [1.0], prior_a=3.0, prior_b=1.0)
    assert abs(p - 0.75) < 1e-7


def test_argument_errors(L):
    f = L.dflash_adaptive_block_size
    import ctypes
    i32, f32 = ctypes.c_int32, ctypes.c_float
    a, b = (i32 * 1)(3), (i32 * 1)(4)
    c, t = (i32 * 1)(8), (f32 * 1)(1.0)
    assert f(a, b, 1, c, t, 1, 1.0, 1.0, None) == 8
    assert f(None, b, 1, c, t, 1, 1.0, 1.0, None) == -1          # NULL with a count
    assert f(a, b, 1, c, t, 0, 1.0, 1.0, None) == -1             # no candidate
    assert f(a, b, 1, c, (f32 * 1)(0.0), 1, 1.0, 1.0, None) == -1   # time not > 0
    assert f(a, b, 1, c, t, 1, -1.0, 1.0, None) == -1            # negative prior
    assert f((i32 * 1)(5), b, 1, c, t, 1, 1.0, 1.0, None) == -1  # a > its block
    assert f(a, (i32 * 1)(17), 1, c, t, 1, 1.0, 1.0, None) == -4  # block past 16
    assert f(a, b, 1, (i32 * 1)(0), t, 1, 1.0, 1.0, None) == -4  # candidate block 0
