"""Scalar building blocks of the oracle, in float64 (test infrastructure only).

* bf16_round: round-to-nearest-even of an fp64 value straight to bfloat16
  (8 significant bits, fp32's exponent range).  It is applied only where the
  GPU stores bfloat16: KV-pool writes and the LM-head input.
* rope: rotary position embedding, rotate-half pairing (x_j, x_{j+d/2}),
  frequency base^(-2j/d), angle = position * frequency.  The pages say only
  that context reaches the draft through its K/V ([Note] 三大核心创新 §2);
  rotary positions are the reading taken for a Qwen3-shaped draft.
* rmsnorm: x / sqrt(mean(x^2) + eps) * gain.
* silu, logsumexp, log_softmax: textbook definitions.
"""
import numpy as np

F64 = np.float64


def bf16_round(x):
    """Nearest bfloat16 value of ``x`` (ties to even), returned as float64.

    frexp gives x = m * 2**e with 0.5 <= |m| < 1; bfloat16 keeps 8
    significant bits, so m*256 is rounded to an integer (np.rint rounds
    halves to even) and scaled back.  Subnormal bfloat16 values are not
    needed by any workload here (magnitudes stay far above 2**-126).
    """
    x = np.asarray(x, dtype=F64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def rope_angles(pos, d, base):
    """Angles [..., d/2]: pos * base**(-2j/d) for j < d/2, in float64."""
    j = np.arange(d // 2, dtype=F64)
    freq = np.power(F64(base), -2.0 * j / d)
    return np.asarray(pos, dtype=F64)[..., None] * freq


def rope(x, pos, base):
    """Rotate each (x_j, x_{j+d/2}) pair of the last axis by angle pos*freq_j.

    ``pos`` broadcasts against x[..., 0].
    """
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    th = rope_angles(pos, d, base)
    c, s = np.cos(th), np.sin(th)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rmsnorm(x, gain, eps):
    x = np.asarray(x, dtype=F64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(gain, dtype=F64)


def silu(x):
    return x / (1.0 + np.exp(-x))


def logsumexp(z, axis=-1):
    z = np.asarray(z, dtype=F64)
    m = np.max(z, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=axis, keepdims=True))).squeeze(axis)


def log_softmax(z, axis=-1):
    z = np.asarray(z, dtype=F64)
    return z - np.expand_dims(logsumexp(z, axis), axis)


def split_hilo(x):
    """(hi, lo) with hi = bf16(x) and lo = bf16(x - hi): used only by tests that
    bound the error of a two-term bfloat16 operand against fp64."""
    hi = bf16_round(x)
    return hi, bf16_round(np.asarray(x, F64) - hi)
