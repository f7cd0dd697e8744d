"""Oracle of block verification (test infrastructure only).

[Blog] "2. Flash Verification" and the loop in "核心创新": the target scores
the context plus the whole draft block in one forward and decides at once how
much of the block to keep; [Note] 整体架构 ends each step with accept/reject;
[Deep] 4.3 defines acceptance length as the mean number of accepted block
tokens.  Row i of the target logits is the target's prediction for block
position i given the tokens before it; row B follows the last block token.

Greedy (temperature 0): a is the first position whose target argmax differs
from the draft token (B if none); the output is the a accepted draft tokens
followed by the target's own token at position a (the bonus), then -1.

Sampled (temperature T > 0): speculative sampling (Leviathan et al. 2023, the
lineage root named in [Note] "与 Speculative Decoding 系列的关系"), which keeps
the output distributed exactly as the target's: p = softmax(z_target/T),
q = softmax(z_draft/T); position i is accepted iff u_i0 * q(d_i) < p(d_i)
(the multiplicative form of u < p/q); at the first rejection the output token
is drawn from max(0, p - q) renormalised; if all B are accepted the bonus is
drawn from p of row B.  Draws use the supplied uniforms u_i1 by inverse CDF:
the smallest k with sum_{v<=k} w_v > u * sum_v w_v.
"""
import numpy as np

F64 = np.float64


def verify_greedy(target_logits, draft_tokens):
    """target_logits [bt, B+1, V]; draft_tokens [bt, B] -> (accept_len [bt], out [bt, B+1])."""
    z = np.asarray(target_logits)
    d = np.asarray(draft_tokens)
    bt, B = d.shape
    y = np.argmax(z, axis=-1)                   # first maximum = lowest index
    acc = np.empty(bt, dtype=np.int64)
    out = np.full((bt, B + 1), -1, dtype=np.int64)
    for b in range(bt):
        a = 0
        while a < B and y[b, a] == d[b, a]:
            a += 1
        acc[b] = a
        out[b, :a] = d[b, :a]
        out[b, a] = y[b, a]
    return acc, out


def _softmax(z, T):
    x = np.asarray(z, F64) / T
    x = x - x.max()
    e = np.exp(x)
    return e / e.sum()


def inverse_cdf(w, u):
    """Smallest k with cumsum(w)[k] > u * sum(w); also returns the distance of
    u*sum(w) to the nearest cumulative boundary, relative to sum(w)."""
    c = np.cumsum(np.asarray(w, F64))
    tot = c[-1]
    t = u * tot
    k = int(np.searchsorted(c, t, side="right"))
    k = min(k, len(c) - 1)
    lo = c[k - 1] if k > 0 else 0.0
    margin = min(abs(t - lo), abs(c[k] - t)) / tot
    return k, margin


def verify_sampled(target_logits, draft_logits, draft_tokens, uniforms, temperature):
    """Lossless speculative-sampling verification.

    target_logits [bt, B+1, V], draft_logits [bt, B, V], draft_tokens [bt, B],
    uniforms [bt, B+1, 2] in [0, 1).  Returns (accept_len, out, margin) where
    margin[b] is the smallest relative distance of any decision this sequence
    took to its threshold (|u q - p| / p for the accept tests, CDF distance
    for the draw); the caller excludes decisions closer than its tolerance.
    """
    zt, zd = np.asarray(target_logits), np.asarray(draft_logits)
    d, U = np.asarray(draft_tokens), np.asarray(uniforms, F64)
    T = float(temperature)
    bt, B = d.shape
    acc = np.empty(bt, dtype=np.int64)
    out = np.full((bt, B + 1), -1, dtype=np.int64)
    margin = np.full(bt, np.inf)
    for b in range(bt):
        a, tok = B, None
        for i in range(B):
            p = _softmax(zt[b, i], T)
            q = _softmax(zd[b, i], T)
            t = int(d[b, i])
            lhs = U[b, i, 0] * q[t]
            margin[b] = min(margin[b], abs(lhs - p[t]) / max(p[t], lhs, 1e-300))
            if lhs < p[t]:
                continue
            a = i
            tok, m = inverse_cdf(np.maximum(p - q, 0.0), U[b, i, 1])
            margin[b] = min(margin[b], m)
            break
        if tok is None:
            tok, m = inverse_cdf(_softmax(zt[b, B], T), U[b, B, 1])
            margin[b] = min(margin[b], m)
        acc[b] = a
        out[b, :a] = d[b, :a]
        out[b, a] = tok
    return acc, out, margin
