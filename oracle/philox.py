"""Counter-based random numbers for the draft's sampling at temperature > 0
(test infrastructure only).

Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw ("Parallel random
numbers: as easy as 1, 2, 3", SC'11): a 4x32-bit counter and a 2x32-bit key
go through ten rounds; each round multiplies counter words 0 and 2 by two
fixed odd constants, swaps the halves of the 64-bit products with the other
two words xor the key, and the key is advanced by two Weyl constants between
rounds.  Both the oracle and the GPU implement it from that definition, so a
draw is a pure function of (seed, counter) on either side.

Gumbel-max sampling (a textbook identity): argmax_v (z_v/T + G_v) with G_v
i.i.d. standard Gumbel is an exact draw from softmax(z/T).  The pages ask for
lossless drafting at high temperature ([Note] 消融实验结论 mentions sampling
at high temperature); how the draft draws its tokens is not stated, and this
is the reading taken.

Counter layout for draft noise: key = (seed mod 2^32, seed >> 32),
counter = (v // 4, position i, denoise step s, sequence b), word v % 4.
u = ((x >> 8) + 0.5) * 2^-24 lies strictly inside (0, 1), G = -ln(-ln u).
"""
import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint32(0x9E3779B9)
W1 = np.uint32(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """ctr: uint32 array [..., 4]; key: uint32 array broadcastable to [..., 2].

    Returns uint32 [..., 4].
    """
    c = np.array(ctr, dtype=np.uint32, copy=True)
    k = np.broadcast_to(np.asarray(key, dtype=np.uint32), c.shape[:-1] + (2,)).copy()
    c0, c1, c2, c3 = (c[..., i].astype(np.uint64) for i in range(4))
    k0, k1 = k[..., 0].astype(np.uint64), k[..., 1].astype(np.uint64)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(W0)) & MASK32
            k1 = (k1 + np.uint64(W1)) & MASK32
        p0 = M0 * c0          # < 2^64, exact in uint64
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def uniform24(x):
    """Map uint32 words to floats strictly inside (0, 1): ((x>>8)+0.5)/2^24."""
    x = np.asarray(x, dtype=np.uint32)
    return ((x >> np.uint32(8)).astype(np.float64) + 0.5) * (2.0 ** -24)


def gumbel_noise(seed, b, s, i, vocab):
    """Standard Gumbel noise G[v], v < vocab, for sequence b, step s, position i."""
    seed = int(seed)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    nblk = (vocab + 3) // 4
    ctr = np.zeros((nblk, 4), dtype=np.uint32)
    ctr[:, 0] = np.arange(nblk, dtype=np.uint32)
    ctr[:, 1] = i
    ctr[:, 2] = s
    ctr[:, 3] = b
    words = philox4x32_10(ctr, key).reshape(-1)[:vocab]
    u = uniform24(words)
    return -np.log(-np.log(u))
