"""Pins of the oracle's injection and draft: brute-force twins on tiny shapes,
closed forms and invariants (CPU only)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from oracle import bf16_round, rmsnorm, rope
from block_diffusion_drafter_injection_amd import synth
import brute

TINY = synth.ModelDims(hidden=32, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=8, intermediate=48,
                       vocab=37, n_fuse=2, target_hidden=16, rope_base=1e4, dtype="bf16")


def np_weights(dims, seed, std=0.02):
    W = synth.make_weights(dims, seed, "cpu", std=std)
    out = {}
    for k, v in W.items():
        if isinstance(v, list):
            out[k] = [t.float().numpy().astype(np.float64) for t in v]
        else:
            out[k] = v.float().numpy().astype(np.float64)
    return out


def np_hiddens(dims, n, seed):
    return synth.make_hiddens(dims, n, seed).float().numpy().astype(np.float64)


def rand_pool(dims, T, seed, scale=1.0):
    K, V = synth.make_pool_values(dims, T, seed, k_std=scale, v_std=scale)
    return K.float().numpy().astype(np.float64), V.float().numpy().astype(np.float64)


def with_qk_gains(dims, W, seed):
    """Random (non-unit) QK-norm gains, so a swapped or misplaced gain changes the result."""
    rng = np.random.default_rng(seed)
    W = dict(W)
    W["q_norm"] = [1.0 + 0.3 * rng.standard_normal(dims.head_dim) for _ in range(dims.n_layers)]
    W["k_norm"] = [1.0 + 0.3 * rng.standard_normal(dims.head_dim) for _ in range(dims.n_layers)]
    return W


@pytest.mark.parametrize("dtype,qk", [("bf16", False), ("fp32", False), ("bf16", True), ("fp32", True)])
def test_inject_matches_brute(dtype, qk):
    dims = replace(TINY, dtype=dtype, qk_norm=qk)
    W = np_weights(dims, 11, std=0.3)
    if qk:
        W = with_qk_gains(dims, W, 111)
    x = np_hiddens(dims, 6, 12)
    pos = np.array([0, 1, 5, 16, 17, 300])
    K, V = oracle.inject(dims, W, x, pos)
    Kb, Vb = brute.inject(dims, W, x.tolist(), pos.tolist())
    assert np.allclose(K, np.array(Kb), rtol=1e-12, atol=1e-12)
    assert np.allclose(V, np.array(Vb), rtol=1e-12, atol=1e-12)
    if dtype == "bf16":
        assert np.array_equal(bf16_round(K), K) and np.array_equal(bf16_round(V), V)


def test_qk_norm_closed_forms():
    # unit gains: every stored key head has rms 1 (RoPE is a rotation, so it keeps the norm)
    dims = replace(TINY, dtype="fp32", qk_norm=True)
    W = np_weights(dims, 17, std=0.3)
    x = np_hiddens(dims, 9, 18)
    K, V = oracle.inject(dims, W, x, np.arange(100, 109))
    rms = np.sqrt(np.mean(K * K, axis=-1))
    # the fp64 head norm misses 1 only by the eps inside the root: rms = r / sqrt(r^2 + eps)
    kv = (W["w_kv"] @ (W["w_fc"] @ x.T)).T.reshape(9, dims.n_layers, 2, dims.n_kv_heads, dims.head_dim)
    r2 = np.mean(kv[:, :, 0] ** 2, axis=-1).transpose(1, 0, 2)
    assert np.allclose(rms, np.sqrt(r2 / (r2 + dims.rms_eps)), rtol=1e-12)
    # values are untouched by QK-norm
    _, V0 = oracle.inject(replace(dims, qk_norm=False), W, x, np.arange(100, 109))
    assert np.array_equal(V, V0)
    # query and key scaled by any positive factor give the same normalised head (up to eps)
    Wq = dict(W)
    Wq["w_kv"] = W["w_kv"] * 4.0
    K4, _ = oracle.inject(dims, Wq, x, np.arange(100, 109))
    assert np.allclose(K4, K, rtol=1e-6, atol=1e-9)


def test_incremental_injection_equals_one_shot():
    W = np_weights(TINY, 13, std=0.3)
    x = np_hiddens(TINY, 40, 14)
    pos = np.arange(40)
    K1, V1 = oracle.inject(TINY, W, x, pos)
    parts = [(0, 17), (17, 18), (18, 29), (29, 40)]
    Ks, Vs = zip(*[oracle.inject(TINY, W, x[a:b], pos[a:b]) for a, b in parts])
    assert np.array_equal(np.concatenate(Ks, axis=1), K1)
    assert np.array_equal(np.concatenate(Vs, axis=1), V1)


def test_inject_position_zero_is_unrotated_projection():
    W = np_weights(TINY, 15, std=0.3)
    x = np_hiddens(TINY, 1, 16)
    K, V = oracle.inject(TINY, W, x, np.array([0]))
    kv = (W["w_kv"] @ (W["w_fc"] @ x[0])).reshape(TINY.n_layers, 2, TINY.n_kv_heads, TINY.head_dim)
    assert np.array_equal(K[:, 0], bf16_round(kv[:, 0]))
    assert np.array_equal(V[:, 0], bf16_round(kv[:, 1]))


def test_attention_closed_forms():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((6, 16)) * 3
    keys = rng.standard_normal((50, 16)) * 3
    vals = rng.standard_normal((50, 16))
    o, p = oracle.attention_group(q, keys, vals, 0.25, return_probs=True)
    assert np.allclose(p.sum(-1), 1.0, rtol=1e-14)                     # rows sum to 1
    assert np.all(p >= 0)
    o1 = oracle.attention_group(q, keys[:1], vals[:1], 0.25)
    assert np.allclose(o1, np.broadcast_to(vals[0], o1.shape), rtol=1e-15)   # one key -> its value
    oe = oracle.attention_group(q, np.tile(keys[:1], (50, 1)), vals, 0.25)
    assert np.allclose(oe, np.broadcast_to(vals.mean(0), oe.shape), rtol=1e-13)  # equal keys -> mean
    oz = oracle.attention_group(np.zeros_like(q), keys, vals, 0.25)
    assert np.allclose(oz, np.broadcast_to(vals.mean(0), oz.shape), rtol=1e-13)  # zero query -> mean
    perm = rng.permutation(50)
    assert np.allclose(oracle.attention_group(q, keys[perm], vals[perm], 0.25), o, rtol=1e-13)


@pytest.mark.parametrize("dtype,qk", [("bf16", False), ("fp32", False), ("bf16", True), ("fp32", True)])
def test_forward_matches_brute(dtype, qk):
    dims = replace(TINY, dtype=dtype, qk_norm=qk)
    W = np_weights(dims, 21, std=0.3)
    if qk:
        W = with_qk_gains(dims, W, 121)
    ctx = [0, 5, 11]
    pools = [rand_pool(dims, T, 30 + T, scale=2.0) for T in ctx]
    rng = np.random.default_rng(22)
    tau = rng.integers(0, dims.vocab, size=(3, 4))
    tau[0, 1] = dims.mask_token_id
    y = oracle.forward_hidden(dims, W, pools, ctx, tau)
    yb = np.array(brute.forward(dims, W, pools, ctx, tau.tolist()))
    if dtype == "bf16":
        # both round the same fp64 value to bf16; a rounding-boundary case could differ by
        # one bf16 ulp, so require equality on all but a tiny fraction and closeness everywhere
        assert np.mean(y != yb) < 0.01
        assert np.allclose(y, yb, rtol=2 ** -7, atol=0)
    else:
        assert np.allclose(y, yb, rtol=1e-10, atol=1e-12)


def test_forward_closed_form_without_mixing():
    """w_o = 0 and w_down = 0 make every layer a no-op: y = store(RMSNorm(E[tau]))."""
    W = np_weights(TINY, 23, std=0.3)
    for l in range(TINY.n_layers):
        W["w_o"][l] = np.zeros_like(W["w_o"][l])
        W["w_down"][l] = np.zeros_like(W["w_down"][l])
    W["final_norm"] = np.linspace(0.5, 1.5, TINY.hidden)
    pools = [rand_pool(TINY, 9, 40)]
    tau = np.array([[3, 36, 0, 36]])
    y = oracle.forward_hidden(TINY, W, pools, [9], tau)
    ref = bf16_round(rmsnorm(W["embed"][tau[0]], W["final_norm"], TINY.rms_eps))
    assert np.array_equal(y[0], ref)


def test_forward_uniform_attention_closed_form():
    """With w_q = 0 every score is 0, so each head's output is the plain mean of
    its kv head's values over all context tokens and all block tokens."""
    dims = replace(TINY, n_layers=1, dtype="fp32", hidden=32, n_q_heads=4, head_dim=8, n_kv_heads=2)
    W = np_weights(dims, 24, std=0.3)
    W["w_q"][0] = np.zeros_like(W["w_q"][0])
    W["w_o"][0] = np.eye(dims.hidden)            # n_q*d == hidden: o goes straight to the residual
    W["w_down"][0] = np.zeros_like(W["w_down"][0])
    W["attn_norm"][0] = np.ones(dims.hidden)
    T = 7
    Kc, Vc = rand_pool(dims, T, 41)
    tau = np.array([[1, 2, 36]])
    y = oracle.forward_hidden(dims, W, [(Kc, Vc)], [T], tau)
    h0 = W["embed"][tau[0]]
    u = rmsnorm(h0, np.ones(dims.hidden), dims.rms_eps)
    nkvd = dims.n_kv_heads * dims.head_dim
    vblk = (u @ W["w_kv"][nkvd:2 * nkvd].T).reshape(3, dims.n_kv_heads, dims.head_dim)
    allv = np.concatenate([Vc[0], vblk], axis=0)           # [T+B, n_kv, d]
    mean = allv.mean(0)                                    # [n_kv, d]
    g = dims.n_q_heads // dims.n_kv_heads
    o = np.concatenate([mean[n // g] for n in range(dims.n_q_heads)])
    ref = rmsnorm(h0 + o, W["final_norm"], dims.rms_eps)
    assert np.allclose(y[0], ref, rtol=1e-12, atol=1e-13)


def test_single_step_denoise_is_forward_plus_argmax():
    W = np_weights(TINY, 25, std=0.3)
    pools = [rand_pool(TINY, T, 50 + T) for T in (4, 13)]
    r = oracle.draft_block(TINY, W, pools, [4, 13], block_size=5, n_steps=1)
    tau0 = np.full((2, 5), TINY.mask_token_id)
    y = oracle.forward_hidden(TINY, W, pools, [4, 13], tau0)
    z = y.reshape(10, -1) @ W["lm_head"].T
    assert np.array_equal(r["tokens"].reshape(-1), np.argmax(z, -1))
    assert np.allclose(r["logits"].reshape(10, -1), z, rtol=1e-13)
    lse = np.log(np.exp(z - z.max(-1, keepdims=True)).sum(-1)) + z.max(-1)
    assert np.allclose(r["conf"][:, 0].reshape(-1), z.max(-1) - lse, rtol=1e-12)


def test_two_step_commit_schedule():
    W = np_weights(TINY, 26, std=0.3)
    pools = [rand_pool(TINY, T, 60 + T) for T in (0, 3, 20)]
    B, S = 5, 2
    r = oracle.draft_block(TINY, W, pools, [0, 3, 20], block_size=B, n_steps=S)
    assert oracle.commit_counts(B, S) == [2, 3]
    assert oracle.commit_counts(16, 2) == [8, 8] and oracle.commit_counts(4, 3) == [1, 1, 2]
    for b in range(3):
        ca = r["committed_at"][b]
        assert sorted(ca.tolist()) == [0, 0, 1, 1, 1]
        first = np.nonzero(ca == 0)[0]
        # step 0 commits the two most confident positions (ties to the lower position)
        c0 = r["conf"][b, 0]
        order = sorted(range(B), key=lambda i: (-c0[i], i))
        assert sorted(order[:2]) == first.tolist()
        assert np.array_equal(r["tokens"][b, first], r["cand"][b, 0, first])
        # committed positions are not re-predicted at step 1
        assert np.all(np.isnan(r["conf"][b, 1, first])) and np.all(r["cand"][b, 1, first] == -1)
        rest = np.nonzero(ca == 1)[0]
        assert np.array_equal(r["tokens"][b, rest], r["cand"][b, 1, rest])
    # step 1 is the forward of the partly committed block
    tau1 = np.where(r["committed_at"] == 0, r["tokens"], TINY.mask_token_id)
    y = oracle.forward_hidden(TINY, W, pools, [0, 3, 20], tau1)
    z = y @ W["lm_head"].T
    rest = r["committed_at"] == 1
    assert np.array_equal(r["tokens"][rest], np.argmax(z, -1)[rest])


def test_repredict_schedule_is_iterated_forward_plus_argmax():
    # every re-predict step is one forward of the previous step's tokens (the
    # first of the all-[MASK] block) and an argmax; forwards by the loop twin
    W = np_weights(TINY, 27, std=0.3)
    ctx = [2, 11]
    pools = [rand_pool(TINY, T, 70 + T) for T in ctx]
    B, S = 4, 3
    r = oracle.draft_block(TINY, W, pools, ctx, block_size=B, n_steps=S, schedule="repredict")
    tau = np.full((2, B), TINY.mask_token_id)
    for s in range(S):
        y = np.array(brute.forward(TINY, W, pools, ctx, tau))
        z = y @ W["lm_head"].T
        assert np.array_equal(r["cand"][:, s], np.argmax(z, -1)), s
        lse = np.log(np.exp(z - z.max(-1, keepdims=True)).sum(-1)) + z.max(-1)
        assert np.allclose(r["conf"][:, s], z.max(-1) - lse, rtol=1e-9, atol=1e-12)
        tau = np.argmax(z, -1)
    assert np.array_equal(r["tokens"], tau)
    assert np.allclose(r["logits"], z, rtol=1e-9, atol=1e-12)
    assert np.all(r["committed_at"] == S - 1) and np.all(np.isinf(r["boundary_gap"]))


def test_repredict_special_cases():
    W = np_weights(TINY, 28, std=0.3)
    ctx = [0, 9]
    pools = [rand_pool(TINY, T, 80 + T) for T in ctx]
    # one step: both readings are a single forward plus argmax
    a = oracle.draft_block(TINY, W, pools, ctx, block_size=6, n_steps=1, schedule="repredict")
    b = oracle.draft_block(TINY, W, pools, ctx, block_size=6, n_steps=1)
    assert np.array_equal(a["tokens"], b["tokens"]) and np.array_equal(a["logits"], b["logits"])
    assert np.array_equal(a["conf"], b["conf"])
    # token-independent embeddings: the block's input never changes, so re-predicting is a no-op
    W1 = dict(W)
    W1["embed"] = np.repeat(W["embed"][:1], TINY.vocab, axis=0)
    r = oracle.draft_block(TINY, W1, pools, ctx, block_size=6, n_steps=3, schedule="repredict")
    for s in (1, 2):
        assert np.array_equal(r["cand"][:, s], r["cand"][:, 0])
        assert np.array_equal(r["conf"][:, s], r["conf"][:, 0])
    with pytest.raises(ValueError):
        oracle.draft_block(TINY, W, pools, ctx, block_size=6, n_steps=1, schedule="other")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_target_forward_matches_brute(dtype):
    dims = replace(TINY, dtype=dtype)
    W = np_weights(dims, 31, std=0.3)
    ctx = [0, 7]
    pools = [rand_pool(dims, T, 90 + T, scale=2.0) for T in ctx]
    tok = np.random.default_rng(32).integers(0, dims.vocab, size=(2, 5))
    z, _, _, _ = oracle.target_forward(dims, W, pools, ctx, tok)
    yb = np.array(brute.forward(dims, W, pools, ctx, tok.tolist(), causal=True))
    zb = yb @ W["lm_head"].T
    scale = np.max(np.abs(zb), axis=-1, keepdims=True)
    # the LM-head input is rounded to bf16 on both sides; a rounding-boundary case may differ by one ulp
    assert np.max(np.abs(z - zb) / scale) < (2e-2 if dtype == "bf16" else 1e-10)


def test_target_forward_causality_and_closed_forms():
    dims = replace(TINY, dtype="fp32")
    W = np_weights(dims, 33, std=0.3)
    ctx = [3, 12]
    pools = [rand_pool(dims, T, 95 + T, scale=2.0) for T in ctx]
    tok = np.random.default_rng(34).integers(0, dims.vocab, size=(2, 6))
    L = dims.n_layers
    z, hid, K, V = oracle.target_forward(dims, W, pools, ctx, tok, capture_layers=(0, L - 1))
    # causal: dropping later tokens leaves the earlier rows unchanged
    z3, hid3, K3, V3 = oracle.target_forward(dims, W, pools, ctx, tok[:, :3], capture_layers=(0, L - 1))
    for a, b in ((z3, z[:, :3]), (hid3, hid[:, :3]), (K3, K[:, :, :3]), (V3, V[:, :, :3])):
        assert np.allclose(a, b, rtol=1e-11, atol=1e-12)
    # one token: causal and bidirectional attention coincide
    y1 = oracle.forward_hidden(dims, W, pools, ctx, tok[:, :1])
    assert np.allclose(z[:, :1], y1 @ W["lm_head"].T, rtol=1e-10, atol=1e-12)
    # the last captured layer is the residual the final norm reads
    H = dims.hidden
    assert np.allclose(rmsnorm(hid[..., H:], W["final_norm"], dims.rms_eps) @ W["lm_head"].T, z, rtol=1e-9,
                       atol=1e-10)
    # layer-0 keys and values come straight from the embedding: RoPE(Wk RMSNorm(E[t])), Wv RMSNorm(E[t])
    nkv, d = dims.n_kv_heads, dims.head_dim
    u = rmsnorm(W["embed"][tok], W["attn_norm"][0], dims.rms_eps)
    kv0 = u @ W["w_kv"][:2 * nkv * d].T
    pos = np.array(ctx)[:, None] + np.arange(6)[None, :]
    k0 = rope(kv0[..., :nkv * d].reshape(2, 6, nkv, d), pos[:, :, None], dims.rope_base)
    assert np.allclose(K[0], k0, rtol=1e-11, atol=1e-12)
    assert np.allclose(V[0], kv0[..., nkv * d:].reshape(2, 6, nkv, d), rtol=1e-11, atol=1e-12)


def test_lm_head_ties_pick_lowest_index():
    W = np_weights(TINY, 27, std=0.3)
    W["lm_head"][9] = W["lm_head"][30]
    W["lm_head"][4] = W["lm_head"][30]
    W["lm_head"][30] *= 1.0
    # make row 30 (and its copies 4 and 9) dominant for every input: scale it up
    for i in (4, 9, 30):
        W["lm_head"][i] = W["lm_head"][30] * 0 + 5.0 * np.sign(np.arange(TINY.hidden) % 2 - 0.5)
    W["final_norm"] = np.ones(TINY.hidden)
    pools = [rand_pool(TINY, 6, 70)]
    # force y to correlate with the tied row: embeddings of the mask equal that direction
    W["embed"][TINY.mask_token_id] = np.sign(np.arange(TINY.hidden) % 2 - 0.5)
    for l in range(TINY.n_layers):
        W["w_o"][l][:] = 0
        W["w_down"][l][:] = 0
    r = oracle.draft_block(TINY, W, pools, [6], block_size=3, n_steps=1)
    assert np.all(r["tokens"] == 4)


def test_temperature_draws_are_gumbel_max():
    W = np_weights(TINY, 28, std=0.3)
    pools = [rand_pool(TINY, T, 80 + T) for T in (2, 9)]
    T = 0.7
    r = oracle.draft_block(TINY, W, pools, [2, 9], block_size=4, n_steps=1, temperature=T, seed=1234)
    tau0 = np.full((2, 4), TINY.mask_token_id)
    z = oracle.forward_hidden(TINY, W, pools, [2, 9], tau0) @ W["lm_head"].T
    for b in range(2):
        for i in range(4):
            g = oracle.gumbel_noise(1234, b, 0, i, TINY.vocab)
            tok = int(np.argmax(z[b, i] / T + g))
            assert r["tokens"][b, i] == tok
            zt = z[b, i] / T
            assert np.isclose(r["conf"][b, 0, i], zt[tok] - oracle.logsumexp(zt), rtol=1e-12)


def test_synthetic_match_rate_gives_truncated_geometric_acceptance():
    """E[a] = p(1-p^B)/(1-p) when every target row agrees with the draft token
    independently with probability p (rows after a mismatch do not count)."""
    p, B, V, n = 0.75, 8, 64, 4000
    draft = torch.randint(0, V, (n, B), generator=torch.Generator().manual_seed(0))
    z = synth.make_greedy_target_logits(draft, V, p, seed=9)
    acc, _ = oracle.verify_greedy(z.numpy(), draft.numpy())
    expect = p * (1 - p ** B) / (1 - p)
    sd = np.std(acc) / np.sqrt(n)
    assert abs(acc.mean() - expect) < 4 * sd


@pytest.mark.parametrize("chunk", [1, 7, 16, 36, 37, 100])
def test_lm_head_chunks_match_explicit_dots(chunk):
    """The LM head is computed over vocabulary chunks; every column of every row, whatever
    the chunk size (one column, ragged last chunk, one chunk, larger than the vocabulary),
    equals the plain dot product of the row with that vocabulary row, summed by a loop."""
    W = np_weights(TINY, 29, std=0.3)
    rng = np.random.default_rng(31)
    y = rng.standard_normal((3, TINY.hidden))
    z = oracle.lm_head_logits(TINY, W, y, chunk=chunk)
    assert z.shape == (3, TINY.vocab)
    for r in range(3):
        for v in range(TINY.vocab):
            ref = 0.0
            for c in range(TINY.hidden):
                ref += float(y[r, c]) * float(W["lm_head"][v, c])
            assert abs(z[r, v] - ref) <= 1e-12 * max(1.0, abs(ref)), (r, v, chunk)


def test_lm_head_default_chunks_over_a_large_vocabulary():
    """A vocabulary spanning three default chunks (16384 columns each, ragged last one):
    the chunked product equals one whole-matrix product, and the columns on both sides of
    each chunk edge equal their explicit dot products."""
    dims = replace(TINY, hidden=8, vocab=2 * 16384 + 5)
    rng = np.random.default_rng(32)
    W = {"lm_head": rng.standard_normal((dims.vocab, dims.hidden))}
    y = rng.standard_normal((4, dims.hidden))
    z = oracle.lm_head_logits(dims, W, y)
    assert np.allclose(z, y @ W["lm_head"].T, rtol=1e-13, atol=1e-13)
    for v in (0, 16383, 16384, 16385, 32767, 32768, dims.vocab - 1):
        for r in range(4):
            ref = sum(float(y[r, c]) * float(W["lm_head"][v, c]) for c in range(dims.hidden))
            assert abs(z[r, v] - ref) <= 1e-12 * max(1.0, abs(ref)), (r, v)


def test_anchored_single_step_is_forward_plus_argmax():
    """With an anchor, block position 0 holds the given token from the start: one step
    equals the brute-force forward of [anchor, MASK, ...] plus argmax on positions 1..B-1,
    and position 0 keeps the anchor."""
    W = np_weights(TINY, 33, std=0.3)
    ctx = [4, 13]
    pools = [rand_pool(TINY, T, 90 + T) for T in ctx]
    anchor = np.array([5, 17])
    B = 5
    r = oracle.draft_block(TINY, W, pools, ctx, block_size=B, n_steps=1, anchor=anchor)
    tau0 = np.full((2, B), TINY.mask_token_id)
    tau0[:, 0] = anchor
    y = np.array(brute.forward(TINY, W, pools, ctx, tau0.tolist()))
    z = y @ W["lm_head"].T
    assert np.array_equal(r["tokens"][:, 0], anchor)
    assert np.array_equal(r["tokens"][:, 1:], np.argmax(z[:, 1:], -1))
    assert np.all(r["committed_at"][:, 0] == -1) and np.all(r["committed_at"][:, 1:] == 0)
    assert np.all(np.isnan(r["conf"][:, 0, 0])) and np.all(r["cand"][:, 0, 0] == -1)


@pytest.mark.parametrize("B,S", [(8, 2), (5, 2), (16, 3), (4, 3)])
def test_anchored_progressive_schedule_commits_over_the_open_positions(B, S):
    W = np_weights(TINY, 34, std=0.3)
    ctx = [0, 7, 21]
    pools = [rand_pool(TINY, T, 95 + T) for T in ctx]
    anchor = np.array([1, 36, 12])
    r = oracle.draft_block(TINY, W, pools, ctx, block_size=B, n_steps=S, anchor=anchor)
    want = oracle.commit_counts(B - 1, S)
    assert sum(want) == B - 1
    for b in range(3):
        assert r["tokens"][b, 0] == anchor[b] and r["committed_at"][b, 0] == -1
        got = [int(np.sum(r["committed_at"][b] == s)) for s in range(S)]
        assert got == want
        for s in range(S):
            assert np.isnan(r["conf"][b, s, 0])            # the anchor is never open
            done = r["committed_at"][b] < s
            done[0] = True
            assert np.all(np.isnan(r["conf"][b, s][done]))
            assert not np.any(np.isnan(r["conf"][b, s][~done]))


def test_anchored_repredict_keeps_the_anchor():
    W = np_weights(TINY, 35, std=0.3)
    ctx = [3, 9]
    pools = [rand_pool(TINY, T, 97 + T) for T in ctx]
    anchor = np.array([2, 30])
    r1 = oracle.draft_block(TINY, W, pools, ctx, block_size=6, n_steps=1, anchor=anchor, schedule="repredict")
    p1 = oracle.draft_block(TINY, W, pools, ctx, block_size=6, n_steps=1, anchor=anchor)
    assert np.array_equal(r1["tokens"], p1["tokens"])
    r3 = oracle.draft_block(TINY, W, pools, ctx, block_size=6, n_steps=3, anchor=anchor, schedule="repredict")
    assert np.array_equal(r3["tokens"][:, 0], anchor)
    # each step re-predicts positions 1.. from the previous step's block, the anchor kept
    tau = np.full((2, 6), TINY.mask_token_id)
    tau[:, 0] = anchor
    for s in range(3):
        y = np.array(brute.forward(TINY, W, pools, ctx, tau.tolist()))
        tau[:, 1:] = np.argmax(y @ W["lm_head"].T, -1)[:, 1:]
        assert np.array_equal(r3["cand"][:, s, 1:], tau[:, 1:])
    assert np.array_equal(r3["tokens"], tau)
