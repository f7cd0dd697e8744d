"""The closed drafter loop, with a target model in it instead of synthetic logits and
hidden states: draft a block (its first position the last committed token) ->
dflash_target_forward over the block (full logits, the captured layer outputs, the
block's K/V appended to the target's cache) -> dflash_verify_block on those logits ->
dflash_advance_context -> dflash_inject_kv of the captured states of the a+1 tokens the
target has now processed -> the next draft, anchored on the bonus token.  Only the
initial contexts are synthetic.

Every step is checked call by call against the oracle chain on identical inputs
(oracle.draft_block on the draft pool the GPU had injected by then, oracle.target_forward
on the target cache it had by then, oracle.verify_greedy on the oracle's own logits,
oracle.inject of the GPU's captured rows).  Entries at positions below a sequence's
committed length never change once written, so the final pools' prefixes are every
earlier step's pools."""
import time
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from block_diffusion_drafter_injection_amd import binding as B
from block_diffusion_drafter_injection_amd import synth
from gpu_util import (TIE, Drafter, alloc_pool, compare_draft, compare_forward_outputs, compare_pool_entries,
                      f64, pack_pool, page_plan, unpack_pool)

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def np64(W):
    return {k: ([t.double().cpu().numpy() for t in v] if isinstance(v, list) else v.double().cpu().numpy())
            for k, v in W.items()}


def run_gpu(dd, td, Wd, Wt, ctx0, steps, Bk, S, caps, seed):
    """The loop on the GPU.  ctx0[b] committed tokens to start with, the last of them the
    first anchor; both pools hold positions 0 .. ctx0[b]-2 (synthetic setup)."""
    bt = len(ctx0)
    inj0 = [c - 1 for c in ctx0]
    grow = (steps + 1) * Bk
    table, n_pages = page_plan(inj0, grow, seed=seed)
    tab = torch.from_numpy(table).cuda()
    pool_d = alloc_pool(dd, n_pages)
    pool_t = alloc_pool(td, n_pages)
    cap = max(inj0) + grow
    dr = Drafter(dd, Wd, max_batch=bt, block_size=Bk, max_ctx=cap, max_inject=max(sum(inj0), bt * Bk))
    seq0 = torch.from_numpy(np.concatenate([np.full(c, b) for b, c in enumerate(inj0)]).astype(np.int32)).cuda()
    pos0 = torch.from_numpy(np.concatenate([np.arange(c) for c in inj0]).astype(np.int32)).cuda()
    dr.inject(synth.make_hiddens(dd, sum(inj0), seed, "cuda"), seq0, pos0, pool_d, n_pages, tab, bt)
    Kt, Vt = synth.make_pool_values(td, sum(inj0), seed + 1, "cuda")
    off = 0
    for b, c in enumerate(inj0):
        pack_pool(td, pool_t, n_pages, table, b, Kt[:, off:off + c], Vt[:, off:off + c])
        off += c
    del Kt, Vt
    tcfg, tw = B.make_config(td), B.Weights(Wt)
    tws_bytes = B.dflash_workspace_size(tcfg, bt, Bk, 0, cap)
    tws = torch.empty(tws_bytes, dtype=torch.uint8, device="cuda")
    vws_bytes = B.dflash_verify_workspace_size(bt, Bk - 1, td.vocab)
    vws = torch.empty(vws_bytes, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(seed + 2)
    anchor = torch.randint(0, dd.vocab, (bt,), generator=g, device="cuda", dtype=torch.int32)
    ctx = torch.tensor(inj0, dtype=torch.int32, device="cuda")
    F = len(caps)
    z = torch.empty(bt, Bk, td.vocab, dtype=torch.float32, device="cuda")
    hid = torch.empty(bt, Bk, F * td.hidden, dtype=torch.bfloat16, device="cuda")
    acc = torch.empty(bt, dtype=torch.int32, device="cuda")
    out = torch.empty(bt, Bk, dtype=torch.int32, device="cuda")
    seq = torch.empty(bt * Bk, dtype=torch.int32, device="cuda")
    pos = torch.empty_like(seq)
    rec = []
    for st in range(steps):
        r = dict(inj=ctx.cpu().numpy().copy(), anchor=anchor.cpu().numpy().copy())
        tok, _, _ = dr.draft(pool_d, n_pages, tab, ctx, cap, Bk, S, want_logits=False, anchor=anchor)
        B.dflash_target_forward(tcfg, tw, pool_t, n_pages, tab, table.shape[1], ctx, cap, bt, Bk, tok, caps, z, hid,
                                tws, tws_bytes)
        drafted = tok[:, 1:].contiguous()
        B.dflash_verify_block(bt, Bk - 1, td.vocab, z, drafted, 0.0, None, None, acc, out, vws, vws_bytes)
        B.dflash_advance_context(bt, Bk - 1, acc, ctx, seq, pos)
        B.dflash_inject_kv(dr.cfg, dr.w, hid.view(bt * Bk, F * td.hidden), seq, pos, bt * Bk, pool_d, n_pages, tab,
                           bt, table.shape[1], dr.ws, dr.ws_bytes)
        anchor = out.gather(1, acc.long().unsqueeze(1)).squeeze(1).contiguous()
        torch.cuda.synchronize()
        r.update(tok=tok.cpu().numpy(), z=z.cpu().numpy(), hid=f64(hid), acc=acc.cpu().numpy().copy(),
                 out=out.cpu().numpy().copy())
        rec.append(r)
    final = ctx.cpu().numpy()
    return dict(rec=rec, final=final, pool_d=pool_d, pool_t=pool_t, table=table, n_pages=n_pages)


def check_oracle(dd, td, Wd, Wt, g, Bk, S, caps, sample, forward_rule):
    """The oracle chain along the GPU's trajectory for the sequences in `sample`."""
    table, n_pages = g["table"], g["n_pages"]
    steps = len(g["rec"])
    end = {b: int(g["final"][b]) + Bk for b in sample}
    gd = {b: unpack_pool(dd, g["pool_d"], n_pages, table, b, int(g["final"][b])) for b in sample}
    gt = {b: unpack_pool(td, g["pool_t"], n_pages, table, b, end[b]) for b in sample}
    alive = {b: True for b in sample}
    stats = dict(pairs=0, dropped=0, accepted=0)
    t0 = time.time()
    for st, r in enumerate(g["rec"]):
        live = [b for b in sample if alive[b]]
        if not live:
            break
        inj = [int(r["inj"][b]) for b in live]
        # draft on the GPU's draft pool, anchored on the GPU's anchor
        res = oracle.draft_block(dd, Wd, [(gd[b][0][:, :c], gd[b][1][:, :c]) for b, c in zip(live, inj)], inj, Bk,
                                 S, want_logits=False, anchor=r["anchor"][live])
        # target forward on the GPU's target cache over the GPU's block
        zo, ho, Ko, Vo = oracle.target_forward(td, Wt, [(gt[b][0][:, :c], gt[b][1][:, :c]) for b, c in zip(live, inj)],
                                               inj, r["tok"][live], capture_layers=caps)
        a_o, out_o = oracle.verify_greedy(zo, r["tok"][live][:, 1:])
        for k, b in enumerate(live):
            tok_g = r["tok"][b]
            tie_d = any(res["gap"][k, s, i] < TIE for s in range(S) for i in range(1, Bk)
                        if res["committed_at"][k, i] == s) or np.any(res["boundary_gap"][k, :S - 1] < TIE)
            top2 = np.sort(zo[k], axis=-1)[:, -2:]
            tie_t = bool(np.any(top2[:, 1] - top2[:, 0] < TIE))
            same = np.array_equal(tok_g, res["tokens"][k]) and r["acc"][b] == a_o[k] and \
                np.array_equal(r["out"][b], out_o[k])
            if not same:
                assert tie_d or tie_t, (f"step {st} seq {b}: GPU {tok_g} a={r['acc'][b]} {r['out'][b]}, oracle "
                                        f"{res['tokens'][k]} a={a_o[k]} {out_o[k]} without a near-tie")
                alive[b] = False
                stats["dropped"] += 1
                continue
            # target logits within tolerance, captured states and appended K/V by the forward rule
            zg = r["z"][b].astype(np.float64)
            rel = np.max(np.abs(zg - zo[k]), axis=-1) / np.max(np.abs(zo[k]), axis=-1)
            assert rel.max() <= 2e-2, (st, b, rel.max())
            forward_rule(r["hid"][b], ho[k], f"step {st} seq {b} captured")
            c, a = inj[k], int(a_o[k])
            forward_rule(gt[b][0][:, c:c + a + 1], Ko[:, k, :a + 1], f"step {st} seq {b} appended K")
            forward_rule(gt[b][1][:, c:c + a + 1], Vo[:, k, :a + 1], f"step {st} seq {b} appended V")
            # injection of the GPU's captured rows 0..a (identical inputs)
            Kn, Vn = oracle.inject(dd, Wd, r["hid"][b][:a + 1], np.arange(c, c + a + 1))
            compare_pool_entries(gd[b][0][:, c:c + a + 1], Kn, dd.dtype, f"step {st} seq {b} injected K")
            compare_pool_entries(gd[b][1][:, c:c + a + 1], Vn, dd.dtype, f"step {st} seq {b} injected V")
            stats["pairs"] += 1
            stats["accepted"] += a
        if st % 4 == 0:
            log(f"  oracle chain step {st}/{steps}: {stats} ({time.time() - t0:.1f}s)")
    return stats


def test_closed_loop_small_shape():
    """Draft: the small bf16 shape over a vocabulary of 4 (random-init models then agree
    often enough for acceptances above 0; the LM head then has a single partial column
    tile).  Target: 4 random-init layers of width 384 (the draft's fused-layer width),
    layers 0, 2, 3 captured.  Batch 6, block 8 (anchor + 7), 12 steps, every sequence
    checked every step.  Captured states and appended K/V come out of a multi-layer
    forward, so they are held to the multi-layer rule."""
    V = 4
    dd = synth.small_dims(vocab=V)
    td = synth.ModelDims(hidden=384, n_layers=4, n_q_heads=4, n_kv_heads=2, head_dim=128, intermediate=768,
                         vocab=V, n_fuse=1, target_hidden=384, rope_base=1e6)
    caps, Bk, S, steps, seed = [0, 2, 3], 8, 2, 12, 61
    ctx0 = [2, 17, 40, 77, 150, 33]
    Wd = synth.make_weights(dd, seed, "cuda")
    Wt = synth.make_weights(td, seed + 5, "cuda", std=0.05)
    t0 = time.time()
    g = run_gpu(dd, td, Wd, Wt, ctx0, steps, Bk, S, caps, seed)
    accs = np.array([r["acc"] for r in g["rec"]])
    log(f"closed loop on the GPU: {time.time() - t0:.1f}s, acceptance per step {accs.tolist()}")
    assert np.all((accs >= 0) & (accs <= Bk - 1))
    assert np.array_equal(g["final"], np.array(ctx0) - 1 + (accs + 1).sum(0))
    stats = check_oracle(dd, td, np64(Wd), np64(Wt), g, Bk, S, caps, list(range(len(ctx0))),
                         compare_forward_outputs)
    log(f"closed loop vs oracle chain: {stats}")
    assert stats["pairs"] >= steps * len(ctx0) // 2
    assert accs.sum() > 0


def test_closed_loop_8b_layer_shape():
    """The Qwen3-8B-shaped draft (5 layers, five fused layers of 4096) fed by a random-init
    target with Qwen3-8B layers (6 of them, layers 0, 1, 2, 4, 5 captured), batch 8, block
    16 (anchor + 15), contexts of a few hundred to a thousand tokens, 8 steps; the oracle
    chain checks three sequences every step."""
    dd = synth.QWEN3_8B_SHAPE
    td = replace(synth.QWEN3_8B_SHAPE, n_layers=6, n_fuse=1)
    caps, Bk, S, steps, seed = [0, 1, 2, 4, 5], 16, 2, 8, 71
    rng = np.random.default_rng(seed)
    ctx0 = rng.integers(200, 1100, size=8).tolist()
    t0 = time.time()
    Wd = synth.make_weights(dd, seed, "cuda")
    Wt = synth.make_weights(td, seed + 5, "cuda")
    g = run_gpu(dd, td, Wd, Wt, ctx0, steps, Bk, S, caps, seed)
    accs = np.array([r["acc"] for r in g["rec"]])
    log(f"closed loop on the GPU: {time.time() - t0:.1f}s, acceptance per step {accs.tolist()}")
    assert np.all((accs >= 0) & (accs <= Bk - 1))
    sample = [0, int(np.argmin(ctx0)), int(np.argmax(ctx0))]
    sample = sorted(set(sample))
    Wd64, Wt64 = np64(Wd), np64(Wt)
    log(f"oracle weights ready {time.time() - t0:.1f}s; sequences {sample}")
    stats = check_oracle(dd, td, Wd64, Wt64, g, Bk, S, caps, sample, compare_forward_outputs)
    log(f"closed loop vs oracle chain: {stats} {time.time() - t0:.1f}s")
    assert stats["pairs"] >= steps * len(sample) // 2
