"""Device-side step loop: dflash_advance_context against its definition, and a
loop of draft -> verify -> advance -> inject that never returns to the host,
run eagerly and as a replayed HIP graph, against the loop whose injection
lists the host builds from the acceptance lengths.  Tokens, acceptance
lengths and the final pool must be identical bit for bit: the injection GEMMs
split K by N and K only, so a row's K/V do not depend on how many rows share
the call.  The oracle then replays the same trajectory step by step (draft on
the pool the GPU had injected by then, verification against the same target
logits, its own injection of the committed rows), so the device loop is pinned
to the fp64 definition and not only to the host-driven loop."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_drafter_injection_amd import binding as B
from block_diffusion_drafter_injection_amd import synth
from gpu_util import TIE, Drafter, alloc_pool, compare_pool_entries, f64, np_weights, page_plan, unpack_pool

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def test_advance_context_matches_definition():
    rng = np.random.default_rng(7)
    for bt, Bk in [(1, 4), (5, 8), (33, 16)]:
        acc = rng.integers(-2, Bk + 3, size=bt).astype(np.int32)       # out-of-range values are clamped
        ctx = rng.integers(0, 5000, size=bt).astype(np.int32)
        d_acc = torch.from_numpy(acc).cuda()
        d_ctx = torch.from_numpy(ctx).cuda()
        seq = torch.full((bt * (Bk + 1),), 12345, dtype=torch.int32, device="cuda")
        pos = torch.full_like(seq, 12345)
        B.dflash_advance_context(bt, Bk, d_acc, d_ctx, seq, pos)
        torch.cuda.synchronize()
        a = np.clip(acc, 0, Bk)
        j = np.arange(Bk + 1)[None, :]
        want_seq = np.where(j <= a[:, None], np.arange(bt)[:, None], -1).reshape(-1)
        want_pos = (ctx[:, None] + j).reshape(-1)
        assert np.array_equal(seq.cpu().numpy(), want_seq)
        assert np.array_equal(pos.cpu().numpy(), want_pos)
        assert np.array_equal(d_ctx.cpu().numpy(), ctx + a + 1)


class Loop:
    """State of one step loop over a copy of the initial pool."""

    def __init__(self, dims, W, pool0, n_pages, table, ctx0, Bk, S, cap):
        self.dims, self.Bk, self.S, self.cap = dims, Bk, S, cap
        self.bt = len(ctx0)
        self.dr = Drafter(dims, W, max_batch=self.bt, block_size=Bk, max_ctx=cap,
                          max_inject=self.bt * (Bk + 1))
        self.pool = pool0.clone()
        self.n_pages, self.table = n_pages, table
        self.ctx = torch.tensor(ctx0, dtype=torch.int32, device="cuda")
        self.tok = torch.empty(self.bt, Bk, dtype=torch.int32, device="cuda")
        self.acc = torch.empty(self.bt, dtype=torch.int32, device="cuda")
        self.out = torch.empty(self.bt, Bk + 1, dtype=torch.int32, device="cuda")
        self.seq = torch.empty(self.bt * (Bk + 1), dtype=torch.int32, device="cuda")
        self.pos = torch.empty_like(self.seq)
        self.vws_bytes = B.dflash_verify_workspace_size(self.bt, Bk, dims.vocab)
        self.vws = torch.empty(self.vws_bytes, dtype=torch.uint8, device="cuda")

    def draft_verify(self, z, zmax, zmin, coin):
        d = self.dr
        B.dflash_draft_block(d.cfg, d.w, self.pool, self.n_pages, self.table, self.table.shape[1], self.ctx,
                             self.cap, self.bt, self.Bk, self.S, 0.0, 0, self.tok, None, None, d.ws, d.ws_bytes)
        # target logits of this block: position i agrees with the draft token where coin is set
        idx = self.tok.long().unsqueeze(-1)
        keep = z[:, :self.Bk].gather(-1, idx)
        z[:, :self.Bk].scatter_(-1, idx, torch.where(coin, zmax, zmin).unsqueeze(-1))
        B.dflash_verify_block(self.bt, self.Bk, self.dims.vocab, z, self.tok, 0.0, None, None, self.acc, self.out,
                              self.vws, self.vws_bytes)
        z[:, :self.Bk].scatter_(-1, idx, keep)

    def device_advance_inject(self, hid):
        d = self.dr
        B.dflash_advance_context(self.bt, self.Bk, self.acc, self.ctx, self.seq, self.pos)
        B.dflash_inject_kv(d.cfg, d.w, hid, self.seq, self.pos, self.bt * (self.Bk + 1), self.pool, self.n_pages,
                           self.table, self.bt, self.table.shape[1], d.ws, d.ws_bytes)

    def host_advance_inject(self, hid):
        a = self.acc.cpu().numpy().astype(np.int64)
        c = self.ctx.cpu().numpy().astype(np.int64)
        rows = np.concatenate([b * (self.Bk + 1) + np.arange(a[b] + 1) for b in range(self.bt)])
        seq = np.concatenate([np.full(a[b] + 1, b) for b in range(self.bt)]).astype(np.int32)
        pos = np.concatenate([c[b] + np.arange(a[b] + 1) for b in range(self.bt)]).astype(np.int32)
        d = self.dr
        B.dflash_inject_kv(d.cfg, d.w, hid[torch.from_numpy(rows).cuda()].contiguous(),
                           torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), len(seq), self.pool,
                           self.n_pages, self.table, self.bt, self.table.shape[1], d.ws, d.ws_bytes)
        self.ctx.copy_(torch.from_numpy((c + a + 1).astype(np.int32)).cuda())

    def record(self):
        torch.cuda.synchronize()
        return self.tok.cpu().numpy().copy(), self.acc.cpu().numpy().copy(), self.out.cpu().numpy().copy()


def test_device_loop_and_graph_replay_match_host_loop():
    dims = synth.small_dims()
    bt, Bk, S, K = 4, 8, 2, 6
    ctx0 = [40, 77, 16, 131]
    cap = max(ctx0) + (K + 1) * (Bk + 1)
    log(f"device loop: small model, batch {bt}, block {Bk}, {K} steps, contexts {ctx0}")
    W = synth.make_weights(dims, 31, "cuda")
    table_np, n_pages = page_plan([cap] * bt, 0, seed=32)
    table = torch.from_numpy(table_np).cuda()
    pool0 = alloc_pool(dims, n_pages)
    fh = dims.n_fuse * dims.target_hidden
    setup = Drafter(dims, W, max_batch=bt, block_size=Bk, max_ctx=cap, max_inject=sum(ctx0))
    seq0 = torch.from_numpy(np.concatenate([np.full(c, b) for b, c in enumerate(ctx0)]).astype(np.int32)).cuda()
    pos0 = torch.from_numpy(np.concatenate([np.arange(c) for c in ctx0]).astype(np.int32)).cuda()
    setup.inject(synth.make_hiddens(dims, sum(ctx0), 33, "cuda"), seq0, pos0, pool0, n_pages, table, bt)
    hid = [synth.make_hiddens(dims, bt * (Bk + 1), 100 + k, "cuda").view(bt * (Bk + 1), fh) for k in range(K)]
    g = torch.Generator(device="cuda").manual_seed(34)
    z = torch.randn(bt, Bk + 1, dims.vocab, generator=g, device="cuda")
    zmax = z[:, :Bk].amax(-1) + 1.0
    zmin = z[:, :Bk].amin(-1) - 1.0
    coins = [torch.rand(bt, Bk, generator=g, device="cuda") < 0.75 for _ in range(K)]

    host = Loop(dims, W, pool0, n_pages, table, ctx0, Bk, S, cap)
    ref = []
    for k in range(K):
        host.draft_verify(z, zmax, zmin, coins[k])
        ref.append(host.record())
        host.host_advance_inject(hid[k])
    torch.cuda.synchronize()
    log(f"host loop acceptance per step: {[r[1].tolist() for r in ref]}")
    assert sum(int(r[1].sum()) for r in ref) > 0

    dev = Loop(dims, W, pool0, n_pages, table, ctx0, Bk, S, cap)
    for k in range(K):
        dev.draft_verify(z, zmax, zmin, coins[k])
        got = dev.record()
        for a, b in zip(got, ref[k]):
            assert np.array_equal(a, b), f"device loop differs at step {k}"
        dev.device_advance_inject(hid[k])
    torch.cuda.synchronize()
    assert torch.equal(dev.ctx, host.ctx)
    log("device-side loop equals the host loop")

    gl = Loop(dims, W, pool0, n_pages, table, ctx0, Bk, S, cap)
    hid_s = torch.empty_like(hid[0])
    coin_s = torch.empty_like(coins[0])
    hid_s.copy_(hid[0])
    coin_s.copy_(coins[0])
    # warm the libraries on a side stream before capture, then undo its effect on the state
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gl.draft_verify(z, zmax, zmin, coin_s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gl.draft_verify(z, zmax, zmin, coin_s)
        gl.device_advance_inject(hid_s)
    for k in range(K):
        hid_s.copy_(hid[k])
        coin_s.copy_(coins[k])
        graph.replay()
        got = gl.record()
        for a, b in zip(got, ref[k]):
            assert np.array_equal(a, b), f"graph replay differs at step {k}"
    torch.cuda.synchronize()
    assert torch.equal(gl.ctx, host.ctx)
    used = np.unique(table_np[table_np >= 0])
    pa = host.pool.view(n_pages, -1)[used].view(torch.int16)
    for other, name in ((dev, "device loop"), (gl, "graph replay")):
        assert torch.equal(other.pool.view(n_pages, -1)[used].view(torch.int16), pa), f"{name} pool differs"
    log(f"graph replay equals the host loop over {K} steps; pools bitwise equal")

    # The oracle along the same trajectory.  Positions below a sequence's length never
    # change once injected, so the prefix of the final pool is the pool of every earlier
    # step: each oracle draft reads exactly what the GPU draft read.
    Wn = np_weights(W)
    final = [int(c) for c in gl.ctx.cpu().tolist()]
    gkv = [unpack_pool(dims, gl.pool, n_pages, table_np, b, final[b]) for b in range(bt)]
    hid0 = f64(synth.make_hiddens(dims, sum(ctx0), 33, "cuda"))
    own, off = [], 0
    for c in ctx0:
        own.append(oracle.inject(dims, Wn, hid0[off:off + c], np.arange(c)))
        off += c
    zc, zmaxc, zminc = f64(z), f64(zmax), f64(zmin)
    ctx = list(ctx0)
    alive = np.ones(bt, dtype=bool)
    pairs = 0
    for k in range(K):
        pools = [(gkv[b][0][:, :ctx[b]], gkv[b][1][:, :ctx[b]]) for b in range(bt)]
        res = oracle.draft_block(dims, Wn, pools, ctx, Bk, S, want_logits=False)
        tok_o = res["tokens"]
        coin = coins[k].cpu().numpy()
        zk = zc.copy()
        for b in range(bt):
            for i in range(Bk):
                zk[b, i, tok_o[b, i]] = zmaxc[b, i] if coin[b, i] else zminc[b, i]
        a_o, out_o = oracle.verify_greedy(zk, tok_o)
        tok_g, acc_g, out_g = ref[k]
        for b in range(bt):
            if not alive[b]:
                continue
            same = np.array_equal(tok_g[b], tok_o[b]) and acc_g[b] == a_o[b] and np.array_equal(out_g[b], out_o[b])
            if not same:
                near = any(res["gap"][b, s, i] < TIE for s in range(S) for i in range(Bk)
                           if res["committed_at"][b, i] == s) or np.any(res["boundary_gap"][b, :S - 1] < TIE)
                assert near, f"step {k} seq {b}: GPU {tok_g[b]} a={acc_g[b]} oracle {tok_o[b]} a={a_o[b]}"
                alive[b] = False
                continue
            pairs += 1
        hk = f64(hid[k])
        for b in range(bt):
            n = int(a_o[b]) + 1
            Kn, Vn = oracle.inject(dims, Wn, hk[b * (Bk + 1):b * (Bk + 1) + n], np.arange(ctx[b], ctx[b] + n))
            own[b] = (np.concatenate([own[b][0], Kn], 1), np.concatenate([own[b][1], Vn], 1))
            ctx[b] += n
    log(f"oracle replay of the device loop: {pairs} of {K * bt} (step, sequence) pairs bit-exact, "
        f"{int((~alive).sum())} dropped after a near-tie")
    assert pairs >= (K * bt) // 2
    for b in range(bt):
        if alive[b]:
            assert ctx[b] == final[b]
            compare_pool_entries(gkv[b][0], own[b][0], dims.dtype, f"seq {b} K")
            compare_pool_entries(gkv[b][1], own[b][1], dims.dtype, f"seq {b} V")
