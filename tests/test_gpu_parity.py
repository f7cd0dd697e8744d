"""GPU parity of the three C-ABI calls against the fp64 oracle on seeded inputs
at sizes the oracle finishes in seconds: several GEMM / attention tiles,
ragged contexts (0, partial pages, many pages), ragged vocabulary."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_drafter_injection_amd import binding as Bn
from block_diffusion_drafter_injection_amd import synth
from gpu_util import (Drafter, alloc_pool, compare_draft, compare_pool_entries, ctx_tensor, f64, np_weights,
                      pack_pool, page_plan, unpack_pool, verify)

pytestmark = pytest.mark.gpu

SMALL = synth.small_dims()


def _dims(name):
    return {"tiny": synth.TINY, "small": SMALL}[name]


def _with_qk(dims, W, seed):
    """QK-norm on, with random (non-unit) gains so a misplaced gain shows."""
    from dataclasses import replace
    dims = replace(dims, qk_norm=True)
    g = torch.Generator(device="cpu").manual_seed(seed)
    W = dict(W)
    for k in ("q_norm", "k_norm"):
        W[k] = [(1.0 + 0.3 * torch.randn(dims.head_dim, generator=g)).float().cuda() for _ in range(dims.n_layers)]
    return dims, W


def _tokens(ctx, device="cuda"):
    seq = np.concatenate([np.full(c, b) for b, c in enumerate(ctx)]).astype(np.int32)
    pos = np.concatenate([np.arange(c) for c in ctx]).astype(np.int32)
    return torch.from_numpy(seq).to(device), torch.from_numpy(pos).to(device)


@pytest.mark.parametrize("name,ctx,chunk,qk", [("tiny", [64], 4096, False), ("small", [37, 0, 70, 131], 64, False),
                                               ("small", [5, 300], 4096, False), ("tiny", [64, 20], 4096, True),
                                               ("small", [37, 150], 64, True)])
def test_inject_matches_oracle(name, ctx, chunk, qk):
    dims = _dims(name)
    W = synth.make_weights(dims, 7, "cuda")
    if qk:
        dims, W = _with_qk(dims, W, 70)
    table, n_pages = page_plan(ctx, 0, seed=3)
    tab = torch.from_numpy(table).cuda()
    pool = alloc_pool(dims, n_pages)
    hid = synth.make_hiddens(dims, sum(ctx), 8, "cuda")
    seq, pos = _tokens(ctx)
    dr = Drafter(dims, W, max_batch=len(ctx), block_size=8, max_ctx=max(ctx), max_inject=chunk)
    dr.inject(hid, seq, pos, pool, n_pages, tab, len(ctx))
    torch.cuda.synchronize()
    Wn = np_weights(W)
    x = f64(hid)
    off = 0
    for b, c in enumerate(ctx):
        if c == 0:
            continue
        Ko, Vo = oracle.inject(dims, Wn, x[off:off + c], np.arange(c))
        K, V = unpack_pool(dims, pool, n_pages, table, b, c)
        compare_pool_entries(K, Ko, dims.dtype, f"K b={b}")
        compare_pool_entries(V, Vo, dims.dtype, f"V b={b}")
        off += c


def test_incremental_injection_is_bitwise_one_shot():
    dims = SMALL
    W = synth.make_weights(dims, 9, "cuda")
    ctx = [150, 97]
    table, n_pages = page_plan(ctx, 0, seed=4)
    tab = torch.from_numpy(table).cuda()
    hid = synth.make_hiddens(dims, sum(ctx), 10, "cuda")
    seq, pos = _tokens(ctx)
    dr = Drafter(dims, W, max_batch=2, block_size=8, max_ctx=150, max_inject=4096)
    one = alloc_pool(dims, n_pages)
    dr.inject(hid, seq, pos, one, n_pages, tab, 2)
    inc = alloc_pool(dims, n_pages)
    n = seq.numel()
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(0)).cuda()  # any order, any split
    for a, b in [(0, 1), (1, 60), (60, 61), (61, 200), (200, n)]:
        idx = perm[a:b]
        dr.inject(hid[idx].contiguous(), seq[idx].contiguous(), pos[idx].contiguous(), inc, n_pages, tab, 2)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), inc.view(torch.int16))


@pytest.mark.parametrize("ctx,n_decoy", [([150, 97], 120), ([700, 600], 900)])
def test_injection_skips_marked_rows_bitwise(ctx, n_decoy):
    """Rows with tok_seq = -1 are dropped before the GEMMs (packed out on the device):
    the same rows with decoys marked -1 spread among them (decoys aim at positions the real
    rows write, so a decoy that got through would change the pool) give the one-shot pool
    bit for bit; a call whose rows are all marked leaves the pool untouched.  The larger
    case has more than 1024 rows, so the packing runs over several blocks."""
    dims = SMALL
    W = synth.make_weights(dims, 11, "cuda")
    table, n_pages = page_plan(ctx, 0, seed=6)
    tab = torch.from_numpy(table).cuda()
    hid = synth.make_hiddens(dims, sum(ctx), 12, "cuda")
    seq, pos = _tokens(ctx)
    n = seq.numel()
    dr = Drafter(dims, W, max_batch=len(ctx), block_size=8, max_ctx=max(ctx), max_inject=n + n_decoy)
    one = alloc_pool(dims, n_pages)
    dr.inject(hid, seq, pos, one, n_pages, tab, len(ctx))
    g = torch.Generator().manual_seed(n_decoy)
    total = n + n_decoy
    real_at = torch.sort(torch.randperm(total, generator=g)[:n]).values   # keeps the real rows' order
    is_real = torch.zeros(total, dtype=torch.bool)
    is_real[real_at] = True
    mseq = torch.full((total,), -1, dtype=torch.int32)
    mpos = pos.cpu()[torch.randint(0, n, (total,), generator=g)].to(torch.int32)
    mhid = synth.make_hiddens(dims, total, 13, "cuda")
    mseq[real_at] = seq.cpu()
    mpos[real_at] = pos.cpu()
    mhid[real_at.cuda()] = hid
    assert (~is_real).sum().item() == n_decoy
    mixed = alloc_pool(dims, n_pages)
    dr.inject(mhid, mseq.cuda(), mpos.cuda(), mixed, n_pages, tab, len(ctx))
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), mixed.view(torch.int16))
    # every row marked: nothing is written
    before = mixed.clone()
    dr.inject(mhid, torch.full_like(mseq, -1).cuda(), mpos.cuda(), mixed, n_pages, tab, len(ctx))
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), mixed.view(torch.int16))


def _draft_case(dims, ctx, B, S, T, seed, want_logits=True, schedule="progressive", qk=False, anchor=None):
    W = synth.make_weights(dims, seed, "cuda")
    if qk:
        dims, W = _with_qk(dims, W, seed + 5)
    table, n_pages = page_plan(ctx, 0, seed=seed + 1)
    tab = torch.from_numpy(table).cuda()
    pool = alloc_pool(dims, n_pages)
    K, V = synth.make_pool_values(dims, max(sum(ctx), 1), seed + 2, "cuda")
    pools = []
    off = 0
    for b, c in enumerate(ctx):
        Kb, Vb = K[:, off:off + c], V[:, off:off + c]
        if c:
            pack_pool(dims, pool, n_pages, table, b, Kb, Vb)
        pools.append((f64(Kb), f64(Vb)))
        off += c
    dr = Drafter(dims, W, max_batch=len(ctx), block_size=B, max_ctx=max(ctx), schedule=schedule)
    anc = None if anchor is None else torch.tensor(anchor, dtype=torch.int32, device="cuda")
    tok, lg, cf = dr.draft(pool, n_pages, tab, ctx_tensor(ctx), max(ctx), B, S, T, seed=1234 + seed,
                           want_logits=want_logits, anchor=anc)
    torch.cuda.synchronize()
    res = oracle.draft_block(dims, np_weights(W), pools, ctx, B, S, temperature=T, seed=1234 + seed,
                             schedule=schedule, anchor=anchor)
    return res, tok.cpu().numpy(), (f64(lg) if lg is not None else None), f64(cf), (dr, pool, n_pages, tab)


@pytest.mark.parametrize("name,ctx,B,S,T", [
    ("tiny", [64], 4, 2, 0.0),
    ("tiny", [64, 3], 4, 1, 0.0),
    ("small", [0, 37, 300], 8, 2, 0.0),
    ("small", [130, 16, 1], 16, 2, 0.0),
    ("small", [45, 200], 16, 3, 0.0),
    ("small", [77, 8], 8, 2, 1.0),
    ("tiny", [64], 4, 2, 0.7),
    ("small", [200], 8, 2, 0.0),          # one sequence: K sliced inside the workgroup (at most 16 rows)
    ("small", [31], 16, 2, 1.0),
])
def test_draft_matches_oracle(name, ctx, B, S, T):
    dims = _dims(name)
    res, tok, lg, cf, _ = _draft_case(dims, ctx, B, S, T, seed=20 + B + S)
    out = compare_draft(dims, S, res, tok, lg, cf)
    print(f"draft {name} ctx={ctx} B={B} S={S} T={T}: {out}")
    assert out["compared"] >= tok.size // 2


@pytest.mark.parametrize("inter,T", [(4608, 0.0), (5120, 1.0)])
def test_draft_one_sequence_long_down_projection(inter, T):
    """One sequence with an MLP wide enough that each of the down projection's eight
    K splits is longer than two batches of eight 32-deep steps (the at-most-16-row GEMM
    that copies the split's activation fragments to LDS once)."""
    from dataclasses import replace
    dims = replace(SMALL, intermediate=inter)
    res, tok, lg, cf, _ = _draft_case(dims, [90], 8, 2, T, seed=140 + inter % 7)
    out = compare_draft(dims, 2, res, tok, lg, cf)
    print(f"draft one sequence, intermediate {inter}, T={T}: {out}")
    assert out["compared"] >= tok.size // 2


@pytest.mark.parametrize("hidden,ctx", [
    (512, [20, 5, 33, 12, 40, 8, 27, 16]),      # 128 rows of 512: 256 threads, one quad each
    (1536, [40, 3, 17, 60, 9, 33, 25, 70]),     # 128 rows of 1536: two quads per thread
    (6144, [12, 40, 7, 22, 31, 5, 18, 26]),     # 128 rows of 6144: 512 threads, four quads each
    (6144, [30, 11]),                           # 32 rows of 6144: 1024 threads, two quads each
])
def test_draft_rmsnorm_row_widths(hidden, ctx):
    """Every launch shape of the RMSNorm (threads per row and quads per thread follow the
    row count and width), each folding the K-split partials of the O and down projections:
    the draft against the oracle at hidden sizes and batches that select them."""
    from dataclasses import replace
    dims = replace(SMALL, hidden=hidden)
    res, tok, lg, cf, _ = _draft_case(dims, ctx, 16, 2, 0.0, seed=170 + hidden % 11 + len(ctx))
    out = compare_draft(dims, 2, res, tok, lg, cf)
    print(f"draft hidden {hidden} ctx={ctx}: {out}")
    assert out["compared"] >= tok.size // 2


@pytest.mark.parametrize("name,ctx,B,S,T", [
    ("tiny", [64, 5], 4, 2, 0.0),
    ("small", [77], 8, 2, 0.0),           # one sequence: the skinny (at most 16 rows) GEMMs
    ("small", [0, 37, 300], 8, 2, 0.0),
    ("small", [130, 16], 16, 3, 0.0),
    ("small", [77, 8], 8, 2, 1.0),
])
def test_draft_repredict_matches_oracle(name, ctx, B, S, T):
    dims = _dims(name)
    res, tok, lg, cf, _ = _draft_case(dims, ctx, B, S, T, seed=60 + B + S, schedule="repredict")
    out = compare_draft(dims, S, res, tok, lg, cf, schedule="repredict")
    print(f"draft (re-predict) {name} ctx={ctx} B={B} S={S} T={T}: {out}")
    assert out["compared"] >= tok.size // 2


@pytest.mark.parametrize("name,ctx,B,S,d", [
    ("tiny", [64, 9], 4, 2, 64),          # fp32: in-place QK-norm, VALU attention
    ("small", [0, 37, 300], 8, 2, 128),   # bf16, head_dim 128: QK-norm in the query prep, MFMA attention
    ("small", [150], 16, 2, 128),         # one sequence: skinny GEMMs feeding the query prep
    ("small", [130, 16], 16, 2, 64),      # bf16, head_dim 64: in-place QK-norm, VALU attention
])
def test_draft_qk_norm_matches_oracle(name, ctx, B, S, d):
    from dataclasses import replace
    dims = _dims(name)
    if d != dims.head_dim:
        dims = replace(dims, head_dim=d)
    res, tok, lg, cf, _ = _draft_case(dims, ctx, B, S, 0.0, seed=80 + B, qk=True)
    out = compare_draft(dims, S, res, tok, lg, cf)
    print(f"draft (QK-norm) {name} d={d} ctx={ctx} B={B} S={S}: {out}")
    assert out["compared"] >= tok.size // 2


@pytest.mark.parametrize("name,ctx,B,S,T,schedule", [
    ("tiny", [64, 3], 4, 2, 0.0, "progressive"),
    ("small", [0, 37, 300], 8, 2, 0.0, "progressive"),
    ("small", [130, 16], 16, 3, 0.0, "progressive"),
    ("small", [77], 16, 2, 0.0, "progressive"),       # one sequence: the skinny GEMMs
    ("small", [77, 8], 8, 2, 1.0, "progressive"),
    ("small", [45, 200], 8, 2, 0.0, "repredict"),
    ("small", [9, 40], 2, 1, 0.0, "progressive"),     # one drafted position
])
def test_draft_with_anchor_matches_oracle(name, ctx, B, S, T, schedule):
    """Block position 0 given (the last committed token of a closed loop), the other
    B-1 positions denoised: tokens, logits and confidences against the oracle."""
    dims = _dims(name)
    rng = np.random.default_rng(B * 7 + S)
    anchor = rng.integers(0, dims.vocab, size=len(ctx)).tolist()
    res, tok, lg, cf, _ = _draft_case(dims, ctx, B, S, T, seed=110 + B + S, schedule=schedule, anchor=anchor)
    assert np.array_equal(tok[:, 0], anchor)
    assert np.all(np.isnan(cf[:, :, 0]))
    out = compare_draft(dims, S, res, tok, lg, cf, schedule=schedule)
    print(f"anchored draft {name} ctx={ctx} B={B} S={S} T={T} {schedule}: {out}")
    assert out["compared"] >= tok.size // 2


def test_incremental_injection_with_qk_norm_is_bitwise_one_shot():
    dims, W = _with_qk(SMALL, synth.make_weights(SMALL, 9, "cuda"), 90)
    ctx = [150, 97]
    table, n_pages = page_plan(ctx, 0, seed=4)
    tab = torch.from_numpy(table).cuda()
    hid = synth.make_hiddens(dims, sum(ctx), 10, "cuda")
    seq, pos = _tokens(ctx)
    dr = Drafter(dims, W, max_batch=2, block_size=8, max_ctx=150, max_inject=4096)
    one = alloc_pool(dims, n_pages)
    dr.inject(hid, seq, pos, one, n_pages, tab, 2)
    inc = alloc_pool(dims, n_pages)
    for a, b in [(0, 3), (3, 100), (100, seq.numel())]:
        dr.inject(hid[a:b].contiguous(), seq[a:b].contiguous(), pos[a:b].contiguous(), inc, n_pages, tab, 2)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), inc.view(torch.int16))


def test_draft_is_deterministic():
    dims = SMALL
    res, tok, lg, cf, (dr, pool, n_pages, tab) = _draft_case(dims, [33, 90], 8, 2, 0.0, seed=40)
    tok2, lg2, cf2 = dr.draft(pool, n_pages, tab, ctx_tensor([33, 90]), 90, 8, 2)
    torch.cuda.synchronize()
    assert np.array_equal(tok, tok2.cpu().numpy())
    assert np.array_equal(lg, f64(lg2), equal_nan=True)
    assert np.array_equal(cf, f64(cf2), equal_nan=True)


@pytest.mark.parametrize("bt,B,V,p", [(5, 8, 5003, 0.7), (3, 1, 100, 0.5), (32, 16, 151936, 0.75)])
def test_greedy_verify_matches_oracle(bt, B, V, p):
    g = torch.Generator(device="cuda").manual_seed(bt * 100 + B)
    draft = torch.randint(0, V, (bt, B), generator=g, device="cuda", dtype=torch.int32)
    zt = synth.make_greedy_target_logits(draft, V, p, seed=bt + B, device="cuda")
    acc, out = verify(zt, draft)
    torch.cuda.synchronize()
    acc_o, out_o = oracle.verify_greedy(zt.cpu().numpy(), draft.cpu().numpy())
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    assert np.array_equal(out.cpu().numpy(), out_o)


@pytest.mark.parametrize("bt,B,V,T", [(6, 8, 5003, 1.0), (4, 4, 777, 0.5), (32, 16, 151936, 1.0)])
def test_sampled_verify_matches_oracle(bt, B, V, T):
    zd, zt = synth.make_sampled_logits(bt, B, V, seed=bt + V, device="cuda")
    draft = synth.sample_tokens(zd, T, seed=bt)
    U = synth.make_uniforms(bt, B, seed=V, device="cuda")
    acc, out = verify(zt, draft, T, zd, U)
    torch.cuda.synchronize()
    acc_o, out_o, margin = oracle.verify_sampled(zt.cpu().numpy(), zd.cpu().numpy(), draft.cpu().numpy(),
                                                 U.cpu().numpy(), T)
    keep = margin > 1e-9
    assert keep.sum() >= bt - 1
    assert np.array_equal(acc.cpu().numpy()[keep], acc_o[keep])
    assert np.array_equal(out.cpu().numpy()[keep], out_o[keep])
    print(f"sampled verify bt={bt} B={B}: mean accept {acc_o.mean():.2f}, excluded {int((~keep).sum())}")


@pytest.mark.parametrize("case", ["v1", "v64_peaked", "v100_flat", "equal", "last_index", "v5003_b1"])
def test_sampled_verify_edge_cases(case):
    """Sampled verification at the edges of its draw: a one-token vocabulary, vocabularies
    smaller than one draw segment, very peaked and very flat distributions, p = q (every
    draft token accepted, bonus drawn from p), and residual mass only at the last index."""
    bt, B, V, T = {"v1": (3, 4, 1, 1.0), "v64_peaked": (4, 16, 64, 0.05), "v100_flat": (5, 8, 100, 4.0),
                   "equal": (4, 8, 777, 1.0), "last_index": (4, 6, 5003, 1.0), "v5003_b1": (7, 1, 5003, 1.0)}[case]
    zd, zt = synth.make_sampled_logits(bt, B, V, seed=7 * V + B, device="cuda")
    draft = synth.sample_tokens(zd, T, seed=bt + B)
    if case == "equal":
        zt = torch.cat([zd, zt[:, B:]], dim=1).contiguous()
    if case == "last_index":
        # the draft puts its mass on token 0 and drafts it; the target prefers token V-1, so
        # the first test rejects (u q < p fails for u >= p/q) and max(0, p - q) sits at V-1
        zd = torch.full((bt, B, V), -30.0, device="cuda")
        zd[:, :, 0] = 30.0
        zt = torch.full((bt, B + 1, V), -30.0, device="cuda")
        zt[:, :, V - 1] = 30.0
        draft = torch.zeros(bt, B, dtype=torch.int32, device="cuda")
    U = synth.make_uniforms(bt, B, seed=V + B, device="cuda")
    acc, out = verify(zt, draft, T, zd, U)
    torch.cuda.synchronize()
    acc_o, out_o, margin = oracle.verify_sampled(zt.cpu().numpy(), zd.cpu().numpy(), draft.cpu().numpy(),
                                                 U.cpu().numpy(), T)
    keep = margin > 1e-9
    assert keep.sum() >= bt - 1
    assert np.array_equal(acc.cpu().numpy()[keep], acc_o[keep])
    assert np.array_equal(out.cpu().numpy()[keep], out_o[keep])
    a = acc.cpu().numpy()
    o = out.cpu().numpy()
    assert np.all((a >= 0) & (a <= B))
    assert np.all((o[np.arange(bt), a] >= 0) & (o[np.arange(bt), a] < V))
    if case == "v1":
        assert np.all(a == B) and np.all(o == 0)
    if case == "equal":
        assert np.all(a == B)
    if case == "last_index":
        assert np.all(a == 0) and np.all(o[:, 0] == V - 1)


@pytest.mark.parametrize("n_tok_case,qk", [(0, False), (17, False), (9, True)])
def test_target_forward_matches_oracle(n_tok_case, qk):
    """Target-side verify forward (causal block over the target's own cache): logits, the
    captured layer outputs and the K/V it appends to the pool, against the oracle; then
    the same call on a prefix of the tokens reproduces the earlier rows (causality)."""
    from dataclasses import replace
    dims = replace(SMALL, n_layers=3)
    W = synth.make_weights(dims, 95, "cuda")
    if qk:   # a Qwen3-style target: QK-norm with random gains
        dims, W = _with_qk(dims, W, 99)
    ctx, n, caps = [37, 130, 0], 5, [0, 2]
    if n_tok_case:
        n = n_tok_case
    bt = len(ctx)
    table, n_pages = page_plan(ctx, n, seed=96)
    tab = torch.from_numpy(table).cuda()
    K, V = synth.make_pool_values(dims, sum(ctx), 97, "cuda")
    pools, off = [], 0
    pool = alloc_pool(dims, n_pages)
    for b, c in enumerate(ctx):
        Kb, Vb = K[:, off:off + c], V[:, off:off + c]
        if c:
            pack_pool(dims, pool, n_pages, table, b, Kb, Vb)
        pools.append((f64(Kb), f64(Vb)))
        off += c
    g = torch.Generator(device="cuda").manual_seed(98)
    tokens = torch.randint(0, dims.vocab, (bt, n), generator=g, device="cuda", dtype=torch.int32)
    cfg, w = Bn.make_config(dims), Bn.Weights(W)
    ws_bytes = Bn.dflash_workspace_size(cfg, bt, n, 0, max(ctx))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    def run(pool_, ntok):
        z = torch.empty(bt, ntok, dims.vocab, dtype=torch.float32, device="cuda")
        hid = torch.empty(bt, ntok, len(caps) * dims.hidden, dtype=torch.bfloat16, device="cuda")
        Bn.dflash_target_forward(cfg, w, pool_, n_pages, tab, table.shape[1], ctx_tensor(ctx), max(ctx), bt, ntok,
                                tokens[:, :ntok].contiguous(), caps, z, hid, ws, ws_bytes)
        return z, hid

    pool0 = pool.clone()
    z, hid = run(pool, n)
    torch.cuda.synchronize()
    zo, ho, Ko, Vo = oracle.target_forward(dims, np_weights(W), pools, ctx, tokens.cpu().numpy(), capture_layers=caps)
    zg = f64(z)
    rel = np.max(np.abs(zg - zo), axis=-1) / np.max(np.abs(zo), axis=-1)
    print(f"target forward: logits max rel err {rel.max():.2e}")
    assert rel.max() <= 2e-2
    # argmax rows (what greedy verification reads) agree away from near-ties
    top2 = np.sort(zo, axis=-1)[..., -2:]
    clear = (top2[..., 1] - top2[..., 0]) > 1e-3
    assert np.array_equal(np.argmax(zg, -1)[clear], np.argmax(zo, -1)[clear])
    compare_pool_entries(f64(hid), ho, dims.dtype, "captured hidden")
    for b, c in enumerate(ctx):
        Kg, Vg = unpack_pool(dims, pool, n_pages, table, b, c + n)
        compare_pool_entries(Kg[:, c:], Ko[:, b], dims.dtype, f"appended K b={b}")
        compare_pool_entries(Vg[:, c:], Vo[:, b], dims.dtype, f"appended V b={b}")
        Kc, Vc = unpack_pool(dims, pool, n_pages, table, b, c)
        assert np.array_equal(Kc, pools[b][0]) and np.array_equal(Vc, pools[b][1])   # context untouched
    # causality: the first three tokens alone give the same first three rows
    z3, hid3 = run(pool0, 3)
    torch.cuda.synchronize()
    rel3 = np.max(np.abs(f64(z3) - zg[:, :3]), axis=-1) / np.max(np.abs(zo[:, :3]), axis=-1)
    assert rel3.max() <= 1e-3, rel3.max()


def test_unmapped_context_pages_are_left_out():
    """Context pages the block table leaves unmapped (-1) are skipped by the MFMA context
    kernel, as by the VALU one: the draft equals the oracle's over the context with those
    tokens removed (block positions still ctx_len + i).  Physical page 0 is kept unused and
    NaN-poisoned, so the page read in place of an unmapped first page holds NaN: its
    scores must be masked and its values zeroed, or the output turns NaN."""
    dims = SMALL
    ctx, B, S = [100, 70], 8, 2
    unmapped = {0: [0, 3], 1: [2]}
    W = synth.make_weights(dims, 51, "cuda")
    pages = [(c + 15) // 16 for c in ctx]
    n_pages = 1 + sum(pages)
    table = np.zeros((len(ctx), max(pages)), dtype=np.int32)
    nxt = 1
    for b, npg in enumerate(pages):
        table[b, :npg] = np.arange(nxt, nxt + npg)
        nxt += npg
    pool = alloc_pool(dims, n_pages)          # NaN everywhere, physical page 0 stays so
    K, V = synth.make_pool_values(dims, sum(ctx), 52, "cuda")
    pools, off = [], 0
    for b, c in enumerate(ctx):
        Kb, Vb = K[:, off:off + c], V[:, off:off + c]
        pack_pool(dims, pool, n_pages, table, b, Kb, Vb)
        keep = np.ones(c, dtype=bool)
        for lp in unmapped[b]:
            keep[16 * lp:16 * lp + 16] = False
            table[b, lp] = -1
        # the oracle slices the first ctx_len tokens of what it is given: the kept ones
        pools.append((f64(Kb)[:, keep], f64(Vb)[:, keep]))
        off += c
    tab = torch.from_numpy(table).cuda()
    dr = Drafter(dims, W, max_batch=len(ctx), block_size=B, max_ctx=max(ctx))
    tok, lg, cf = dr.draft(pool, n_pages, tab, ctx_tensor(ctx), max(ctx), B, S)
    torch.cuda.synchronize()
    assert torch.isfinite(lg).all()
    res = oracle.draft_block(dims, np_weights(W), pools, ctx, B, S)
    out = compare_draft(dims, S, res, tok.cpu().numpy(), f64(lg), f64(cf))
    print(f"unmapped pages {unmapped}: {out}")
    assert out["compared"] >= tok.numel() // 2


@pytest.mark.parametrize("V", [4096, 5003])
def test_greedy_verify_misaligned_logits(V):
    """Target logits at a base that is 4- but not 16-byte aligned (an offset view): the
    row kernel must not take its 128-bit path, and the result equals the oracle's."""
    bt, B = 5, 8
    g = torch.Generator(device="cuda").manual_seed(V)
    draft = torch.randint(0, V, (bt, B), generator=g, device="cuda", dtype=torch.int32)
    zt = synth.make_greedy_target_logits(draft, V, 0.7, seed=V, device="cuda")
    buf = torch.empty(zt.numel() + 1, dtype=torch.float32, device="cuda")
    zo = buf[1:].view(zt.shape)
    zo.copy_(zt)
    assert zo.data_ptr() % 16 != 0
    acc, out = verify(zo, draft)
    torch.cuda.synchronize()
    acc_o, out_o = oracle.verify_greedy(zt.cpu().numpy(), draft.cpu().numpy())
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    assert np.array_equal(out.cpu().numpy(), out_o)
