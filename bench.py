"""Benchmark of the block-diffusion drafter step on one MI355X.

One step = the whole hot path over one batch: inject the a+1 newly accepted
tokens of every sequence into the paged KV pool, draft a block (two denoise
forwards), verify it greedily against target logits.  Inputs are seeded
synthetic tensors resident in HBM; the target logits of each step are made
from a pre-drawn N(0,1) base by forcing each block position to agree with
the draft token with the workload's match probability (this stands in for
the target model, which is outside the path, and is excluded from the timed
intervals by HIP events).

Prints one JSON line (see --help for options).
"""
import argparse
import json
import re
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # dense bf16 MFMA, FLOP/s
PEAK_FP32 = 157.3e12
PEAK_HBM = 8.0e12       # B/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_shape_b16_bs32")
    ap.add_argument("--roofline-kernel", default="auto",
                    help="kernel class timed for the roofline object (auto: the one with the largest time)")
    ap.add_argument("--cpu-baseline", type=int, default=1, help="time the fp64 oracle on a bounded sample")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="after the timed steps, run one plain device copy of COPY_BYTES (for HBM counter scaling)")
    ap.add_argument("--summarize-sq", nargs=3, metavar=("DIR1", "DIR2", "DIR3"),
                    help="write profiles/sq_counters_*.md from the three shader-sequencer counter passes")
    ap.add_argument("--summarize-verify", metavar="TRACE_DIR",
                    help="write profiles/kernel_stats_sampled_verify_*.md from a --longctx 1 kernel trace")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="turn rocprofv3 csv output into profiles/ summaries and exit")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--target", type=int, default=1,
                    help="also time the target-side verify forward of a Qwen3-8B-shaped 36-layer target")
    ap.add_argument("--longctx", type=int, default=1,
                    help="also time the draft call and sampled verification of the long-context workload")
    ap.add_argument("--batch1", type=int, default=1,
                    help="also time the draft call of the Qwen3-4B-shaped batch-1 block-8 workload")
    ap.add_argument("--ceilings", type=int, default=1,
                    help="measure the vendor GEMM rate and a device copy's HBM rate on this GPU, and price "
                         "the draft's executed work against them")
    ap.add_argument("--device-loop", type=int, default=1,
                    help="also time the step loop kept on the GPU (dflash_advance_context, HIP graph replay)")
    ap.add_argument("--block-sweep", type=int, default=1,
                    help="also time the draft call alone at block sizes 4, 8 and 16 on the same batch and pool")
    ap.add_argument("--incremental", type=int, default=1,
                    help="also time the incremental workload (block 8, lognormal contexts, shared prefixes)")
    ap.add_argument("--tiny", type=int, default=1, help="also time the tiny fp32 workload (absolute latency)")
    ap.add_argument("--closed", type=int, default=1,
                    help="also time the closed step with a 36-layer Qwen3-8B-shaped target in the loop")
    return ap.parse_args()


COPY_BYTES = 1 << 29          # 512 MiB read + 512 MiB written by the calibration copy
# Kernel name patterns (regular expressions) of each timed class: GEMM kernels
# end their template arguments with (operand planes, epilogue kind), the
# large-tile kernel then with its count of weight stages.
KERNEL_NAMES = {
    "attn": r"attn_ctx_mfma_kernel",
    "gemm_qkv": r"gemm_\w+_kernel<[^>]*, 2, 0(, \d)?>",
    "gemm_o": r"gemm_\w+_kernel<[^>]*, 2, 1(, \d)?>",
    "gemm_down": r"gemm_\w+_kernel<[^>]*, 2, 1(, \d)?>",
    "gemm_gateup": r"gemm_\w+_kernel<[^>]*, 2, 2(, \d)?>",
    "lmhead": r"gemm_\w+_kernel<[^>]*, 1, 3(, \d)?>",
}
KERNEL_SOURCES = ["common.h", "kernels.h", "gemm.hip", "attention.hip", "elementwise.hip", "verify.hip", "api.cpp"]


def pct(xs):
    """median, p10 and p90 of a list of per-call times (ms)"""
    import numpy as np
    q = np.percentile(np.asarray(xs, dtype=np.float64), [50, 10, 90])
    return {"median": round(float(q[0]), 4), "p10": round(float(q[1]), 4), "p90": round(float(q[2]), 4), "n": len(xs)}


def source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_diffusion_drafter_injection_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload, cls):
    return os.path.join(ROOT, "profiles", f"traffic_{cls}_{workload}.json")


def work_per_class(dims, bt, B, S, ctx, n_new):
    """Algorithmic work of each kernel class over one step: dict cls -> (amount, unit, bound, launches).

    GEMMs: 2*M*N*K flops (the second MFMA of a hi/lo operand is not counted).
    Attention: K and V bytes of every context token read once per layer per forward.
    """
    H, L, I, V = dims.hidden, dims.n_layers, dims.intermediate, dims.vocab
    nq, nkv, d = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    M = bt * B
    el = 2 if dims.dtype == "bf16" else 4
    out = {}
    out["gemm_qkv"] = (2.0 * M * (nq + 2 * nkv) * d * H * L * S, "flop", L * S)
    out["gemm_o"] = (2.0 * M * H * nq * d * L * S, "flop", L * S)
    out["gemm_gateup"] = (2.0 * M * 2 * I * H * L * S, "flop", L * S)
    out["gemm_down"] = (2.0 * M * H * I * L * S, "flop", L * S)
    opens, done = [], 0
    for s in range(S):
        opens.append(B - done)
        done += (s + 1) * B // S - s * B // S
    out["lmhead"] = (sum(2.0 * bt * o * V * H for o in opens), "flop", S)
    out["attn"] = (float(sum(ctx)) * nkv * d * 2 * el * L * S, "byte", L * S)
    out["inject_fc"] = (2.0 * n_new * H * dims.n_fuse * dims.target_hidden, "flop", 1)
    out["inject_kv"] = (2.0 * n_new * L * 2 * nkv * d * H, "flop", 1)
    out["verify"] = (float(bt) * (B + 1) * V * 4, "byte", 1)
    return out


def draft_roofline_ms(dims, bt, B, S, ctx, peak=None, hbm=PEAK_HBM, executed=False):
    """Roofline time of one draft call: the sum over its kernels of max(flops / MFMA peak,
    HBM bytes / HBM peak), with weights streamed once per forward, every context token's
    K and V read once per layer and forward, and the LM head over the still-open rows only.
    executed=True counts the layer GEMMs' second (lo-plane) MFMA as work, as the kernels
    execute it (bf16 only)."""
    H, L, I, V = dims.hidden, dims.n_layers, dims.intermediate, dims.vocab
    nq, nkv, d = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    el = 2 if dims.dtype == "bf16" else 4
    if peak is None:
        peak = PEAK_BF16 if dims.dtype == "bf16" else PEAK_FP32
    planes = 2.0 if (executed and dims.dtype == "bf16") else 1.0
    M = bt * B
    gemms = [((nq + 2 * nkv) * d, H), (H, nq * d), (2 * I, H), (H, I)]
    t, done = 0.0, 0
    for s in range(S):
        for N, K in gemms:
            t += L * max(planes * 2.0 * M * N * K / peak, N * K * el / hbm)
        t += L * float(sum(ctx)) * nkv * d * 2 * el / hbm
        rows = bt * (B - done)
        t += max(2.0 * rows * V * H / peak, V * H * el / hbm)
        done += (s + 1) * B // S - s * B // S
    return t * 1e3


def measured_ceilings(dims, bt, B):
    """What this GPU sustains on plain library work, measured live: the bf16 rate of the
    vendor GEMM (torch.matmul, hipBLASLt) on a large square product and on each of the
    draft's GEMM shapes (one bf16 plane), and the HBM rate of a 1 GiB device copy
    (bytes read + written)."""
    import torch
    dev = "cuda"

    def timed(fn, n):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n / 1e3

    out = {}
    H, I, V = dims.hidden, dims.intermediate, dims.vocab
    nq, nkv, d = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    M = bt * B
    shapes = {"square_8192": (8192, 8192, 8192), "qkv": (M, (nq + 2 * nkv) * d, H), "o": (M, H, nq * d),
              "gate_up": (M, 2 * I, H), "down": (M, H, I), "lm_head": (M, V, H)}
    gemm = {}
    for name, (m, n, k) in shapes.items():
        a = torch.randn(m, k, device=dev, dtype=torch.bfloat16)
        w = torch.randn(n, k, device=dev, dtype=torch.bfloat16)
        sec = timed(lambda: torch.matmul(a, w.t()), 10)
        gemm[name] = {"m": m, "n": n, "k": k, "us": round(sec * 1e6, 1), "tflops": round(2.0 * m * n * k / sec / 1e12, 1)}
        del a, w
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    sec = timed(lambda: dst.copy_(src), 10)
    out["hbm_copy_gbs"] = round(2.0 * src.numel() * 4 / sec / 1e9, 1)
    del src, dst
    out["mfma_bf16_tflops"] = gemm["square_8192"]["tflops"]
    out["vendor_gemm"] = gemm
    torch.cuda.empty_cache()
    return out


def main():
    a = parse()
    if a.summarize_sq:
        summarize_sq(*a.summarize_sq)
        return
    if a.summarize_verify:
        summarize_verify(a.summarize_verify)
        return
    if a.summarize:
        summarize(*a.summarize)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only; it has no multi-GPU mode "
                                   "(the draft step would shard by sequence with no exchange)", "n_gpus": a.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    from block_diffusion_drafter_injection_amd import binding as Bn
    from block_diffusion_drafter_injection_amd import synth

    wl = synth.WORKLOADS[a.workload]
    dims = wl.dims
    bt, B, S = wl.batch, wl.block_size, wl.n_steps
    dev = "cuda"
    torch.manual_seed(a.seed)
    t_setup = time.time()
    W = synth.make_weights(dims, wl.seed, dev)
    cfg, w = Bn.make_config(dims), Bn.Weights(W)
    ctx0 = synth.context_lengths(wl).numpy().astype(np.int64)
    grow = (2 * a.steps + a.warmup + 12) * (B + 1)
    max_ctx = int(ctx0.max()) + grow
    pages_per = (max_ctx + 15) // 16
    n_pages = bt * pages_per
    table = torch.arange(n_pages, dtype=torch.int32, device=dev).view(bt, pages_per)
    pool = torch.zeros(Bn.pool_elems(dims, n_pages), dtype=dims.torch_dtype, device=dev)
    max_inject = 8192
    ws_bytes = Bn.dflash_workspace_size(cfg, bt, B, max_inject, max_ctx)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    vws_bytes = Bn.dflash_verify_workspace_size(bt, B, dims.vocab)
    vws = torch.empty(vws_bytes, dtype=torch.uint8, device=dev)

    # one-shot injection of the initial contexts (setup, untimed)
    for b in range(bt):
        c = int(ctx0[b])
        hid = synth.make_hiddens(dims, c, wl.seed * 1000 + b, dev)
        seq = torch.full((c,), b, dtype=torch.int32, device=dev)
        pos = torch.arange(c, dtype=torch.int32, device=dev)
        Bn.dflash_inject_kv(cfg, w, hid, seq, pos, c, pool, n_pages, table, bt, pages_per, ws, ws_bytes)
        del hid
    torch.cuda.synchronize()

    new_hid = synth.make_hiddens(dims, bt * (B + 1), wl.seed + 77, dev)
    g = torch.Generator(device=dev).manual_seed(3000 + wl.seed)
    z0 = torch.randn(bt, B + 1, dims.vocab, generator=g, device=dev, dtype=torch.float32)
    zmax = z0[:, :B].amax(-1) + 1.0
    zmin = z0[:, :B].amin(-1) - 1.0
    ctx = ctx0.copy()
    ctx_dev = torch.tensor(ctx, dtype=torch.int32, device=dev)
    tok = torch.empty(bt, B, dtype=torch.int32, device=dev)
    acc = torch.empty(bt, dtype=torch.int32, device=dev)
    outt = torch.empty(bt, B + 1, dtype=torch.int32, device=dev)
    pin_seq = torch.empty(bt * (B + 1), dtype=torch.int32, pin_memory=True)
    pin_pos = torch.empty(bt * (B + 1), dtype=torch.int32, pin_memory=True)
    dev_seq = torch.empty(bt * (B + 1), dtype=torch.int32, device=dev)
    dev_pos = torch.empty(bt * (B + 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    last_acc = np.zeros(bt, dtype=np.int64)     # before the first step nothing is pending
    first = True
    setup_s = time.time() - t_setup

    def step(ev):
        nonlocal first, ctx
        # tokens accepted by the previous step: a+1 per sequence at positions ctx .. ctx+a
        if first:
            n_new = 0
        else:
            seqs = np.concatenate([np.full(int(x) + 1, b) for b, x in enumerate(last_acc)])
            poss = np.concatenate([np.arange(ctx[b], ctx[b] + int(x) + 1) for b, x in enumerate(last_acc)])
            n_new = len(seqs)
            pin_seq[:n_new] = torch.from_numpy(seqs.astype(np.int32))
            pin_pos[:n_new] = torch.from_numpy(poss.astype(np.int32))
            dev_seq[:n_new].copy_(pin_seq[:n_new], non_blocking=True)
            dev_pos[:n_new].copy_(pin_pos[:n_new], non_blocking=True)
            ctx = ctx + last_acc + 1
            ctx_dev.copy_(torch.from_numpy(ctx.astype(np.int32)), non_blocking=True)
        ev[0].record(stream)
        if n_new:
            Bn.dflash_inject_kv(cfg, w, new_hid, dev_seq, dev_pos, n_new, pool, n_pages, table, bt, pages_per, ws,
                                ws_bytes)
        Bn.dflash_draft_block(cfg, w, pool, n_pages, table, pages_per, ctx_dev, max_ctx, bt, B, S, 0.0, 0, tok,
                              None, None, ws, ws_bytes)
        ev[1].record(stream)
        # target logits for this block (stand-in for the target model; not timed)
        coin = torch.rand(bt, B, generator=g, device=dev) < wl.p_match
        val = torch.where(coin, zmax, zmin)
        idx = tok.long().unsqueeze(-1)
        keep = z0[:, :B].gather(-1, idx)
        z0[:, :B].scatter_(-1, idx, val.unsqueeze(-1))
        ev[2].record(stream)
        Bn.dflash_verify_block(bt, B, dims.vocab, z0, tok, 0.0, None, None, acc, outt, vws, vws_bytes)
        ev[3].record(stream)
        z0[:, :B].scatter_(-1, idx, keep)
        first = False
        return n_new

    def run(n, sel=None):
        nonlocal last_acc
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        dl = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        accs, news = [], []
        for i in range(n):
            news.append(step(evs[i]))
            a_np = acc.cpu().numpy().astype(np.int64)      # the scheduler needs the acceptance
            last_acc = a_np
            accs.append(a_np)
        torch.cuda.synchronize()
        hot = [evs[i][0].elapsed_time(evs[i][1]) + evs[i][2].elapsed_time(evs[i][3]) for i in range(n)]
        return hot, accs, news

    # warmup
    run(a.warmup)
    # pick the roofline kernel
    cls = a.roofline_kernel
    if cls == "auto":
        best, cls = -1.0, "attn"
        for c in ["attn", "gemm_gateup", "lmhead", "gemm_down", "gemm_qkv", "gemm_o"]:
            Bn.dflash_prof_select(c)
            run(1)
            ms, n = Bn.dflash_prof_collect()
            if ms > best:
                best, cls = ms, c
        Bn.dflash_prof_select("none")

    # draft-only latency (separate, back-to-back calls on the current state, each between its own events)
    nd = 20
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nd)]
    for e0_, e1_ in dev_ev:
        e0_.record(stream)
        Bn.dflash_draft_block(cfg, w, pool, n_pages, table, pages_per, ctx_dev, max_ctx, bt, B, S, 0.0, 0, tok, None,
                              None, ws, ws_bytes)
        e1_.record(stream)
    torch.cuda.synchronize()
    draft_calls = [e0_.elapsed_time(e1_) for e0_, e1_ in dev_ev]
    draft_ms = float(np.mean(draft_calls))

    # timed region
    Bn.dflash_prof_select(cls)
    ctx_before = ctx.copy()
    torch.cuda.synchronize()
    t0 = time.time()
    hot, accs, news = run(a.steps)
    torch.cuda.synchronize()
    wall = time.time() - t0
    kms, kn = Bn.dflash_prof_collect()
    Bn.dflash_prof_select("none")

    if a.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_step = float(np.mean(hot))
    accepted = float(np.mean([np.sum(x + 1) for x in accs]))
    value = accepted / (ms_step / 1e3)
    n_new_mean = float(np.mean(news))
    work = work_per_class(dims, bt, B, S, (ctx_before + ctx) / 2.0, n_new_mean)
    t_roof = draft_roofline_ms(dims, bt, B, S, ctx_before)   # the state the draft-only timing ran on
    amount, unit, launches_per_step = work[cls]
    bound = "hbm" if unit == "byte" else "mfma"
    peak = PEAK_HBM if unit == "byte" else (PEAK_BF16 if dims.dtype == "bf16" else PEAK_FP32)
    achieved = amount * a.steps / (kms / 1e3) if kms > 0 else 0.0
    roof = {"kernel": cls, "bound": bound,
            "achieved": round(achieved / (1e9 if unit == "byte" else 1e12), 2),
            "peak": round(peak / (1e9 if unit == "byte" else 1e12), 1),
            "unit": "GB/s" if unit == "byte" else "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": load_traffic(wl.name, cls),
            "launches": kn, "avg_launch_us": round(kms * 1e3 / max(kn, 1), 2)}

    res = {
        "metric": "accepted tok/s of the drafter step (inject a+1, 2-step block draft, greedy verify)",
        "value": round(value, 1), "unit": "tok/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dims.dtype == "bf16" else "f32", "data": "synthetic (seeded random-init weights, "
        "N(0,1) target hiddens, forced-match target logits)",
        "config": {"workload": wl.name, "batch": bt, "block": B, "denoise_steps": S, "hidden": dims.hidden,
                   "layers": dims.n_layers, "vocab": dims.vocab, "ctx_start": int(ctx0.mean()),
                   "p_match": wl.p_match},
        "draft_ms": round(draft_ms, 4),
        "draft_latency_ms": pct(draft_calls),
        "step_latency_ms": pct(hot),
        "drafted_tok_s": round(bt * B / (draft_ms / 1e3), 1),
        "mean_accept_plus_bonus": round(accepted / bt, 3),
        "wall_ms_per_step": round(wall * 1e3 / a.steps, 3),
        "roofline": roof,
        "draft_roofline": {"t_roof_ms": round(t_roof, 4), "draft_ms": round(draft_ms, 4),
                           "frac": round(t_roof / draft_ms, 4),
                           "definition": "sum over the draft's kernels of max(flops/2.5 PFLOP/s, bytes/8 TB/s)"},
    }
    if a.ceilings and dims.dtype == "bf16":
        c = measured_ceilings(dims, bt, B)
        t_ex = draft_roofline_ms(dims, bt, B, S, ctx_before, peak=c["mfma_bf16_tflops"] * 1e12,
                                 hbm=c["hbm_copy_gbs"] * 1e9, executed=True)
        res["measured_ceilings"] = c
        # the roofline kernel against what this GPU sustains on library work, with the
        # hi/lo layer GEMMs' second MFMA counted as executed work
        if roof["unit"] == "TFLOP/s":
            ex = roof["achieved"] * (2.0 if cls in ("gemm_qkv", "gemm_o", "gemm_gateup", "gemm_down") else 1.0)
            roof["executed"] = round(ex, 2)
            roof["frac_executed_of_measured"] = round(ex / c["mfma_bf16_tflops"], 4)
        else:
            roof["frac_of_measured"] = round(roof["achieved"] / c["hbm_copy_gbs"], 4)
        res["draft_roofline"]["measured"] = {
            "t_roof_ms": round(t_ex, 4), "frac": round(t_ex / draft_ms, 4),
            "definition": "sum over the draft's kernels of max(executed flops (hi/lo counted twice) / the "
                          "vendor GEMM's bf16 rate on an 8192^3 product, bytes / a 1 GiB device copy's rate)"}
    if a.device_loop:
        res["device_loop"] = device_loop(a, Bn, cfg, w, dims, bt, B, S, pool, n_pages, table, pages_per, max_ctx,
                                         ctx_dev, acc, tok, outt, new_hid, z0, zmax, zmin, wl.p_match, g, ws,
                                         ws_bytes, vws, vws_bytes)
    if a.block_sweep:
        sweep = []
        for Bs in (4, 8, 16):
            wsb = Bn.dflash_workspace_size(cfg, bt, Bs, max_inject, max_ctx)
            wss = ws if wsb <= ws_bytes else torch.empty(wsb, dtype=torch.uint8, device=dev)
            toks = torch.empty(bt, Bs, dtype=torch.int32, device=dev)
            for _ in range(2):
                Bn.dflash_draft_block(cfg, w, pool, n_pages, table, pages_per, ctx_dev, max_ctx, bt, Bs, S, 0.0, 0,
                                      toks, None, None, wss, max(wsb, 0))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(nd):
                Bn.dflash_draft_block(cfg, w, pool, n_pages, table, pages_per, ctx_dev, max_ctx, bt, Bs, S, 0.0, 0,
                                      toks, None, None, wss, max(wsb, 0))
            e1.record(stream)
            torch.cuda.synchronize()
            ms_b = e0.elapsed_time(e1) / nd
            tr = draft_roofline_ms(dims, bt, Bs, S, ctx)
            sweep.append({"block": Bs, "draft_ms": round(ms_b, 4), "drafted_tok_s": round(bt * Bs / (ms_b / 1e3), 1),
                          "t_roof_ms": round(tr, 4), "frac": round(tr / ms_b, 4)})
            del wss
        res["block_sweep"] = sweep
        # the adaptive block size this run's acceptances call for, with the measured draft times
        # of each block size as the step times (host policy, dflash_adaptive_block_size)
        a_obs = np.concatenate(accs).astype(int).tolist()
        choice, p_hat = Bn.dflash_adaptive_block_size(a_obs, [B] * len(a_obs), [x["block"] for x in sweep],
                                                      [x["draft_ms"] for x in sweep])
        res["adaptive_block"] = {
            "p_match_estimate": round(p_hat, 4), "choice": choice,
            "predicted_accepted_tok_s": {str(x["block"]): round(
                bt * sum(p_hat ** k for k in range(x["block"] + 1)) / (x["draft_ms"] / 1e3), 1) for x in sweep}}
    if a.block_sweep:
        # the other denoise reading on the same batch and pool: every step re-predicts every
        # position, so the second step's LM head covers all rows
        cfg_rp = Bn.make_config(dims, "repredict")
        for _ in range(2):
            Bn.dflash_draft_block(cfg_rp, w, pool, n_pages, table, pages_per, ctx_dev, max_ctx, bt, B, S, 0.0, 0,
                                  tok, None, None, ws, ws_bytes)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(nd):
            Bn.dflash_draft_block(cfg_rp, w, pool, n_pages, table, pages_per, ctx_dev, max_ctx, bt, B, S, 0.0, 0,
                                  tok, None, None, ws, ws_bytes)
        e1.record(stream)
        torch.cuda.synchronize()
        res["repredict_schedule"] = {"draft_ms": round(e0.elapsed_time(e1) / nd, 4),
                                     "note": "same batch and pool; every step re-predicts every position"}
        # the same draft with QK-norm layers (unit gains; timing only, the pool was injected without it)
        from dataclasses import replace as _replace
        dims_qk = _replace(dims, qk_norm=True)
        W_qk = dict(W, q_norm=[torch.ones(dims.head_dim, device=dev) for _ in range(dims.n_layers)],
                    k_norm=[torch.ones(dims.head_dim, device=dev) for _ in range(dims.n_layers)])
        cfg_qk, w_qk = Bn.make_config(dims_qk), Bn.Weights(W_qk)
        for _ in range(2):
            Bn.dflash_draft_block(cfg_qk, w_qk, pool, n_pages, table, pages_per, ctx_dev, max_ctx, bt, B, S, 0.0, 0,
                                  tok, None, None, ws, ws_bytes)
        e0.record(stream)
        for _ in range(nd):
            Bn.dflash_draft_block(cfg_qk, w_qk, pool, n_pages, table, pages_per, ctx_dev, max_ctx, bt, B, S, 0.0, 0,
                                  tok, None, None, ws, ws_bytes)
        e1.record(stream)
        torch.cuda.synchronize()
        res["qk_norm"] = {"draft_ms": round(e0.elapsed_time(e1) / nd, 4),
                          "note": "same batch and pool with per-head RMSNorm of queries and keys (query prep)"}
    if a.batch1 and a.workload != "qwen3_4b_shape_b8":
        res["batch1_block8"] = batch1_latency(Bn, nd)
    if a.longctx and a.workload == "qwen3_8b_shape_b16_bs32":
        res["longctx_sampled"] = longctx_bench(Bn, nd, W)
    if a.incremental and a.workload == "qwen3_8b_shape_b16_bs32":
        res["incremental_b8"] = incremental_bench(a, Bn, W)
    if a.tiny:
        res["tiny_fp32_b4"] = tiny_bench(a, Bn)
    if a.target:
        res["target_forward"] = target_forward_bench(Bn, nd)
    if a.closed and a.workload == "qwen3_8b_shape_b16_bs32":
        res["closed_step"] = closed_step_bench(a, Bn, W)
    if a.cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(dims, W, wl, B, S, int(ctx_before[0]))
    res["setup_s"] = round(setup_s, 1)
    print(json.dumps(res))


def host_step_loop(Bn, cfg, w, dims, bt, B, S, pool, n_pages, table, max_pages, max_ctx, ctx0, new_hid, ws,
                   ws_bytes, p_match, steps, warmup, seed):
    """The drafter step driven from the host, as the main measurement runs it: inject the
    previous step's a+1 accepted tokens of every sequence (their rows of new_hid), draft a
    block, verify it greedily against target logits that agree with each draft token with
    probability p_match (the stand-in for the target model, outside the timed intervals).
    Returns ms per step (inject + draft + verify, HIP events on the stream), the draft-only
    time on the final state, and the accepted tokens (a+1 summed over sequences) per step."""
    import numpy as np
    import torch
    dev = "cuda"
    stream = torch.cuda.current_stream()
    g = torch.Generator(device=dev).manual_seed(seed)
    z0 = torch.randn(bt, B + 1, dims.vocab, generator=g, device=dev, dtype=torch.float32)
    zmax = z0[:, :B].amax(-1) + 1.0
    zmin = z0[:, :B].amin(-1) - 1.0
    ctx = np.asarray(ctx0, dtype=np.int64).copy()
    ctx_dev = torch.tensor(ctx, dtype=torch.int32, device=dev)
    tok = torch.empty(bt, B, dtype=torch.int32, device=dev)
    acc = torch.empty(bt, dtype=torch.int32, device=dev)
    outt = torch.empty(bt, B + 1, dtype=torch.int32, device=dev)
    vws_bytes = Bn.dflash_verify_workspace_size(bt, B, dims.vocab)
    vws = torch.empty(vws_bytes, dtype=torch.uint8, device=dev)
    pin_seq = torch.empty(bt * (B + 1), dtype=torch.int32, pin_memory=True)
    pin_pos = torch.empty(bt * (B + 1), dtype=torch.int32, pin_memory=True)
    dev_seq = torch.empty(bt * (B + 1), dtype=torch.int32, device=dev)
    dev_pos = torch.empty(bt * (B + 1), dtype=torch.int32, device=dev)
    last = None
    hot, accs = [], []
    for i in range(warmup + steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        n_new = 0
        if last is not None:
            seqs = np.concatenate([np.full(int(x) + 1, b) for b, x in enumerate(last)])
            poss = np.concatenate([np.arange(ctx[b], ctx[b] + int(x) + 1) for b, x in enumerate(last)])
            n_new = len(seqs)
            pin_seq[:n_new] = torch.from_numpy(seqs.astype(np.int32))
            pin_pos[:n_new] = torch.from_numpy(poss.astype(np.int32))
            dev_seq[:n_new].copy_(pin_seq[:n_new], non_blocking=True)
            dev_pos[:n_new].copy_(pin_pos[:n_new], non_blocking=True)
            ctx = ctx + last + 1
            ctx_dev.copy_(torch.from_numpy(ctx.astype(np.int32)), non_blocking=True)
        ev[0].record(stream)
        if n_new:
            Bn.dflash_inject_kv(cfg, w, new_hid, dev_seq, dev_pos, n_new, pool, n_pages, table, bt, max_pages, ws,
                                ws_bytes)
        Bn.dflash_draft_block(cfg, w, pool, n_pages, table, max_pages, ctx_dev, max_ctx, bt, B, S, 0.0, 0, tok, None,
                              None, ws, ws_bytes)
        ev[1].record(stream)
        coin = torch.rand(bt, B, generator=g, device=dev) < p_match
        idx = tok.long().unsqueeze(-1)
        keep = z0[:, :B].gather(-1, idx)
        z0[:, :B].scatter_(-1, idx, torch.where(coin, zmax, zmin).unsqueeze(-1))
        ev[2].record(stream)
        Bn.dflash_verify_block(bt, B, dims.vocab, z0, tok, 0.0, None, None, acc, outt, vws, vws_bytes)
        ev[3].record(stream)
        z0[:, :B].scatter_(-1, idx, keep)
        last = acc.cpu().numpy().astype(np.int64)     # the scheduler needs the acceptance
        torch.cuda.synchronize()
        if i >= warmup:
            hot.append(ev[0].elapsed_time(ev[1]) + ev[2].elapsed_time(ev[3]))
            accs.append(int(np.sum(last + 1)))
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nd = 5
    d0.record(stream)
    for _ in range(nd):
        Bn.dflash_draft_block(cfg, w, pool, n_pages, table, max_pages, ctx_dev, max_ctx, bt, B, S, 0.0, 0, tok, None,
                              None, ws, ws_bytes)
    d1.record(stream)
    torch.cuda.synchronize()
    return float(np.mean(hot)), d0.elapsed_time(d1) / nd, accs, ctx


def incremental_bench(a, Bn, W):
    """The incremental workload: batch 32, block 8, two denoise steps, contexts lognormal
    (median 2048, clamped to [512, 8192]) in the paged pool, eight groups of four sequences
    sharing a 512-token prefix (32 physical pages named by four block-table rows, injected
    once); every step injects only the a+1 tokens the previous verification committed, then
    drafts and verifies.  Same Qwen3-8B-shaped weights as the main measurement."""
    import numpy as np
    import torch
    from block_diffusion_drafter_injection_amd import synth
    wl = synth.WORKLOADS["incremental_8b_shape_b8_bs32"]
    dims, bt, B, S, dev = wl.dims, wl.batch, wl.block_size, wl.n_steps, "cuda"
    cfg, w = Bn.make_config(dims), Bn.Weights(W)
    ctx0 = synth.context_lengths(wl).numpy().astype(np.int64)
    steps, warm = a.steps, a.warmup
    grow = (steps + warm + 2) * (B + 1)
    shared_pages, group = wl.shared_prefix // 16, wl.group_size
    need = [(int(c) + grow + 15) // 16 for c in ctx0]
    max_pages = max(need)
    table = np.full((bt, max_pages), -1, dtype=np.int32)
    nxt = 0
    for g0 in range(0, bt, group):
        table[g0:g0 + group, :shared_pages] = np.arange(nxt, nxt + shared_pages)
        nxt += shared_pages
    for b in range(bt):
        table[b, shared_pages:need[b]] = np.arange(nxt, nxt + need[b] - shared_pages)
        nxt += need[b] - shared_pages
    n_pages = nxt
    tab = torch.from_numpy(table).to(dev)
    pool = torch.zeros(Bn.pool_elems(dims, n_pages), dtype=dims.torch_dtype, device=dev)
    max_ctx = int(ctx0.max()) + grow
    ws_bytes = Bn.dflash_workspace_size(cfg, bt, B, 8192, max_ctx)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    # initial contexts (setup, untimed): each shared prefix injected once, by the group's first sequence
    for b in range(bt):
        start = wl.shared_prefix if b % group else 0
        c = int(ctx0[b])
        hid = synth.make_hiddens(dims, c - start, wl.seed * 1000 + b, dev)
        Bn.dflash_inject_kv(cfg, w, hid, torch.full((c - start,), b, dtype=torch.int32, device=dev),
                            torch.arange(start, c, dtype=torch.int32, device=dev), c - start, pool, n_pages, tab, bt,
                            max_pages, ws, ws_bytes)
        del hid
    new_hid = synth.make_hiddens(dims, bt * (B + 1), wl.seed + 77, dev)
    torch.cuda.synchronize()
    ms, draft_ms, accs, ctx_end = host_step_loop(Bn, cfg, w, dims, bt, B, S, pool, n_pages, tab, max_pages, max_ctx,
                                                 ctx0, new_hid, ws, ws_bytes, wl.p_match, steps, warm, 3000 + wl.seed)
    accepted = float(np.mean(accs))
    t_roof = draft_roofline_ms(dims, bt, B, S, ctx_end)
    unique_pages = float(np.sum(ctx_end)) - (bt - bt // group) * wl.shared_prefix
    del pool, ws, new_hid
    torch.cuda.empty_cache()
    return {"workload": wl.name, "batch": bt, "block": B, "denoise_steps": S, "ctx_min": int(ctx0.min()),
            "ctx_max": int(ctx0.max()), "ctx_mean": round(float(ctx0.mean()), 1), "shared_prefix": wl.shared_prefix,
            "group_size": group, "steps": steps,
            "ms_per_step": round(ms, 4), "accepted_tok_s": round(accepted / (ms / 1e3), 1),
            "mean_accept_plus_bonus": round(accepted / bt, 3),
            "draft_ms": round(draft_ms, 4), "drafted_tok_s": round(bt * B / (draft_ms / 1e3), 1),
            "t_roof_ms": round(t_roof, 4), "frac": round(t_roof / draft_ms, 4),
            "note": "step = inject a+1 committed tokens per sequence + draft + greedy verify; the roofline "
                    "counts every sequence's context K/V once per layer and forward (shared prefix pages too), "
                    f"the pool holding {int(unique_pages)} distinct tokens"}


def tiny_bench(a, Bn):
    """The tiny fp32 workload (hidden 256, 2 layers, vocab 1024, block 4, two denoise steps,
    batch 1, context 64): absolute latencies, since its work is far below any roofline (the
    call is a chain of short kernels, so launch latency sets its time)."""
    import numpy as np
    import torch
    from block_diffusion_drafter_injection_amd import synth
    wl = synth.WORKLOADS["tiny_fp32_b4"]
    dims, bt, B, S, dev = wl.dims, wl.batch, wl.block_size, wl.n_steps, "cuda"
    ctx0 = synth.context_lengths(wl).numpy().astype(np.int64)
    W = synth.make_weights(dims, wl.seed, dev)
    cfg, w = Bn.make_config(dims), Bn.Weights(W)
    steps, warm = max(a.steps, 20), max(a.warmup, 3)
    grow = (steps + warm + 2) * (B + 1)
    max_ctx = int(ctx0.max()) + grow
    max_pages = (max_ctx + 15) // 16
    tab = torch.arange(max_pages, dtype=torch.int32, device=dev).view(1, -1)
    pool = torch.zeros(Bn.pool_elems(dims, max_pages), dtype=dims.torch_dtype, device=dev)
    ws_bytes = Bn.dflash_workspace_size(cfg, bt, B, 256, max_ctx)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    c = int(ctx0[0])
    Bn.dflash_inject_kv(cfg, w, synth.make_hiddens(dims, c, wl.seed * 1000, dev),
                        torch.zeros(c, dtype=torch.int32, device=dev), torch.arange(c, dtype=torch.int32, device=dev),
                        c, pool, max_pages, tab, 1, max_pages, ws, ws_bytes)
    new_hid = synth.make_hiddens(dims, bt * (B + 1), wl.seed + 77, dev)
    torch.cuda.synchronize()
    ms, draft_ms, accs, _ = host_step_loop(Bn, cfg, w, dims, bt, B, S, pool, max_pages, tab, max_pages, max_ctx, ctx0,
                                           new_hid, ws, ws_bytes, wl.p_match, steps, warm, 3000 + wl.seed)
    accepted = float(np.mean(accs))
    del pool, ws, W, w
    torch.cuda.empty_cache()
    return {"workload": wl.name, "dtype": "f32", "batch": bt, "block": B, "ctx": c, "steps": steps,
            "draft_ms": round(draft_ms, 4), "ms_per_step": round(ms, 4),
            "accepted_tok_s": round(accepted / (ms / 1e3), 1), "mean_accept_plus_bonus": round(accepted / bt, 3),
            "note": "absolute latency (fp32 VALU kernels; far below every roofline)"}


def closed_step_bench(a, Bn, W):
    """The drafter step with a target model in the loop: the Qwen3-8B-shaped draft (block 16:
    the last committed token as anchor plus 15 drafted positions) and a random-init
    Qwen3-8B-shaped 36-layer target, batch 32, contexts 4096.  One step: draft ->
    dflash_target_forward over the block (full logits, five captured layers, K/V appended to
    the target's cache) -> greedy verification of the 15 drafted tokens ->
    dflash_advance_context -> injection of the captured states of the a+1 processed tokens ->
    the bonus token becomes the next anchor.  Everything on the device, timed with events.
    Random-init draft and target agree on almost no token, so a is about 0 and each step
    commits about one token per sequence: the figure is the step's time, not a speed-up."""
    import numpy as np
    import torch
    from dataclasses import replace
    from block_diffusion_drafter_injection_amd import synth
    dd = synth.QWEN3_8B_SHAPE
    td = replace(synth.QWEN3_8B_SHAPE, n_layers=36, n_fuse=1)
    caps = [1, 9, 17, 25, 33]
    bt, Bk, S, ctx, dev = 32, 16, 2, 4096, "cuda"
    steps, warm = a.steps, a.warmup
    Wt = synth.make_weights(td, 7, dev)
    dcfg, dw = Bn.make_config(dd), Bn.Weights(W)
    tcfg, tw = Bn.make_config(td), Bn.Weights(Wt)
    inj = ctx - 1
    grow = (steps + warm + 2) * Bk
    pages_per = (inj + grow + 15) // 16
    n_pages = bt * pages_per
    table = torch.arange(n_pages, dtype=torch.int32, device=dev).view(bt, pages_per)
    # both caches filled directly (values of the spread injection produces; setup, untimed)
    pool_d = torch.empty(Bn.pool_elems(dd, n_pages), dtype=torch.bfloat16, device=dev).normal_(0.0, 3.6)
    pool_t = torch.empty(Bn.pool_elems(td, n_pages), dtype=torch.bfloat16, device=dev).normal_(0.0, 3.6)
    max_ctx = inj + grow
    dws_bytes = Bn.dflash_workspace_size(dcfg, bt, Bk, bt * Bk, max_ctx)
    dws = torch.empty(dws_bytes, dtype=torch.uint8, device=dev)
    tws_bytes = Bn.dflash_workspace_size(tcfg, bt, Bk, 0, max_ctx)
    tws = torch.empty(tws_bytes, dtype=torch.uint8, device=dev)
    vws_bytes = Bn.dflash_verify_workspace_size(bt, Bk - 1, td.vocab)
    vws = torch.empty(vws_bytes, dtype=torch.uint8, device=dev)
    ctx_dev = torch.full((bt,), inj, dtype=torch.int32, device=dev)
    anchor = torch.randint(0, dd.vocab, (bt,), device=dev, dtype=torch.int32)
    tok = torch.empty(bt, Bk, dtype=torch.int32, device=dev)
    drafted = torch.empty(bt, Bk - 1, dtype=torch.int32, device=dev)
    z = torch.empty(bt, Bk, td.vocab, dtype=torch.float32, device=dev)
    hid = torch.empty(bt, Bk, len(caps) * td.hidden, dtype=torch.bfloat16, device=dev)
    acc = torch.empty(bt, dtype=torch.int32, device=dev)
    out = torch.empty(bt, Bk, dtype=torch.int32, device=dev)
    seq = torch.empty(bt * Bk, dtype=torch.int32, device=dev)
    pos = torch.empty_like(seq)
    F = len(caps)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        Bn.dflash_draft_block(dcfg, dw, pool_d, n_pages, table, pages_per, ctx_dev, max_ctx, bt, Bk, S, 0.0, 0, tok,
                              None, None, dws, dws_bytes, anchor=anchor)
        if ev:
            ev[1].record(stream)
        Bn.dflash_target_forward(tcfg, tw, pool_t, n_pages, table, pages_per, ctx_dev, max_ctx, bt, Bk, tok, caps, z,
                                 hid, tws, tws_bytes)
        if ev:
            ev[2].record(stream)
        drafted.copy_(tok[:, 1:])
        Bn.dflash_verify_block(bt, Bk - 1, td.vocab, z, drafted, 0.0, None, None, acc, out, vws, vws_bytes)
        Bn.dflash_advance_context(bt, Bk - 1, acc, ctx_dev, seq, pos)
        Bn.dflash_inject_kv(dcfg, dw, hid.view(bt * Bk, F * td.hidden), seq, pos, bt * Bk, pool_d, n_pages, table, bt,
                            pages_per, dws, dws_bytes)
        anchor.copy_(out.gather(1, acc.long().unsqueeze(1)).squeeze(1))
        if ev:
            ev[3].record(stream)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    ctx_start = int(ctx_dev.min().item())
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    tot = torch.zeros(bt, dtype=torch.int64, device=dev)
    for i in range(steps):
        step(evs[i])
        tot += acc.long() + 1
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[3]) for e in evs]
    d_ms = [e[0].elapsed_time(e[1]) for e in evs]
    t_ms = [e[1].elapsed_time(e[2]) for e in evs]
    committed = float(tot.sum().item()) / steps
    # rooflines: the draft's, and one causal target forward of bt*Bk rows (weights once,
    # every context K/V once per layer, the LM head over every row)
    H, L, I, V = td.hidden, td.n_layers, td.intermediate, td.vocab
    nq, nkv, d = td.n_q_heads, td.n_kv_heads, td.head_dim
    M = bt * Bk
    tt = 0.0
    for N, K in [((nq + 2 * nkv) * d, H), (H, nq * d), (2 * I, H), (H, I)]:
        tt += L * max(2.0 * M * N * K / PEAK_BF16, N * K * 2 / PEAK_HBM)
    tt += L * float(bt * ctx_start) * nkv * d * 2 * 2 / PEAK_HBM
    tt += max(2.0 * M * V * H / PEAK_BF16, V * H * 2 / PEAK_HBM)
    td_roof = draft_roofline_ms(dd, bt, Bk, S, [ctx_start] * bt)
    del Wt, tw, pool_d, pool_t, dws, tws, z, hid
    torch.cuda.empty_cache()
    return {"batch": bt, "block": Bk, "anchor": True, "drafted_per_seq": Bk - 1, "ctx_start": ctx_start + 1,
            "target_layers": L, "captured_layers": caps, "steps": steps,
            "ms_per_step": round(float(np.mean(ms)), 4), "draft_ms": round(float(np.mean(d_ms)), 4),
            "target_forward_ms": round(float(np.mean(t_ms)), 4),
            "verify_advance_inject_ms": round(float(np.mean(ms)) - float(np.mean(d_ms)) - float(np.mean(t_ms)), 4),
            "committed_tok_s": round(committed / (float(np.mean(ms)) / 1e3), 1),
            "mean_accept_plus_bonus": round(committed / bt, 3),
            "draft_t_roof_ms": round(td_roof, 4), "target_t_roof_ms": round(tt * 1e3, 4),
            "step_frac": round((td_roof + tt * 1e3) / float(np.mean(ms)), 4),
            "note": "random-init draft and target: acceptance about 0, so the committed rate is about one token "
                    "per sequence per step; the step time is the figure"}


def target_forward_bench(Bn, nd):
    """dflash_target_forward of a random-init Qwen3-8B-shaped target (36 layers) over batch 32
    x 17 tokens (the last committed token and a block of 16) at context 4096, capturing five
    layers' outputs, with its roofline (weights once, every context K/V once per layer)."""
    import torch
    from dataclasses import replace
    from block_diffusion_drafter_injection_amd import synth
    dims = replace(synth.QWEN3_8B_SHAPE, n_layers=36)
    bt, n, ctx, dev = 32, 17, 4096, "cuda"
    caps = [1, 9, 17, 25, 33]
    W = synth.make_weights(dims, 7, dev)
    cfg, w = Bn.make_config(dims), Bn.Weights(W)
    pages_per = (ctx + n + 15) // 16
    n_pages = bt * pages_per
    table = torch.arange(n_pages, dtype=torch.int32, device=dev).view(bt, pages_per)
    pool = torch.randn(Bn.pool_elems(dims, n_pages), device=dev, dtype=torch.bfloat16).mul_(3.6)
    ws_bytes = Bn.dflash_workspace_size(cfg, bt, n, 0, ctx)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ctx_dev = torch.full((bt,), ctx, dtype=torch.int32, device=dev)
    tokens = torch.randint(0, dims.vocab, (bt, n), device=dev, dtype=torch.int32)
    z = torch.empty(bt, n, dims.vocab, dtype=torch.float32, device=dev)
    hid = torch.empty(bt, n, len(caps) * dims.hidden, dtype=torch.bfloat16, device=dev)

    def call():
        Bn.dflash_target_forward(cfg, w, pool, n_pages, table, pages_per, ctx_dev, ctx, bt, n, tokens, caps, z, hid,
                                 ws, ws_bytes)
    for _ in range(2):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(nd):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / nd
    # roofline of one causal forward of bt*n rows (the LM head over every row)
    H, L, I, V = dims.hidden, dims.n_layers, dims.intermediate, dims.vocab
    nq, nkv, d = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    M = bt * n
    t = 0.0
    for N, K in [((nq + 2 * nkv) * d, H), (H, nq * d), (2 * I, H), (H, I)]:
        t += L * max(2.0 * M * N * K / PEAK_BF16, N * K * 2 / PEAK_HBM)
    t += L * float(bt * ctx) * nkv * d * 2 * 2 / PEAK_HBM
    t += max(2.0 * M * V * H / PEAK_BF16, V * H * 2 / PEAK_HBM)
    del W, w, pool, ws, z, hid
    torch.cuda.empty_cache()
    return {"layers": L, "batch": bt, "n_tok": n, "ctx": ctx, "captured_layers": caps, "ms": round(ms, 4),
            "t_roof_ms": round(t * 1e3, 4), "frac": round(t * 1e3 / ms, 4),
            "note": "random-init Qwen3-8B-shaped target, causal over the 17 verified positions, full logits, "
                    "K/V appended to its own cache"}


def longctx_bench(Bn, nd, W):
    """Draft call at T = 1 (Gumbel-max) and sampled verification of the long-context workload:
    batch 32, block 16, contexts uniform in [16384, 32768], on the Qwen3-8B-shaped weights
    (the same shapes as the main workload).  The 16 GB pool is filled with random values
    directly (N(0, 3.6^2), the spread injection produces): injecting 790k tokens is setup,
    and the values do not change the work.  Target logits are N(0, 1) stand-ins."""
    import torch
    from block_diffusion_drafter_injection_amd import synth
    wl = synth.WORKLOADS["longctx_sampled_8b_shape_b16_bs32"]
    dims, bt, B, S, T, dev = wl.dims, wl.batch, wl.block_size, wl.n_steps, wl.temperature, "cuda"
    ctx = synth.context_lengths(wl).tolist()
    cfg, w = Bn.make_config(dims), Bn.Weights(W)
    pages = [(c + 15) // 16 for c in ctx]
    n_pages = sum(pages)
    pool = torch.empty(Bn.pool_elems(dims, n_pages), dtype=dims.torch_dtype, device=dev).normal_(0.0, 3.6)
    table = torch.zeros(bt, max(pages), dtype=torch.int32)
    nxt = 0
    for b in range(bt):
        table[b, :pages[b]] = torch.arange(nxt, nxt + pages[b], dtype=torch.int32)
        nxt += pages[b]
    table = table.to(dev)
    ctx_dev = torch.tensor(ctx, dtype=torch.int32, device=dev)
    ws_bytes = Bn.dflash_workspace_size(cfg, bt, B, 0, max(ctx))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    tok = torch.empty(bt, B, dtype=torch.int32, device=dev)
    lg = torch.empty(bt, B, dims.vocab, dtype=torch.float32, device=dev)

    def draft():
        Bn.dflash_draft_block(cfg, w, pool, n_pages, table, table.shape[1], ctx_dev, max(ctx), bt, B, S, T, 2024,
                              tok, lg, None, ws, ws_bytes)

    g = torch.Generator(device=dev).manual_seed(11)
    zt = torch.randn(bt, B + 1, dims.vocab, generator=g, device=dev)
    u = torch.rand(bt, B + 1, 2, generator=g, device=dev)
    vws_bytes = Bn.dflash_verify_workspace_size(bt, B, dims.vocab)
    vws = torch.empty(max(vws_bytes, 1), dtype=torch.uint8, device=dev)
    acc = torch.empty(bt, dtype=torch.int32, device=dev)
    outt = torch.empty(bt, B + 1, dtype=torch.int32, device=dev)

    def verify():
        Bn.dflash_verify_block(bt, B, dims.vocab, zt, tok, T, lg, u, acc, outt, vws, vws_bytes)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = {}
    for name, fn in (("draft", draft), ("verify", verify)):
        for _ in range(2):
            fn()
        e0.record()
        for _ in range(nd):
            fn()
        e1.record()
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / nd
    t_roof = draft_roofline_ms(dims, bt, B, S, ctx)
    kv_gb = float(sum(ctx)) * dims.n_layers * dims.n_kv_heads * dims.head_dim * 2 * 2 * S / 1e9
    # verify reads the target and draft logits once: HBM roofline of that pass
    v_roof = (zt.numel() + lg.numel()) * 4 / PEAK_HBM * 1e3
    del pool, ws, lg, zt
    torch.cuda.empty_cache()
    return {"workload": wl.name, "batch": bt, "block": B, "temperature": T, "ctx_min": min(ctx), "ctx_max": max(ctx),
            "draft_ms": round(times["draft"], 4), "drafted_tok_s": round(bt * B / (times["draft"] / 1e3), 1),
            "t_roof_ms": round(t_roof, 4), "frac": round(t_roof / times["draft"], 4),
            "context_kv_gb_per_draft": round(kv_gb, 2),
            "verify_ms": round(times["verify"], 4), "verify_t_roof_ms": round(v_roof, 4),
            "verify_frac": round(v_roof / times["verify"], 4),
            "note": "draft with out_logits (the sampled verify reads them); pool filled directly"}


def batch1_latency(Bn, nd):
    """Draft-call latency of the Qwen3-4B-shaped workload (one sequence, block 8, two denoise
    steps, context 2048) on its own weights and pool, with the roofline of that call."""
    import torch
    from block_diffusion_drafter_injection_amd import synth
    wl = synth.WORKLOADS["qwen3_4b_shape_b8"]
    dims, B, S, dev = wl.dims, wl.block_size, wl.n_steps, "cuda"
    ctx = int(synth.context_lengths(wl)[0])
    W = synth.make_weights(dims, wl.seed, dev)
    cfg, w = Bn.make_config(dims), Bn.Weights(W)
    n_pages = (ctx + B + 15) // 16
    table = torch.arange(n_pages, dtype=torch.int32, device=dev).view(1, -1)
    pool = torch.zeros(Bn.pool_elems(dims, n_pages), dtype=dims.torch_dtype, device=dev)
    ws_bytes = Bn.dflash_workspace_size(cfg, 1, B, ctx, ctx)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    hid = synth.make_hiddens(dims, ctx, wl.seed * 1000, dev)
    Bn.dflash_inject_kv(cfg, w, hid, torch.zeros(ctx, dtype=torch.int32, device=dev),
                        torch.arange(ctx, dtype=torch.int32, device=dev), ctx, pool, n_pages, table, 1, n_pages, ws,
                        ws_bytes)
    ctx_dev = torch.tensor([ctx], dtype=torch.int32, device=dev)
    tok = torch.empty(1, B, dtype=torch.int32, device=dev)
    for _ in range(3):
        Bn.dflash_draft_block(cfg, w, pool, n_pages, table, n_pages, ctx_dev, ctx, 1, B, S, 0.0, 0, tok, None, None,
                              ws, ws_bytes)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(nd * 4):
        Bn.dflash_draft_block(cfg, w, pool, n_pages, table, n_pages, ctx_dev, ctx, 1, B, S, 0.0, 0, tok, None, None,
                              ws, ws_bytes)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (nd * 4)
    tok_eager = tok.clone()
    # the same call captured once as a HIP graph and replayed: no host launch work
    # between its kernels (the library enqueues everything on the caller's stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        Bn.dflash_draft_block(cfg, w, pool, n_pages, table, n_pages, ctx_dev, ctx, 1, B, S, 0.0, 0, tok, None, None,
                              ws, ws_bytes)
    for _ in range(2):
        graph.replay()
    e0.record()
    for _ in range(nd * 4):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / (nd * 4)
    same = bool(torch.equal(tok, tok_eager))
    t_roof = draft_roofline_ms(dims, 1, B, S, [ctx])
    del graph, W, w, pool, ws, hid
    torch.cuda.empty_cache()
    return {"workload": wl.name, "batch": 1, "block": B, "ctx": ctx, "draft_ms": round(ms, 4),
            "drafted_tok_s": round(B / (ms / 1e3), 1), "t_roof_ms": round(t_roof, 4), "frac": round(t_roof / ms, 4),
            "graph_draft_ms": round(ms_graph, 4), "graph_frac": round(t_roof / ms_graph, 4),
            "graph_tokens_match_eager": same,
            "note": "weight streaming bound (M = 8 rows); the call is a chain of about a hundred small kernels, "
                    "timed called directly and as a replayed HIP graph of the same call"}


def device_loop(a, Bn, cfg, w, dims, bt, B, S, pool, n_pages, table, pages_per, max_ctx, ctx_dev, acc, tok, outt,
                new_hid, z0, zmax, zmin, p_match, g, ws, ws_bytes, vws, vws_bytes):
    """The step loop kept on the GPU: draft -> target logits (stand-in) -> verify ->
    dflash_advance_context -> inject the committed rows, captured once as a HIP graph and
    replayed a.steps times back to back with no host work in between.  The previous
    (host-driven) step's committed tokens are injected first, untimed."""
    import torch
    K = a.steps
    seq = torch.empty(bt * (B + 1), dtype=torch.int32, device="cuda")
    pos = torch.empty_like(seq)
    coins = torch.rand(K + 1, bt, B, generator=g, device="cuda") < p_match
    step = torch.zeros(1, dtype=torch.int64, device="cuda")
    hist = torch.zeros(K + 1, bt, dtype=torch.int32, device="cuda")
    n_rows = bt * (B + 1)

    def advance_inject():
        Bn.dflash_advance_context(bt, B, acc, ctx_dev, seq, pos)
        Bn.dflash_inject_kv(cfg, w, new_hid, seq, pos, n_rows, pool, n_pages, table, bt, pages_per, ws, ws_bytes)

    def body():
        Bn.dflash_draft_block(cfg, w, pool, n_pages, table, pages_per, ctx_dev, max_ctx, bt, B, S, 0.0, 0, tok,
                              None, None, ws, ws_bytes)
        coin = coins.index_select(0, step).squeeze(0)
        idx = tok.long().unsqueeze(-1)
        keep = z0[:, :B].gather(-1, idx)
        z0[:, :B].scatter_(-1, idx, torch.where(coin, zmax, zmin).unsqueeze(-1))
        Bn.dflash_verify_block(bt, B, dims.vocab, z0, tok, 0.0, None, None, acc, outt, vws, vws_bytes)
        z0[:, :B].scatter_(-1, idx, keep)
        hist.index_copy_(0, step, acc.unsqueeze(0))
        step.add_(1)
        advance_inject()

    advance_inject()          # the host-driven loop's last committed tokens
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()                # one eager step, so every kernel has run before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    step.zero_()
    graph.replay()            # warm replay
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    e0.record()
    for _ in range(K):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.time() - t0
    ms = e0.elapsed_time(e1) / K
    accepted = float(hist[1:K + 1].sum().item()) + bt * K
    return {"graph": True, "steps": K, "ms_per_step": round(ms, 4), "wall_ms_per_step": round(wall * 1e3 / K, 4),
            "accepted_tok_s": round(accepted / K / (ms / 1e3), 1),
            "mean_accept_plus_bonus": round(accepted / K / bt, 3),
            "note": "injection rows of all block+1 verified positions, those past the accepted prefix "
                    "marked -1 and packed out on the device, so the injection GEMMs run on the accepted "
                    "rows only; includes the target-logit stand-in kernels"}


def load_traffic(workload, cls):
    """HBM bytes per launch of the kernel from the committed counter summary, or None if
    there is none or the kernel sources changed since the counters were taken."""
    f = traffic_file(workload, cls)
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash():
        return None
    return t["bytes_per_launch"]


def _read_csv(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def summarize(trace_dir, fetch_dir, write_dir):
    """profiles/ summaries from rocprofv3 csv output: kernel time table of the benchmark run,
    and HBM traffic per launch of each timed kernel class, scaled by the calibration copy."""
    import glob
    import numpy as np
    wl_name = parse_workload_from(trace_dir)
    stats = _read_csv(glob.glob(os.path.join(trace_dir, "*kernel_stats.csv"))[0])
    counters = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _read_csv(glob.glob(os.path.join(d, "*counter_collection.csv"))[0])
        per = {}
        for r in rows:
            if r["Counter_Name"] != name:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        counters[name] = per
    copy_name = [k for k in counters["FETCH_SIZE"] if "copy" in k.lower() and "bfloat16" not in k.lower()]
    big = None
    for k in copy_name:
        vals = counters["FETCH_SIZE"][k]
        if big is None or max(vals) > big[1]:
            big = (k, max(vals))
    fetch_scale = COPY_BYTES / (big[1] * 1024.0)
    wvals = counters["WRITE_SIZE"].get(big[0], [0.0])
    write_scale = COPY_BYTES / (max(wvals) * 1024.0) if max(wvals) > 0 else None
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    h = source_hash()
    lines = [f"# rocprofv3 kernel statistics, {wl_name}", "",
             "Command (run from the repository root, output csv):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d <TRACE_DIR> -o run -- "
             "python bench.py --steps 5 --warmup 2 --cpu-baseline 0 --device-loop 0 --block-sweep 0 --ceilings 0 --batch1 0 --target 0 --longctx 0 --incremental 0 --tiny 0 --closed 0", "",
             f"Kernel sources hash: {h}", "",
             "| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:20]:
        nm = r["Name"].replace("dflash::", "")
        nm = nm.split("(")[0] if "dflash" in r["Name"] else nm[:60]
        lines.append(f"| `{nm}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.1f} |")
    with open(os.path.join(ROOT, "profiles", f"kernel_stats_{wl_name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    tl = [f"# HBM traffic per launch, {wl_name}", "",
          "Commands (repository root, csv output):", "",
          "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -o p -- "
          "python bench.py --steps 2 --warmup 1 --cpu-baseline 0 --device-loop 0 --block-sweep 0 --ceilings 0 --batch1 0 --target 0 --longctx 0 --incremental 0 --tiny 0 --closed 0 --copy-calibration 1",
          "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -o p -- "
          "python bench.py --steps 2 --warmup 1 --cpu-baseline 0 --device-loop 0 --block-sweep 0 --ceilings 0 --batch1 0 --target 0 --longctx 0 --incremental 0 --tiny 0 --closed 0 --copy-calibration 1",
          "    python bench.py --summarize <TRACE_DIR> <FETCH_DIR> <WRITE_DIR>", "",
          f"Calibration: a {COPY_BYTES >> 20} MiB device copy (`{big[0][:60]}`) reads FETCH_SIZE = "
          f"{big[1]:.0f} KiB -> fetch scale {fetch_scale:.4f}; WRITE_SIZE scale "
          f"{write_scale if write_scale is None else round(write_scale, 4)}.", "",
          f"Kernel sources hash: {h}", "",
          "| class | kernel | FETCH KiB/launch | WRITE KiB/launch | scaled MB/launch |", "|---|---|---|---|---|"]
    for cls, pat in KERNEL_NAMES.items():
        ks = [k for k in counters["FETCH_SIZE"] if re.search(pat, k)]
        if not ks:
            continue
        f = float(np.mean([v for k in ks for v in counters["FETCH_SIZE"][k]]))
        w = float(np.mean([v for k in ks for v in counters["WRITE_SIZE"].get(k, [0.0])]))
        by = f * 1024 * fetch_scale + w * 1024 * (write_scale or 1.0)
        tl.append(f"| {cls} | `{pat}` | {f:.0f} | {w:.0f} | {by / 1e6:.1f} |")
        with open(traffic_file(wl_name, cls), "w") as fh:
            json.dump({"workload": wl_name, "class": cls, "kernel": pat, "fetch_kib": f, "write_kib": w,
                       "fetch_scale": fetch_scale, "write_scale": write_scale, "bytes_per_launch": round(by),
                       "source_hash": h}, fh, indent=1)
    with open(os.path.join(ROOT, "profiles", f"hbm_traffic_{wl_name}.md"), "w") as fh:
        fh.write("\n".join(tl) + "\n")
    print("\n".join(lines + [""] + tl))


PROFILE_OFF = ("--cpu-baseline 0 --device-loop 0 --block-sweep 0 --ceilings 0 --batch1 0 --target 0 --longctx 0 "
               "--incremental 0 --tiny 0 --closed 0")
SQ_PASSES = [
    "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_LDS SQ_INSTS_LDS "
    "SQ_WAVE_CYCLES SQ_WAIT_ANY",
    "SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_ACTIVE_INST_VALU SQ_WAIT_INST_ANY SQ_INSTS_VMEM "
    "SQ_ACTIVE_INST_ANY",
    "SQ_WAVES SQ_BUSY_CYCLES SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_MISC "
    "SQ_INST_CYCLES_SALU GRBM_GUI_ACTIVE",
]
SQ_CLASSES = [
    ("LM head (`gemm_fl_kernel<256, 256, 4, 2, 1, 3, 3>`, both denoise steps)", r"gemm_fl_kernel<256, 256, 4, 2, 1, 3, 3>"),
    ("gate/up (SwiGLU) (`gemm_fl_kernel<128, 384, 2, 4, 2, 2, 2>`)", r"gemm_fl_kernel<128, 384, 2, 4, 2, 2, 2>"),
    ("O and down (residual) (`gemm_fl_kernel<128, 256, 2, 4, 2, 1, 2>`)", r"gemm_fl_kernel<128, 256, 2, 4, 2, 1, 2>"),
    ("q/k/v (`gemm_fl_kernel<128, 384, 2, 4, 2, 0, 2>`)", r"gemm_fl_kernel<128, 384, 2, 4, 2, 0, 2>"),
    ("attention context (`attn_ctx_mfma_kernel<128, 4>`)", r"attn_ctx_mfma_kernel<128, 4>"),
    ("attention finish (`attn_finish_kernel`)", r"attn_finish_kernel"),
    ("query prep (`attn_qprep_kernel`)", r"attn_qprep_kernel"),
    ("RMSNorm (`rmsnorm_kernel`)", r"rmsnorm_kernel"),
]


def _counter_classes(d):
    """Per kernel class, the mean over its dispatches of each counter (summed over the rows of a dispatch)."""
    import collections
    import glob
    import numpy as np
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    name = {}
    for r in _read_csv(glob.glob(os.path.join(d, "*counter_collection.csv"))[0]):
        per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        name[r["Dispatch_Id"]] = r["Kernel_Name"]
    cls = collections.defaultdict(lambda: collections.defaultdict(list))
    for dd, c in per.items():
        for label, pat in SQ_CLASSES:
            if re.search(pat, name[dd]):
                for k, v in c.items():
                    cls[label][k].append(v)
                break
    return {l: {k: float(np.mean(v)) for k, v in c.items()} for l, c in cls.items()}


def summarize_sq(d1, d2, d3):
    """profiles/sq_counters_*.md from the three counter passes of SQ_PASSES."""
    p1, p2, p3 = _counter_classes(d1), _counter_classes(d2), _counter_classes(d3)
    wl_name = parse_workload_from(d1)
    lines = [f"# Shader-sequencer counters per kernel, {wl_name}", "",
             "Three counter passes over the same short benchmark run (repository root, csv output; each pass stays "
             "within the per-block counter limits), then the summary:", ""]
    for i, ctr in enumerate(SQ_PASSES, 1):
        lines.append(f"    rocprofv3 --pmc {ctr} --output-format csv -d <DIR{i}> -o p -- python bench.py --steps 1 "
                     f"--warmup 1 {PROFILE_OFF}")
    lines += ["    python bench.py --summarize-sq <DIR1> <DIR2> <DIR3>", "",
              f"Kernel sources hash: {source_hash()}", "",
              "Derived per dispatch (each counter summed over the rows the tool reports for the dispatch), averaged "
              "over the dispatches of each kernel. The GRBM_GUI_ACTIVE value is the sum over the 8 XCDs, so it is "
              "divided by 8 to get the dispatch's cycles:", "",
              "- MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs);",
              "- LDS indexed busy % = SQ_LDS_IDX_ACTIVE / (cycles x 256 CUs) (ds_read/ds_write only; the direct "
              "global->LDS copies are not indexed operations and are not in it);",
              "- bank-conflict cycles % = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE;",
              "- wave time waiting % = SQ_WAIT_ANY / SQ_WAVE_CYCLES (both in quad-cycles);",
              "- instructions per wave = SQ_INSTS_* / SQ_WAVES (\"other VALU\" excludes the MFMAs, which the VALU "
              "count includes).", "",
              "| kernel | cycles per XCD (µs at 2.1 GHz) | MFMA busy % | LDS indexed busy % | bank-conflict cycles % "
              "of LDS | wave time waiting % | MFMA / wave | other VALU / wave | SALU / wave | LDS instr / wave |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    for label, _ in SQ_CLASSES:
        a, b, c = p1.get(label), p2.get(label), p3.get(label)
        if not (a and b and c):
            continue
        cyc = c["GRBM_GUI_ACTIVE"] / 8
        waves = max(c["SQ_WAVES"], 1.0)
        lines.append(
            f"| {label} | {cyc / 2100:.0f} | {100 * a['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.0f} | "
            f"{100 * a['SQ_LDS_IDX_ACTIVE'] / (cyc * 256):.0f} | "
            f"{100 * a['SQ_LDS_BANK_CONFLICT'] / max(a['SQ_LDS_IDX_ACTIVE'], 1):.0f} | "
            f"{100 * a['SQ_WAIT_ANY'] / max(a['SQ_WAVE_CYCLES'], 1):.0f} | {b['SQ_INSTS_MFMA'] / waves:.0f} | "
            f"{(b['SQ_INSTS_VALU'] - b['SQ_INSTS_MFMA']) / waves:.0f} | {b['SQ_INSTS_SALU'] / waves:.0f} | "
            f"{b['SQ_INSTS_LDS'] / waves:.0f} |")
    with open(os.path.join(ROOT, "profiles", f"sq_counters_{wl_name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_verify(trace_dir):
    """profiles/kernel_stats_sampled_verify_*.md: the sampled-verification kernels of a --longctx 1 trace."""
    import glob
    rows = _read_csv(glob.glob(os.path.join(trace_dir, "*kernel_stats.csv"))[0])
    wl = "longctx_sampled_8b_shape_b16_bs32"
    lines = [f"# rocprofv3 kernel statistics, sampled verification of {wl}", "",
             "Command (run from the repository root, output csv), then the summary:", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d <TRACE_DIR> -o run -- python bench.py "
             "--steps 2 --warmup 1 " + PROFILE_OFF.replace("--longctx 0", "--longctx 1"),
             "    python bench.py --summarize-verify <TRACE_DIR>", "",
             f"Kernel sources hash: {source_hash()}", "",
             "The sampled-verification kernels run only in the `longctx_sampled` section of that command (batch 32, "
             "block 16, vocabulary 151936, T = 1: 330 MB of target and 311 MB of draft logits per call); the rows "
             "below are those kernels from `run_kernel_stats.csv`.", "",
             "| kernel | calls | avg us | total ms |", "|---|---|---|---|"]
    tot = 0.0
    for w in ["lse_rows_kernel", "draw_select_kernel", "draw_segments_kernel", "lse_merge_kernel"]:
        for r in rows:
            if r["Name"].split("(")[0].endswith(w):
                avg = float(r["AverageNs"]) / 1e3
                tot += avg
                lines.append(f"| `{w}` | {r['Calls']} | {avg:.1f} | {float(r['TotalDurationNs']) / 1e6:.2f} |")
    lines += ["", f"Sum of the per-call averages: {tot:.1f} us per verification (641 MB of logits; 80 us at 8 TB/s)."]
    with open(os.path.join(ROOT, "profiles", f"kernel_stats_sampled_verify_{wl}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def parse_workload_from(trace_dir):
    """Workload name recorded by the benchmark run next to the trace (default workload otherwise)."""
    f = os.path.join(trace_dir, "workload.txt")
    if os.path.exists(f):
        return open(f).read().strip()
    return "qwen3_8b_shape_b16_bs32"


def cpu_baseline(dims, W, wl, B, S, ctx, min_seconds=10.0, max_seqs=4):
    """The fp64 oracle, as it stands, on a bounded sample of the workload: one sequence
    at a time (inject 4 new tokens, draft one block, verify it) until min_seconds of work
    or max_seqs sequences.  Throughput = accepted tokens / oracle time."""
    import numpy as np
    import torch
    import oracle
    from block_diffusion_drafter_injection_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    Wn = {k: ([t.float().cpu().numpy() for t in v] if isinstance(v, list) else v.float().cpu().numpy())
          for k, v in W.items()}
    spent, accepted, n = 0.0, 0, 0
    while n < max_seqs and (spent < min_seconds or n == 0):
        K, V = synth.make_pool_values(dims, ctx, 99 + n, "cpu")
        K, V = K.double().numpy(), V.double().numpy()
        x = synth.make_hiddens(dims, 4, 98 + n, "cpu").double().numpy()
        t0 = time.time()
        Kn, Vn = oracle.inject(dims, Wn, x, np.arange(ctx, ctx + 4))
        K = np.concatenate([K, Kn], axis=1)
        V = np.concatenate([V, Vn], axis=1)
        r = oracle.draft_block(dims, Wn, [(K, V)], [ctx + 4], B, S, want_logits=False)
        tok = torch.from_numpy(r["tokens"].astype(np.int32))
        zt = synth.make_greedy_target_logits(tok, dims.vocab, wl.p_match, seed=5 + n).numpy()
        acc, _ = oracle.verify_greedy(zt, r["tokens"])
        spent += time.time() - t0
        accepted += int(acc[0]) + 1
        n += 1
    return {"value": round(accepted / spent, 4), "unit": "tok/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} of {wl.batch} sequences, one step each (inject 4 tokens, {S}-step block-{B} "
                      f"draft at context {ctx}, greedy verify): {accepted} accepted tokens in {spent:.1f} s"}


if __name__ == "__main__":
    main()
