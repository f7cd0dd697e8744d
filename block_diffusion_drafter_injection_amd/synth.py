"""Seeded synthetic inputs for the draft step: workload definitions, random-init
weights, target hidden states, target/draft logits, uniforms, context lengths.

This module holds no arithmetic of the method itself; it only draws inputs.
Both the HIP library (through the binding) and the CPU oracle (in the tests)
are fed from it.  Draws use torch generators on the requested device so the
large workloads can be generated in device memory directly; the same call
on the same device and seed gives the same values.

Shapes follow the workloads named below: random-init weights N(0, 0.02)
rounded to bfloat16 (fp32 for the tiny workload), RMSNorm gains 1, target
hidden states N(0, 1), and target logits whose argmax agrees with the draft
token at a chosen per-position rate (a stand-in for the code-generation
prompts the pages measure on, whose acceptance lengths the pages rate at
"> 3 acceptable, > 4 excellent").
"""
from dataclasses import dataclass, field, replace
import math

import torch


@dataclass(frozen=True)
class ModelDims:
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_fuse: int
    target_hidden: int
    rope_base: float
    dtype: str = "bf16"          # 'bf16' or 'fp32': storage type of weights, inputs and KV pool
    rms_eps: float = 1e-6
    page_size: int = 16
    qk_norm: bool = False        # per-head RMSNorm of queries and keys before RoPE (Qwen3 layers)

    @property
    def mask_token_id(self):
        return self.vocab - 1

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


@dataclass(frozen=True)
class Workload:
    name: str
    dims: ModelDims
    batch: int
    block_size: int
    n_steps: int
    ctx: tuple                    # ('fixed', n) | ('lognormal', median, sigma, lo, hi) | ('uniform', lo, hi)
    temperature: float = 0.0
    p_match: float = 0.5          # greedy verify: chance a target row agrees with the draft token
    loop_steps: int = 1           # inject -> draft -> verify rounds
    shared_prefix: int = 0        # tokens of prefix shared by each group of sequences
    group_size: int = 1
    seed: int = 0


TINY = ModelDims(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512,
                 vocab=1024, n_fuse=3, target_hidden=256, rope_base=1e4, dtype="fp32")
QWEN3_4B_SHAPE = ModelDims(hidden=2560, n_layers=5, n_q_heads=32, n_kv_heads=8, head_dim=128,
                           intermediate=9728, vocab=151936, n_fuse=5, target_hidden=2560, rope_base=1e6)
QWEN3_8B_SHAPE = ModelDims(hidden=4096, n_layers=5, n_q_heads=32, n_kv_heads=8, head_dim=128,
                           intermediate=12288, vocab=151936, n_fuse=5, target_hidden=4096, rope_base=1e6)

WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_b4", TINY, batch=1, block_size=4, n_steps=2, ctx=("fixed", 64),
                 p_match=0.5, seed=1),
        Workload("qwen3_4b_shape_b8", QWEN3_4B_SHAPE, batch=1, block_size=8, n_steps=2,
                 ctx=("fixed", 2048), p_match=0.7, seed=2),
        Workload("qwen3_8b_shape_b16_bs32", QWEN3_8B_SHAPE, batch=32, block_size=16, n_steps=2,
                 ctx=("fixed", 4096), p_match=0.75, seed=3),
        Workload("incremental_8b_shape_b8_bs32", QWEN3_8B_SHAPE, batch=32, block_size=8, n_steps=2,
                 ctx=("lognormal", 2048, math.log(16) / 4, 512, 8192), p_match=0.75,
                 loop_steps=64, shared_prefix=512, group_size=4, seed=4),
        Workload("longctx_sampled_8b_shape_b16_bs32", QWEN3_8B_SHAPE, batch=32, block_size=16,
                 n_steps=2, ctx=("uniform", 16384, 32768), temperature=1.0, seed=5),
    ]
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def context_lengths(w: Workload, device="cpu"):
    """Per-sequence context lengths (int64 tensor on the CPU)."""
    kind = w.ctx[0]
    if kind == "fixed":
        return torch.full((w.batch,), int(w.ctx[1]), dtype=torch.int64)
    g = _gen("cpu", 5000 + w.seed)
    if kind == "uniform":
        lo, hi = w.ctx[1], w.ctx[2]
        return torch.randint(lo, hi + 1, (w.batch,), generator=g, dtype=torch.int64)
    if kind == "lognormal":
        med, sig, lo, hi = w.ctx[1:]
        x = torch.exp(math.log(med) + sig * torch.randn(w.batch, generator=g, dtype=torch.float64))
        return torch.clamp(torch.round(x), lo, hi).to(torch.int64)
    raise ValueError(kind)


def make_weights(d: ModelDims, seed, device="cpu", std=0.02):
    """Random-init draft weights in the storage dtype (matrices N(0, std), gains 1)."""
    g = _gen(device, 1000 + seed)
    dt = d.torch_dtype
    H, L, I = d.hidden, d.n_layers, d.intermediate
    nq, nkv, hd = d.n_q_heads, d.n_kv_heads, d.head_dim

    def mat(n, k):
        return (torch.randn(n, k, generator=g, device=device, dtype=torch.float32) * std).to(dt)

    def gain(n):
        return torch.ones(n, device=device, dtype=torch.float32)

    W = dict(
        w_fc=mat(H, d.n_fuse * d.target_hidden),
        w_kv=mat(L * 2 * nkv * hd, H),
        embed=mat(d.vocab, H),
        final_norm=gain(H),
        lm_head=mat(d.vocab, H),
        attn_norm=[], w_q=[], w_o=[], mlp_norm=[], w_gate=[], w_up=[], w_down=[],
    )
    if d.qk_norm:
        W["q_norm"] = [gain(hd) for _ in range(L)]
        W["k_norm"] = [gain(hd) for _ in range(L)]
    for _ in range(L):
        W["attn_norm"].append(gain(H))
        W["w_q"].append(mat(nq * hd, H))
        W["w_o"].append(mat(H, nq * hd))
        W["mlp_norm"].append(gain(H))
        W["w_gate"].append(mat(I, H))
        W["w_up"].append(mat(I, H))
        W["w_down"].append(mat(H, I))
    return W


def make_hiddens(d: ModelDims, n_tok, seed, device="cpu"):
    """Target hidden states of n_tok tokens, F layers concatenated: [n_tok, F*Ht], N(0,1)."""
    g = _gen(device, 2000 + seed)
    return torch.randn(n_tok, d.n_fuse * d.target_hidden, generator=g, device=device,
                       dtype=torch.float32).to(d.torch_dtype)


def make_pool_values(d: ModelDims, n_tok, seed, device="cpu", k_std=3.6, v_std=3.6):
    """Synthetic logical KV contents [L, n_tok, n_kv, d] (K and V), in the storage dtype.

    The default spread matches what injection produces from N(0,1) hiddens
    through N(0, 0.02) weights at the Qwen3-8B shape (about 3.6).
    """
    g = _gen(device, 7000 + seed)
    shp = (d.n_layers, n_tok, d.n_kv_heads, d.head_dim)
    K = (torch.randn(shp, generator=g, device=device, dtype=torch.float32) * k_std).to(d.torch_dtype)
    V = (torch.randn(shp, generator=g, device=device, dtype=torch.float32) * v_std).to(d.torch_dtype)
    return K, V


def make_greedy_target_logits(draft_tokens, vocab, p_match, seed, device="cpu"):
    """Target logits [bt, B+1, V] fp32 from N(0,1): each row i < B is made to agree
    with draft token i with probability p_match (that entry set to row max + 1),
    otherwise made to disagree (that entry set to row min - 1).  Row B is plain."""
    dt = draft_tokens.to(device=device, dtype=torch.int64)
    bt, B = dt.shape
    g = _gen(device, 3000 + seed)
    z = torch.randn(bt, B + 1, vocab, generator=g, device=device, dtype=torch.float32)
    coin = torch.rand(bt, B, generator=g, device=device, dtype=torch.float32) < p_match
    zb = z[:, :B]
    hi = zb.max(dim=-1).values + 1.0
    lo = zb.min(dim=-1).values - 1.0
    val = torch.where(coin, hi, lo)
    zb.scatter_(-1, dt.unsqueeze(-1), val.unsqueeze(-1))
    return z


def make_sampled_logits(bt, B, vocab, seed, device="cpu", spread=0.6):
    """Draft logits [bt, B, V] ~ N(0,1); target logits [bt, B+1, V]: rows i < B are the
    draft row plus spread*N(0,1), row B is N(0,1)."""
    g = _gen(device, 3000 + seed)
    zd = torch.randn(bt, B, vocab, generator=g, device=device, dtype=torch.float32)
    zt = torch.empty(bt, B + 1, vocab, device=device, dtype=torch.float32)
    zt[:, :B] = zd + spread * torch.randn(bt, B, vocab, generator=g, device=device, dtype=torch.float32)
    zt[:, B] = torch.randn(bt, vocab, generator=g, device=device, dtype=torch.float32)
    return zd, zt


def sample_tokens(logits, temperature, seed):
    """Draw one token per row of logits [..., V] from softmax(logits/T) (torch.multinomial)."""
    g = _gen(logits.device, 8000 + seed)
    flat = torch.softmax(logits.reshape(-1, logits.shape[-1]).double() / temperature, dim=-1)
    return torch.multinomial(flat, 1, generator=g).reshape(logits.shape[:-1]).to(torch.int32)


def make_uniforms(bt, B, seed, device="cpu"):
    """Uniforms [bt, B+1, 2] in [0, 1), fp32."""
    g = _gen(device, 4000 + seed)
    return torch.rand(bt, B + 1, 2, generator=g, device=device, dtype=torch.float32)


def small_dims(**kw):
    """A small bf16 shape that still spans several GEMM/attention tiles and
    ragged tails (vocab and contexts not multiples of any tile)."""
    base = ModelDims(hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                     intermediate=1024, vocab=5003, n_fuse=3, target_hidden=384, rope_base=1e6)
    return replace(base, **kw)
