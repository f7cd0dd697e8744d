"""Plain fp64 CPU oracle for the block-diffusion draft step with KV injection.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; the only thing both sides have in common is the seeded input they
are handed.

Sources (the method's description, cited by page title and section):

* [Note]  "DFlash: Block Diffusion for Flash Speculative Decoding" (study note,
  notebook-dae.pages.dev), sections "整体架构", "三大核心创新" (1 context
  feature extraction, 2 KV injection, 3 block diffusion decoding) and
  "Immediate Materialization".
* [Blog]  "DFlash：用“块扩散”魔法，让大模型推理速度起飞！" (blog.veyvin.com),
  sections "核心创新" (the draft/verify loop) and "2. Flash Verification".
* [Deep]  "DFlash + Spec V2 深度解析" (ai-master.cc), sections "2.2 DFlash 的解法：
  KV 注入", "2.3 块扩散：并行生成 block", "4.2 训练配置", "4.3 评估指标".

Everything is computed in float64.  Where the GPU stores a value in bfloat16
(the injected KV pool and the LM-head input) the oracle rounds its own fp64
value to the nearest bfloat16 (ties to even) at the same point; everything
else stays fp64.  The readings taken where the pages are silent are listed in
each function's docstring.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
brute-force loops on tiny inputs, closed forms and invariants.  Faithfulness
to DFlash's trained drafter itself is parity-unpinned: the pages print no
worked example.
"""
from .numerics import bf16_round, rope, rmsnorm, silu, log_softmax, logsumexp, split_hilo
from .philox import philox4x32_10, gumbel_noise, uniform24
from .model import (inject, forward_hidden, lm_head_logits, draft_block, attention_group,
                    commit_counts, target_forward)
from .verify import verify_greedy, verify_sampled, inverse_cdf

__all__ = [
    "bf16_round", "rope", "rmsnorm", "silu", "log_softmax", "logsumexp", "split_hilo",
    "philox4x32_10", "gumbel_noise", "uniform24",
    "inject", "forward_hidden", "lm_head_logits", "draft_block", "attention_group", "commit_counts",
    "target_forward",
    "verify_greedy", "verify_sampled", "inverse_cdf",
]
