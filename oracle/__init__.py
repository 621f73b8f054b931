"""CPU oracle of the speculative-decoding verify step.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  The library's product path never calls it, and it shares
no code with the HIP path: no kernels, headers, helpers, tables or constant
generators.  The only thing both sides share is the seeded input package
`synth`, which holds no part of the method's arithmetic.

Everything is plain PyTorch CPU arithmetic in float64 over bf16 weights that are
upcast exactly.  The single place where the oracle rounds is the KV cache, which
is stored in bf16 because the cache is state of the 16-bit model that replay must
reproduce.

Sources (cited by page title and section; no line numbers):
  [ShardFlow]  "I Got 28 TPS Out of Free Kaggle GPUs: Here's What It Took" (dev.to)
  [Sangama]    "Qwen3.5-397B on 20 GPUs, through a relay" (sangama.pages.dev)
The decoder layer itself (pre-norm RMSNorm, rotate-half RoPE, grouped-query
attention, SwiGLU, q/k/v biases, untied or tied head) is the Qwen2.5 layer of
the models the ShardFlow page runs (Qwen2.5-7B target, Qwen2.5-0.5B drafter).

Pins: see tests/test_oracle_*.py.  Every function here is pinned by at least one
closed form, invariant, brute-force enumeration or independent library routine.
"""
from .decoder import (
    Model,
    KVCache,
    round_bf16,
    rms_norm,
    rope_angles,
    rope,
    silu,
    swiglu,
    causal_gqa_attention,
    forward,
)
from .spec import (
    argmax_lowest,
    top_gap,
    accept_prefix,
    verify,
    prefill,
    greedy_decode,
    greedy_continuation,
    rollback,
    set_next,
    speculative_decode,
    model_draft_round,
    snapshot,
    restore,
    snapshot_verify,
)
from .ngram import propose
from . import nf4

__all__ = [
    "Model", "KVCache", "round_bf16", "rms_norm", "rope_angles", "rope", "silu", "swiglu",
    "causal_gqa_attention", "forward", "argmax_lowest", "top_gap", "accept_prefix", "verify",
    "prefill", "greedy_decode", "greedy_continuation", "rollback", "set_next",
    "speculative_decode", "model_draft_round", "snapshot", "restore", "snapshot_verify", "propose", "nf4",
]
