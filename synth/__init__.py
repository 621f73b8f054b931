"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This package generates data only: model shapes, random-init weights, prompts,
draft corruptions, synthetic KV-cache contents and prompt-lookup histories.  It
holds none of the decoder's arithmetic (no norms, no attention, no argmax, no
accept rule), so that the CPU oracle and the HIP path can both be fed from it
without sharing any part of the method.

Every generator is a pure function of an integer seed.  Large tensors are
generated in fixed 2**22-element chunks, each from its own PCG64 stream keyed
by (seed, tensor name, chunk index), so the bytes do not depend on the number
of threads used.
"""
from .shapes import (Shape, TINY, QWEN05B, QWEN05B_UNTIED, QWEN7B, QWEN7B_HALF, QWEN14B, QWEN14B_2L, SHAPES, tensor_names,
                     tensor_shape)
from .gen import (
    bf16_normal,
    model_weights,
    prompt_ids,
    corrupt_draft,
    synthetic_kv,
    lookup_history,
    batch_contexts,
    rejected_suffix,
    seeds,
    with_head_gain,
    near_copy,
    history_successors,
    successor_stack,
    perturb_successors,
    nf4_tensor,
    nf4_model_weights,
)

__all__ = [
    "Shape", "TINY", "QWEN05B", "QWEN05B_UNTIED", "QWEN7B", "QWEN7B_HALF", "QWEN14B", "QWEN14B_2L", "SHAPES", "tensor_names", "tensor_shape",
    "bf16_normal", "model_weights", "prompt_ids", "corrupt_draft", "synthetic_kv", "lookup_history",
    "batch_contexts", "rejected_suffix", "seeds", "with_head_gain", "near_copy", "history_successors", "successor_stack", "perturb_successors", "nf4_tensor", "nf4_model_weights",
]
