"""Decoder shapes of the workloads and the names/shapes of their weight tensors.

Weights follow the usual [out_features][in_features] layout of a linear layer.
Tensor names:
  embed                         [vocab][hidden]
  l{i}.ln1, l{i}.ln2            [hidden]            RMSNorm gains
  l{i}.wq / l{i}.bq             [n_q*head_dim][hidden] / [n_q*head_dim]
  l{i}.wk / l{i}.bk             [n_kv*head_dim][hidden] / [n_kv*head_dim]
  l{i}.wv / l{i}.bv             [n_kv*head_dim][hidden] / [n_kv*head_dim]
  l{i}.wo                       [hidden][n_q*head_dim]
  l{i}.wg, l{i}.wu              [ffn][hidden]       SwiGLU gate / up
  l{i}.wd                       [hidden][ffn]       down
  final_norm                    [hidden]            (full stacks only)
  lm_head                       [vocab][hidden]     (full stacks with an untied head only)
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Shape:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_base: float
    rms_eps: float = 1e-6
    tied_head: bool = False   # LM head reuses the embedding matrix
    has_head: bool = True     # False: hidden-state-only shard (no final norm, no head)
    qkv_bias: bool = True

    @property
    def q_dim(self):
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    def param_count(self):
        return sum(_numel(tensor_shape(self, n)) for n in tensor_names(self))


def _numel(shape):
    n = 1
    for s in shape:
        n *= s
    return n


# Two-layer decoder used for exhaustive correctness runs.
TINY = Shape("tiny", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=1024,
             vocab=4096, rope_base=10000.0)
# Qwen2.5-0.5B dimensions (draft model, tied head).
QWEN05B = Shape("qwen2.5-0.5b", n_layers=24, hidden=896, n_q_heads=14, n_kv_heads=2, head_dim=64,
                ffn=4864, vocab=151936, rope_base=1e6, tied_head=True)
# Qwen2.5-7B dimensions (verifier, untied head).
QWEN7B = Shape("qwen2.5-7b", n_layers=28, hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128,
               ffn=18944, vocab=152064, rope_base=1e6)
# First half of the 7B stack (embedding + layers 0..13), emitting hidden states.
QWEN7B_HALF = replace(QWEN7B, name="qwen2.5-7b-half", n_layers=14, has_head=False)

# Qwen2.5-14B dimensions (NF4 verifier; untied head).
QWEN14B = Shape("qwen2.5-14b", n_layers=48, hidden=5120, n_q_heads=40, n_kv_heads=8, head_dim=128,
                ffn=13824, vocab=152064, rope_base=1e6)
# Two layers of the 14B stack with its full embedding and head: every kernel at its real shape.
QWEN14B_2L = replace(QWEN14B, name="qwen2.5-14b-2l", n_layers=2)

# The 0.5B shape with an untied LM head: the drafter of a successor-planted pair (a planted
# head must differ from the embedding); a step reads the same bytes as the tied shape.
QWEN05B_UNTIED = replace(QWEN05B, name="qwen2.5-0.5b-untied", tied_head=False)
SHAPES = {s.name: s for s in (TINY, QWEN05B, QWEN05B_UNTIED, QWEN7B, QWEN7B_HALF, QWEN14B, QWEN14B_2L)}


def tensor_names(shape):
    names = ["embed"]
    for i in range(shape.n_layers):
        p = f"l{i}."
        names += [p + "ln1", p + "wq"]
        if shape.qkv_bias:
            names += [p + "bq"]
        names += [p + "wk"]
        if shape.qkv_bias:
            names += [p + "bk"]
        names += [p + "wv"]
        if shape.qkv_bias:
            names += [p + "bv"]
        names += [p + "wo", p + "ln2", p + "wg", p + "wu", p + "wd"]
    if shape.has_head:
        names += ["final_norm"]
        if not shape.tied_head:
            names += ["lm_head"]
    return names


def tensor_shape(shape, name):
    H, Q, KV, F, V = shape.hidden, shape.q_dim, shape.kv_dim, shape.ffn, shape.vocab
    if name in ("embed", "lm_head"):
        return (V, H)
    if name == "final_norm":
        return (H,)
    base = name.split(".", 1)[1]
    return {
        "ln1": (H,), "ln2": (H,),
        "wq": (Q, H), "bq": (Q,),
        "wk": (KV, H), "bk": (KV,),
        "wv": (KV, H), "bv": (KV,),
        "wo": (H, Q),
        "wg": (F, H), "wu": (F, H),
        "wd": (H, F),
    }[base]
