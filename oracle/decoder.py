"""Oracle decoder stack (float64 torch CPU).  TEST INFRASTRUCTURE ONLY.

One forward pass scores n tokens at n absolute positions against a static,
pre-allocated KV cache (ShardFlow, "Why It Kept Breaking (and How I Fixed It)",
fix 1: a fixed-size cache allocated up front; fix 3: the positions of the tokens
are given explicitly).  The keys and values of the n tokens are written into the
cache first; each token then attends to every cached position up to and
including its own, which is the causal rule that lets the verifier check all
drafts in one pass (ShardFlow, "Speculative Decoding: The Idea"; Sangama,
"Speculative decoding: correct, but slower (for now)").
"""
import math

import numpy as np
import torch

F64 = torch.float64


def round_bf16(x):
    """Round float64 values to the nearest bf16 value, ties to even, in one step.

    x = m * 2**e with 0.5 <= |m| < 1; bf16 keeps 8 significant bits, so m*256 is
    rounded to an integer (torch.round rounds half to even).
    """
    m, e = torch.frexp(x)
    return torch.ldexp(torch.round(m * 256.0), e - 8)


def rms_norm(x, gain, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gain."""
    return x / torch.sqrt((x * x).mean(dim=-1, keepdim=True) + eps) * gain


def rope_angles(positions, head_dim, base):
    """theta[p, i] = p * base**(-2i/head_dim) for i < head_dim/2, in float64."""
    i = torch.arange(head_dim // 2, dtype=F64)
    inv_freq = torch.pow(torch.tensor(float(base), dtype=F64), -2.0 * i / head_dim)
    return torch.as_tensor(positions, dtype=F64)[:, None] * inv_freq[None, :]


def rope(x, theta):
    """Rotate-half RoPE.  x: [n, heads, head_dim]; theta: [n, head_dim/2].

    Dimension i is paired with i + head_dim/2 and the pair is rotated by theta_i:
      x_i'        = x_i cos - x_{i+d/2} sin
      x_{i+d/2}'  = x_{i+d/2} cos + x_i sin
    """
    half = x.shape[-1] // 2
    c = torch.cos(theta)[:, None, :]
    s = torch.sin(theta)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)


def silu(z):
    return z / (1.0 + torch.exp(-z))


def swiglu(gate, up):
    """SwiGLU activation: silu(gate) * up."""
    return silu(gate) * up


def causal_gqa_attention(q, k_cache, v_cache, positions):
    """Causal grouped-query attention over a cache.

    q: [n, n_q, d] float64; k_cache, v_cache: [n_kv, P, d] float64; positions: n ints.
    Query head h reads KV head h // (n_q / n_kv).  Row r attends to cache
    positions 0..positions[r] with scores q.k / sqrt(d) and a softmax over them.
    """
    n, n_q, d = q.shape
    n_kv = k_cache.shape[0]
    group = n_q // n_kv
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(d)
    for r in range(n):
        p = int(positions[r])
        for g in range(n_kv):
            qg = q[r, g * group:(g + 1) * group, :]            # [group, d]
            keys = k_cache[g, :p + 1, :]                        # [p+1, d]
            vals = v_cache[g, :p + 1, :]
            s = (qg @ keys.T) * scale                           # [group, p+1]
            w = torch.softmax(s, dim=-1)
            out[r, g * group:(g + 1) * group, :] = w @ vals
    return out


def _bf16_bits_to_f64(a):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.to(F64)


class Model:
    """A decoder shape plus its weights as bf16 bit arrays (numpy uint16).

    get(name) returns the tensor upcast exactly to float64.  With cache=True the
    float64 copies are kept (small models); otherwise they are rebuilt per use.
    """

    def __init__(self, shape, weights, cache=False):
        self.shape = shape
        self.w = weights
        self._cache = {} if cache else None

    def get(self, name):
        if self._cache is not None and name in self._cache:
            return self._cache[name]
        t = _bf16_bits_to_f64(self.w[name])
        if self._cache is not None:
            self._cache[name] = t
        return t

    def head_name(self):
        return "embed" if self.shape.tied_head else "lm_head"


class KVCache:
    """Static KV cache: K and V as bf16 [n_layers][n_kv][capacity][head_dim].

    `length` is the number of committed positions; `next_token` is the pending
    token that will occupy position `length` in the next pass.
    """

    def __init__(self, shape, capacity, dtype=torch.bfloat16):
        """dtype=torch.float64 keeps unrounded K/V; it exists only to compare the
        stack against an unrounded float64 reference implementation."""
        self.shape = shape
        self.capacity = capacity
        dims = (shape.n_layers, shape.n_kv_heads, capacity, shape.head_dim)
        self.k = torch.zeros(dims, dtype=dtype)
        self.v = torch.zeros(dims, dtype=dtype)
        self.length = 0
        self.next_token = 0

    def load(self, k_bits, v_bits, n_pos, next_token=0):
        """Fill positions 0..n_pos-1 from bf16 bit arrays [layers][n_kv][>=n_pos][d]."""
        k = torch.from_numpy(np.ascontiguousarray(k_bits[:, :, :n_pos]).view(np.int16)).view(torch.bfloat16)
        v = torch.from_numpy(np.ascontiguousarray(v_bits[:, :, :n_pos]).view(np.int16)).view(torch.bfloat16)
        self.k[:, :, :n_pos] = k
        self.v[:, :, :n_pos] = v
        self.length = n_pos
        self.next_token = int(next_token)

    def copy(self):
        c = KVCache.__new__(KVCache)
        c.shape, c.capacity = self.shape, self.capacity
        c.k, c.v = self.k.clone(), self.v.clone()
        c.length, c.next_token = self.length, self.next_token
        return c


def forward(model, cache, tokens, positions):
    """Score `tokens` at absolute `positions`; write their K/V into `cache`.

    Returns float64 logits [n, vocab] for a stack with a head, or the residual
    stream after the last layer [n, hidden] for a hidden-state-only stack.
    The cache length is not changed here; the accept/commit rule does that.
    """
    S = model.shape
    n = len(tokens)
    pos = [int(p) for p in positions]
    if max(pos) >= cache.capacity:
        raise ValueError("position beyond cache capacity")
    tok = torch.as_tensor(np.asarray(tokens, dtype=np.int64))
    x = model.get("embed")[tok]                                     # [n, H]
    theta = rope_angles(pos, S.head_dim, S.rope_base)
    pidx = torch.as_tensor(pos, dtype=torch.long)
    for l in range(S.n_layers):
        p = f"l{l}."
        a = rms_norm(x, model.get(p + "ln1"), S.rms_eps)
        q = a @ model.get(p + "wq").T
        k = a @ model.get(p + "wk").T
        v = a @ model.get(p + "wv").T
        if S.qkv_bias:
            q = q + model.get(p + "bq")
            k = k + model.get(p + "bk")
            v = v + model.get(p + "bv")
        q = rope(q.view(n, S.n_q_heads, S.head_dim), theta)
        k = rope(k.view(n, S.n_kv_heads, S.head_dim), theta)
        v = v.view(n, S.n_kv_heads, S.head_dim)
        # The cache stores bf16; every read below sees the stored values.
        if cache.k.dtype == torch.bfloat16:
            k, v = round_bf16(k), round_bf16(v)
        cache.k[l][:, pidx, :] = k.permute(1, 0, 2).to(cache.k.dtype)
        cache.v[l][:, pidx, :] = v.permute(1, 0, 2).to(cache.v.dtype)
        hi = max(pos) + 1
        kc = cache.k[l][:, :hi, :].to(F64)
        vc = cache.v[l][:, :hi, :].to(F64)
        o = causal_gqa_attention(q, kc, vc, pos)
        x = x + o.reshape(n, S.q_dim) @ model.get(p + "wo").T
        a = rms_norm(x, model.get(p + "ln2"), S.rms_eps)
        h = swiglu(a @ model.get(p + "wg").T, a @ model.get(p + "wu").T)
        x = x + h @ model.get(p + "wd").T
    if not S.has_head:
        return x
    a = rms_norm(x, model.get("final_norm"), S.rms_eps)
    return a @ model.get(model.head_name()).T
