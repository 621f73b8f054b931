"""Seeded generators.  Data only: nothing here computes any step of the decoder.

bf16 tensors are returned as numpy uint16 arrays holding the bf16 bit patterns;
callers view them as torch.bfloat16 (CPU or GPU) without conversion.
"""
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .shapes import tensor_names, tensor_shape

CHUNK = 1 << 22
WEIGHT_STD = 0.02
BF16_ONE = 0x3F80


def seeds(config_index):
    """Sub-seeds of workload `config_index` (1-based): weights, prompt, draft, contexts, kv."""
    base = 1000 * int(config_index)
    return {"weights": base + 1, "prompt": base + 2, "draft": base + 3, "contexts": base + 4,
            "kv": base + 5}


def _f32_to_bf16_bits(f):
    """Round float32 values to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    u = f.view(np.uint32)
    u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def _stream(seed, name, chunk):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(seed) & 0xFFFFFFFF, zlib.crc32(name.encode()), int(chunk)])))


def _threads(threads):
    if threads:
        return threads
    return max(1, min(16, os.cpu_count() or 1))


def bf16_normal(shape, std, seed, name, threads=None, pool=None):
    """bf16(std * z), z ~ N(0,1) float32, as uint16 bits; chunked so bytes are thread-count independent."""
    n = 1
    for s in shape:
        n *= int(s)
    out = np.empty(n, dtype=np.uint16)
    std32 = np.float32(std)

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        z = _stream(seed, name, c).standard_normal(hi - lo, dtype=np.float32)
        z *= std32
        out[lo:hi] = _f32_to_bf16_bits(z)

    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    elif pool is not None:
        list(pool.map(fill, range(nchunks)))
    else:
        with ThreadPoolExecutor(_threads(threads)) as p:
            list(p.map(fill, range(nchunks)))
    return out.reshape(shape)


def model_weights(shape, seed, names=None, threads=None):
    """All weight tensors of `shape` (or the subset `names`).

    Linear, bias and embedding tensors are bf16(0.02*z); RMSNorm gains are 1.0.
    A tensor's bytes depend only on (seed, tensor name), so the hidden-only half
    stack is exactly the first layers of the full stack under the same seed.
    """
    names = tensor_names(shape) if names is None else names
    out = {}
    with ThreadPoolExecutor(_threads(threads)) as pool:
        for name in names:
            shp = tensor_shape(shape, name)
            if name.endswith("ln1") or name.endswith("ln2") or name == "final_norm":
                out[name] = np.full(shp, BF16_ONE, dtype=np.uint16)
            else:
                out[name] = bf16_normal(shp, WEIGHT_STD, seed, name, pool=pool)
    return out


def with_head_gain(weights, gain):
    """A copy of `weights` whose final RMSNorm gain is bf16(gain) everywhere: every logit is
    scaled by the gain, which widens the spread between the top choices (random-init stacks
    otherwise have logits far flatter than a trained model's)."""
    out = dict(weights)
    out["final_norm"] = np.full_like(weights["final_norm"], _f32_to_bf16_bits(np.array([gain], np.float32))[0])
    return out


def history_successors(hist, vocab, seed):
    """succ[t] = the id that most often follows t in `hist` (ties: the smallest such id); an
    id never followed by anything there gets a seeded uniform id."""
    rng = np.random.Generator(np.random.PCG64(seed))
    succ = rng.integers(0, vocab, size=vocab, dtype=np.int64)
    h = np.asarray(hist, dtype=np.int64)
    keys, counts = np.unique(h[:-1] * vocab + h[1:], return_counts=True)
    a, b = keys // vocab, keys % vocab
    order = np.lexsort((b, -counts, a))        # by a, then most frequent, then smallest b
    a, b = a[order], b[order]
    first = np.ones(len(a), dtype=bool)
    first[1:] = a[1:] != a[:-1]
    succ[a[first]] = b[first]
    return succ.astype(np.int32)


def perturb_successors(succ, frac, seed):
    """A copy of succ with a seeded fraction `frac` of the ids given a uniform new successor:
    the map of a drafter that agrees with the verifier's on about 1 - frac of the ids."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.array(succ, dtype=np.int32)
    hit = rng.random(len(out)) < frac
    out[hit] = rng.integers(0, len(out), size=int(hit.sum()), dtype=np.int64).astype(np.int32)
    return out


def successor_stack(weights, succ, shift=8, threads=None):
    """A stack (untied head) whose greedy next token is succ[current token], a stand-in for a
    trained model that has learned a history's successor statistics (random-init weights follow
    no text, so a prompt-lookup drafter never finds what they will say).  Every layer's
    projections and biases are scaled by 2**-shift, an exponent shift (exact for every result in
    the normal range; results below it, which N(0, 0.02) weights never produce, become signed
    zeros), which keeps the residual stream within about 1% of the current token's embedding
    after 28 layers; the LM head's row v is the sum of the embeddings of the ids u with
    succ[u] = v (the embedding row itself when there is one such u, zero when there is none),
    so that embedding scores its successor highest by a wide margin (|e|^2 against the e.e' of
    unrelated rows).  The embedding, norms and all shapes are those of `weights`, so a pass
    costs the same."""
    def scaled(u):
        e = (u >> np.uint16(7)) & np.uint16(0xFF)
        return np.where(e > shift, u - np.uint16(shift << 7), u & np.uint16(0x8000)).astype(np.uint16)
    out = dict(weights)
    names = [n for n in weights if n.split(".")[-1] in ("wq", "wk", "wv", "wo", "wg", "wu", "wd", "bq", "bk", "bv")]
    with ThreadPoolExecutor(_threads(threads)) as pool:
        for name, arr in zip(names, pool.map(lambda n: scaled(weights[n]), names)):
            out[name] = arr
    emb = weights["embed"]
    succ = np.asarray(succ, dtype=np.int64)
    order = np.argsort(succ, kind="stable")
    rows, starts, sizes = np.unique(succ[order], return_index=True, return_counts=True)
    head = np.zeros_like(emb)
    one = sizes == 1
    head[rows[one]] = emb[order[starts[one]]]
    for v, s0, n in zip(rows[~one], starts[~one], sizes[~one]):
        acc = (emb[order[s0:s0 + n]].astype(np.uint32) << np.uint32(16)).view(np.float32).sum(axis=0, dtype=np.float32)
        head[v] = _f32_to_bf16_bits(acc)
    out["lm_head"] = head
    return out


def near_copy(weights, other, eps):
    """A stack close to `weights`: every projection becomes bf16(w + eps * o), o the same
    tensor of `other`; embeddings, norms and the head are shared.  Used as a drafter that
    agrees with the target often but not always."""
    def f32(u):
        return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)
    out = dict(weights)
    for name, w in weights.items():
        if name.split(".")[-1] in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            out[name] = _f32_to_bf16_bits(f32(w) + np.float32(eps) * f32(other[name]))
    return out


NF4_QUANTIZED = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def nf4_tensor(shape, seed, name, threads=None, pool=None):
    """Synthetic NF4 projection [rows][n_in] with the statistics of a quantized bf16(0.02 z)
    matrix: codes uint8 [rows][n_in / 2] (two per byte, even input in the low nibble), each
    code uniform over the 16 levels (NF4 levels bound equal-probability bins of a normal
    weight), and scales as bf16 bits [rows][n_in / 64]: 0.02 times the largest |z| of 64
    standard normals, drawn by inverting that maximum's distribution function."""
    from scipy.special import ndtri
    rows, n_in = int(shape[0]), int(shape[1])
    codes = np.empty(rows * n_in // 2, dtype=np.uint8)
    scales = np.empty(rows * n_in // 64, dtype=np.uint16)
    nc = (codes.size + CHUNK - 1) // CHUNK
    ns = (scales.size + CHUNK - 1) // CHUNK

    def fill(c):
        if c < nc:
            lo, hi = c * CHUNK, min(codes.size, (c + 1) * CHUNK)
            codes[lo:hi] = _stream(seed, name + "/codes", c).integers(0, 256, hi - lo, dtype=np.uint8)
        else:
            c -= nc
            lo, hi = c * CHUNK, min(scales.size, (c + 1) * CHUNK)
            u = _stream(seed, name + "/scales", c).random(hi - lo)
            m = ndtri(0.5 * (1.0 + u ** (1.0 / 64.0)))
            scales[lo:hi] = _f32_to_bf16_bits((WEIGHT_STD * m).astype(np.float32))

    if nc + ns <= 1:
        for c in range(nc + ns):
            fill(c)
    elif pool is not None:
        list(pool.map(fill, range(nc + ns)))
    else:
        with ThreadPoolExecutor(_threads(threads)) as p:
            list(p.map(fill, range(nc + ns)))
    return codes.reshape(rows, n_in // 2), scales.reshape(rows, n_in // 64)


def nf4_model_weights(shape, seed, names=None, threads=None):
    """All weights of `shape` with the projections (q, k, v, o, gate, up, down) in NF4 as
    (codes, scales) pairs from nf4_tensor; embeddings, norms, biases and the head as in
    model_weights."""
    names = tensor_names(shape) if names is None else names
    out = {}
    with ThreadPoolExecutor(_threads(threads)) as pool:
        for name in names:
            shp = tensor_shape(shape, name)
            if name.split(".")[-1] in NF4_QUANTIZED:
                out[name] = nf4_tensor(shp, seed, name, pool=pool)
            elif name.endswith("ln1") or name.endswith("ln2") or name == "final_norm":
                out[name] = np.full(shp, BF16_ONE, dtype=np.uint16)
            else:
                out[name] = bf16_normal(shp, WEIGHT_STD, seed, name, pool=pool)
    return out


def prompt_ids(vocab, n, seed):
    """n token ids uniform in [0, vocab)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def corrupt_draft(continuation, vocab, rng):
    """Replace one token of a K-token continuation at a uniform slot p in 0..K (K = no change).

    The replacement at p is (g + 1 + U{0..V-2}) mod V, so it always differs from g.
    Returns (draft int32[K], p).
    """
    d = np.array(continuation, dtype=np.int64).copy()
    K = len(d)
    p = int(rng.integers(0, K + 1))
    if p < K:
        d[p] = (d[p] + 1 + int(rng.integers(0, vocab - 1))) % vocab
    return d.astype(np.int32), p


def rejected_suffix(rng, k):
    """Number of rejected drafts r ~ U{0..k}."""
    return int(rng.integers(0, k + 1))


def synthetic_kv(shape, n_pos, seed, std=1.0, n_layers=None, threads=None):
    """Synthetic cache contents: K and V, each uint16 bf16 bits [layers][n_kv][n_pos][head_dim]."""
    L = shape.n_layers if n_layers is None else n_layers
    shp = (L, shape.n_kv_heads, n_pos, shape.head_dim)
    k = bf16_normal(shp, std, seed, "kv.k", threads=threads)
    v = bf16_normal(shp, std, seed, "kv.v", threads=threads)
    return k, v


def lookup_history(vocab, n, seed, n_spans=16, span_len=32, p_sub=0.10):
    """A token stream that repeats itself: spans drawn with replacement from a pool of
    `n_spans` random `span_len`-token spans, each token replaced with probability
    `p_sub` by a uniform id.  Gives a prompt-lookup drafter something to find."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pool = rng.integers(0, vocab, size=(n_spans, span_len), dtype=np.int64)
    out = []
    while len(out) < n:
        out.extend(pool[int(rng.integers(0, n_spans))].tolist())
    out = np.array(out[:n], dtype=np.int64)
    sub = rng.random(n) < p_sub
    out[sub] = rng.integers(0, vocab, size=int(sub.sum()), dtype=np.int64)
    return out.astype(np.int32)


def batch_contexts(n_seqs, lo, hi, seed):
    """Per-sequence context lengths uniform in lo..hi (inclusive)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=n_seqs, dtype=np.int64).astype(np.int32)
