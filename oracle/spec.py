"""Oracle accept / commit / rollback rules and the greedy reference.  TEST INFRASTRUCTURE ONLY.

Round structure (ShardFlow, "Speculative Decoding: The Idea"): a drafter guesses
K tokens, the verifier checks all of them in one pass, and the agreed prefix is
committed in one round trip.  The verifier returns its own greedy choice at
every position (Sangama, "Speculative decoding: correct, but slower (for now)"),
so the caller can count how many guesses were right.

Reading taken where the pages leave it open: after M agreed drafts, the
verifier's own choice at the first disagreement (or after the last draft) is
committed too, so a round always commits M+1 tokens.  Under greedy decoding this
emits exactly the plain greedy sequence, which is the correctness criterion the
Sangama page states.

Rollback is an index update (ShardFlow, "Why It Kept Breaking", fix 4: the cache
is rewound in place to the last accepted position); cache entries past the
committed length are stale and are overwritten by later passes.
"""
import numpy as np
import torch

from .decoder import forward


def argmax_lowest(z):
    """Per-row argmax of z [n, V]; the lowest index wins an exact tie."""
    z = torch.as_tensor(z)
    best = z.max(dim=-1, keepdim=True).values
    idx = torch.arange(z.shape[-1]).expand_as(z)
    big = torch.full_like(idx, z.shape[-1])
    return torch.where(z == best, idx, big).min(dim=-1).values


def top_gap(z):
    """Per-row gap between the largest and second-largest logit."""
    top2 = torch.topk(torch.as_tensor(z), 2, dim=-1).values
    return top2[:, 0] - top2[:, 1]


def accept_prefix(draft, target, k):
    """Length M of the longest prefix with draft[j] == target[j], capped at k.

    draft[j] is the (j+1)-th guessed token; target[j] is the verifier's choice
    for that slot, i.e. its argmax at the position of the token before it.
    """
    m = 0
    while m < k and int(draft[m]) == int(target[m]):
        m += 1
    return m


def verify(model, cache, draft, k=None, commit=True, force_accept=False):
    """One verify pass over T = len(draft)+1 positions starting at cache.length.

    Tokens are [next_token, d_1..d_k, 0 ... 0]: slots past k hold token 0, and
    causality keeps them from affecting real slots.  Returns a dict with
    logits/hidden [T, .], target [T], accepted M and the pre-pass length.
    On commit: length += M+1, next_token = target[M].  force_accept sets M = k
    (used to feed known tokens, e.g. a prompt).
    """
    K = len(draft)
    k = K if k is None else int(k)
    if not 0 <= k <= K:
        raise ValueError("k out of range")
    L = cache.length
    T = K + 1
    if L + T > cache.capacity:
        raise ValueError("capacity")
    toks = [cache.next_token] + [int(d) for d in draft[:k]] + [0] * (K - k)
    out = forward(model, cache, toks, list(range(L, L + T)))
    res = {"L": L, "tokens": toks}
    if not model.shape.has_head:
        res["hidden"] = out
        if commit:
            cache.length = L + k + 1
        return res
    target = argmax_lowest(out)
    M = k if force_accept else accept_prefix(draft, target, k)
    res.update(logits=out, target=target, accepted=M, gap=top_gap(out))
    if commit:
        cache.length = L + M + 1
        cache.next_token = int(target[M])
    return res


def prefill(model, cache, tokens):
    """Score a prompt from position 0; commit all of it.  next_token = argmax at the last position."""
    n = len(tokens)
    if n < 1 or n > cache.capacity:
        raise ValueError("bad prompt length")
    out = forward(model, cache, [int(t) for t in tokens], list(range(n)))
    cache.length = n
    if model.shape.has_head:
        cache.next_token = int(argmax_lowest(out[-1:])[0])
    return out


def rollback(cache, pos):
    """In-place rewind: the committed length becomes pos (0 <= pos <= length)."""
    if not 0 <= pos <= cache.length:
        raise ValueError("rollback position beyond committed length")
    cache.length = int(pos)


def snapshot(cache, T):
    """The state one pass of T positions overwrites: committed length, pending token, and the
    cache's K/V rows at positions [length, length + T) (clipped to the capacity).  [Sangama]
    "Speculative decoding: correct, but slower (for now)": every worker saves its state
    before the guesses are checked."""
    L = cache.length
    hi = min(L + T, cache.capacity)
    return {"length": L, "next_token": cache.next_token,
            "k": cache.k[:, :, L:hi].clone(), "v": cache.v[:, :, L:hi].clone()}


def restore(cache, snap):
    """Put a snapshot back: its K/V rows at its length, then its length and pending token."""
    L = snap["length"]
    n = snap["k"].shape[2]
    cache.k[:, :, L:L + n] = snap["k"]
    cache.v[:, :, L:L + n] = snap["v"]
    cache.length = L
    cache.next_token = snap["next_token"]


def snapshot_verify(model, cache, draft, k):
    """One verify with the snapshot form of rollback (same page and section as snapshot()):
    save the state, check the k drafts (the pass commits as verify() does), and when some
    were rejected restore the snapshot and replay only the accepted drafts, a pass over the
    pending token and d_1..d_M whose last target is the new pending token.  Returns the
    checking pass's result dict."""
    snap = snapshot(cache, k + 1)
    res = verify(model, cache, draft, k)
    M = res["accepted"]
    if M < k:
        restore(cache, snap)
        verify(model, cache, [int(t) for t in draft[:M]], M, force_accept=True)
    return res


def set_next(cache, token):
    cache.next_token = int(token)


def greedy_decode(model, cache, n):
    """Plain greedy decoding: n single-token passes.  Returns the n tokens fed."""
    fed = []
    for _ in range(n):
        fed.append(cache.next_token)
        verify(model, cache, [], 0)
    return fed


def greedy_continuation(model, cache, K):
    """The K tokens plain greedy decoding would emit after the pending token (cache untouched)."""
    c = cache.copy()
    out = []
    for _ in range(K):
        verify(model, c, [], 0)
        out.append(c.next_token)
    return out


def speculative_decode(model, cache, n_tokens, draft_fn, K):
    """Decode with speculation until at least n_tokens tokens are emitted.

    draft_fn(cache) -> (draft list of length K, k).  Returns the emitted stream
    (the tokens fed at positions L0, L0+1, ...), truncated to n_tokens.
    """
    emitted = []
    while len(emitted) < n_tokens:
        d, k = draft_fn(cache)
        d = list(d) + [0] * (K - len(d))
        first = cache.next_token
        r = verify(model, cache, d, k)
        emitted.extend([first] + [int(t) for t in d[:r["accepted"]]])
    return emitted[:n_tokens]


def model_draft_round(drafter, dcache, verifier, vcache, K):
    """One speculative round with a model drafter (ShardFlow, "Speculative Decoding: The Idea":
    a small model guesses K tokens, the large one checks them in one pass and the agreed prefix
    is committed).  Both caches start at the same length L and pending token.

    The drafter takes K greedy single-token steps (d_1..d_K), the verifier verifies them and
    commits M+1 tokens, and the drafter's cache is rewound in place to the committed stream
    (ShardFlow, "Why It Kept Breaking", fix 4).  Reading taken where the pages leave it open:
    after M < K accepted drafts, the drafter's cache already holds positions L..L+M of the
    committed stream, so its length becomes L+M+1; after all K, it has not yet consumed d_K,
    so it takes one more step (feeding d_K at L+K) first.  Either way its pending token becomes
    the verifier's.  Returns verify()'s result dict for the verifier plus "draft" and
    "draft_gap" (the drafter's top-1/top-2 gap at each of its K choices).
    """
    if dcache.length != vcache.length or dcache.next_token != vcache.next_token:
        raise ValueError("drafter and verifier caches are not at the same point")
    L = dcache.length
    d, gaps = [], []
    for _ in range(K):
        rd = verify(drafter, dcache, [], 0)
        d.append(dcache.next_token)
        gaps.append(float(rd["gap"][0]))
    r = verify(verifier, vcache, d, K)
    M = r["accepted"]
    if M < K:
        rollback(dcache, L + M + 1)
    else:
        verify(drafter, dcache, [], 0)
    set_next(dcache, vcache.next_token)
    r["draft"] = d
    r["draft_gap"] = gaps
    return r
