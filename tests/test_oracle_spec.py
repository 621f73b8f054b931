"""Pins of the oracle's decoder stack and its accept / commit / rollback rules (CPU only).

Invariants fixed by the pages: speculative output equals plain greedy output
token for token (Sangama, "Speculative decoding: correct, but slower (for now)");
an in-place rewind followed by a replay reproduces the cache (ShardFlow, "Why It
Kept Breaking", fix 4; Sangama, same section: restore and replay the accepted
tokens).  The whole stack is also checked against an independent float64
implementation of the same decoder architecture (transformers' Qwen2).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth

F64 = torch.float64


# ---------------------------------------------------------------- argmax / accept

def test_argmax_lowest_index_on_ties():
    z = torch.tensor([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-1.0, -2.0, -0.5, -0.5]], dtype=F64)
    assert oracle.argmax_lowest(z).tolist() == [1, 0, 2]


def test_argmax_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(200):
        z = rng.integers(-3, 4, size=(3, 7)).astype(np.float64)
        got = oracle.argmax_lowest(torch.from_numpy(z)).tolist()
        want = [min(i for i in range(7) if z[r, i] == z[r].max()) for r in range(3)]
        assert got == want


def test_top_gap():
    z = torch.tensor([[0.0, 2.5, 1.0], [4.0, 4.0, 0.0]], dtype=F64)
    assert oracle.top_gap(z).tolist() == [1.5, 0.0]


def test_accept_prefix_brute_force():
    # Every draft/target pair over a 3-token vocabulary, K = 3, every k.
    K = 3
    for d in itertools.product(range(3), repeat=K):
        for t in itertools.product(range(3), repeat=K + 1):
            for k in range(K + 1):
                want = max(m for m in range(k + 1) if list(d[:m]) == list(t[:m]))
                assert oracle.accept_prefix(d, t, k) == want


# ---------------------------------------------------------------- stack vs independent implementation

def test_stack_matches_transformers_qwen2(tiny):
    from transformers import Qwen2Config, Qwen2ForCausalLM
    S = synth.TINY
    cfg = Qwen2Config(vocab_size=S.vocab, hidden_size=S.hidden, intermediate_size=S.ffn,
                      num_hidden_layers=S.n_layers, num_attention_heads=S.n_q_heads,
                      num_key_value_heads=S.n_kv_heads, max_position_embeddings=256,
                      rope_theta=S.rope_base, rms_norm_eps=S.rms_eps, tie_word_embeddings=False,
                      attn_implementation="eager")
    hf = Qwen2ForCausalLM(cfg).to(F64).eval()
    sd = {"model.embed_tokens.weight": tiny.get("embed"), "model.norm.weight": tiny.get("final_norm"),
          "lm_head.weight": tiny.get("lm_head")}
    for i in range(S.n_layers):
        p, q = f"l{i}.", f"model.layers.{i}."
        for ours, theirs in [("wq", "self_attn.q_proj.weight"), ("bq", "self_attn.q_proj.bias"),
                             ("wk", "self_attn.k_proj.weight"), ("bk", "self_attn.k_proj.bias"),
                             ("wv", "self_attn.v_proj.weight"), ("bv", "self_attn.v_proj.bias"),
                             ("wo", "self_attn.o_proj.weight"), ("wg", "mlp.gate_proj.weight"),
                             ("wu", "mlp.up_proj.weight"), ("wd", "mlp.down_proj.weight"),
                             ("ln1", "input_layernorm.weight"), ("ln2", "post_attention_layernorm.weight")]:
            sd[q + theirs] = tiny.get(p + ours)
    missing, unexpected = hf.load_state_dict(sd, strict=False)
    assert not unexpected and all("rotary" in m for m in missing), (missing, unexpected)
    toks = synth.prompt_ids(S.vocab, 40, 77)
    with torch.no_grad():
        want = hf(torch.as_tensor(toks[None].astype(np.int64))).logits[0]
    cache = oracle.KVCache(S, 64, dtype=F64)
    got = oracle.forward(tiny, cache, toks, list(range(40)))
    # The library computes RoPE angles in float32; everything else is float64.
    assert (got - want).abs().max().item() < 1e-5
    assert got.abs().max().item() > 0.1


def test_stack_with_gqa_heads_permuted_is_different(tiny):
    # Guard against a transposed GQA mapping going unnoticed: swapping the two KV
    # heads' weights must change the logits.
    S = synth.TINY
    w = dict(tiny.w)
    d = S.head_dim
    for name in ("l0.wk", "l0.wv"):
        a = w[name].copy()
        w[name] = np.concatenate([a[d:], a[:d]])
    for name in ("l0.bk", "l0.bv"):
        a = w[name].copy()
        w[name] = np.concatenate([a[d:], a[:d]])
    m2 = oracle.Model(S, w)
    toks = synth.prompt_ids(S.vocab, 8, 5)
    a = oracle.forward(tiny, oracle.KVCache(S, 16), toks, range(8))
    b = oracle.forward(m2, oracle.KVCache(S, 16), toks, range(8))
    assert (a - b).abs().max().item() > 1e-3


# ---------------------------------------------------------------- invariants I1-I4

def _prefilled(model, n=24, seed=11, cap=128):
    c = oracle.KVCache(model.shape, cap)
    oracle.prefill(model, c, synth.prompt_ids(model.shape.vocab, n, seed))
    return c


def test_I4_multi_position_equals_single_token_decode(tiny):
    c = _prefilled(tiny)
    cont = oracle.greedy_continuation(tiny, c, 4)
    c1 = c.copy()
    r = oracle.verify(tiny, c1, cont, 4, commit=False)
    c2 = c.copy()
    toks = [c.next_token] + cont
    for i, t in enumerate(toks):
        z = oracle.forward(tiny, c2, [t], [c.length + i])
        assert (z[0] - r["logits"][i]).abs().max().item() < 1e-10


def test_I2_own_greedy_continuation_is_fully_accepted(tiny):
    c = _prefilled(tiny)
    for K in (1, 4, 8):
        cc = c.copy()
        cont = oracle.greedy_continuation(tiny, cc, K)
        r = oracle.verify(tiny, cc, cont, K)
        assert r["accepted"] == K
        assert cc.length == c.length + K + 1
        assert int(r["target"][K]) == cc.next_token


def test_I1_speculative_equals_greedy(tiny):
    base = _prefilled(tiny, seed=12)
    ref = oracle.greedy_decode(tiny, base.copy(), 30)
    rng = np.random.default_rng(3)
    K = 4
    drafts = {
        "perfect": lambda c: (oracle.greedy_continuation(tiny, c, K), K),
        "random": lambda c: (list(rng.integers(0, synth.TINY.vocab, K)), K),
        "corrupted": lambda c: (list(synth.corrupt_draft(oracle.greedy_continuation(tiny, c, K),
                                                          synth.TINY.vocab, rng)[0]), K),
        "short": lambda c: (oracle.greedy_continuation(tiny, c, K)[:2], 2),
        "empty": lambda c: ([], 0),
    }
    for name, fn in drafts.items():
        got = oracle.speculative_decode(tiny, base.copy(), 30, fn, K)
        assert got == ref, name


def test_corrupted_draft_accepts_exactly_p(tiny):
    c = _prefilled(tiny, seed=13)
    rng = np.random.default_rng(9)
    seen = set()
    for _ in range(12):
        cont = oracle.greedy_continuation(tiny, c, 4)
        d, p = synth.corrupt_draft(cont, synth.TINY.vocab, rng)
        r = oracle.verify(tiny, c, d, 4)
        assert r["accepted"] == p
        seen.add(p)
    assert len(seen) >= 3


def test_I3_rollback_and_replay_reproduce_cache(tiny):
    c = _prefilled(tiny, seed=14)
    L0, nxt0 = c.length, c.next_token
    snap_k, snap_v = c.k.clone(), c.v.clone()
    cont = oracle.greedy_continuation(tiny, c, 4)
    r1 = oracle.verify(tiny, c, cont, 4)                  # writes L0..L0+4, commits 5
    k_after, v_after = c.k.clone(), c.v.clone()
    junk = list(np.random.default_rng(1).integers(0, synth.TINY.vocab, 4))
    oracle.verify(tiny, c, junk, 4)                       # more writes past the commit
    oracle.rollback(c, L0)
    oracle.set_next(c, nxt0)
    # Rollback is an index write: positions < L0 are untouched.
    assert torch.equal(c.k[:, :, :L0], snap_k[:, :, :L0])
    r2 = oracle.verify(tiny, c, cont, 4)
    assert torch.equal(c.k[:, :, :L0 + 5], k_after[:, :, :L0 + 5])
    assert torch.equal(c.v[:, :, :L0 + 5], v_after[:, :, :L0 + 5])
    assert torch.equal(r1["logits"], r2["logits"])
    assert c.length == L0 + 5


def test_rollback_and_capacity_errors(tiny):
    c = oracle.KVCache(synth.TINY, 16)
    oracle.prefill(tiny, c, [1, 2, 3])
    with pytest.raises(ValueError):
        oracle.rollback(c, 4)
    with pytest.raises(ValueError):
        oracle.verify(tiny, c, [0] * 13, 13)
    oracle.verify(tiny, c, [0] * 12, 12, commit=False)    # 3 + 13 = 16 fits exactly


def test_pad_slots_do_not_change_real_slots(tiny):
    c = _prefilled(tiny, seed=15)
    a = oracle.verify(tiny, c.copy(), [5, 6, 0, 0], 2, commit=False)["logits"][:3]
    b = oracle.verify(tiny, c.copy(), [5, 6, 99, 1234], 2, commit=False)["logits"][:3]
    assert (a - b).abs().max().item() == 0.0


def test_hidden_only_stack_is_prefix_of_full_stack():
    # The half shard (layers 0..n-1, no head) returns the residual stream that the
    # full stack feeds into layer n; checked on a two-layer stack cut after layer 0.
    from dataclasses import replace
    full = replace(synth.TINY, name="t2")
    half = replace(synth.TINY, name="t1", n_layers=1, has_head=False)
    w = synth.model_weights(full, 5)
    mf, mh = oracle.Model(full, w), oracle.Model(half, {k: v for k, v in w.items()})
    toks = [3, 1, 4, 1, 5]
    xh = oracle.forward(mh, oracle.KVCache(half, 8), toks, range(5))
    # Recompute the full stack with layer 1 replaced by identity maps: zero its out-projections.
    w0 = dict(w)
    w0["l1.wo"] = np.zeros_like(w["l1.wo"])
    w0["l1.wd"] = np.zeros_like(w["l1.wd"])
    z = oracle.forward(oracle.Model(full, w0), oracle.KVCache(full, 8), toks, range(5))
    zh = oracle.rms_norm(xh, mf.get("final_norm"), full.rms_eps) @ mf.get("lm_head").T
    assert (z - zh).abs().max().item() < 1e-12


def test_bf16_cache_holds_rounded_layer0_kv(tiny):
    """Reading of the cache precision: K (after RoPE) and V are rounded to bf16 once on
    append.  Layer 0's K/V depend only on the embedding and layer-0 weights, so a bf16
    cache must hold exactly bf16(the float64 cache's layer-0 values)."""
    S = synth.TINY
    toks = synth.prompt_ids(S.vocab, 12, 91)
    c16 = oracle.KVCache(S, 16)
    c64 = oracle.KVCache(S, 16, dtype=F64)
    oracle.forward(tiny, c16, toks, range(12))
    oracle.forward(tiny, c64, toks, range(12))
    for got, ref in ((c16.k[0, :, :12], c64.k[0, :, :12]), (c16.v[0, :, :12], c64.v[0, :, :12])):
        want = oracle.round_bf16(ref).to(torch.bfloat16)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    # and a later layer differs from plain rounding (the rounded cache feeds attention)
    assert not torch.equal(c16.k[1, :, :12].double(), oracle.round_bf16(c64.k[1, :, :12]))


# ---------------------------------------------------------------- model-drafter rounds

def _round_pair(drafter, verifier, seed=21, n=20):
    prompt = synth.prompt_ids(verifier.shape.vocab, n, seed)
    dc, vc = oracle.KVCache(drafter.shape, 160), oracle.KVCache(verifier.shape, 160)
    oracle.prefill(drafter, dc, prompt)
    oracle.prefill(verifier, vc, prompt)
    oracle.set_next(dc, vc.next_token)   # the verifier's choice after the prompt is the stream's
    return dc, vc


def _emit(drafter, verifier, K, rounds, seed=21):
    """Stream committed by `rounds` model-drafter rounds, and the per-round accepted counts."""
    dc, vc = _round_pair(drafter, verifier, seed)
    out, accepted = [], []
    for _ in range(rounds):
        first = vc.next_token
        r = oracle.model_draft_round(drafter, dc, verifier, vc, K)
        out += [first] + [int(t) for t in r["draft"][:r["accepted"]]]
        accepted.append(r["accepted"])
        assert dc.length == vc.length and dc.next_token == vc.next_token
    return out, accepted, dc, vc


def test_model_draft_round_with_itself_accepts_everything_and_equals_greedy(tiny):
    K = 4
    out, accepted, _, _ = _emit(tiny, tiny, K, 5)
    assert accepted == [K] * 5
    _, vc = _round_pair(tiny, tiny)
    assert out == oracle.greedy_decode(tiny, vc, len(out))


def test_model_draft_round_with_another_drafter_equals_greedy():
    drafter = oracle.Model(synth.TINY, synth.model_weights(synth.TINY, synth.seeds(2)["weights"]), cache=True)
    verifier = oracle.Model(synth.TINY, synth.model_weights(synth.TINY, synth.seeds(1)["weights"]), cache=True)
    out, accepted, dc, _ = _emit(drafter, verifier, 4, 6)
    _, vc = _round_pair(drafter, verifier)
    assert out == oracle.greedy_decode(verifier, vc, len(out))
    # The rewound drafter cache holds exactly the committed stream: its next greedy token
    # equals that of a fresh drafter cache that consumed the same stream.
    fresh = oracle.KVCache(synth.TINY, 160)
    prompt = synth.prompt_ids(synth.TINY.vocab, 20, 21)
    oracle.prefill(drafter, fresh, [int(t) for t in prompt] + out)
    oracle.set_next(fresh, dc.next_token)
    assert fresh.length == dc.length
    ra = oracle.verify(drafter, dc.copy(), [], 0, commit=False)
    rb = oracle.verify(drafter, fresh, [], 0, commit=False)
    assert (ra["logits"] - rb["logits"]).abs().max().item() < 1e-6


def test_model_draft_round_with_a_near_copy_drafter_takes_both_branches_and_equals_greedy():
    """A drafter close to the verifier (each projection w + 0.05 o, head gain 32): rounds
    that reject part of the draft and rounds that accept all of it both occur, and the
    committed stream is still the verifier's greedy one."""
    wv = synth.with_head_gain(synth.model_weights(synth.TINY, synth.seeds(1)["weights"]), 32.0)
    wd = synth.near_copy(wv, synth.model_weights(synth.TINY, synth.seeds(2)["weights"]), 0.05)
    verifier = oracle.Model(synth.TINY, wv, cache=True)
    drafter = oracle.Model(synth.TINY, wd, cache=True)
    out, accepted, _, _ = _emit(drafter, verifier, 4, 8)
    assert 4 in accepted and min(accepted) < 4
    _, vc = _round_pair(drafter, verifier)
    assert out == oracle.greedy_decode(verifier, vc, len(out))


def test_head_gain_scales_every_logit():
    """The final RMSNorm gain multiplies the head's input, so a gain of 32 (a power of two:
    exact through bf16 rounding) scales every logit by exactly 32."""
    w1 = synth.model_weights(synth.TINY, synth.seeds(1)["weights"])
    prompt = synth.prompt_ids(synth.TINY.vocab, 12, 5)
    z = []
    for w in (w1, synth.with_head_gain(w1, 32.0)):
        c = oracle.KVCache(synth.TINY, 16)
        z.append(oracle.prefill(oracle.Model(synth.TINY, w, cache=True), c, prompt))
    assert (z[1] - 32.0 * z[0]).abs().max().item() <= 1e-9 * z[1].abs().max().item()


# ---------------------------------------------------------------- snapshot rollback

def _corrupted_rounds(model, cache, K, rounds, seed):
    """Per round: the model's own K-token continuation with one seeded corruption."""
    rng = np.random.default_rng(seed)
    for _ in range(rounds):
        d, _ = synth.corrupt_draft(oracle.greedy_continuation(model, cache, K), model.shape.vocab, rng)
        yield d


def test_snapshot_restore_returns_every_byte(tiny):
    """Save, a committing verify that writes K+1 K/V rows, restore: the whole cache (both
    arrays, every position), the length and the pending token are as before."""
    K = 4
    c = oracle.KVCache(synth.TINY, 64)
    oracle.prefill(tiny, c, synth.prompt_ids(synth.TINY.vocab, 20, 21))
    before = c.copy()
    snap = oracle.snapshot(c, K + 1)
    oracle.verify(tiny, c, [1, 2, 3, 4], K)
    assert c.length > before.length and not torch.equal(c.k, before.k)
    oracle.restore(c, snap)
    assert torch.equal(c.k, before.k) and torch.equal(c.v, before.v)
    assert (c.length, c.next_token) == (before.length, before.next_token)


def test_snapshot_verify_equals_in_place_verify_and_greedy(tiny):
    """Rounds with the snapshot form of rollback (save, check, restore, replay the accepted
    drafts) reach the same length, pending token and committed K/V as the in-place form
    (commit M+1, leave the rest stale), and their committed stream is plain greedy decoding."""
    K = 4
    prompt = synth.prompt_ids(synth.TINY.vocab, 20, 21)
    a, b = oracle.KVCache(synth.TINY, 96), oracle.KVCache(synth.TINY, 96)
    oracle.prefill(tiny, a, prompt)
    oracle.prefill(tiny, b, prompt)
    stream, accepted = [], []
    for d in _corrupted_rounds(tiny, a, K, 8, 5):
        first = a.next_token
        ra = oracle.verify(tiny, a, d, K)
        rb = oracle.snapshot_verify(tiny, b, d, K)
        assert ra["accepted"] == rb["accepted"]
        assert (a.length, a.next_token) == (b.length, b.next_token)
        n = a.length
        assert (a.k[:, :, :n].double() - b.k[:, :, :n].double()).abs().max().item() == 0.0
        assert (a.v[:, :, :n].double() - b.v[:, :, :n].double()).abs().max().item() == 0.0
        stream += [first] + [int(t) for t in d[:ra["accepted"]]]
        accepted.append(ra["accepted"])
    assert min(accepted) < K                      # the restore-and-replay branch ran
    g = oracle.KVCache(synth.TINY, 96)
    oracle.prefill(tiny, g, prompt)
    assert stream == oracle.greedy_decode(tiny, g, len(stream))


# ---------------------------------------------------------------- prefill's pending token, cache loading

def test_prefill_pending_token_is_the_greedy_choice_after_the_last_prompt_token(tiny):
    """After a prompt of n tokens the pending token is the argmax (lowest index on ties) of the
    logits at position n-1: the same choice a single-token pass makes when the last prompt
    token is fed on top of a prefill of the first n-1 (so taking any other row of the prefill's
    logits, e.g. position 0, fails here: the chosen prompt makes those choices differ)."""
    S = synth.TINY
    prompt = synth.prompt_ids(S.vocab, 21, 404)
    c1 = oracle.KVCache(S, 64)
    z = oracle.prefill(tiny, c1, prompt)
    assert c1.length == 21
    assert c1.next_token == int(oracle.argmax_lowest(z)[-1])
    assert int(oracle.argmax_lowest(z)[0]) != c1.next_token
    c2 = oracle.KVCache(S, 64)
    oracle.prefill(tiny, c2, prompt[:-1])
    oracle.set_next(c2, int(prompt[-1]))
    r = oracle.verify(tiny, c2, [], 0)
    assert int(r["target"][0]) == c1.next_token
    assert (r["logits"][0] - z[-1]).abs().max().item() < 1e-10
    assert (c2.length, c2.next_token) == (c1.length, c1.next_token)


def test_kvcache_load_places_exactly_the_given_positions(tiny):
    """KVCache.load copies positions [0, n_pos) of bf16 bit arrays [layer][kv head][pos][dim]
    into the cache and nothing else: a cache loaded from another cache's exported bits holds
    the same bytes, zeros past n_pos (the source's junk there is not taken), the given length
    and pending token, and verifies to exactly the same logits."""
    S = synth.TINY
    src = _prefilled(tiny, n=30, seed=405, cap=64)
    kb = src.k.view(torch.int16).numpy().view(np.uint16).copy()
    vb = src.v.view(torch.int16).numpy().view(np.uint16).copy()
    kb[:, :, 30:] = 0x3F80        # junk (bf16 1.0) past the loaded positions
    vb[:, :, 30:] = 0xBF80
    c = oracle.KVCache(S, 48)
    c.load(kb, vb, 30, next_token=src.next_token)
    assert (c.length, c.next_token) == (30, src.next_token)
    assert torch.equal(c.k[:, :, :30].view(torch.int16), src.k[:, :, :30].view(torch.int16))
    assert torch.equal(c.v[:, :, :30].view(torch.int16), src.v[:, :, :30].view(torch.int16))
    assert not c.k[:, :, 30:].view(torch.int16).any() and not c.v[:, :, 30:].view(torch.int16).any()
    # Element order: layer, kv head, position, dim (a swapped axis would move this value).
    assert c.k[1, 0, 7, 5].item() == src.k[1, 0, 7, 5].item() != c.k[0, 1, 7, 5].item()
    d = [9, 8, 7, 6]
    ra = oracle.verify(tiny, src.copy(), d, 4, commit=False)
    rb = oracle.verify(tiny, c, d, 4, commit=False)
    assert torch.equal(ra["logits"], rb["logits"])
