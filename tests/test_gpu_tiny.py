"""GPU parity of the whole verify path on the two-layer decoder, through the C ABI.

Workload: 2 layers, hidden 256, 4 query / 2 KV heads, head_dim 64, FFN 1024,
vocab 4096, RoPE base 10000; a 64-token uniform prompt; 16 verify steps with
K=4 drafts, each the oracle's greedy continuation with one token replaced at a
seeded slot (4 = none); a 128-position static cache.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GAP, LOGIT_TOL, Pair, accepted_decided, check_targets, need_gpu, say

pytestmark = pytest.mark.gpu

S = synth.TINY


@pytest.fixture(scope="module")
def pair():
    need_gpu()
    say("[tiny] building engine")
    p = Pair(S, 1, capacity=128, k_max=4)
    yield p
    p.close()


def _reset(pair, prompt):
    sfb, eng = pair.sfb, pair.eng
    c = oracle.KVCache(S, 128)
    oracle.prefill(pair.model, c, prompt)
    nxt = sfb.sf_prefill(eng.cache, 0, prompt)
    return c, nxt


def test_prefill_matches_oracle(pair):
    sfb, eng = pair.sfb, pair.eng
    for n in (1, 5, 64, 100, 127):
        say(f"[tiny] prefill n={n}")
        prompt = synth.prompt_ids(S.vocab, n, 2000 + n)
        c = oracle.KVCache(S, 128)
        z = oracle.prefill(pair.model, c, prompt)
        nxt = sfb.sf_prefill(eng.cache, 0, prompt)
        gap = oracle.top_gap(z[-1:])[0].item()
        if gap > GAP:
            assert nxt == c.next_token, (n, nxt, c.next_token, gap)
        assert sfb.sf_cache_state(eng.cache, 0) == (n, nxt)


def _kv(sfb, cache, n, cap):
    shape = (S.n_layers, S.n_kv_heads, cap, S.head_dim)
    kg = torch.zeros(shape, dtype=torch.int16, device="cuda")
    vg = torch.zeros_like(kg)
    sfb.sf_kv_read(cache, 0, kg, vg, n, cap)
    torch.cuda.synchronize()
    return kg.cpu()[:, :, :n], vg.cpu()[:, :, :n]


def test_prefill_chunk_sizes_agree_bitwise_and_match_oracle(monkeypatch):
    """A 1100-token prompt in passes of 512 positions (the default: 512 + 512 + 76) and of 64
    (18 passes) writes bit-identical K/V and picks the same next token: every GEMM splits k
    the same way at any row count and attention spans are fixed by absolute position.  Both
    match the oracle's cache within 0.02."""
    sfb = need_gpu()
    n, cap = 1100, 1152
    p = Pair(S, 1, capacity=cap, k_max=4)
    monkeypatch.setenv("SF_PREFILL_CHUNK", "64")
    c64 = sfb.sf_cache_alloc(p.eng.model, 1, cap, 4)
    try:
        prompt = synth.prompt_ids(S.vocab, n, 4100)
        say(f"[tiny] prefill {n} in passes of 512 and of 64")
        nxt = sfb.sf_prefill(p.eng.cache, 0, prompt)
        nxt64 = sfb.sf_prefill(c64, 0, prompt)
        assert nxt == nxt64
        ka, va = _kv(sfb, p.eng.cache, n, cap)
        kb, vb = _kv(sfb, c64, n, cap)
        assert torch.equal(ka, kb) and torch.equal(va, vb)
        c = oracle.KVCache(S, cap)
        z = oracle.prefill(p.model, c, prompt)
        if oracle.top_gap(z[-1:])[0].item() > GAP:
            assert nxt == c.next_token
        assert (ka.view(torch.bfloat16).double() - c.k[:, :, :n].double()).abs().max().item() <= 0.02
        assert (va.view(torch.bfloat16).double() - c.v[:, :, :n].double()).abs().max().item() <= 0.02
        assert sfb.sf_cache_state(p.eng.cache, 0) == (n, nxt)
        assert sfb.sf_cache_state(c64, 0) == (n, nxt)
    finally:
        sfb.sf_cache_free(c64)
        p.close()


def test_c1_lockstep_16_steps(pair):
    """The tiny workload end to end: eager debug pass (logits), graph pass (accepted,
    targets), and the oracle, step by step; both sides are then forced to the oracle's
    (length, pending token) so a near-tie cannot desynchronise them."""
    sfb, eng, K = pair.sfb, pair.eng, pair.K
    prompt = synth.prompt_ids(S.vocab, 64, synth.seeds(1)["prompt"])
    c, nxt = _reset(pair, prompt)
    if nxt != c.next_token:
        sfb.sf_set_next(eng.cache, 0, c.next_token)
    rng = np.random.default_rng(synth.seeds(1)["draft"])
    logits = torch.empty((K + 1, S.vocab), dtype=torch.float32, device="cuda")
    n_exact = n_tot = 0
    m_checked = 0
    worst = 0.0
    for step in range(16):
        L = c.length
        cont = oracle.greedy_continuation(pair.model, c, K)
        draft, p = synth.corrupt_draft(cont, S.vocab, rng)
        say(f"[tiny] step {step} L={L} p={p}")
        acc_e, tgt_e = sfb.sf_verify(eng.cache, draft[None], None, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT,
                                     dev_out=logits)
        torch.cuda.synchronize()
        acc_g, tgt_g = sfb.sf_verify(eng.cache, draft[None], None, sfb.SF_NO_COMMIT)
        # The graph replays the same kernels as the eager pass: identical results.
        assert acc_g[0] == acc_e[0] and (tgt_g == tgt_e).all()
        r = oracle.verify(pair.model, c, draft, K)
        assert r["accepted"] == p                       # construction of the drafts
        err = (logits.double().cpu() - r["logits"]).abs().max().item()
        worst = max(worst, err)
        assert err <= LOGIT_TOL, (step, err)
        ne, nt = check_targets(tgt_g[0], r, K)
        n_exact += ne
        n_tot += nt
        if accepted_decided(r, int(acc_g[0]), K):
            assert acc_g[0] == r["accepted"], (step, acc_g[0], r["accepted"])
            m_checked += 1
        # Lockstep: commit the oracle's decision on the GPU.
        sfb.sf_verify(eng.cache, draft[None], np.array([r["accepted"]]), sfb.SF_FORCE_ACCEPT)
        sfb.sf_set_next(eng.cache, 0, c.next_token)
        assert sfb.sf_cache_state(eng.cache, 0) == (c.length, c.next_token)
    say(f"[tiny] exact-rule slots {n_exact}/{n_tot}, accepted counts checked {m_checked}/16, "
        f"max |dlogit| {worst:.4g}")
    assert n_exact >= n_tot // 4


def test_replay_is_bitwise_deterministic(pair):
    sfb, eng, K = pair.sfb, pair.eng, pair.K
    prompt = synth.prompt_ids(S.vocab, 40, 77)
    _reset(pair, prompt)
    d = np.array([[5, 6, 7, 8]], dtype=np.int32)
    a = torch.empty((K + 1, S.vocab), dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    sfb.sf_verify(eng.cache, d, None, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT, dev_out=a)
    sfb.sf_verify(eng.cache, d, None, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT, dev_out=b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_rollback_and_replay_reproduce_cache_bytes(pair):
    sfb, eng, K = pair.sfb, pair.eng, pair.K
    prompt = synth.prompt_ids(S.vocab, 30, 78)
    _, nxt = _reset(pair, prompt)
    L0 = 30
    d = np.array([[11, 12, 13, 14]], dtype=np.int32)
    acc1, tgt1 = sfb.sf_verify(eng.cache, d, None, sfb.SF_FORCE_ACCEPT)     # commits L0..L0+4
    shape = (S.n_layers, S.n_kv_heads, 64, S.head_dim)
    k1 = torch.zeros(shape, dtype=torch.int16, device="cuda")
    v1 = torch.zeros_like(k1)
    sfb.sf_kv_read(eng.cache, 0, k1, v1, L0 + 5, 64)
    junk = np.array([[100, 200, 300, 400]], dtype=np.int32)
    sfb.sf_verify(eng.cache, junk, None, 0)                                  # more writes
    sfb.sf_rollback(eng.cache, 0, L0)
    sfb.sf_set_next(eng.cache, 0, nxt)
    assert sfb.sf_cache_state(eng.cache, 0) == (L0, nxt)
    acc2, tgt2 = sfb.sf_verify(eng.cache, d, None, sfb.SF_FORCE_ACCEPT)
    k2 = torch.zeros_like(k1)
    v2 = torch.zeros_like(k1)
    sfb.sf_kv_read(eng.cache, 0, k2, v2, L0 + 5, 64)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert (tgt1 == tgt2).all() and acc1[0] == acc2[0] == 4


def test_kv_append_matches_oracle_cache(pair):
    """The K (after RoPE) and V the pass appends equal the oracle's, element by element,
    to a few bf16 ulps."""
    sfb, eng = pair.sfb, pair.eng
    prompt = synth.prompt_ids(S.vocab, 50, 79)
    c, _ = _reset(pair, prompt)
    shape = (S.n_layers, S.n_kv_heads, 64, S.head_dim)
    kg = torch.zeros(shape, dtype=torch.int16, device="cuda")
    vg = torch.zeros_like(kg)
    sfb.sf_kv_read(eng.cache, 0, kg, vg, 50, 64)
    torch.cuda.synchronize()
    kg = kg.cpu().view(torch.bfloat16).double()[:, :, :50]
    vg = vg.cpu().view(torch.bfloat16).double()[:, :, :50]
    ko = c.k[:, :, :50].double()
    vo = c.v[:, :, :50].double()
    assert (kg - ko).abs().max().item() <= 0.02 * max(1.0, ko.abs().max().item())
    assert (vg - vo).abs().max().item() <= 0.02 * max(1.0, vo.abs().max().item())


def test_draft_steps_match_oracle_greedy(pair):
    """The captured single-token graph, stepped in lockstep with the oracle's greedy
    decoding; then n steps in one call equal n single calls bitwise."""
    sfb, eng = pair.sfb, pair.eng
    prompt = synth.prompt_ids(S.vocab, 48, 80)
    c, nxt = _reset(pair, prompt)
    sfb.sf_set_next(eng.cache, 0, c.next_token)
    checked = 0
    for i in range(24):
        tok = int(sfb.sf_draft_step(eng.cache, 1)[0][0])
        r = oracle.verify(pair.model, c, [], 0)
        if r["gap"][0] > GAP:
            assert tok == c.next_token, (i, tok, c.next_token)
            checked += 1
        sfb.sf_set_next(eng.cache, 0, c.next_token)
        assert sfb.sf_cache_state(eng.cache, 0) == (c.length, c.next_token)
    say(f"[tiny] draft steps checked under the gap rule: {checked}/24")
    assert checked >= 2
    base_len, base_next = sfb.sf_cache_state(eng.cache, 0)
    many = sfb.sf_draft_step(eng.cache, 12)[0].tolist()
    sfb.sf_rollback(eng.cache, 0, base_len)
    sfb.sf_set_next(eng.cache, 0, base_next)
    one = [int(sfb.sf_draft_step(eng.cache, 1)[0][0]) for _ in range(12)]
    assert many == one


def test_gpu_speculative_equals_gpu_greedy(pair):
    """I1 on the GPU itself: verify passes and single-token steps produce bitwise-equal
    decisions, so speculative decoding emits exactly the greedy stream."""
    sfb, eng, K = pair.sfb, pair.eng, pair.K
    prompt = synth.prompt_ids(S.vocab, 20, 81)
    sfb.sf_prefill(eng.cache, 0, prompt)
    greedy = sfb.sf_draft_step(eng.cache, 40)[0].tolist()
    nxt0 = sfb.sf_prefill(eng.cache, 0, prompt)
    stream = [nxt0] + greedy
    # Speculate with drafts taken from the greedy stream, some of them corrupted.
    rng = np.random.default_rng(5)
    emitted = [nxt0]
    pos = 0
    while len(emitted) < 30:
        d = np.array(stream[pos + 1:pos + 1 + K], dtype=np.int32)
        j = int(rng.integers(0, K + 1))
        if j < K:
            d[j] = (d[j] + 1) % S.vocab
        acc, tgt = sfb.sf_verify(eng.cache, d[None])
        M = int(acc[0])
        assert M == j if j < K else M == K
        emitted += [int(t) for t in d[:M]] + [int(tgt[0][M])]
        pos += M + 1
    assert emitted[:30] == stream[:30]


def test_errors_leave_state_unchanged(pair):
    sfb, eng, K = pair.sfb, pair.eng, pair.K
    sfb.sf_prefill(eng.cache, 0, synth.prompt_ids(S.vocab, 124, 82))
    st = sfb.sf_cache_state(eng.cache, 0)
    with pytest.raises(sfb.SFError) as e:
        sfb.sf_verify(eng.cache, np.zeros((1, K), np.int32))        # 124 + 5 > 128
    assert e.value.code == sfb.SF_E_CAPACITY
    with pytest.raises(sfb.SFError) as e:
        sfb.sf_rollback(eng.cache, 0, 125)
    assert e.value.code == sfb.SF_E_STATE
    with pytest.raises(sfb.SFError) as e:
        sfb.sf_set_next(eng.cache, 0, S.vocab)
    assert e.value.code == sfb.SF_E_ARG
    sfb.sf_rollback(eng.cache, 0, 100)
    with pytest.raises(sfb.SFError) as e:
        sfb.sf_verify(eng.cache, np.array([[1, 2, S.vocab, 3]], np.int32))
    assert e.value.code == sfb.SF_E_ARG
    with pytest.raises(sfb.SFError) as e:
        sfb.sf_verify(eng.cache, np.zeros((1, K), np.int32), np.array([K + 1]))
    assert e.value.code == sfb.SF_E_ARG
    with pytest.raises(sfb.SFError) as e:
        sfb.sf_draft_step(eng.cache, 29)                              # 100 + 29 > 128
    assert e.value.code == sfb.SF_E_CAPACITY
    assert sfb.sf_cache_state(eng.cache, 0) == (100, st[1])


def test_four_wave_workgroups_split_k_and_64_row_chunks(monkeypatch):
    """The GEMM kernels with 8-tile batches, every GEMM with 4-wave workgroups, QKV / O / down
    split over two workgroups per block (partials + reduce kernels), and prefill chunks of 64
    rows."""
    need_gpu()
    monkeypatch.setenv("SF_PREFILL_CHUNK", "64")
    monkeypatch.setenv("SF_KH", "8")     # 8-tile batches
    for v in ("SF_NW_QKV", "SF_NW_O", "SF_NW_GU", "SF_NW_D", "SF_NW_HEAD"):
        monkeypatch.setenv(v, "4")
    for v in ("SF_SP_QKV", "SF_SP_O", "SF_SP_D"):
        monkeypatch.setenv(v, "2")
    p = Pair(S, 1, capacity=128, k_max=4)
    try:
        for n in (64, 100):
            say(f"[tiny/nw4] prefill n={n}")
            prompt = synth.prompt_ids(S.vocab, n, 3000 + n)
            c = oracle.KVCache(S, 128)
            z = oracle.prefill(p.model, c, prompt)
            nxt = p.sfb.sf_prefill(p.eng.cache, 0, prompt)
            if oracle.top_gap(z[-1:])[0].item() > GAP:
                assert nxt == c.next_token
            shape = (S.n_layers, S.n_kv_heads, 128, S.head_dim)
            kg = torch.zeros(shape, dtype=torch.int16, device="cuda")
            vg = torch.zeros_like(kg)
            p.sfb.sf_kv_read(p.eng.cache, 0, kg, vg, n, 128)
            torch.cuda.synchronize()
            kg = kg.cpu().view(torch.bfloat16).double()[:, :, :n]
            vg = vg.cpu().view(torch.bfloat16).double()[:, :, :n]
            assert (kg - c.k[:, :, :n].double()).abs().max().item() <= 0.02
            assert (vg - c.v[:, :, :n].double()).abs().max().item() <= 0.02
        d = np.array([[1, 2, 3, 4]], dtype=np.int32)
        logits = torch.empty((5, S.vocab), dtype=torch.float32, device="cuda")
        p.sfb.sf_verify(p.eng.cache, d, None, p.sfb.SF_DEBUG_LOGITS | p.sfb.SF_NO_COMMIT, dev_out=logits)
        torch.cuda.synchronize()
        r = oracle.verify(p.model, c, d[0], 4, commit=False)
        assert (logits.double().cpu() - r["logits"]).abs().max().item() <= LOGIT_TOL
    finally:
        p.close()


def test_largest_capacity_and_longest_draft():
    """Capacity 16384 with K=15 drafts: the span merge sees up to 256 position spans (four
    register slots of 64).  Seeded synthetic K/V fill contexts on both sides of the 64-,
    128- and 192-span boundaries and the last ones the capacity allows."""
    need_gpu()
    K, cap = 15, 16384
    p = Pair(S, 1, capacity=cap, k_max=K)
    try:
        kb, vb = synth.synthetic_kv(S, cap - K - 1, synth.seeds(1)["kv"])
        kd = torch.from_numpy(np.ascontiguousarray(kb).view(np.int16)).cuda()
        vd = torch.from_numpy(np.ascontiguousarray(vb).view(np.int16)).cuda()
        rng = np.random.default_rng(synth.seeds(1)["draft"])
        for ctx in (4080, 4096, 8177, 12300, cap - K - 1):
            say(f"[tiny/cap] ctx={ctx}")
            nxt = int(rng.integers(0, S.vocab))
            p.sfb.sf_kv_write(p.eng.cache, 0, kd, vd, ctx, kb.shape[2])
            p.sfb.sf_set_next(p.eng.cache, 0, nxt)
            d = rng.integers(0, S.vocab, size=(1, K)).astype(np.int32)
            logits = torch.empty((K + 1, S.vocab), dtype=torch.float32, device="cuda")
            acc, tgt = p.sfb.sf_verify(p.eng.cache, d, None, p.sfb.SF_DEBUG_LOGITS | p.sfb.SF_NO_COMMIT,
                                       dev_out=logits)
            torch.cuda.synchronize()
            c = oracle.KVCache(S, ctx + K + 1)
            c.load(kb, vb, ctx, next_token=nxt)
            r = oracle.verify(p.model, c, d[0], K, commit=False)
            err = (logits.double().cpu() - r["logits"]).abs().max().item()
            say(f"[tiny/cap] ctx={ctx} max |dlogit| {err:.3g}")
            assert err <= LOGIT_TOL
            check_targets(tgt[0], r, K)
    finally:
        p.close()


@pytest.mark.parametrize("planted", [False, True], ids=["random", "successor"])
def test_prompt_lookup_loop_commits_the_greedy_stream(planted):
    """The prompt-lookup loop the benchmark runs, at the tiny shape: prefill a repeating
    history, then committing verifies whose drafts the n-gram proposer finds in the committed
    stream (pending token included).  Proposals equal the oracle proposer's on the same
    stream, and the committed stream is plain greedy decoding of the oracle, token for token
    while its choices clear the gap ([ShardFlow] "Speculative Decoding: The Idea": the output
    is the target model's own; [Sangama] "Speculative decoding: correct, but slower (for
    now)": the client's n-gram guesses).  Two stacks: random-init weights with head gain 32,
    and the successor-planted stack the benchmark's loop uses (greedy next = the history's
    most frequent successor), under which the drafts are mostly accepted."""
    sfb = need_gpu()
    K = 8
    prompt = synth.lookup_history(S.vocab, 160, 5151)
    w = synth.model_weights(S, synth.seeds(1)["weights"])
    if planted:
        w = synth.successor_stack(w, synth.history_successors(prompt, S.vocab, 5152))
    else:
        w = synth.with_head_gain(w, 32.0)
    model = oracle.Model(S, w, cache=True)
    eng = sfb.Engine(S, w, n_seqs=1, capacity=512, k_max=K)
    try:
        nxt = sfb.sf_prefill(eng.cache, 0, prompt)
        toks = [int(t) for t in prompt]
        stream, accepted = [], []
        for _ in range(40):
            h = np.array(toks + [nxt], dtype=np.int32)
            prop = sfb.sf_ngram_propose(h, 2, 4, K)
            assert prop.tolist() == oracle.propose(h.tolist(), 2, 4, K)
            d = np.zeros((1, K), dtype=np.int32)
            d[0, :len(prop)] = prop
            acc, tgt = sfb.sf_verify(eng.cache, d, np.array([len(prop)], dtype=np.int32), 0)
            M = int(acc[0])
            stream += [nxt] + [int(t) for t in prop[:M]]
            toks += [nxt] + [int(t) for t in prop[:M]]
            accepted.append(M)
            nxt = int(tgt[0][M])
        assert sfb.sf_cache_state(eng.cache, 0) == (len(prompt) + len(stream), nxt)
        # Every committed token is the oracle's greedy choice after the committed prefix
        # (the oracle is fed the GPU's stream, so a near-tie does not desynchronise the rest).
        c = oracle.KVCache(S, 512)
        z = oracle.prefill(model, c, prompt)
        gap = oracle.top_gap(z[-1:])[0].item()
        n_cmp = 0
        for i, t in enumerate(stream):
            if gap > GAP:
                assert t == c.next_token, (i, t, c.next_token)
                n_cmp += 1
            oracle.set_next(c, t)
            gap = oracle.verify(model, c, [], 0)["gap"][0].item()
        say(f"[tiny] lookup loop ({'successor' if planted else 'random'}): {len(stream)} tokens in 40 steps, "
            f"accepted {sum(accepted)}, {n_cmp} checked against the oracle's greedy choice")
        assert n_cmp >= (3 * len(stream)) // 4 and sum(accepted) > 0
        if planted:
            assert n_cmp == len(stream) and sum(accepted) >= 2 * len(accepted)
    finally:
        eng.close()
