"""GPU parity at the Qwen2.5-7B shape through the C ABI.

Full stack (28 layers, hidden 3584, 28 q / 4 KV heads, head_dim 128, SwiGLU 18944,
vocab 152064, untied head) in the launch configuration the benchmark times: one
sequence, K=8 drafts, capacity 8208, captured-graph replay.  Contexts hold seeded
synthetic K/V; drafts come from the prompt-lookup proposer over a seeded history.
Every logit of the 9 positions is compared with the float64 oracle (max-abs
<= 0.05) and tokens / accepted counts bit-exactly where the oracle's gap > 0.1.

First-half shard (embedding + layers 0..13, hidden-state output) at context 1024:
rows of x/rms(x) compared with max-abs <= 0.05.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GAP, LOGIT_TOL, accepted_decided, check_targets, need_gpu, say

pytestmark = pytest.mark.gpu

S = synth.QWEN7B
K = 8
CAP = 8192 + 16


@pytest.fixture(scope="module")
def weights():
    need_gpu()
    say("[7b] generating weights")
    return synth.model_weights(S, synth.seeds(4)["weights"])


@pytest.fixture(scope="module")
def kv():
    return synth.synthetic_kv(S, 8192, synth.seeds(4)["kv"])


@pytest.fixture(scope="module")
def hist():
    return synth.lookup_history(S.vocab, 8193, synth.seeds(4)["prompt"])


@pytest.fixture(scope="module")
def eng(weights):
    sfb = need_gpu()
    say("[7b] packing weights")
    e = sfb.Engine(S, weights, n_seqs=1, capacity=CAP, k_max=K)
    yield e
    e.close()


def _load_ctx(sfb, cache, kv, ctx, nxt, n_layers=None):
    kb, vb = kv
    if n_layers is not None:
        kb, vb = kb[:n_layers], vb[:n_layers]
    kd = torch.from_numpy(np.ascontiguousarray(kb).view(np.int16)).cuda()
    vd = torch.from_numpy(np.ascontiguousarray(vb).view(np.int16)).cuda()
    sfb.sf_kv_write(cache, 0, kd, vd, ctx, kb.shape[2])
    sfb.sf_set_next(cache, 0, nxt)
    torch.cuda.synchronize()


def _oracle_cache(kv, ctx, nxt, shape=S, capacity=None):
    c = oracle.KVCache(shape, capacity or ctx + K + 1)
    c.load(kv[0][:shape.n_layers], kv[1][:shape.n_layers], ctx, next_token=nxt)
    return c


@pytest.mark.parametrize("ctx", [512, 2048, 8192])
def test_full_stack_verify_matches_oracle(eng, weights, kv, hist, ctx):
    sfb = need_gpu()
    nxt = int(hist[ctx])
    prop = sfb.sf_ngram_propose(hist[:ctx + 1], 2, 4, K)
    d = np.zeros(K, dtype=np.int32)
    d[:len(prop)] = prop
    k = len(prop)
    say(f"[7b] ctx={ctx} k={k}")
    _load_ctx(sfb, eng.cache, kv, ctx, nxt)
    logits = torch.empty((K + 1, S.vocab), dtype=torch.float32, device="cuda")
    acc_e, tgt_e = sfb.sf_verify(eng.cache, d[None], np.array([k]), sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT,
                                 dev_out=logits)
    acc_g, tgt_g = sfb.sf_verify(eng.cache, d[None], np.array([k]), sfb.SF_NO_COMMIT)
    torch.cuda.synchronize()
    assert acc_g[0] == acc_e[0] and (tgt_g == tgt_e).all()
    model = oracle.Model(S, weights)
    say(f"[7b] ctx={ctx} oracle")
    r = oracle.verify(model, _oracle_cache(kv, ctx, nxt), d, k, commit=False)
    err = (logits.double().cpu() - r["logits"]).abs().max().item()
    ne, nt = check_targets(tgt_g[0], r, K)
    say(f"[7b] ctx={ctx} max |dlogit| {err:.4g}; exact-rule slots {ne}/{nt}; accepted gpu {acc_g[0]} "
        f"oracle {r['accepted']}")
    assert err <= LOGIT_TOL
    if accepted_decided(r, int(acc_g[0]), k):
        assert acc_g[0] == r["accepted"]

    # Second pass: the first draft replaced by the model's own choice after the pending
    # token, so at least one draft is accepted; committed on the device.
    d2 = d.copy()
    d2[0] = int(r["target"][0])
    acc2, tgt2 = sfb.sf_verify(eng.cache, d2[None], np.array([max(k, 1)]))
    r2 = oracle.verify(model, _oracle_cache(kv, ctx, nxt), d2, max(k, 1), commit=True)
    check_targets(tgt2[0], r2, K)
    if accepted_decided(r2, int(acc2[0]), max(k, 1)):
        assert acc2[0] == r2["accepted"] >= 1
        assert sfb.sf_cache_state(eng.cache, 0) == (ctx + r2["accepted"] + 1, int(r2["target"][r2["accepted"]]))


def test_prefill_one_and_two_passes_match_oracle(eng, weights, monkeypatch):
    """A 70-token prompt as one 70-row pass (the batched GEMM kernel) and as passes of 64 + 6
    rows (the single-group kernel) writes bit-identical K/V, within 0.02 relative of the
    oracle's cache."""
    sfb = need_gpu()
    prompt = synth.prompt_ids(S.vocab, 70, 4242)
    say("[7b] prefill 70")
    nxt = sfb.sf_prefill(eng.cache, 0, prompt)
    shape = (S.n_layers, S.n_kv_heads, 70, S.head_dim)
    kg = torch.zeros(shape, dtype=torch.int16, device="cuda")
    vg = torch.zeros_like(kg)
    sfb.sf_kv_read(eng.cache, 0, kg, vg, 70, 70)
    monkeypatch.setenv("SF_PREFILL_CHUNK", "64")
    c64 = sfb.sf_cache_alloc(eng.model, 1, 80, K)
    try:
        assert sfb.sf_prefill(c64, 0, prompt) == nxt
        k64 = torch.zeros_like(kg)
        v64 = torch.zeros_like(kg)
        sfb.sf_kv_read(c64, 0, k64, v64, 70, 70)
        torch.cuda.synchronize()
        assert torch.equal(kg, k64) and torch.equal(vg, v64)
    finally:
        sfb.sf_cache_free(c64)
    c = oracle.KVCache(S, 80)
    z = oracle.prefill(oracle.Model(S, weights), c, prompt)
    gap = oracle.top_gap(z[-1:])[0].item()
    if gap > GAP:
        assert nxt == c.next_token
    kg = kg.cpu().view(torch.bfloat16).double()
    vg = vg.cpu().view(torch.bfloat16).double()
    ko, vo = c.k[:, :, :70].double(), c.v[:, :, :70].double()
    rel_k = ((kg - ko).norm() / ko.norm()).item()
    rel_v = ((vg - vo).norm() / vo.norm()).item()
    say(f"[7b] prefill: next gpu {nxt} oracle {c.next_token} gap {gap:.3f}; KV rel err k {rel_k:.2e} v {rel_v:.2e}")
    # bf16 GEMM inputs and a bf16 cache: relative rounding ~2^-9 per element, a few of them per layer.
    assert rel_k < 0.02 and rel_v < 0.02
    assert sfb.sf_cache_state(eng.cache, 0) == (70, nxt)


def test_half_stack_hidden_states_match_oracle(weights, kv, hist):
    """The first-half shard's step as the benchmark runs it: a committing verify from 1024
    positions, a rollback that keeps the pending token and two drafts with a new pending
    token, and a second verify on top; both passes' hidden states against the oracle doing
    the same (max |d(x/rms x)| within the logit tolerance)."""
    sfb = need_gpu()
    H = synth.QWEN7B_HALF
    ctx = 1024
    say("[7b-half] engine")
    e = sfb.Engine(H, weights, n_seqs=1, capacity=4096, k_max=K)
    model = oracle.Model(H, weights)
    oc = _oracle_cache(kv, ctx, int(hist[ctx]), H, capacity=ctx + 2 * (K + 1) + 8)

    def check(xg, xo, what):
        ng = xg / xg.pow(2).mean(-1, keepdim=True).sqrt()
        no = xo / xo.pow(2).mean(-1, keepdim=True).sqrt()
        err = (ng - no).abs().max().item()
        say(f"[7b-half] {what}: max |d(x/rms x)| {err:.4g}")
        assert err <= LOGIT_TOL

    try:
        nxt = int(hist[ctx])
        _load_ctx(sfb, e.cache, kv, ctx, nxt, n_layers=H.n_layers)
        d = hist[ctx + 1:ctx + 1 + K].astype(np.int32)
        hid = torch.empty((K + 1, H.hidden), dtype=torch.int16, device="cuda")
        sfb.sf_verify(e.cache, d[None], None, 0, dev_out=hid)
        torch.cuda.synchronize()
        # Hidden-state stacks commit all k+1 positions; the caller then rewinds.
        assert sfb.sf_cache_state(e.cache, 0)[0] == ctx + K + 1
        sfb.sf_rollback(e.cache, 0, ctx + 3)
        assert sfb.sf_cache_state(e.cache, 0)[0] == ctx + 3
        say("[7b-half] oracle")
        r = oracle.verify(model, oc, d, K, commit=True)
        check(hid.cpu().view(torch.bfloat16).double(), r["hidden"], "first pass")
        # the second step on top of the rewound cache, with a new pending token
        oracle.rollback(oc, ctx + 3)
        t2 = int(hist[ctx + 40])
        oracle.set_next(oc, t2)
        sfb.sf_set_next(e.cache, 0, t2)
        d2 = hist[ctx + 41:ctx + 41 + K].astype(np.int32)
        sfb.sf_verify(e.cache, d2[None], None, 0, dev_out=hid)
        torch.cuda.synchronize()
        assert sfb.sf_cache_state(e.cache, 0)[0] == ctx + 3 + K + 1
        r2 = oracle.verify(model, oc, d2, K, commit=True)
        check(hid.cpu().view(torch.bfloat16).double(), r2["hidden"], "after the rollback")
    finally:
        e.close()


def test_batched_32_sequences_matches_oracle_and_single_runs(weights, kv):
    """32 sequences x 9 positions (288 rows, the row-grouped GEMM path) at contexts drawn
    from U{256..8192}: eight sequences (the shortest and longest context and six between)
    against the oracle, and the shortest and longest bitwise equal to the same sequence
    verified alone."""
    sfb = need_gpu()
    Bn = 32
    rng = np.random.default_rng(synth.seeds(5)["contexts"])
    ctx = rng.integers(256, 8192 + 1, size=Bn)
    nxt = rng.integers(0, S.vocab, size=Bn)
    drafts = rng.integers(0, S.vocab, size=(Bn, K)).astype(np.int32)
    say(f"[7b-batched] contexts {ctx.min()}..{ctx.max()}")
    eng = sfb.Engine(S, weights, n_seqs=Bn, capacity=CAP, k_max=K)
    one = sfb.Engine(S, weights, n_seqs=1, capacity=CAP, k_max=K)
    try:
        kd = torch.from_numpy(np.ascontiguousarray(kv[0]).view(np.int16)).cuda()
        vd = torch.from_numpy(np.ascontiguousarray(kv[1]).view(np.int16)).cuda()
        for b in range(Bn):
            sfb.sf_kv_write(eng.cache, b, kd, vd, int(ctx[b]), kv[0].shape[2])
            sfb.sf_set_next(eng.cache, b, int(nxt[b]))
        logits = torch.empty((Bn * (K + 1), S.vocab), dtype=torch.float32, device="cuda")
        acc, tgt = sfb.sf_verify(eng.cache, drafts, None, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT, dev_out=logits)
        acc_g, tgt_g = sfb.sf_verify(eng.cache, drafts, None, sfb.SF_NO_COMMIT)
        torch.cuda.synchronize()
        assert (acc_g == acc).all() and (tgt_g == tgt).all()
        model = oracle.Model(S, weights)
        one_logits = torch.empty((K + 1, S.vocab), dtype=torch.float32, device="cuda")
        ends = (int(np.argmin(ctx)), int(np.argmax(ctx)))
        order = np.argsort(ctx)
        between = [int(order[i]) for i in np.linspace(1, Bn - 2, 6).round().astype(int)]
        for b in list(ends) + between:
            if b in ends:
                sfb.sf_kv_write(one.cache, 0, kd, vd, int(ctx[b]), kv[0].shape[2])
                sfb.sf_set_next(one.cache, 0, int(nxt[b]))
                a1, t1 = sfb.sf_verify(one.cache, drafts[b:b + 1], None, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT,
                                       dev_out=one_logits)
                torch.cuda.synchronize()
                assert torch.equal(one_logits.cpu(), logits.view(Bn, K + 1, S.vocab)[b].cpu()), f"sequence {b}"
                assert a1[0] == acc[b] and (t1[0] == tgt[b]).all()
            say(f"[7b-batched] seq {b} ctx {ctx[b]}: oracle")
            r = oracle.verify(model, _oracle_cache(kv, int(ctx[b]), int(nxt[b])), drafts[b], K, commit=False)
            err = (logits.view(Bn, K + 1, S.vocab)[b].double().cpu() - r["logits"]).abs().max().item()
            say(f"[7b-batched] seq {b} max |dlogit| {err:.3g}")
            assert err <= LOGIT_TOL
            check_targets(tgt[b], r, K)
            if accepted_decided(r, int(acc[b]), K):
                assert acc[b] == r["accepted"]
    finally:
        eng.close()
        one.close()
