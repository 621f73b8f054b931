"""GPU parity of the graph-replayed single-token draft loop at the Qwen2.5-0.5B shape
(24 layers, hidden 896, 14 q / 2 KV heads, head_dim 64, SwiGLU 4864, vocab 151936,
tied head), through the C ABI.

A 512-token uniform prompt is prefilled on both sides; then rounds of 8 draft steps
run in lockstep with the oracle's greedy decoding, each round followed by the
in-place rollback of a seeded 0..8 rejected suffix and a seeded correction token.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GAP, need_gpu, say

pytestmark = pytest.mark.gpu

S = synth.QWEN05B


@pytest.fixture(scope="module")
def weights():
    need_gpu()
    say("[0.5b] weights")
    return synth.model_weights(S, synth.seeds(2)["weights"])


@pytest.fixture(scope="module")
def setup(weights):
    sfb = need_gpu()
    model = oracle.Model(S, weights, cache=True)
    say("[0.5b] engine")
    eng = sfb.Engine(S, weights, n_seqs=1, capacity=2048, k_max=8)
    yield sfb, model, eng
    eng.close()


def _round_rollback(rng, L):
    """Seeded outcome of a round that fed positions L..L+7: (new length, new pending token or None)."""
    r = synth.rejected_suffix(rng, 8)
    if r == 0:
        return L + 8, None
    M = 8 - r
    return L + 1 + M, int(rng.integers(0, S.vocab))


def test_draft_rounds_lockstep_with_oracle(setup):
    sfb, model, eng = setup
    prompt = synth.prompt_ids(S.vocab, 512, synth.seeds(2)["prompt"])
    say("[0.5b] prefill")
    nxt = sfb.sf_prefill(eng.cache, 0, prompt)
    c = oracle.KVCache(S, 2048)
    z = oracle.prefill(model, c, prompt)
    if oracle.top_gap(z[-1:])[0].item() > GAP:
        assert nxt == c.next_token
    sfb.sf_set_next(eng.cache, 0, c.next_token)
    rng = np.random.default_rng(synth.seeds(2)["draft"])
    checked = total = 0
    for rnd in range(4):
        L = c.length
        say(f"[0.5b] round {rnd} L={L}")
        for i in range(8):
            tok = int(sfb.sf_draft_step(eng.cache, 1)[0][0])
            r = oracle.verify(model, c, [], 0)
            total += 1
            if r["gap"][0] > GAP:
                assert tok == c.next_token, (rnd, i, tok, c.next_token)
                checked += 1
            sfb.sf_set_next(eng.cache, 0, c.next_token)
        new_len, new_next = _round_rollback(rng, L)
        oracle.rollback(c, new_len)
        sfb.sf_rollback(eng.cache, 0, new_len)
        if new_next is not None:
            oracle.set_next(c, new_next)
            sfb.sf_set_next(eng.cache, 0, new_next)
        assert sfb.sf_cache_state(eng.cache, 0) == (c.length, c.next_token)
    say(f"[0.5b] draft tokens checked under the gap rule: {checked}/{total}")
    assert checked >= total // 4


def test_64_rounds_graph_loop_with_rollback(setup):
    """The full draft workload on the GPU alone: 64 rounds of one 8-step graph-replay call
    plus a seeded rollback; n steps in one call equal n single-step calls bitwise."""
    sfb, model, eng = setup
    prompt = synth.prompt_ids(S.vocab, 512, synth.seeds(2)["prompt"])
    sfb.sf_prefill(eng.cache, 0, prompt)
    rng = np.random.default_rng(synth.seeds(2)["draft"] + 1)
    for rnd in range(64):
        L, nx = sfb.sf_cache_state(eng.cache, 0)
        toks = sfb.sf_draft_step(eng.cache, 8)[0].tolist()
        if rnd % 16 == 0:
            sfb.sf_rollback(eng.cache, 0, L)
            sfb.sf_set_next(eng.cache, 0, nx)
            one = [int(sfb.sf_draft_step(eng.cache, 1)[0][0]) for _ in range(8)]
            assert one == toks
        assert sfb.sf_cache_state(eng.cache, 0) == (L + 8, toks[-1])
        new_len, new_next = _round_rollback(rng, L)
        sfb.sf_rollback(eng.cache, 0, new_len)
        if new_next is not None:
            sfb.sf_set_next(eng.cache, 0, new_next)
    ln, _ = sfb.sf_cache_state(eng.cache, 0)
    say(f"[0.5b] after 64 rounds: length {ln}")
    assert 512 < ln <= 512 + 64 * 8


def test_draft_pass_logits_and_prefill_match_oracle(setup):
    """The drafter at logit level (tied head, V=151936, head_dim 64).  A second cache of the
    same model with k_max=0 runs exactly the draft step's one-row pass; after a 512-token
    prefill its debug logits, at the prefill's pending token and after each of four lockstep
    steps, are within 0.05 of the oracle's, and the graph-replayed draft step returns their
    argmax (same kernels, same bits).  The prefill's K/V are within 0.02 relative of the
    oracle's cache."""
    sfb, model, eng = setup
    c0 = sfb.sf_cache_alloc(eng.model, 1, 2048, 0)
    try:
        prompt = synth.prompt_ids(S.vocab, 512, synth.seeds(2)["prompt"] + 9)
        say("[0.5b] prefill (logit check)")
        nxt = sfb.sf_prefill(c0, 0, prompt)
        c = oracle.KVCache(S, 2048)
        z = oracle.prefill(model, c, prompt)
        if oracle.top_gap(z[-1:])[0].item() > GAP:
            assert nxt == c.next_token
        shape = (S.n_layers, S.n_kv_heads, 512, S.head_dim)
        kg = torch.zeros(shape, dtype=torch.int16, device="cuda")
        vg = torch.zeros_like(kg)
        sfb.sf_kv_read(c0, 0, kg, vg, 512, 512)
        torch.cuda.synchronize()
        kg = kg.cpu().view(torch.bfloat16).double()
        vg = vg.cpu().view(torch.bfloat16).double()
        ko, vo = c.k[:, :, :512].double(), c.v[:, :, :512].double()
        rel_k = ((kg - ko).norm() / ko.norm()).item()
        rel_v = ((vg - vo).norm() / vo.norm()).item()
        say(f"[0.5b] prefill KV rel err k {rel_k:.2e} v {rel_v:.2e}")
        assert rel_k < 0.02 and rel_v < 0.02
        sfb.sf_set_next(c0, 0, c.next_token)
        logits = torch.empty((1, S.vocab), dtype=torch.float32, device="cuda")
        worst = 0.0
        for i in range(5):
            sfb.sf_verify(c0, np.zeros((1, 0), np.int32), None, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT,
                          dev_out=logits)
            torch.cuda.synchronize()
            zg = logits.cpu()
            r = oracle.verify(model, c, [], 0)
            err = (zg.double() - r["logits"]).abs().max().item()
            worst = max(worst, err)
            assert err <= 0.05, (i, err)
            tok = int(sfb.sf_draft_step(c0, 1)[0][0])
            assert tok == int(oracle.argmax_lowest(zg)[0]), i
            if r["gap"][0] > GAP:
                assert tok == c.next_token
            sfb.sf_set_next(c0, 0, c.next_token)
            assert sfb.sf_cache_state(c0, 0) == (c.length, c.next_token)
        say(f"[0.5b] draft-pass max |dlogit| {worst:.4g}")
    finally:
        sfb.sf_cache_free(c0)
