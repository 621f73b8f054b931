"""GPU parity of the device-resident speculative round (sf_round_*): drafter steps, verify,
accept and the drafter's rewind in one captured graph, against the oracle's model-drafter
round, round by round, through the C-ABI.

Inputs: two-layer stacks whose final-norm gain is 32 (every logit scaled by 32, so top-1/top-2
gaps are as wide as a trained model's instead of a random-init stack's).  Drafters: a near
copy of the verifier (each projection w + 0.05 o: mixed acceptance, both the rejection and the
all-accepted branch), a far copy (0.3: mostly rejected), and the verifier itself (every draft
accepted: the drafter's catch-up step every round).  Parity rule as elsewhere: accepted
counts, next tokens and both caches' positions bit-exact while every decision involved (the
drafter's K choices and the verifier's deciding slots) clears the oracle's top-1/top-2 gap of
0.1; the first round with a closer decision ends the comparison.
"""
import pytest
import torch

import oracle
import synth
from gpu_util import GAP, accepted_decided, need_gpu, say

pytestmark = pytest.mark.gpu

S = synth.TINY
K = 4
CAP = 256


HEAD_GAIN = 32.0
DRAFTERS = {"near": 0.05, "far": 0.3, "self": 0.0}


def _setup(sfb, drafter):
    wv = synth.with_head_gain(synth.model_weights(S, synth.seeds(1)["weights"]), HEAD_GAIN)
    eps = DRAFTERS[drafter]
    wd = wv if eps == 0 else synth.near_copy(wv, synth.model_weights(S, synth.seeds(2)["weights"]), eps)
    stream = torch.cuda.Stream()
    v = sfb.Engine(S, wv, n_seqs=1, capacity=CAP, k_max=K, stream=stream)
    d = sfb.Engine(S, wd, n_seqs=1, capacity=CAP, k_max=0, stream=stream)
    ov, od = oracle.Model(S, wv, cache=True), oracle.Model(S, wd, cache=True)
    prompt = synth.prompt_ids(S.vocab, 20, 21)
    nv = sfb.sf_prefill(v.cache, 0, prompt)
    sfb.sf_prefill(d.cache, 0, prompt)
    vc, dc = oracle.KVCache(S, CAP), oracle.KVCache(S, CAP)
    zv = oracle.prefill(ov, vc, prompt)
    oracle.prefill(od, dc, prompt)
    assert oracle.top_gap(zv[-1:])[0].item() > GAP
    assert nv == vc.next_token
    sfb.sf_set_next(d.cache, 0, nv)
    oracle.set_next(dc, vc.next_token)
    return stream, v, d, ov, od, vc, dc


@pytest.mark.parametrize("drafter", list(DRAFTERS))
def test_round_matches_oracle_round_by_round(drafter):
    sfb = need_gpu()
    stream, v, d, ov, od, vc, dc = _setup(sfb, drafter)
    rnd = sfb.sf_round_create(d.cache, v.cache, K)
    try:
        compared, accepted = 0, []
        for i in range(12):
            L = vc.length
            sfb.sf_round_run(rnd, 1)
            stream.synchronize()
            vlen, vnext = sfb.sf_cache_state(v.cache, 0)
            M = vlen - L - 1                     # a round commits M + 1 positions
            r = oracle.model_draft_round(od, dc, ov, vc, K)
            decided = min(r["draft_gap"]) > GAP and accepted_decided(r, M, K) and r["gap"][min(M, K)].item() > GAP
            if not decided:
                say(f"[round] round {i}: a decision within the gap; comparison ends here")
                break
            assert M == r["accepted"], f"round {i}"
            assert vnext == int(r["target"][M]), f"round {i}"
            assert (vlen, vnext) == (vc.length, vc.next_token), f"round {i}"
            assert sfb.sf_cache_state(d.cache, 0) == (dc.length, dc.next_token), f"round {i}"
            compared += 1
            accepted.append(M)
        say(f"[round] {drafter} drafter: {compared} rounds compared, accepted {accepted}")
        assert compared >= 6
        if drafter == "self":
            assert all(m == K for m in accepted)
        if drafter == "near":
            assert K in accepted and min(accepted) < K   # both branches of the round
    finally:
        sfb.sf_round_free(rnd)
        d.close()
        v.close()


def test_several_rounds_in_one_call_and_state_checks():
    sfb = need_gpu()
    stream, v, d, ov, od, vc, dc = _setup(sfb, "near")
    rnd = sfb.sf_round_create(d.cache, v.cache, K)
    try:
        sfb.sf_round_run(rnd, 3)
        stream.synchronize()
        for _ in range(3):
            r = oracle.model_draft_round(od, dc, ov, vc, K)
            M = r["accepted"]
            assert min(r["draft_gap"]) > GAP and accepted_decided(r, M, K) and r["gap"][M].item() > GAP
        assert sfb.sf_cache_state(v.cache, 0) == (vc.length, vc.next_token)
        assert sfb.sf_cache_state(d.cache, 0) == (dc.length, dc.next_token)
        # Out of step: the round refuses to start.
        sfb.sf_set_next(d.cache, 0, (vc.next_token + 1) % S.vocab)
        with pytest.raises(sfb.SFError) as e:
            sfb.sf_round_run(rnd, 1)
        assert e.value.code == sfb.SF_E_STATE
        sfb.sf_set_next(d.cache, 0, vc.next_token)
        # Capacity: rounds that could run past the capacity are refused before any launch.
        with pytest.raises(sfb.SFError) as e:
            sfb.sf_round_run(rnd, CAP)
        assert e.value.code == sfb.SF_E_CAPACITY
    finally:
        sfb.sf_round_free(rnd)
        d.close()
        v.close()


def test_round_create_rejects_bad_pairs():
    sfb = need_gpu()
    wv = synth.with_head_gain(synth.model_weights(S, synth.seeds(1)["weights"]), HEAD_GAIN)
    v = sfb.Engine(S, wv, n_seqs=1, capacity=CAP, k_max=K)
    other = sfb.Engine(S, wv, n_seqs=1, capacity=CAP, k_max=K)   # its own stream
    try:
        for args in [(v.cache, v.cache, K), (other.cache, v.cache, K), (v.cache, v.cache, 0)]:
            with pytest.raises(sfb.SFError) as e:
                sfb.sf_round_create(*args)
            assert e.value.code == sfb.SF_E_ARG
    finally:
        other.close()
        v.close()
