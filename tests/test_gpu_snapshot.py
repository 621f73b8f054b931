"""GPU parity of the snapshot form of rollback (sf_snapshot_save / sf_snapshot_restore plus a
replay of the accepted drafts) through the C-ABI: against the in-place index rewind on the
GPU (bit-identical state and K/V) and against the oracle's snapshot_verify round by round.

Inputs: the tiny stack with a final-norm gain of 32 (every logit x32 exactly, so the top-1 /
top-2 gaps clear the 0.1 decision threshold as a trained model's do), a 20-token prompt, and
per round the oracle's own 4-token greedy continuation with one seeded corruption.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GAP, accepted_decided, need_gpu, say

pytestmark = pytest.mark.gpu

S = synth.TINY
K = 4
CAP = 128


def _kv(sfb, cache, n):
    shape = (S.n_layers, S.n_kv_heads, CAP, S.head_dim)
    kg = torch.zeros(shape, dtype=torch.int16, device="cuda")
    vg = torch.zeros_like(kg)
    sfb.sf_kv_read(cache, 0, kg, vg, n, CAP)
    torch.cuda.synchronize()
    return kg.cpu()[:, :, :n], vg.cpu()[:, :, :n]


def _setup(sfb):
    w = synth.with_head_gain(synth.model_weights(S, synth.seeds(1)["weights"]), 32.0)
    eng = sfb.Engine(S, w, n_seqs=1, capacity=CAP, k_max=K)
    snap_cache = sfb.sf_cache_alloc(eng.model, 1, CAP, K)
    om = oracle.Model(S, w, cache=True)
    prompt = synth.prompt_ids(S.vocab, 20, 21)
    oc = oracle.KVCache(S, CAP)
    z = oracle.prefill(om, oc, prompt)
    assert oracle.top_gap(z[-1:])[0].item() > GAP
    for c in (eng.cache, snap_cache):
        assert sfb.sf_prefill(c, 0, prompt) == oc.next_token
    return eng, snap_cache, om, oc


def test_restore_returns_the_saved_rows_and_state():
    sfb = need_gpu()
    eng, sc, om, oc = _setup(sfb)
    try:
        fresh = sfb.sf_cache_alloc(eng.model, 1, CAP, K)
        with pytest.raises(sfb.SFError) as e:
            sfb.sf_snapshot_restore(fresh)         # nothing saved yet
        assert e.value.code == sfb.SF_E_STATE
        sfb.sf_cache_free(fresh)
        L, nx = sfb.sf_cache_state(sc, 0)
        k0, v0 = _kv(sfb, sc, L + K + 1)
        sfb.sf_snapshot_save(sc)
        sfb.sf_verify(sc, np.array([[5, 6, 7, 8]], dtype=np.int32), [K], sfb.SF_FORCE_ACCEPT)
        assert sfb.sf_cache_state(sc, 0) != (L, nx)
        k1, _ = _kv(sfb, sc, L + K + 1)
        assert not torch.equal(k0, k1)             # the pass wrote rows L..L+K
        sfb.sf_snapshot_restore(sc)
        assert sfb.sf_cache_state(sc, 0) == (L, nx)
        k2, v2 = _kv(sfb, sc, L + K + 1)
        assert torch.equal(k0, k2) and torch.equal(v0, v2)
    finally:
        sfb.sf_cache_free(sc)
        eng.close()


def test_snapshot_rounds_match_in_place_rounds_and_oracle():
    sfb = need_gpu()
    eng, sc, om, oc = _setup(sfb)
    rng = np.random.default_rng(7)
    try:
        compared, accepted = 0, []
        for i in range(10):
            d, _ = synth.corrupt_draft(oracle.greedy_continuation(om, oc, K), S.vocab, rng)
            dd = d[None].astype(np.int32)
            acc_a, _ = sfb.sf_verify(eng.cache, dd, [K])                     # in-place rewind
            sfb.sf_snapshot_save(sc)
            acc_b, _ = sfb.sf_verify(sc, dd, [K])
            M = int(acc_b[0])
            if M < K:
                sfb.sf_snapshot_restore(sc)
                sfb.sf_verify(sc, dd, [M], sfb.SF_FORCE_ACCEPT)              # replay d_1..d_M
            assert int(acc_a[0]) == M, f"round {i}"
            st = sfb.sf_cache_state(eng.cache, 0)
            assert sfb.sf_cache_state(sc, 0) == st, f"round {i}"
            ka, va = _kv(sfb, eng.cache, st[0])
            kb, vb = _kv(sfb, sc, st[0])
            assert torch.equal(ka, kb) and torch.equal(va, vb), f"round {i}"
            r = oracle.snapshot_verify(om, oc, d, K)
            if not (accepted_decided(r, M, K) and r["gap"][min(M, K)].item() > GAP):
                say(f"[snapshot] round {i}: a decision within the gap; oracle comparison ends here")
                break
            assert M == r["accepted"] and st == (oc.length, oc.next_token), f"round {i}"
            compared += 1
            accepted.append(M)
        say(f"[snapshot] {compared} rounds compared with the oracle, accepted {accepted}")
        assert compared >= 6 and min(accepted) < K
    finally:
        sfb.sf_cache_free(sc)
        eng.close()
