"""GPU parity of NF4 verification (sf_model_create_nf4: 4-bit NormalFloat projections decoded
inside the GEMM) against the oracle's NF4 stack, through the C ABI.

Inputs: synthetic NF4 projections (codes uniform over the 16 levels, per-64 scales drawn as
0.02 times the largest |z| of 64 normals), bf16 embeddings, biases and head.  Tiny stack with
a final-norm gain of 32 (every logit x32 exactly, so top-1/top-2 gaps clear 0.1 as a trained
model's do); two layers at the Qwen2.5-14B shape (hidden 5120, 40 query / 8 KV heads, FFN
13824, vocab 152064) with the full embedding and head.  Rule: logits max-abs <= 0.05; targets,
accepted counts and positions bit-exact where the oracle's top-1/top-2 gap exceeds 0.1.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GAP, LOGIT_TOL, accepted_decided, check_targets, need_gpu, say
from oracle import nf4

pytestmark = pytest.mark.gpu


def _verify_vs_oracle(sfb, eng, om, oc, d, k, K, tag):
    logits = torch.empty((K + 1, om.shape.vocab), dtype=torch.float32, device="cuda")
    acc_e, tgt_e = sfb.sf_verify(eng.cache, d[None], np.array([k]), sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT,
                                 dev_out=logits)
    acc, tgt = sfb.sf_verify(eng.cache, d[None], np.array([k]), sfb.SF_NO_COMMIT)
    torch.cuda.synchronize()
    assert acc[0] == acc_e[0] and (tgt == tgt_e).all()
    r = oracle.verify(om, oc, d, k)
    err = (logits.double().cpu() - r["logits"]).abs().max().item()
    ne, nt = check_targets(tgt[0], r, K)
    say(f"[{tag}] max |dlogit| {err:.3g}; exact-rule slots {ne}/{nt}; accepted gpu {acc[0]} oracle {r['accepted']}")
    assert err <= LOGIT_TOL
    # Lockstep: commit the oracle's decision on the GPU.
    sfb.sf_verify(eng.cache, d[None], np.array([r["accepted"]]), sfb.SF_FORCE_ACCEPT)
    sfb.sf_set_next(eng.cache, 0, oc.next_token)
    assert sfb.sf_cache_state(eng.cache, 0) == (oc.length, oc.next_token)
    return int(acc[0]), r


def test_nf4_tiny_prefill_and_lockstep_verify():
    sfb = need_gpu()
    S, K, CAP = synth.TINY, 4, 256
    w = synth.with_head_gain(synth.nf4_model_weights(S, synth.seeds(1)["weights"]), 32.0)
    eng = sfb.Engine(S, w, n_seqs=1, capacity=CAP, k_max=K)
    try:
        om = nf4.Nf4Model(S, w, cache=True)
        prompt = synth.prompt_ids(S.vocab, 100, 31)           # two prefill passes (64 + 36)
        oc = oracle.KVCache(S, CAP)
        z = oracle.prefill(om, oc, prompt)
        nxt = sfb.sf_prefill(eng.cache, 0, prompt)
        assert oracle.top_gap(z[-1:])[0].item() > GAP and nxt == oc.next_token
        shape = (S.n_layers, S.n_kv_heads, CAP, S.head_dim)
        kg = torch.zeros(shape, dtype=torch.int16, device="cuda")
        vg = torch.zeros_like(kg)
        sfb.sf_kv_read(eng.cache, 0, kg, vg, 100, CAP)
        torch.cuda.synchronize()
        kg = kg.cpu().view(torch.bfloat16).double()[:, :, :100]
        vg = vg.cpu().view(torch.bfloat16).double()[:, :, :100]
        assert (kg - oc.k[:, :, :100].double()).abs().max().item() <= 0.02 * max(1.0, oc.k.double().abs().max().item())
        assert (vg - oc.v[:, :, :100].double()).abs().max().item() <= 0.02 * max(1.0, oc.v.double().abs().max().item())
        rng = np.random.default_rng(11)
        accepted = []
        for step in range(10):
            d, _ = synth.corrupt_draft(oracle.greedy_continuation(om, oc, K), S.vocab, rng)
            M, r = _verify_vs_oracle(sfb, eng, om, oc, d, K, K, f"nf4-tiny step {step}")
            if accepted_decided(r, M, K):
                assert M == r["accepted"]
                accepted.append(M)
        assert len(accepted) >= 6 and min(accepted) < K
    finally:
        eng.close()


def test_nf4_14b_shape_two_layers_verify_matches_oracle():
    """Two layers of the 14B shape with NF4 projections, capacity 576 (9 attention spans x 8 KV
    heads): prefill and two verifies against the oracle's NF4 model.  This capacity once
    faulted when an L2 warm-up walked the bf16 tile layout over NF4 blocks; the case stays as a
    regression test."""
    sfb = need_gpu()
    S, K, CAP = synth.QWEN14B_2L, 8, 576
    say("[nf4-14b-2l] weights")
    w = synth.nf4_model_weights(S, synth.seeds(8)["weights"])
    eng = sfb.Engine(S, w, n_seqs=1, capacity=CAP, k_max=K)
    try:
        om = nf4.Nf4Model(S, w)
        prompt = synth.prompt_ids(S.vocab, 40, 41)
        say("[nf4-14b-2l] prefill")
        nxt = sfb.sf_prefill(eng.cache, 0, prompt)
        oc = oracle.KVCache(S, CAP)
        z = oracle.prefill(om, oc, prompt)
        if oracle.top_gap(z[-1:])[0].item() > GAP:
            assert nxt == oc.next_token
        sfb.sf_set_next(eng.cache, 0, oc.next_token)
        d = synth.prompt_ids(S.vocab, K, 43).astype(np.int32)
        say("[nf4-14b-2l] verify")
        M, r = _verify_vs_oracle(sfb, eng, om, oc, d, K, K, "nf4-14b-2l")
        if accepted_decided(r, M, K):
            assert M == r["accepted"]
        d2 = synth.prompt_ids(S.vocab, K, 44).astype(np.int32)
        say("[nf4-14b-2l] second verify")
        _verify_vs_oracle(sfb, eng, om, oc, d2, K, K, "nf4-14b-2l second")
    finally:
        eng.close()
