"""GPU parity of the batched verify (many sequences in one pass, more than 64 rows), through
the C ABI.

Each sequence has its own length, pending token and drafts in one pool; the pass runs
the row-grouped GEMM path.  Checks: every sequence against the float64 oracle (parity
rule), and bitwise equality with the same sequence verified alone, since a row's
arithmetic must not depend on the other rows of the batch.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GAP, LOGIT_TOL, accepted_decided, check_targets, need_gpu, say

pytestmark = pytest.mark.gpu

S = synth.TINY
B, K, CAP = 16, 4, 512


def _fill(sfb, eng, kv, ctx, nxt):
    kb, vb = kv
    kd = torch.from_numpy(np.ascontiguousarray(kb).view(np.int16)).cuda()
    vd = torch.from_numpy(np.ascontiguousarray(vb).view(np.int16)).cuda()
    for b, (c, t) in enumerate(zip(ctx, nxt)):
        sfb.sf_kv_write(eng.cache, b, kd, vd, int(c), kb.shape[2])
        sfb.sf_set_next(eng.cache, b, int(t))
    torch.cuda.synchronize()


def test_batched_tiny_matches_oracle_and_single_sequence_runs():
    sfb = need_gpu()
    sd = synth.seeds(5)
    rng = np.random.default_rng(sd["contexts"])
    ctx = rng.integers(40, CAP - K - 1, size=B)
    nxt = rng.integers(0, S.vocab, size=B)
    drafts = rng.integers(0, S.vocab, size=(B, K)).astype(np.int32)
    ks = rng.integers(0, K + 1, size=B).astype(np.int32)
    kv = synth.synthetic_kv(S, CAP, sd["kv"])
    w = synth.model_weights(S, sd["weights"])
    say(f"[batched] B={B} K={K} contexts {ctx.min()}..{ctx.max()}")
    eng = sfb.Engine(S, w, n_seqs=B, capacity=CAP, k_max=K)
    one = sfb.Engine(S, w, n_seqs=1, capacity=CAP, k_max=K)
    try:
        _fill(sfb, eng, kv, ctx, nxt)
        logits = torch.empty((B * (K + 1), S.vocab), dtype=torch.float32, device="cuda")
        acc, tgt = sfb.sf_verify(eng.cache, drafts, ks, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT, dev_out=logits)
        acc_g, tgt_g = sfb.sf_verify(eng.cache, drafts, ks, 0)   # graph replay, commits
        torch.cuda.synchronize()
        assert (acc_g == acc).all() and (tgt_g == tgt).all()
        lg = logits.double().cpu().view(B, K + 1, S.vocab)
        model = oracle.Model(S, w)
        one_logits = torch.empty((K + 1, S.vocab), dtype=torch.float32, device="cuda")
        worst = 0.0
        for b in range(B):
            c = oracle.KVCache(S, int(ctx[b]) + K + 1)
            c.load(kv[0], kv[1], int(ctx[b]), next_token=int(nxt[b]))
            r = oracle.verify(model, c, drafts[b], int(ks[b]), commit=True)
            worst = max(worst, (lg[b] - r["logits"]).abs().max().item())
            check_targets(tgt[b], r, K)
            if accepted_decided(r, int(acc[b]), int(ks[b])):
                assert acc[b] == r["accepted"]
                assert sfb.sf_cache_state(eng.cache, b) == (c.length, c.next_token)
            # the same sequence alone
            _fill(sfb, one, kv, [ctx[b]], [nxt[b]])
            a1, t1 = sfb.sf_verify(one.cache, drafts[b:b + 1], ks[b:b + 1], sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT,
                                   dev_out=one_logits)
            torch.cuda.synchronize()
            assert a1[0] == acc[b] and (t1[0] == tgt[b]).all()
            assert torch.equal(one_logits.cpu(), logits.view(B, K + 1, S.vocab)[b].cpu()), f"sequence {b}"
        say(f"[batched] max |dlogit| vs oracle over {B} sequences: {worst:.3g}")
        assert worst <= LOGIT_TOL
    finally:
        eng.close()
        one.close()


def test_largest_batch_64_sequences_512_rows():
    """The largest pass the library takes: 64 sequences x 8 positions (k_max 7, 512 rows, eight
    64-row groups), contexts drawn from U{10..200} and per-sequence k in 0..7.  Eight sampled
    sequences against the oracle, two of them also bitwise against the same sequence verified
    alone, and every sequence's committed state."""
    sfb = need_gpu()
    Bm, Km, cap = 64, 7, 256
    rng = np.random.default_rng(6464)
    ctx = rng.integers(10, 201, size=Bm)
    nxt = rng.integers(0, S.vocab, size=Bm)
    drafts = rng.integers(0, S.vocab, size=(Bm, Km)).astype(np.int32)
    ks = rng.integers(0, Km + 1, size=Bm).astype(np.int32)
    kv = synth.synthetic_kv(S, cap, 6465)
    w = synth.model_weights(S, synth.seeds(5)["weights"])
    eng = sfb.Engine(S, w, n_seqs=Bm, capacity=cap, k_max=Km)
    one = sfb.Engine(S, w, n_seqs=1, capacity=cap, k_max=Km)
    try:
        _fill(sfb, eng, kv, ctx, nxt)
        logits = torch.empty((Bm * (Km + 1), S.vocab), dtype=torch.float32, device="cuda")
        acc, tgt = sfb.sf_verify(eng.cache, drafts, ks, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT, dev_out=logits)
        acc_g, tgt_g = sfb.sf_verify(eng.cache, drafts, ks, 0)   # graph replay, commits
        torch.cuda.synchronize()
        assert (acc_g == acc).all() and (tgt_g == tgt).all()
        lg = logits.double().cpu().view(Bm, Km + 1, S.vocab)
        model = oracle.Model(S, w)
        one_logits = torch.empty((Km + 1, S.vocab), dtype=torch.float32, device="cuda")
        sample = sorted(set([0, Bm - 1] + rng.choice(Bm, size=6, replace=False).tolist()))
        worst = 0.0
        for b in sample:
            c = oracle.KVCache(S, int(ctx[b]) + Km + 1)
            c.load(kv[0], kv[1], int(ctx[b]), next_token=int(nxt[b]))
            r = oracle.verify(model, c, drafts[b], int(ks[b]), commit=True)
            worst = max(worst, (lg[b] - r["logits"]).abs().max().item())
            check_targets(tgt[b], r, Km)
            if accepted_decided(r, int(acc[b]), int(ks[b])):
                assert acc[b] == r["accepted"]
                assert sfb.sf_cache_state(eng.cache, b) == (c.length, c.next_token)
            if b in (sample[0], sample[-1]):
                _fill(sfb, one, kv, [ctx[b]], [nxt[b]])
                sfb.sf_verify(one.cache, drafts[b:b + 1], ks[b:b + 1], sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT,
                              dev_out=one_logits)
                torch.cuda.synchronize()
                assert torch.equal(one_logits.cpu(), logits.view(Bm, Km + 1, S.vocab)[b].cpu()), f"sequence {b}"
        for b in range(Bm):
            L, t = sfb.sf_cache_state(eng.cache, b)
            assert L == int(ctx[b]) + int(acc[b]) + 1 and t == int(tgt[b][int(acc[b])])
        say(f"[batched] 64 x 8 rows: max |dlogit| vs oracle over {len(sample)} sequences: {worst:.3g}")
        assert worst <= LOGIT_TOL
    finally:
        eng.close()
        one.close()


@pytest.mark.parametrize("splits", [(2, 4), (4, 8)], ids=["O2-down4", "O4-down8"])
def test_batched_k_splits_bitwise_single_runs(monkeypatch, splits):
    """More k splits than the tiny shape's defaults (SF_SP_O / SF_SP_D, read when a cache is
    allocated), so the batched residual projections run the LDS-staged kernel with 8 to 32
    k chunks and a last arriver over 2 to 8 splits: 13 sequences x 5 positions (65 rows: one
    64-row group and a one-row tail) bitwise against each sequence verified alone, and one
    sequence against the oracle."""
    sfb = need_gpu()
    sp_o, sp_d = splits
    monkeypatch.setenv("SF_SP_O", str(sp_o))
    monkeypatch.setenv("SF_SP_D", str(sp_d))
    Bs, Ks = 13, 4
    rng = np.random.default_rng(7300 + sp_d)
    ctx = rng.integers(20, CAP - Ks - 1, size=Bs)
    nxt = rng.integers(0, S.vocab, size=Bs)
    drafts = rng.integers(0, S.vocab, size=(Bs, Ks)).astype(np.int32)
    ks = rng.integers(0, Ks + 1, size=Bs).astype(np.int32)
    kv = synth.synthetic_kv(S, CAP, 7301)
    w = synth.model_weights(S, synth.seeds(5)["weights"])
    say(f"[batched splits] O {sp_o}, down {sp_d}: {Bs} x {Ks + 1} rows")
    eng = sfb.Engine(S, w, n_seqs=Bs, capacity=CAP, k_max=Ks)
    one = sfb.Engine(S, w, n_seqs=1, capacity=CAP, k_max=Ks)
    try:
        _fill(sfb, eng, kv, ctx, nxt)
        logits = torch.empty((Bs * (Ks + 1), S.vocab), dtype=torch.float32, device="cuda")
        acc, tgt = sfb.sf_verify(eng.cache, drafts, ks, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT, dev_out=logits)
        torch.cuda.synchronize()
        one_logits = torch.empty((Ks + 1, S.vocab), dtype=torch.float32, device="cuda")
        for b in range(Bs):
            _fill(sfb, one, kv, [ctx[b]], [nxt[b]])
            a1, t1 = sfb.sf_verify(one.cache, drafts[b:b + 1], ks[b:b + 1], sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT,
                                   dev_out=one_logits)
            torch.cuda.synchronize()
            assert a1[0] == acc[b] and (t1[0] == tgt[b]).all()
            assert torch.equal(one_logits.cpu(), logits.view(Bs, Ks + 1, S.vocab)[b].cpu()), f"sequence {b}"
        b = Bs - 1
        c = oracle.KVCache(S, int(ctx[b]) + Ks + 1)
        c.load(kv[0], kv[1], int(ctx[b]), next_token=int(nxt[b]))
        r = oracle.verify(oracle.Model(S, w), c, drafts[b], int(ks[b]), commit=True)
        worst = (logits.double().cpu().view(Bs, Ks + 1, S.vocab)[b] - r["logits"]).abs().max().item()
        check_targets(tgt[b], r, Ks)
        say(f"[batched splits] last sequence max |dlogit| vs oracle: {worst:.3g}")
        assert worst <= LOGIT_TOL
    finally:
        eng.close()
        one.close()
