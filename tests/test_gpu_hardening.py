"""GPU tests of the rules a parity test with the gap exemption cannot reach, and of the error
path, through the C ABI, on the two-layer decoder.

- Exact argmax ties: two LM-head rows made bitwise equal give exactly equal logits, so the
  oracle's top-1/top-2 gap is 0 and the gap rule would skip the slot; the kernels must still
  pick the lower index ([Sangama] "Speculative decoding: correct, but slower (for now)": the
  model's own choice at every position; lowest index is this build's tie reading).  Planted
  inside one 32-column tile, and across tiles with the lower copy on a tile's last column.
- Split-K arrival counters: with every projection split (three ways for down), counters are
  back at zero after every pass and results stay within the oracle's tolerance.
- Injected failures (SF_FAULT=launch / alloc): the call fails with SF_E_HIP / SF_E_NOMEM and
  no sequence's length or pending token moves; the next call works as before.
- A device-resident round over three sequences, one of whose rounds is mixed (some sequences
  accept every draft, others do not), against the oracle sequence by sequence.
- Device drafts outside the vocabulary: clamped into the pass, never accepted.
- K/V copies against work still queued on torch's own stream: sf_kv_read's destination fill
  and sf_kv_write's source copy, each behind a long torch product, are ordered before the copy.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GAP, LOGIT_TOL, accepted_decided, check_targets, need_gpu, say

pytestmark = pytest.mark.gpu

S = synth.TINY
K = 4


def _tie_weights():
    """Head gain 32 (wide gaps) and two planted ties; returns (weights, slot -> expected index,
    draft, prompt, the tied pairs)."""
    w = synth.with_head_gain(synth.model_weights(S, synth.seeds(1)["weights"]), 32.0)
    m = oracle.Model(S, w, cache=True)
    prompt = synth.prompt_ids(S.vocab, 40, 606)
    c = oracle.KVCache(S, 128)
    oracle.prefill(m, c, prompt)
    cont = oracle.greedy_continuation(m, c, K)
    r = oracle.verify(m, c.copy(), cont, K, commit=False)
    t = [int(v) for v in r["target"]]
    # Within a tile: slot 0's choice copied to the first column of its own tile.
    s_in = next(j for j in range(K + 1) if t[j] % 32 != 0)
    low_in = t[s_in] - t[s_in] % 32
    # Across tiles: another slot's choice copied to the last column of an earlier tile.
    s_x = next(j for j in range(K + 1) if j != s_in and t[j] // 32 >= 2 and t[j] != t[s_in])
    low_x = 32 * (t[s_x] // 32 - 1) - 1
    head = w["lm_head"].copy()
    head[low_in] = head[t[s_in]]
    head[low_x] = head[t[s_x]]
    w = dict(w)
    w["lm_head"] = head
    return w, {s_in: (low_in, t[s_in]), s_x: (low_x, t[s_x])}, np.array(cont, dtype=np.int32), prompt


def test_exact_ties_pick_the_lowest_index():
    sfb = need_gpu()
    w, planted, draft, prompt = _tie_weights()
    say(f"[ties] planted (slot: lower, higher) {planted}")
    m = oracle.Model(S, w, cache=True)
    c = oracle.KVCache(S, 128)
    oracle.prefill(m, c, prompt)
    r = oracle.verify(m, c.copy(), draft, K, commit=False)
    z = r["logits"]
    for s, (lo, hi) in planted.items():
        # Exactly tied at the top, clear of everything else.
        assert abs(z[s, lo].item() - z[s, hi].item()) < 1e-9
        others = torch.cat([z[s, :lo], z[s, lo + 1:hi], z[s, hi + 1:]])
        assert z[s, hi].item() - others.max().item() > GAP
        assert int(r["target"][s]) == lo
    eng = sfb.Engine(S, w, n_seqs=1, capacity=128, k_max=K)
    try:
        nxt = sfb.sf_prefill(eng.cache, 0, prompt)
        assert nxt == c.next_token
        logits = torch.empty((K + 1, S.vocab), dtype=torch.float32, device="cuda")
        acc_e, tgt_e = sfb.sf_verify(eng.cache, draft[None], None, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT,
                                     dev_out=logits)
        acc, tgt = sfb.sf_verify(eng.cache, draft[None], None, sfb.SF_NO_COMMIT)
        torch.cuda.synchronize()
        zl = logits.cpu()
        for s, (lo, hi) in planted.items():
            assert zl[s, lo].item() == zl[s, hi].item(), (s, lo, hi)
            assert int(tgt_e[0][s]) == lo and int(tgt[0][s]) == lo, (s, tgt[0], lo)
        check_targets(tgt[0], r, K)
        assert (logits.double().cpu() - z).abs().max().item() <= LOGIT_TOL
        # The accept rule sees the lower index: the draft holds the higher copy at slot 0's
        # position only if slot 0 is the within-tile tie; either way M is the oracle's.
        assert int(acc[0]) == r["accepted"]
        say(f"[ties] targets {tgt[0].tolist()}, accepted {int(acc[0])}")
    finally:
        eng.close()


def test_split_counters_return_to_zero_and_results_hold(monkeypatch):
    """Every projection split over workgroups (QKV and O two ways, down three ways: a count
    that 2^32 is not a multiple of), through verifies, draft steps and a prefill: the arrival
    counters read zero after each, and logits stay within the oracle's tolerance."""
    sfb = need_gpu()
    monkeypatch.setenv("SF_SP_QKV", "2")
    monkeypatch.setenv("SF_SP_O", "2")
    monkeypatch.setenv("SF_SP_D", "3")
    w = synth.model_weights(S, synth.seeds(1)["weights"])
    m = oracle.Model(S, w, cache=True)
    eng = sfb.Engine(S, w, n_seqs=1, capacity=128, k_max=K)
    try:
        prompt = synth.prompt_ids(S.vocab, 33, 707)
        c = oracle.KVCache(S, 128)
        oracle.prefill(m, c, prompt)
        sfb.sf_prefill(eng.cache, 0, prompt)
        sfb.sf_set_next(eng.cache, 0, c.next_token)
        assert sfb.sf_debug_counters(eng.cache) == (0, 0)
        logits = torch.empty((K + 1, S.vocab), dtype=torch.float32, device="cuda")
        rng = np.random.default_rng(7)
        for i in range(6):
            d = rng.integers(0, S.vocab, size=(1, K)).astype(np.int32)
            sfb.sf_verify(eng.cache, d, None, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT, dev_out=logits)
            acc, tgt = sfb.sf_verify(eng.cache, d, None, sfb.SF_NO_COMMIT)
            assert sfb.sf_debug_counters(eng.cache) == (0, 0), f"pass {i}"
            r = oracle.verify(m, c, d[0], K, commit=False)
            assert (logits.double().cpu() - r["logits"]).abs().max().item() <= LOGIT_TOL
            check_targets(tgt[0], r, K)
        sfb.sf_draft_step(eng.cache, 5)
        assert sfb.sf_debug_counters(eng.cache) == (0, 0)
    finally:
        eng.close()


def test_injected_failures_leave_state_unchanged(monkeypatch):
    sfb = need_gpu()
    w = synth.model_weights(S, synth.seeds(1)["weights"])
    eng = sfb.Engine(S, w, n_seqs=1, capacity=128, k_max=K)
    try:
        sfb.sf_prefill(eng.cache, 0, synth.prompt_ids(S.vocab, 30, 808))
        d = np.array([[3, 1, 4, 1]], dtype=np.int32)
        acc0, tgt0 = sfb.sf_verify(eng.cache, d, None, sfb.SF_NO_COMMIT)
        st = sfb.sf_cache_state(eng.cache, 0)
        monkeypatch.setenv("SF_FAULT", "launch")
        calls = [lambda: sfb.sf_verify(eng.cache, d),
                 lambda: sfb.sf_verify(eng.cache, d, None, sfb.SF_DEBUG_LOGITS,
                                       dev_out=torch.empty((K + 1, S.vocab), device="cuda")),
                 lambda: sfb.sf_verify_device(eng.cache, torch.from_numpy(d).cuda()),
                 lambda: sfb.sf_draft_step(eng.cache, 3),
                 lambda: sfb.sf_prefill(eng.cache, 0, [5, 6, 7])]
        for i, f in enumerate(calls):
            with pytest.raises(sfb.SFError) as e:
                f()
            assert e.value.code == sfb.SF_E_HIP, i
            assert "launch" in sfb.sf_last_error()
        monkeypatch.setenv("SF_FAULT", "alloc")
        with pytest.raises(sfb.SFError) as e:
            sfb.sf_cache_alloc(eng.model, 1, 64, 2)
        assert e.value.code == sfb.SF_E_NOMEM
        monkeypatch.delenv("SF_FAULT")
        assert sfb.sf_cache_state(eng.cache, 0) == st
        acc1, tgt1 = sfb.sf_verify(eng.cache, d, None, sfb.SF_NO_COMMIT)
        assert (acc1 == acc0).all() and (tgt1 == tgt0).all()
        assert sfb.sf_cache_state(eng.cache, 0) == st
    finally:
        eng.close()


def test_round_over_three_sequences_with_a_mixed_round():
    """Three sequences (prompts whose oracle rounds are all decided beyond the gap), near-copy
    drafter, K=4, eight rounds one graph replay each.  Round 2 accepts every draft on one
    sequence and fewer on the others; the drafter's catch-up pass then runs for that sequence
    only.  Lengths and pending tokens of both caches match the oracle's round by round."""
    sfb = need_gpu()
    B, CAP = 3, 256
    wv = synth.with_head_gain(synth.model_weights(S, synth.seeds(1)["weights"]), 32.0)
    wd = synth.near_copy(wv, synth.model_weights(S, synth.seeds(2)["weights"]), 0.05)
    ov, od = oracle.Model(S, wv, cache=True), oracle.Model(S, wd, cache=True)
    stream = torch.cuda.Stream()
    v = sfb.Engine(S, wv, n_seqs=B, capacity=CAP, k_max=K, stream=stream)
    d = sfb.Engine(S, wd, n_seqs=B, capacity=CAP, k_max=0, stream=stream)
    rnd = None
    try:
        vcs, dcs = [], []
        for b, seed in enumerate((21, 23, 27)):
            prompt = synth.prompt_ids(S.vocab, 20, seed)
            vc, dc = oracle.KVCache(S, CAP), oracle.KVCache(S, CAP)
            zv = oracle.prefill(ov, vc, prompt)
            oracle.prefill(od, dc, prompt)
            assert oracle.top_gap(zv[-1:])[0].item() > GAP
            oracle.set_next(dc, vc.next_token)
            assert sfb.sf_prefill(v.cache, b, prompt) == vc.next_token
            sfb.sf_prefill(d.cache, b, prompt)
            sfb.sf_set_next(d.cache, b, vc.next_token)
            vcs.append(vc)
            dcs.append(dc)
        rnd = sfb.sf_round_create(d.cache, v.cache, K)
        mixed = 0
        for i in range(8):
            sfb.sf_round_run(rnd, 1)
            stream.synchronize()
            Ms = []
            for b in range(B):
                L = vcs[b].length
                r = oracle.model_draft_round(od, dcs[b], ov, vcs[b], K)
                vlen, vnext = sfb.sf_cache_state(v.cache, b)
                M = vlen - L - 1
                assert min(r["draft_gap"]) > GAP and accepted_decided(r, M, K) and r["gap"][min(M, K)].item() > GAP
                assert M == r["accepted"], (i, b)
                assert (vlen, vnext) == (vcs[b].length, vcs[b].next_token), (i, b)
                assert sfb.sf_cache_state(d.cache, b) == (dcs[b].length, dcs[b].next_token), (i, b)
                Ms.append(M)
            say(f"[round x3] round {i}: accepted {Ms}")
            mixed += (K in Ms) and min(Ms) < K
        assert mixed >= 1
    finally:
        if rnd is not None:
            sfb.sf_round_free(rnd)
        d.close()
        v.close()


def test_device_drafts_outside_the_vocabulary_are_clamped_and_never_accepted():
    """sf_verify_device does not range-check device drafts (they never reach the host): ids
    outside [0, V) feed the clamped id (0 or V-1) into the pass and never count as accepted.
    Targets equal those of a host verify with the clamped drafts; M stops at the first
    out-of-range draft."""
    sfb = need_gpu()
    w = synth.model_weights(S, synth.seeds(1)["weights"])
    eng = sfb.Engine(S, w, n_seqs=2, capacity=128, k_max=K)
    try:
        for b, seed in enumerate((31, 37)):
            sfb.sf_prefill(eng.cache, b, synth.prompt_ids(S.vocab, 24, seed))
        sfb.sf_sync(eng.cache)
        # sequence 0: its own greedy continuation with an out-of-range id at slot 2;
        # sequence 1: a negative id first.
        acc0, tgt0 = sfb.sf_verify(eng.cache, np.zeros((2, K), np.int32), np.zeros(2, np.int32), sfb.SF_NO_COMMIT)
        raw = np.array([[int(tgt0[0][0]), 0, S.vocab + 7, 3], [-5, 1, 2, 3]], dtype=np.int32)
        d = torch.from_numpy(raw).cuda()
        sfb.sf_verify_device(eng.cache, d, None, sfb.SF_NO_COMMIT)
        sfb.sf_sync(eng.cache)
        pa, _ = sfb.sf_results_device(eng.cache)
        res = _read_device(pa, 2 + 2 * (K + 1))
        acc_d, tgt_d = res[:2], res[2:].reshape(2, K + 1)
        clamped = np.clip(raw, 0, S.vocab - 1).astype(np.int32)
        acc_h, tgt_h = sfb.sf_verify(eng.cache, clamped, None, sfb.SF_NO_COMMIT)
        assert (tgt_d == tgt_h).all()
        for b in range(2):
            M = 0
            while M < K and raw[b][M] == tgt_h[b][M]:
                M += 1
            assert int(acc_d[b]) == M, (b, acc_d, M)
        assert int(acc_d[1]) == 0 and int(acc_d[0]) <= 2
    finally:
        eng.close()


def test_kv_copies_wait_for_work_queued_on_other_streams():
    sfb = need_gpu()
    w = synth.model_weights(S, synth.seeds(2)["weights"])
    eng = sfb.Engine(S, w, n_seqs=1, capacity=128, k_max=K)
    n = 60
    shape = (S.n_layers, S.n_kv_heads, 128, S.head_dim)
    try:
        sfb.sf_prefill(eng.cache, 0, synth.prompt_ids(S.vocab, n, 77))
        rk = torch.zeros(shape, dtype=torch.int16, device="cuda")
        rv = torch.zeros_like(rk)
        torch.cuda.synchronize()
        sfb.sf_kv_read(eng.cache, 0, rk, rv, n, 128)
        assert (rk[:, :, :n] != 0).any() and (rv[:, :, :n] != 0).any()
        busy = torch.randn(4096, 4096, device="cuda")
        torch.cuda.synchronize()
        say("[kv order] read into buffers filled behind a long product on torch's stream")
        for _ in range(3):
            kg = torch.empty(shape, dtype=torch.int16, device="cuda")
            vg = torch.empty_like(kg)
            torch.mm(busy, busy)
            kg.fill_(-1)
            vg.fill_(-1)
            sfb.sf_kv_read(eng.cache, 0, kg, vg, n, 128)
            torch.cuda.synchronize()
            assert torch.equal(kg[:, :, :n], rk[:, :, :n]) and torch.equal(vg[:, :, :n], rv[:, :, :n])
        say("[kv order] write from buffers copied behind a long product on torch's stream")
        for _ in range(3):
            sk = torch.zeros(shape, dtype=torch.int16, device="cuda")
            sv = torch.zeros_like(sk)
            torch.cuda.synchronize()
            torch.mm(busy, busy)
            sk.copy_(rk)
            sv.copy_(rv)
            sfb.sf_kv_write(eng.cache, 0, sk, sv, n, 128)
            kg = torch.zeros(shape, dtype=torch.int16, device="cuda")
            vg = torch.zeros_like(kg)
            sfb.sf_kv_read(eng.cache, 0, kg, vg, n, 128)
            torch.cuda.synchronize()
            assert torch.equal(kg[:, :, :n], rk[:, :, :n]) and torch.equal(vg[:, :, :n], rv[:, :, :n])
    finally:
        eng.close()


def _read_device(addr, n):
    """n int32 values at a device address, copied to the host (hipMemcpy, device to host)."""
    import ctypes
    out = np.zeros(n, dtype=np.int32)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    assert hip.hipMemcpy(out.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(addr), n * 4, 2) == 0
    return out
