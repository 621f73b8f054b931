"""The no-allocation verify (sf_verify_device_static) against the entry point it is a variant of
(sf_verify_device), through the C ABI, on the two-layer decoder.

Two caches of one model start from the same state; one runs sf_verify_device (its own
scratch), the other sf_verify_device_static (the library's static device array).  Results,
committed lengths, pending tokens and every K/V byte of the pass must be identical.  Two calls
in a row, the second with a smaller input (fewer sequences, fewer drafts, a smaller cache),
then the first shape again, so stale contents of the shared array cannot leak into a result.
A pass whose working memory exceeds the array is refused before any work.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_targets, need_gpu, say

pytestmark = pytest.mark.gpu

S = synth.TINY


def _kv(sfb, cache, seq, n, cap):
    shape = (S.n_layers, S.n_kv_heads, cap, S.head_dim)
    k = torch.zeros(shape, dtype=torch.int16, device="cuda")
    v = torch.zeros_like(k)
    sfb.sf_kv_read(cache, seq, k, v, n, cap)
    return k, v


def _pair_run(sfb, model, n_seqs, k_max, cap, prompts, drafts, ks, flags):
    """Fresh caches A (sf_verify_device) and B (the static variant) from the same prompts;
    one pass each; returns both results and states."""
    a = sfb.sf_cache_alloc(model, n_seqs, cap, k_max)
    b = sfb.sf_cache_alloc(model, n_seqs, cap, k_max)
    try:
        for s, p in enumerate(prompts):
            assert sfb.sf_prefill(a, s, p) == sfb.sf_prefill(b, s, p)
        d = torch.from_numpy(np.ascontiguousarray(drafts, dtype=np.int32)).cuda()
        kk = torch.from_numpy(np.asarray(ks, dtype=np.int32)).cuda()
        res = torch.full((n_seqs + n_seqs * (k_max + 1),), -7, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()   # the fill runs on torch's stream, the passes on the model stream
        sfb.sf_verify_device(a, d, kk, flags)
        sfb.sf_verify_device_static(b, d, kk, flags, res)
        sfb.sf_sync(a)
        sfb.sf_sync(b)
        # Results of A: accepted then targets, contiguous at its fixed result buffer.
        pa, _ = sfb.sf_results_device(a)
        torch.cuda.synchronize()
        ra = _read_device(pa, res.numel())
        states = []
        for s in range(n_seqs):
            sa, sb = sfb.sf_cache_state(a, s), sfb.sf_cache_state(b, s)
            n = min(cap, sa[0] + k_max + 1)        # every position the pass wrote, committed or not
            ka, va = _kv(sfb, a, s, n, cap)
            kb, vb = _kv(sfb, b, s, n, cap)
            torch.cuda.synchronize()
            states.append((sa, sb, torch.equal(ka, kb) and torch.equal(va, vb)))
        return ra, res.cpu().numpy(), states
    finally:
        sfb.sf_cache_free(a)
        sfb.sf_cache_free(b)


def _read_device(addr, n):
    """n int32 values at a device address, copied to the host (hipMemcpy, device to host)."""
    import ctypes
    out = np.zeros(n, dtype=np.int32)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    assert hip.hipMemcpy(out.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(addr), n * 4, 2) == 0
    return out


def test_static_verify_equals_device_verify_twice_second_smaller():
    sfb = need_gpu()
    w = synth.model_weights(S, synth.seeds(1)["weights"])
    eng = sfb.Engine(S, w, n_seqs=1, capacity=64, k_max=2)
    m = oracle.Model(S, w, cache=True)
    try:
        rng = np.random.default_rng(31)
        cases = [  # (n_seqs, k_max, capacity, flags): the second smaller than the first
            (3, 6, 300, 0),
            (1, 2, 64, 0),
            (3, 6, 300, sfb.SF_NO_COMMIT),
        ]
        for i, (B, Kx, cap, flags) in enumerate(cases):
            prompts = [synth.prompt_ids(S.vocab, int(rng.integers(20, 60)), 900 + 10 * i + s) for s in range(B)]
            drafts = rng.integers(0, S.vocab, size=(B, Kx)).astype(np.int32)
            ks = rng.integers(0, Kx + 1, size=B).astype(np.int32)
            say(f"[no-alloc] call {i}: n_seqs {B}, k_max {Kx}, capacity {cap}, k {ks.tolist()}")
            ra, rb, states = _pair_run(sfb, eng.model, B, Kx, cap, prompts, drafts, ks, flags)
            assert (ra == rb).all(), (ra, rb)
            for s, (sa, sb, kv_same) in enumerate(states):
                assert sa == sb, (s, sa, sb)
                assert kv_same, s
            # And the oracle, for the record: the targets where its gap rule applies.
            for s in range(B):
                c = oracle.KVCache(S, cap)
                oracle.prefill(m, c, prompts[s])
                r = oracle.verify(m, c, drafts[s], int(ks[s]), commit=False)
                check_targets(rb[B + s * (Kx + 1):B + (s + 1) * (Kx + 1)], r, Kx)
    finally:
        eng.close()


def test_static_verify_refuses_a_pass_larger_than_the_array():
    sfb = need_gpu()
    w = synth.model_weights(S, synth.seeds(1)["weights"])
    eng = sfb.Engine(S, w, n_seqs=1, capacity=64, k_max=2)
    big = sfb.sf_cache_alloc(eng.model, 32, 16384, 15)
    try:
        d = torch.zeros((32, 15), dtype=torch.int32, device="cuda")
        res = torch.zeros(32 + 32 * 16, dtype=torch.int32, device="cuda")
        with pytest.raises(sfb.SFError) as e:
            sfb.sf_verify_device_static(big, d, None, 0, res)
        assert e.value.code == sfb.SF_E_CAPACITY and "static" in str(e.value)
        assert sfb.sf_cache_state(big, 0) == (0, 0)
    finally:
        sfb.sf_cache_free(big)
        eng.close()
