"""GPU test of the checking build (libsf_checks.so, SF_CHECKS=1), run in a child process that
loads it through SF_LIB: kernels record violated invariants in a device word instead of only
clamping.  A correct run (prefill, committing verifies of two sequences, a 16-sequence batched
pass, draft steps) records nothing; device drafts outside the vocabulary and a draft count
outside 0..k_max record exactly SF_CHECK_TOKEN | SF_CHECK_K (the pass still clamps them); the
word clears.  Inputs are the tiny decoder's, as in the other GPU tests."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import json, sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import synth
import speculative_decoding_verification_decode_amd as sfb
S = synth.TINY
K = 4
torch.cuda.set_device(0)
out = {"start": sfb.sf_debug_checks(clear=True)}
w = synth.model_weights(S, synth.seeds(1)["weights"])
eng = sfb.Engine(S, w, n_seqs=2, capacity=128, k_max=K)
try:
    for b, seed in enumerate((31, 37)):
        sfb.sf_prefill(eng.cache, b, synth.prompt_ids(S.vocab, 24, seed))
    rng = np.random.default_rng(5)
    for _ in range(6):
        d = rng.integers(0, S.vocab, size=(2, K)).astype(np.int32)
        sfb.sf_verify(eng.cache, d, np.array([K, 2], np.int32), 0)
    print("verify steps done", flush=True)
    sfb.sf_draft_step(eng.cache, 4)
    print("draft steps done", flush=True)
    out["clean"] = sfb.sf_debug_checks()
    d = torch.tensor([[1, S.vocab + 3, 2, 3], [-4, 0, 0, 0]], dtype=torch.int32, device="cuda")
    kk = torch.tensor([K + 3, 1], dtype=torch.int32, device="cuda")
    sfb.sf_verify_device(eng.cache, d, kk, sfb.SF_NO_COMMIT)
    sfb.sf_sync(eng.cache)
    out["bad"] = sfb.sf_debug_checks(clear=True)
    out["cleared"] = sfb.sf_debug_checks()
finally:
    eng.close()
eb = sfb.Engine(S, w, n_seqs=16, capacity=128, k_max=K)
try:
    for b in range(16):
        sfb.sf_prefill(eb.cache, b, synth.prompt_ids(S.vocab, 20 + b, 100 + b))
    d = np.random.default_rng(9).integers(0, S.vocab, size=(16, K)).astype(np.int32)
    sfb.sf_verify(eb.cache, d, None, 0)
    out["batched"] = sfb.sf_debug_checks()
finally:
    eb.close()
print(json.dumps(out), flush=True)
"""


def test_checking_build_records_only_violated_invariants():
    sfb = need_gpu()
    from speculative_decoding_verification_decode_amd import build as b
    assert os.path.exists(b.CHECKS_LIB), "libsf_checks.so must be built before the tests run (build.py --checks)"
    env = dict(os.environ, SF_LIB=b.CHECKS_LIB)
    say("[checks] child process on libsf_checks.so")
    r = subprocess.run([sys.executable, "-u", "-c", CHILD, ROOT], env=env, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    say(f"[checks] {res}")
    assert res["clean"] == 0 and res["batched"] == 0
    assert res["bad"] == (sfb.SF_CHECK_TOKEN | sfb.SF_CHECK_K)
    assert res["cleared"] == 0
