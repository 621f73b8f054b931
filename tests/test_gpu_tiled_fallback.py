"""GPU test: the batched passes' two GEMM kernels give the same bits.  Passes of more than 64
rows run the LDS-staged kernel for the split O and down, the gate/up and the LM head, and the
row-group kernel for every projection when SF_TILED=0 (read once per process, so that side runs
in a child process).  Both walk each output's k range in the compact kernel's chunks and add
the chunk results in the same order, so the logits of a tiny 16-sequence pass (80 rows) and of
a 512-token prefill must agree bit for bit.  At the tiny shape the gate/up (64 blocks of 16 k
tiles), the LM head (128 blocks) and the down projection (two splits of 32 k tiles) take the
staged kernel; the O projection does with SF_SP_O=2."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import synth
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import synth
import speculative_decoding_verification_decode_amd as sfb
S = synth.TINY
B, K, CAP = 16, 4, 1024
torch.cuda.set_device(0)
w = synth.model_weights(S, synth.seeds(5)["weights"])
eng = sfb.Engine(S, w, n_seqs=B, capacity=CAP, k_max=K)
try:
    rng = np.random.default_rng(4242)
    for b in range(B):
        sfb.sf_prefill(eng.cache, b, synth.prompt_ids(S.vocab, int(rng.integers(20, 60)), 500 + b))
    nxt = sfb.sf_prefill(eng.cache, 0, synth.prompt_ids(S.vocab, 600, 77))   # 512 + 88 positions
    d = rng.integers(0, S.vocab, size=(B, K)).astype(np.int32)
    logits = torch.empty((B * (K + 1), S.vocab), dtype=torch.float32, device="cuda")
    sfb.sf_verify(eng.cache, d, None, sfb.SF_DEBUG_LOGITS | sfb.SF_NO_COMMIT, dev_out=logits)
    torch.cuda.synchronize()
    np.save(sys.argv[2], logits.cpu().numpy())
    with open(sys.argv[2] + ".next", "w") as f:
        f.write(str(int(nxt)))
finally:
    eng.close()
print("child done", flush=True)
"""


def _run(tmp_path, tag, tiled):
    env = dict(os.environ)
    env["SF_TILED"] = "1" if tiled else "0"
    env["SF_SP_O"] = "2"   # the tiny shape's O projection is not split by default; split it so that it is staged too
    out = str(tmp_path / f"{tag}.npy")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, out], env=env, capture_output=True, text=True, timeout=240)
    say(r.stdout.strip()[-200:])
    assert r.returncode == 0, r.stderr[-2000:]
    return np.load(out), open(out + ".next").read()


def test_tiled_and_row_group_kernels_agree_bitwise(tmp_path):
    need_gpu()
    a, na = _run(tmp_path, "tiled", True)
    b, nb = _run(tmp_path, "rowgroup", False)
    say(f"[tiled fallback] logits {a.shape}, next tokens {na} / {nb}")
    assert na == nb
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
