"""Helpers shared by the GPU tests: parity rule, engines, and the lockstep step."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

# Parity rule: logits within max-abs 0.05 everywhere; token ids, accepted counts and
# cache positions bit-exact wherever the oracle's top-1/top-2 gap exceeds 0.1.
LOGIT_TOL = 0.05
GAP = 0.1


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_decoding_verification_decode_amd as sfb
    sfb.lib()          # fails loudly if the HIP library is missing
    return sfb


def check_targets(tgt_gpu, res_o, K):
    """Compare GPU targets / accept count with an oracle verify result.  Returns
    (#slots under the exact rule, #slots total, accepted comparable)."""
    gap = res_o["gap"].numpy()
    t_o = res_o["target"].numpy()
    exact = gap > GAP
    n_exact = int(exact.sum())
    bad = [j for j in range(len(t_o)) if exact[j] and int(tgt_gpu[j]) != int(t_o[j])]
    assert not bad, f"target mismatch at slots {bad}: gpu {list(tgt_gpu)} oracle {list(t_o)} gaps {gap}"
    return n_exact, len(t_o)


def accepted_decided(res_o, M_gpu, K):
    """True if every slot that decides M (0..min(M_o, M_gpu), capped at K) clears the gap."""
    M_o = res_o["accepted"]
    hi = min(max(M_o, M_gpu), K - 1) if K > 0 else -1
    gap = res_o["gap"].numpy()
    return all(gap[j] > GAP for j in range(0, hi + 1))


class Pair:
    """An oracle model/cache and a GPU engine with the same weights and state."""

    def __init__(self, shape, seed_cfg, capacity, k_max, n_seqs=1):
        sfb = need_gpu()
        self.sfb = sfb
        self.shape = shape
        w = synth.model_weights(shape, synth.seeds(seed_cfg)["weights"])
        self.model = oracle.Model(shape, w, cache=True)
        self.eng = sfb.Engine(shape, w, n_seqs=n_seqs, capacity=capacity, k_max=k_max)
        self.K = k_max
        self.cap = capacity

    def close(self):
        self.eng.close()
