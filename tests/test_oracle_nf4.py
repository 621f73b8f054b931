"""Pins of the oracle's NF4 weights (CPU only): the level table against the definition of the
4-bit NormalFloat format (QLoRA paper, "4-bit NormalFloat") and its published values, the
dequantization against hand-built examples, and the NF4 stack against the pinned bf16 stack."""
import numpy as np
import pytest
import torch
from scipy.stats import norm

import oracle
import synth
from oracle import nf4


def test_levels_shape_of_the_format():
    v = nf4.levels()
    assert len(v) == 16 and np.all(np.diff(v) > 0)
    assert v[0] == -1.0 and v[-1] == 1.0
    assert np.sum(v == 0.0) == 1 and np.sum(v < 0) == 7 and np.sum(v > 0) == 8


def test_levels_are_normal_quantiles_at_even_probabilities():
    """Mapped back through the normal distribution function (not its inverse, which builds
    them), the positive levels sit at 9 evenly spaced probabilities from 1/2 to 1 - delta and
    the negative ones at 8 from 1/2 down to delta."""
    v = nf4.levels()
    delta = 0.5 * (1 / 30 + 1 / 32)
    zmax = norm.isf(delta)
    p_pos = norm.cdf(v[v >= 0] * zmax)
    p_neg = norm.cdf(v[v <= 0] * zmax)
    assert np.allclose(p_pos, np.linspace(0.5, 1 - delta, 9), atol=1e-12)
    assert np.allclose(p_neg, np.linspace(delta, 0.5, 8), atol=1e-12)


def test_levels_match_published_table():
    """The NF4 values as published with the format (four decimals)."""
    pub = [-1.0, -0.6962, -0.5251, -0.3949, -0.2844, -0.1848, -0.0911, 0.0,
           0.0796, 0.1609, 0.2461, 0.3379, 0.4407, 0.5626, 0.7230, 1.0]
    assert np.abs(nf4.levels() - np.array(pub)).max() < 1.5e-4


def test_table_is_bf16_of_levels():
    t = nf4.table().numpy()
    assert np.abs(t - nf4.levels()).max() < 2 ** -8            # one bf16 rounding, |v| <= 1
    bits = torch.from_numpy(t.astype(np.float32)).view(torch.int32).numpy()
    assert np.all(bits & 0xFFFF == 0)                         # exactly representable in bf16


def test_dequantize_hand_example():
    """Two rows of 128 inputs: nibble order, the 64-input block boundary, per-row scales."""
    t = nf4.table().numpy()
    codes = np.zeros((2, 128), dtype=np.int64)
    codes[0, :] = np.arange(128) % 16
    codes[1, :] = 15 - np.arange(128) % 16
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sc = np.array([[0.5, 2.0], [-0.25, 1.0]], dtype=np.float32)
    sbits = (sc.view(np.uint32) >> 16).astype(np.uint16)      # exact in bf16
    w = nf4.dequantize(packed, sbits, 128).numpy()
    assert w.shape == (2, 128)
    assert w[0, 0] == t[0] * 0.5 and w[0, 1] == t[1] * 0.5 and w[0, 63] == t[15] * 0.5
    assert w[0, 64] == t[0] * 2.0 and w[0, 127] == t[15] * 2.0
    assert w[1, 0] == t[15] * -0.25 and w[1, 64] == t[15] * 1.0
    ref = np.array([[t[c] for c in row] for row in codes]) * np.repeat(sc, 64, axis=1)
    assert np.array_equal(w, ref)


def test_nf4_stack_equals_bf16_stack_on_exact_weights():
    """With power-of-two scales every dequantized weight is a bf16 value, so the NF4 stack must
    give exactly the bf16 stack's logits when that stack holds the same weights as bf16."""
    S = synth.TINY
    w = synth.nf4_model_weights(S, 17)
    rng = np.random.default_rng(3)
    wb = {}
    for name, val in w.items():
        if nf4.is_quantized(name):
            codes, _ = val
            e = rng.integers(-8, -4, size=(codes.shape[0], codes.shape[1] * 2 // 64))
            sbits = ((e + 127) << 7).astype(np.uint16)        # bf16 bits of 2^e
            w[name] = (codes, sbits)
            deq = nf4.dequantize(codes, sbits, codes.shape[1] * 2).float()
            wb[name] = (deq.view(torch.int32) >> 16).numpy().astype(np.uint16)
            assert torch.equal(torch.from_numpy(wb[name].astype(np.int32) << 16).view(torch.float32).double(),
                               deq.double())
        else:
            wb[name] = val
    prompt = synth.prompt_ids(S.vocab, 12, 9)
    za = oracle.prefill(nf4.Nf4Model(S, w, cache=True), oracle.KVCache(S, 16), prompt)
    zb = oracle.prefill(oracle.Model(S, wb, cache=True), oracle.KVCache(S, 16), prompt)
    assert torch.equal(za, zb)


def test_synthetic_nf4_codes_and_scales():
    codes, scales = synth.nf4_tensor((256, 512), 5, "t")
    assert codes.shape == (256, 256) and codes.dtype == np.uint8
    assert scales.shape == (256, 8) and scales.dtype == np.uint16
    n = np.bincount(np.concatenate([(codes & 15).ravel(), (codes >> 4).ravel()]), minlength=16)
    assert n.min() > 0.9 * n.mean()                           # codes uniform over the levels
    s = torch.from_numpy(scales.astype(np.int32) << 16).view(torch.float32).numpy()
    assert 0.02 * 1.8 < np.median(s) < 0.02 * 2.8             # median |max| of 64 normals ~ 2.4
