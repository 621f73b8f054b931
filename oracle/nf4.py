"""4-bit NormalFloat (NF4) weights for the oracle.  TEST INFRASTRUCTURE ONLY (see the package
docstring).

[ShardFlow] "The Numbers" runs the 14.7B-parameter Qwen2.5-14B with 4-bit NF4 quantization on
the same two GPUs.  The pages name the format but do not define it; the definition is the
QLoRA paper's (Dettmers et al., 2023, "4-bit NormalFloat"), restated here:

* 16 levels are quantiles of the standard normal distribution, normalised into [-1, 1], with
  an exact zero: 2^(k-1) + 1 = 9 quantiles on the positive side and 2^(k-1) = 8 on the
  negative side, taken at probabilities spaced evenly from 1/2 out to 1 - delta (delta the
  mean of 1/(2*15) and 1/(2*16)), the two zeros merged into one;
* a weight row is cut into blocks of 64 consecutive inputs; a block stores one scale (its
  absolute maximum) and one 4-bit code per weight;
* the dequantized weight is level[code] * scale.

Readings taken where the paper leaves a choice for this stack: the level table is held in
bf16 (the dtype of the layer arithmetic) and used exactly; block scales are stored as bf16;
embeddings, norms, biases and the LM head stay bf16, as in QLoRA, which quantizes only the
projection matrices.  Storage: codes row-major, two per byte, the even input in the low
nibble; scales [rows][inputs / 64].
"""
import numpy as np
import torch
from scipy.stats import norm

from .decoder import Model, round_bf16, _bf16_bits_to_f64

BLOCK = 64
QUANTIZED = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def levels():
    """The 16 NF4 levels in float64, ascending."""
    delta = 0.5 * (1.0 / (2 * 15) + 1.0 / (2 * 16))
    pos = norm.ppf(np.linspace(0.5, 1.0 - delta, 9))      # 0 and 8 positive quantiles
    neg = -norm.ppf(np.linspace(0.5, 1.0 - delta, 8))     # 0 and 7 negative quantiles
    v = np.unique(np.concatenate([pos, neg]))            # the two zeros merge
    return v / np.abs(v).max()


def table():
    """The level table as the stack uses it: each level rounded to bf16, as float64."""
    return round_bf16(torch.from_numpy(levels())).double()


def unpack_codes(packed, n_in):
    """Codes [rows][n_in] (int64) from bytes [rows][n_in / 2], even input in the low nibble."""
    p = torch.as_tensor(np.asarray(packed, dtype=np.uint8)).long()
    out = torch.empty((p.shape[0], n_in), dtype=torch.long)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequantize(packed, scale_bits, n_in):
    """float64 weights [rows][n_in]: level[code] * scale of the code's 64-input block."""
    codes = unpack_codes(packed, n_in)
    scales = _bf16_bits_to_f64(scale_bits)                # [rows][n_in / 64]
    w = table()[codes]
    return w * scales.repeat_interleave(BLOCK, dim=1)


def is_quantized(name):
    return name.split(".")[-1] in QUANTIZED


class Nf4Model(Model):
    """A decoder whose projection matrices are NF4: weights[name] is (codes, scales) for
    those, bf16 bits for the rest.  get() dequantizes on use (kept with cache=True)."""

    def get(self, name):
        if not is_quantized(name):
            return super().get(name)
        if self._cache is not None and name in self._cache:
            return self._cache[name]
        codes, scales = self.w[name]
        t = dequantize(codes, scales, codes.shape[1] * 2)
        if self._cache is not None:
            self._cache[name] = t
        return t
