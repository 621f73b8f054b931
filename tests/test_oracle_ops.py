"""Pins of the oracle's elementwise and attention operators (CPU only).

Each check reaches the operator through something other than its own formula:
hand-worked values, closed forms, invariants, or an independent library routine.
"""
import math

import numpy as np
import pytest
import torch

import oracle

F64 = torch.float64


# ---------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_float32_bit_rounding():
    # For float32 inputs, rounding to bf16 is also done by torch's float->bf16
    # conversion (round to nearest even on the bit pattern): two independent routes.
    rng = np.random.default_rng(0)
    x32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(F64)
    got = oracle.round_bf16(torch.from_numpy(x32).to(F64))
    assert torch.equal(got, want)


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even neighbour is 1.
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: the even one is 1 + 2^-6.
    x = torch.tensor([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 1 + 2**-8 + 2**-30, 0.0], dtype=F64)
    want = torch.tensor([1.0, 1 + 2**-6, -1.0, 1 + 2**-7, 0.0], dtype=F64)
    assert torch.equal(oracle.round_bf16(x), want)


def test_round_bf16_single_rounding_from_double():
    # A double just above a bf16 tie must round up; rounding via float32 first
    # would land on the tie and round down to even.
    x = torch.tensor([1 + 2**-8 + 2**-40], dtype=F64)
    assert oracle.round_bf16(x).item() == 1 + 2**-7


# ---------------------------------------------------------------- RMSNorm

def test_rms_norm_hand_example():
    x = torch.tensor([[3.0, 4.0]], dtype=F64)
    g = torch.tensor([1.0, 2.0], dtype=F64)
    rms = math.sqrt((9 + 16) / 2)
    y = oracle.rms_norm(x, g, 0.0)
    assert torch.allclose(y, torch.tensor([[3 / rms, 8 / rms]], dtype=F64), atol=1e-15)


def test_rms_norm_invariants_and_library():
    torch.manual_seed(0)
    x = torch.randn(7, 96, dtype=F64) * 5
    ones = torch.ones(96, dtype=F64)
    y = oracle.rms_norm(x, ones, 0.0)
    assert torch.allclose((y * y).mean(-1), torch.ones(7, dtype=F64), atol=1e-12)
    assert torch.allclose(oracle.rms_norm(x * 37.5, ones, 0.0), y, atol=1e-12)
    g = torch.randn(96, dtype=F64)
    lib = torch.nn.functional.rms_norm(x, (96,), weight=g, eps=1e-6)
    assert torch.allclose(oracle.rms_norm(x, g, 1e-6), lib, atol=1e-12)


def test_rms_norm_eps_matters_for_tiny_rows():
    x = torch.full((1, 4), 1e-4, dtype=F64)
    y = oracle.rms_norm(x, torch.ones(4, dtype=F64), 1e-6)
    assert torch.allclose(y, torch.full((1, 4), 1e-4 / math.sqrt(1e-8 + 1e-6), dtype=F64))


# ---------------------------------------------------------------- RoPE

def test_rope_angles_closed_form():
    th = oracle.rope_angles([0, 1, 5], 4, 10000.0)
    want = torch.tensor([[0, 0], [1, 0.01], [5, 0.05]], dtype=F64)
    assert torch.allclose(th, want, atol=1e-15)


def test_rope_identity_at_zero_and_norm_preserved():
    torch.manual_seed(1)
    x = torch.randn(3, 2, 8, dtype=F64)
    th0 = oracle.rope_angles([0, 0, 0], 8, 10000.0)
    assert torch.equal(oracle.rope(x, th0), x)
    th = oracle.rope_angles([3, 100, 7777], 8, 10000.0)
    y = oracle.rope(x, th)
    pn = lambda t: t[..., :4] ** 2 + t[..., 4:] ** 2
    assert torch.allclose(pn(y), pn(x), atol=1e-12)


def test_rope_is_complex_rotation():
    # Pair (x_i, x_{i+d/2}) as the complex number x_i + j x_{i+d/2}; RoPE multiplies it by exp(j theta_i).
    torch.manual_seed(2)
    d = 16
    x = torch.randn(5, 3, d, dtype=F64)
    pos = [0, 1, 2, 31, 4095]
    th = oracle.rope_angles(pos, d, 1e6)
    z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * torch.polar(torch.ones_like(th), th)[:, None, :]
    want = torch.cat([z.real, z.imag], dim=-1)
    assert torch.allclose(oracle.rope(x, th), want, atol=1e-12)


def test_rope_quarter_turn():
    # d=2, position p rotates (1, 0) by p radians: p = pi/2 is not an integer, so use
    # base**0 = 1 and positions 1, 2: (cos p, sin p).
    x = torch.tensor([[[1.0, 0.0]], [[1.0, 0.0]]], dtype=F64)
    th = oracle.rope_angles([1, 2], 2, 10000.0)
    y = oracle.rope(x, th)
    want = torch.tensor([[[math.cos(1), math.sin(1)]], [[math.cos(2), math.sin(2)]]], dtype=F64)
    assert torch.allclose(y, want, atol=1e-15)


def test_rope_relative_position():
    torch.manual_seed(3)
    d = 64
    q = torch.randn(1, 1, d, dtype=F64)
    k = torch.randn(1, 1, d, dtype=F64)
    for (p, r, delta) in [(10, 3, 100), (500, 499, 7000), (0, 0, 12345)]:
        a = (oracle.rope(q, oracle.rope_angles([p], d, 1e6)) * oracle.rope(k, oracle.rope_angles([r], d, 1e6))).sum()
        b = (oracle.rope(q, oracle.rope_angles([p + delta], d, 1e6)) *
             oracle.rope(k, oracle.rope_angles([r + delta], d, 1e6))).sum()
        assert abs(a - b) <= 1e-9 * max(1.0, abs(a))


# ---------------------------------------------------------------- SwiGLU

def test_silu_and_swiglu():
    z = torch.linspace(-30, 30, 601, dtype=F64)
    assert torch.allclose(oracle.silu(z), torch.nn.functional.silu(z), atol=1e-14)
    assert oracle.silu(torch.tensor([0.0], dtype=F64)).item() == 0.0
    assert abs(oracle.silu(torch.tensor([50.0], dtype=F64)).item() - 50.0) < 1e-15 * 50 + 1e-18
    g = torch.tensor([1.0, -2.0], dtype=F64)
    u = torch.tensor([3.0, 5.0], dtype=F64)
    want = torch.tensor([3.0 / (1 + math.exp(-1.0)), 5.0 * -2.0 / (1 + math.exp(2.0))], dtype=F64)
    assert torch.allclose(oracle.swiglu(g, u), want, atol=1e-14)


# ---------------------------------------------------------------- attention

def _attn(q, k, v, pos):
    return oracle.causal_gqa_attention(q, k, v, pos)


def test_attention_single_key_returns_value():
    torch.manual_seed(4)
    q = torch.randn(1, 4, 8, dtype=F64)
    k = torch.randn(2, 1, 8, dtype=F64)
    v = torch.randn(2, 1, 8, dtype=F64)
    out = _attn(q, k, v, [0])
    assert torch.allclose(out[0, :2], v[0, 0].expand(2, 8))
    assert torch.allclose(out[0, 2:], v[1, 0].expand(2, 8))


def test_attention_identical_keys_average_values():
    torch.manual_seed(5)
    q = torch.randn(1, 2, 8, dtype=F64)
    k = torch.randn(1, 1, 8, dtype=F64).expand(1, 6, 8).contiguous()
    v = torch.randn(1, 6, 8, dtype=F64)
    out = _attn(q, k, v, [5])
    assert torch.allclose(out[0], v[0].mean(0).expand(2, 8), atol=1e-14)


def test_attention_is_causal():
    torch.manual_seed(6)
    q = torch.randn(3, 2, 8, dtype=F64)
    k = torch.randn(1, 10, 8, dtype=F64)
    v = torch.randn(1, 10, 8, dtype=F64)
    base = _attn(q, k, v, [4, 5, 6])
    k2, v2 = k.clone(), v.clone()
    k2[:, 6:] += 100.0
    v2[:, 6:] -= 50.0
    alt = _attn(q, k2, v2, [4, 5, 6])
    assert torch.equal(base[:2], alt[:2])
    assert not torch.allclose(base[2], alt[2])


@pytest.mark.parametrize("n_q,n_kv", [(4, 4), (4, 2), (28, 4), (14, 2)])
def test_attention_matches_library_sdpa(n_q, n_kv):
    torch.manual_seed(7)
    n, d = 9, 32
    q = torch.randn(n, n_q, d, dtype=F64)
    k = torch.randn(n_kv, n, d, dtype=F64)
    v = torch.randn(n_kv, n, d, dtype=F64)
    got = _attn(q, k, v, list(range(n)))
    rep = n_q // n_kv
    kk = k.repeat_interleave(rep, dim=0)
    vv = v.repeat_interleave(rep, dim=0)
    want = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2), kk, vv, is_causal=True).permute(1, 0, 2)
    assert torch.allclose(got, want, atol=1e-12)


def test_attention_with_prefix_matches_library():
    # Rows at positions L..L+T-1 over a cache of L+T keys: equal to the last T rows
    # of full causal attention over L+T queries.
    torch.manual_seed(8)
    L, T, n_q, n_kv, d = 20, 5, 6, 2, 16
    qa = torch.randn(L + T, n_q, d, dtype=F64)
    k = torch.randn(n_kv, L + T, d, dtype=F64)
    v = torch.randn(n_kv, L + T, d, dtype=F64)
    got = _attn(qa[L:], k, v, list(range(L, L + T)))
    kk = k.repeat_interleave(n_q // n_kv, 0)
    vv = v.repeat_interleave(n_q // n_kv, 0)
    want = torch.nn.functional.scaled_dot_product_attention(
        qa.permute(1, 0, 2), kk, vv, is_causal=True).permute(1, 0, 2)[L:]
    assert torch.allclose(got, want, atol=1e-12)
