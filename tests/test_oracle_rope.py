"""Pins for the oracle's Chunked RoPE rotation (CPU only).

The rotation R(p) is pinned by
  * hand-derived closed forms that fix the pairing (i with i + D/2), the sign
    of the sine terms and the frequency law theta^(-2i/D);
  * the complex-number form of RoPE (z_i = x_i + j x_{i+D/2} times e^{j p w_i}),
    computed with numpy's complex exp and multiply;
  * Hugging Face transformers' Llama rotary embedding (a library routine, in
    fp32, so a looser tolerance) for the conventions the served models use;
  * Theorem 6 as the pages describe it (re-rotation is exact: attention
    scores depend only on relative position), in fp64 within 1e-5;
  * invariants: per-pair norm preservation, R(0) = I (bit-exact through bf16),
    R(a)R(b) = R(a+b), R(-p)R(p) = I.
"""

import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import bf16_to_f64, expected_rows, f64_to_bf16, rope_inv_freq, rope_rotate


# ---------------------------------------------------------------- closed forms

def test_inv_freq_closed_form():
    w = rope_inv_freq(128, 5e5)
    assert w[0] == 1.0
    assert w.size == 64
    assert math.isclose(w[1], 5e5 ** (-2 / 128), rel_tol=1e-15)
    assert math.isclose(w[-1], 5e5 ** (-126 / 128), rel_tol=1e-15)
    assert np.allclose(w[1:] / w[:-1], 5e5 ** (-2 / 128), rtol=1e-14, atol=0)


@pytest.mark.parametrize("x, p, expect", [
    # D = 4, theta = 1e4: w_0 = 1, w_1 = 1e4^(-1/2) = 0.01.  Element 0 pairs
    # with element 2, element 1 with element 3.
    ([1, 0, 0, 0], 1, [math.cos(1), 0, math.sin(1), 0]),
    ([0, 0, 1, 0], 1, [-math.sin(1), 0, math.cos(1), 0]),
    ([0, 1, 0, 0], 1, [0, math.cos(0.01), 0, math.sin(0.01)]),
    ([0, 0, 0, 1], 1, [0, -math.sin(0.01), 0, math.cos(0.01)]),
    ([0, 1, 0, 0], 100, [0, math.cos(1.0), 0, math.sin(1.0)]),
    ([2, 0, 0, 0], 3, [2 * math.cos(3), 0, 2 * math.sin(3), 0]),
])
def test_closed_form_pairs(x, p, expect):
    y = rope_rotate(np.array(x, np.float64), p, 1e4)
    assert np.allclose(y, expect, rtol=0, atol=1e-15)


def test_d2_is_complex_multiplication():
    # D = 2 has one frequency, w_0 = theta^0 = 1: R(p) is multiplication by e^{jp}
    rng = np.random.default_rng(3)
    for _ in range(200):
        x = rng.standard_normal(2)
        p = int(rng.integers(0, 100000))
        z = complex(x[0], x[1]) * complex(math.cos(p), math.sin(p))
        y = rope_rotate(x, p, 5e5)
        assert abs(y[0] - z.real) <= 1e-12 and abs(y[1] - z.imag) <= 1e-12


@pytest.mark.parametrize("theta", [5e5, 1e6])
def test_complex_form(theta):
    rng = np.random.default_rng(5)
    D = 128
    x = rng.standard_normal((64, D))
    p = rng.integers(0, 4096, 64)
    w = np.exp(-(2.0 * np.arange(D // 2) / D) * np.log(theta))
    z = (x[:, : D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * p[:, None] * w)
    y = rope_rotate(x, p, theta)
    assert np.allclose(y[:, : D // 2], z.real, rtol=0, atol=1e-11)
    assert np.allclose(y[:, D // 2:], z.imag, rtol=0, atol=1e-11)


def test_matches_transformers_llama_rotary():
    torch = pytest.importorskip("torch")
    tr = pytest.importorskip("transformers")
    from transformers.models.llama import modeling_llama as ml
    cfg = tr.LlamaConfig(hidden_size=1024, num_attention_heads=8, num_key_value_heads=8,
                         head_dim=128, max_position_embeddings=8192,
                         rope_parameters={"rope_type": "default", "rope_theta": 500000.0})
    rot = ml.LlamaRotaryEmbedding(cfg)
    rng = np.random.default_rng(9)
    S, H, D = 300, 8, 128
    pos = np.sort(rng.choice(4096, S, replace=False))
    k = rng.standard_normal((1, H, S, D)).astype(np.float32)
    kt = torch.from_numpy(k)
    cos, sin = rot(kt, torch.from_numpy(pos[None, :]).long())
    _, k_hf = ml.apply_rotary_pos_emb(kt, kt, cos, sin, unsqueeze_dim=1)
    ours = rope_rotate(k[0].astype(np.float64), pos[None, :], 5e5)
    # transformers works in fp32 (fp32 frequencies and angles): the angle error
    # grows like p * 2^-24, about 3e-4 rad at p = 4096.
    assert np.max(np.abs(k_hf[0].double().numpy() - ours)) < 5e-3


# ---------------------------------------------------------------- Theorem 6

@settings(max_examples=300, deadline=None)
@given(D=st.sampled_from([2, 64, 128]), theta=st.sampled_from([5e5, 1e6]),
       m=st.integers(0, 200000), n=st.integers(0, 200000), seed=st.integers(0, 2**31))
def test_theorem6_relative_position(D, theta, m, n, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)
    lhs = float(np.dot(rope_rotate(q, m, theta), rope_rotate(k, n, theta)))
    rhs = float(np.dot(q, rope_rotate(k, n - m, theta)))
    assert abs(lhs - rhs) <= 1e-5


# ---------------------------------------------------------------- invariants

def test_norm_preserved_per_pair():
    rng = np.random.default_rng(13)
    D = 128
    x = rng.standard_normal((500, D))
    p = rng.integers(0, 100000, 500)
    y = rope_rotate(x, p, 1e6)
    nx = np.hypot(x[:, :64], x[:, 64:])
    ny = np.hypot(y[:, :64], y[:, 64:])
    assert np.allclose(nx, ny, rtol=1e-14, atol=0)


def test_position_zero_is_identity_through_bf16():
    rng = np.random.default_rng(17)
    bits = f64_to_bf16(rng.standard_normal((40, 8, 128)))
    k, v = expected_rows(bits, bits, np.zeros(40, np.int64), 5e5)
    assert np.array_equal(k, bits)
    assert np.array_equal(v, bits)


def test_composition_and_inverse():
    rng = np.random.default_rng(19)
    x = rng.standard_normal((100, 128))
    a = rng.integers(0, 5000, 100)
    b = rng.integers(0, 5000, 100)
    y = rope_rotate(rope_rotate(x, a, 5e5), b, 5e5)
    assert np.allclose(y, rope_rotate(x, a + b, 5e5), rtol=0, atol=1e-11)
    assert np.allclose(rope_rotate(rope_rotate(x, a, 5e5), -a, 5e5), x, rtol=0, atol=1e-11)


def test_bf16_output_within_half_ulp_of_exact():
    # expected_rows rounds the fp64 rotation once: every output element is the
    # nearest bf16 to the fp64 value, so it is within half a bf16 spacing.
    rng = np.random.default_rng(23)
    bits = f64_to_bf16(rng.standard_normal((64, 8, 128)))
    pos = rng.integers(0, 3000, 64)
    k, _ = expected_rows(bits, bits, pos, 5e5)
    exact = rope_rotate(bf16_to_f64(bits), pos[:, None], 5e5)
    got = bf16_to_f64(k)
    _, e = np.frexp(exact)
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    assert np.all(np.abs(got - exact) <= spacing / 2)
