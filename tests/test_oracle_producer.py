"""Pins of the oracle's producer step (RMS-normalised Lc, rotary-embedded Rc)
against closed forms, invariants and independent library routines.

Page: "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
(colibri PR #299), commit message, attention_rows item: the producer
quantizes the fresh normalised and rotary-embedded latent row.  The page does
not give the forms; the readings are RMS normalisation with a per-channel
weight and eps inside the square root, and rotation of the interleaved pairs
(2i, 2i+1) by fl32(fl32(pos) * fl32(theta^(-2i/64))).
"""
import numpy as np
import pytest

import oracle

KL, KR = 512, 64


def rows(seed, n, scale=1.0):
    return (np.random.default_rng(seed).standard_normal((n, KL + KR)) * scale).astype(np.float32)


def run(x, w=None, eps=1e-6, pos=None, theta=10000.0):
    w = np.ones(KL, np.float32) if w is None else w
    pos = np.zeros(x.shape[0], np.int64) if pos is None else pos
    return oracle.norm_rope_rows(x, w, eps, pos, theta)


def test_unit_weight_gives_unit_rms():
    y = run(rows(1, 16), eps=0.0)
    rms = np.sqrt((y[:, :KL].astype(np.float64) ** 2).mean(axis=1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-6)


def test_lc_matches_torch_rms_norm():
    """torch's rms_norm (library routine) in f64 with the same weight and eps."""
    torch = pytest.importorskip("torch")
    x = rows(2, 32, scale=3.0)
    w = np.random.default_rng(3).uniform(0.5, 1.5, KL).astype(np.float32)
    y = run(x, w=w, eps=1e-3)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x[:, :KL]).double(), (KL,),
                                       weight=torch.from_numpy(w).double(), eps=1e-3).numpy()
    np.testing.assert_allclose(y[:, :KL], ref, rtol=2e-7, atol=0)


def test_eps_inside_the_root():
    """A row of tiny values is dominated by eps: y = w x / sqrt(mean x^2 + eps)."""
    x = np.full((1, KL + KR), 1e-4, np.float32)
    y = run(x, eps=1.0)
    np.testing.assert_allclose(y[0, :KL], 1e-4 / np.sqrt(1e-8 + 1.0), rtol=1e-6)
    z = run(np.zeros((1, KL + KR), np.float32), eps=1e-6)
    assert np.all(z == 0)


def test_power_of_two_scaling_is_invisible():
    x = rows(4, 8)
    a = run(x, eps=0.0)
    b = run(x * np.float32(2.0 ** -20), eps=0.0)
    np.testing.assert_array_equal(a[:, :KL], b[:, :KL])


def test_position_zero_is_identity_on_rc():
    x = rows(5, 8)
    y = run(x, pos=np.zeros(8, np.int64))
    np.testing.assert_array_equal(y[:, KL:], x[:, KL:])


def test_rotation_matches_complex_multiplication():
    """numpy complex product (x_2i + i x_2i+1) e^{i a_i} with the reading's f32 angles."""
    x = rows(6, 20)
    pos = np.random.default_rng(7).integers(0, 262144, 20).astype(np.int64)
    y = run(x, pos=pos)
    f = np.array([np.float32(10000.0 ** (-2.0 * i / KR)) for i in range(KR // 2)], np.float32)
    ang = (pos.astype(np.float32)[:, None] * f[None, :]).astype(np.float32)
    z = (x[:, KL::2].astype(np.float64) + 1j * x[:, KL + 1::2]) * np.exp(1j * ang.astype(np.float64))
    np.testing.assert_allclose(y[:, KL::2], z.real, rtol=0, atol=2e-6)
    np.testing.assert_allclose(y[:, KL + 1::2], z.imag, rtol=0, atol=2e-6)


def test_pair_norms_are_preserved():
    x = rows(8, 16)
    y = run(x, pos=np.arange(16, dtype=np.int64) * 9973)
    n0 = np.hypot(x[:, KL::2].astype(np.float64), x[:, KL + 1::2])
    n1 = np.hypot(y[:, KL::2].astype(np.float64), y[:, KL + 1::2])
    np.testing.assert_allclose(n1, n0, rtol=1e-6)


def test_first_pair_at_position_one_turns_by_one_radian():
    """Pair 0 has frequency theta^0 = 1: (1, 0) at position 1 becomes (cos 1, sin 1);
    pair 31 turns by theta^(-62/64)."""
    x = np.zeros((1, KL + KR), np.float32)
    x[0, KL] = 1.0
    x[0, KL + 62] = 1.0
    y = run(x, pos=np.array([1]))
    assert abs(y[0, KL] - np.cos(1.0)) < 1e-7 and abs(y[0, KL + 1] - np.sin(1.0)) < 1e-7
    a = float(np.float32(10000.0 ** (-62.0 / 64.0)))
    assert abs(y[0, KL + 62] - np.cos(a)) < 1e-7 and abs(y[0, KL + 63] - np.sin(a)) < 1e-7


def test_scores_depend_on_relative_position_only():
    """<rope(q, m), rope(k, n)> is unchanged when both positions shift by the same d."""
    q, k = rows(9, 1), rows(10, 1)
    dots = []
    for m, n in ((37, 5), (137, 105), (1037, 1005)):
        a = run(q, pos=np.array([m]))[0, KL:].astype(np.float64)
        b = run(k, pos=np.array([n]))[0, KL:].astype(np.float64)
        dots.append(a @ b)
    np.testing.assert_allclose(dots, dots[0], rtol=0, atol=5e-4 * np.abs(dots[0]) + 5e-5)
