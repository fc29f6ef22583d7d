"""Pins of the oracle's non-absorbed projection of cache rows (dequantized Lc
times the kv_b weight; Rc read through the decode table).

Page: "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
(colibri PR #299), commit message, attention_rows item: the non-absorbed
prefill dequantizes Lc into an f32 staging row for the kv_b matmul and reads
Rc via the decode table.
"""
import numpy as np
import pytest

import oracle

KL, KR, D = 512, 64, 576


def cache(seed, n):
    x = np.random.default_rng(seed).standard_normal((n, D)).astype(np.float32)
    return oracle.quantize_rows(x)


def bf16(a):
    """Round-to-nearest-even bf16 bits of f32 values (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_value(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_identity_weight_returns_dequantized_lc():
    c, s = cache(1, 24)
    w = bf16(np.eye(KL, dtype=np.float32))
    out, rope = oracle.project_rows(c, s, w)
    dq = oracle.decode(c)
    np.testing.assert_array_equal(out, dq[:, :KL] * s[:, :1].astype(np.float64))
    np.testing.assert_array_equal(rope, dq[:, KL:] * s[:, 1:].astype(np.float64))


def test_matches_numpy_matmul_of_dequantized_rows():
    """numpy's matmul (a library routine) on the dequantized rows and bf16 weights."""
    c, s = cache(2, 40)
    w = bf16(np.random.default_rng(3).standard_normal((96, KL)).astype(np.float32) * 0.05)
    out, _ = oracle.project_rows(c, s, w)
    x = oracle.decode(c)[:, :KL] * s[:, :1].astype(np.float64)
    ref = x @ bf16_value(w).T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_single_column_is_a_dot_product_and_rows_are_independent():
    c, s = cache(4, 5)
    w = bf16(np.random.default_rng(5).standard_normal((3, KL)).astype(np.float32))
    out, _ = oracle.project_rows(c, s, w)
    for m in (0, 4):
        for n in range(3):
            x = oracle.decode(c[m, :KL]) * float(s[m, 0])
            assert abs(out[m, n] - float(np.dot(x, bf16_value(w[n])))) <= 1e-12 * np.abs(x).sum()
        one, _ = oracle.project_rows(c[m:m + 1], s[m:m + 1], w)
        np.testing.assert_array_equal(one[0], out[m])


def test_linear_in_the_weight_and_in_the_scale():
    c, s = cache(6, 8)
    g = np.random.default_rng(7)
    w1 = bf16(g.standard_normal((16, KL)).astype(np.float32))
    w2 = bf16(g.standard_normal((16, KL)).astype(np.float32))
    o1, _ = oracle.project_rows(c, s, w1)
    o2, _ = oracle.project_rows(c, s, w2)
    o12, _ = oracle.project_rows(c, s, np.concatenate([w1, w2]))
    np.testing.assert_array_equal(o12, np.concatenate([o1, o2], axis=1))
    s2 = s.copy()
    s2[:, 0] *= np.float32(4.0)
    o4, _ = oracle.project_rows(c, s2, w1)
    np.testing.assert_array_equal(o4, 4.0 * o1)


def test_guarded_rows_project_to_zero():
    x = np.zeros((2, D), np.float32)
    x[1, :] = 1e-40
    c, s = oracle.quantize_rows(x)
    w = bf16(np.ones((8, KL), np.float32))
    out, rope = oracle.project_rows(c, s, w)
    assert not out.any() and not rope.any()
