"""Pins of the oracle's absorbed-MLA decode (CPU only).

What is pinned (page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with
.coli_kv v2", colibri PR #299): the commit message's attention_rows item --
absorbed score and context loops over the dequantized latent rows, the latent
acting as both key and value -- and its Validation sentence that the KV8=0
path equals plain f32 attention; the PR description's follow-up paragraph
(split-T kernels, merged here by log-sum-exp).

Independent pins: the non-absorbed form of MLA attention with random
up-projections (the absorbed score and context must reproduce it), PyTorch's
scaled_dot_product_attention on the same rows, closed-form special cases
(one token, zero query, one dominant token), and invariances (token
permutation, any split count, causal query == truncated cache).
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_e4m3_latent_amd import workloads

KL, KR = 512, 64
D = KL + KR
SIGMA = np.float32(1.0 / 24.0)


def make_case(seed, B=2, Q=1, H=3, lens=(40, 23)):
    rng = np.random.default_rng(seed)
    lens = np.array(lens[:B], dtype=np.int32)
    start = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    rows = rng.standard_normal((int(lens.sum()), D)).astype(np.float32)
    q_lat = workloads.bf16_bits(rng.standard_normal((B, Q, H, KL)).astype(np.float32) / 24)
    q_rope = workloads.bf16_bits(rng.standard_normal((B, Q, H, KR)).astype(np.float32) / 24)
    return rows, start, lens, q_lat, q_rope


def qf(bits):
    return workloads.bf16_to_f32(bits).astype(np.float64)


def dequant_rows(codes, scales):
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    s = np.concatenate([np.repeat(scales[:, :1], KL, 1), np.repeat(scales[:, 1:], KR, 1)], 1)
    return v * s.astype(np.float64)


def test_kv8_0_equals_non_absorbed_mla():
    """Non-absorbed MLA with random W_UK [H, 512, 512] (invertible) and
    W_UV [H, 16, 512]: k = W_UK Lc, v = W_UV Lc, q_nope chosen with
    W_UK^T q_nope = q_lat.  softmax(s (q_nope.k + q_rope.Rc)) . v must equal
    W_UV applied to the absorbed latent output."""
    rows, start, lens, q_lat, q_rope = make_case(11)
    B, Q, H = 2, 1, 3
    out = oracle.attention_f32rows(q_lat, q_rope, rows, start, lens, Q=1, softmax_scale=SIGMA)
    rng = np.random.default_rng(12)
    for b in range(B):
        X = rows[start[b]:start[b] + lens[b]].astype(np.float64)
        for h in range(H):
            W_uk = rng.standard_normal((KL, KL)) / np.sqrt(KL)
            W_uv = rng.standard_normal((16, KL)) / np.sqrt(KL)
            ql = qf(q_lat[b, 0, h])
            q_nope = np.linalg.solve(W_uk.T, ql)
            k_nope = X[:, :KL] @ W_uk.T
            v = X[:, :KL] @ W_uv.T
            s = float(SIGMA) * (k_nope @ q_nope + X[:, KL:] @ qf(q_rope[b, 0, h]))
            p = np.exp(s - s.max())
            p /= p.sum()
            ref = p @ v
            got = W_uv @ out[b, 0, h]
            assert np.allclose(got, ref, rtol=1e-9, atol=1e-12)


def _sdpa(q, K, V, sigma):
    qt = torch.from_numpy(q.astype(np.float32))[None, None]
    Kt = torch.from_numpy(K.astype(np.float32))[None, None]
    Vt = torch.from_numpy(V.astype(np.float32))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=float(sigma))
    return o[0, 0].double().numpy()


def test_kv8_0_matches_torch_sdpa_f32():
    rows, start, lens, q_lat, q_rope = make_case(13)
    out = oracle.attention_f32rows(q_lat, q_rope, rows, start, lens, softmax_scale=SIGMA)
    for b in range(2):
        X = rows[start[b]:start[b] + lens[b]]
        q = np.concatenate([qf(q_lat[b, 0]), qf(q_rope[b, 0])], axis=1)
        ref = _sdpa(q, X, X[:, :KL], SIGMA)
        assert np.max(np.abs(out[b, 0] - ref)) <= 2e-6 * np.max(np.abs(ref))


def test_kv8_1_matches_sdpa_on_dequantized_rows():
    rows, start, lens, q_lat, q_rope = make_case(14)
    codes, scales = oracle.quantize_rows(rows)
    out = oracle.attention(q_lat, q_rope, codes, scales, start, lens, softmax_scale=SIGMA)
    Xh = dequant_rows(codes, scales)
    for b in range(2):
        X = Xh[start[b]:start[b] + lens[b]]
        q = np.concatenate([qf(q_lat[b, 0]), qf(q_rope[b, 0])], axis=1)
        ref = _sdpa(q, X, X[:, :KL], SIGMA)
        assert np.max(np.abs(out[b, 0] - ref)) <= 2e-6 * np.max(np.abs(ref))
    # and differs from the unquantized result by a quantization-sized amount
    out0 = oracle.attention_f32rows(q_lat, q_rope, rows, start, lens, softmax_scale=SIGMA)
    rel = np.max(np.abs(out - out0)) / np.max(np.abs(out0))
    assert 1e-4 < rel < 0.1


def test_kv8_1_equals_kv8_0_on_representable_rows():
    rng = np.random.default_rng(15)
    vals = oracle.decode(np.arange(127, dtype=np.uint8))
    n = 50
    c = rng.integers(0, 127, size=(n, D))
    c[:, 0] = 126
    c[:, KL] = 126
    sign = np.where(rng.random((n, D)) < 0.5, -1.0, 1.0)
    k = rng.integers(-6, 6, size=(n, 2))
    mult = np.concatenate([np.repeat(2.0 ** k[:, :1], KL, 1), np.repeat(2.0 ** k[:, 1:], KR, 1)], 1)
    rows = (sign * vals[c] * mult).astype(np.float32)
    start = np.array([0, 30], np.int64)
    lens = np.array([30, 20], np.int32)
    _, _, _, q_lat, q_rope = make_case(16)
    codes, scales = oracle.quantize_rows(rows)
    a = oracle.attention(q_lat, q_rope, codes, scales, start, lens)
    b = oracle.attention_f32rows(q_lat, q_rope, rows, start, lens)
    assert np.array_equal(a, b)


def test_single_token_returns_its_lc_row():
    rows, start, lens, q_lat, q_rope = make_case(17, lens=(1, 1))
    codes, scales = oracle.quantize_rows(rows)
    out = oracle.attention(q_lat, q_rope, codes, scales, start, lens)
    Xh = dequant_rows(codes, scales)
    for b in range(2):
        for h in range(3):
            assert np.array_equal(out[b, 0, h], Xh[start[b], :KL])


def test_zero_query_returns_mean_row():
    rows, start, lens, q_lat, q_rope = make_case(18)
    q_lat[:] = 0
    q_rope[:] = 0
    codes, scales = oracle.quantize_rows(rows)
    out = oracle.attention(q_lat, q_rope, codes, scales, start, lens)
    Xh = dequant_rows(codes, scales)
    for b in range(2):
        m = Xh[start[b]:start[b] + lens[b], :KL].mean(axis=0)
        assert np.allclose(out[b, 0, 0], m, rtol=1e-13, atol=1e-15)


def test_dominant_token():
    rows, start, lens, q_lat, q_rope = make_case(19, B=1, H=1, lens=(64,))
    q_lat[:] = 0
    q_rope[:] = 0
    q_lat[0, 0, 0, 5] = workloads.bf16_bits(np.array([8.0], np.float32))[0]
    rows[37, 5] = 200.0  # score margin ~ 8*200/24 = 66
    codes, scales = oracle.quantize_rows(rows)
    out = oracle.attention(q_lat, q_rope, codes, scales, start, lens)
    Xh = dequant_rows(codes, scales)
    assert np.allclose(out[0, 0, 0], Xh[37, :KL], rtol=1e-20, atol=1e-24)


def test_token_permutation_invariance():
    rows, start, lens, q_lat, q_rope = make_case(20, B=1, lens=(70,))
    perm = np.random.default_rng(21).permutation(70)
    a = oracle.attention_f32rows(q_lat, q_rope, rows, start, lens)
    b = oracle.attention_f32rows(q_lat, q_rope, rows[perm], start, lens)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("splits", [2, 7, 64, 70, 200])
def test_split_merge_equals_unsplit(splits):
    rows, start, lens, q_lat, q_rope = make_case(22, lens=(70, 41))
    codes, scales = oracle.quantize_rows(rows)
    a = oracle.attention(q_lat, q_rope, codes, scales, start, lens, num_splits=1)
    b = oracle.attention(q_lat, q_rope, codes, scales, start, lens, num_splits=splits)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15)


def test_causal_query_equals_truncated_cache():
    Q = 4
    rows, start, lens, q_lat, q_rope = make_case(23, Q=Q, lens=(50, 9))
    codes, scales = oracle.quantize_rows(rows)
    out = oracle.attention(q_lat, q_rope, codes, scales, start, lens, Q=Q)
    for b in range(2):
        for i in range(Q):
            n = lens[b] - (Q - 1) + i
            ref = oracle.attention(q_lat[b:b + 1, i:i + 1], q_rope[b:b + 1, i:i + 1], codes,
                                   scales, start[b:b + 1], np.array([n], np.int32), Q=1)
            assert np.array_equal(out[b, i], ref[0, 0])


def test_empty_and_short_ranges_give_zeros():
    Q = 4
    rows, start, lens, q_lat, q_rope = make_case(24, Q=Q, lens=(2, 0))
    codes, scales = oracle.quantize_rows(np.concatenate([rows, rows[:1]]))
    out = oracle.attention(q_lat, q_rope, codes, scales, start, lens, Q=Q)
    # sequence 0 has 2 rows: queries 0, 1 see -1 and 0 rows
    assert not out[0, :2].any() and out[0, 2:].any()
    assert not out[1].any()


def test_selected_rows_equal_full_output():
    Q = 2
    rows, start, lens, q_lat, q_rope = make_case(25, Q=Q, lens=(33, 17))
    codes, scales = oracle.quantize_rows(rows)
    full = oracle.attention(q_lat, q_rope, codes, scales, start, lens, Q=Q)
    sel = np.array([0, 5, 7, 11, 3], np.int64)
    part = oracle.attention(q_lat, q_rope, codes, scales, start, lens, Q=Q, sel=sel)
    assert np.array_equal(part, full.reshape(-1, KL)[sel])
