"""Pins of the oracle's block-scaled (MX) variant: e4m3 elements with one
power-of-two scale per 32 values, stored as a ue8m0 byte (page "Phase 0 toward
V4.1 on a 128 GB Mac: lossless mxfp8 residents and kill-test tooling" (keep
PR #3), mxfp8 residents paragraph: e4m3 bytes and ue8m0 exponents per 32-wide
group, 8.25 bits per value).

Reading: the block exponent E is the smallest integer with amax <= 448 * 2^E
(no finite value saturates, as with the per-row amax/448 scale), clamped to
the ue8m0 range [-127, 127].
"""
import numpy as np
import pytest

import oracle

D = 576


def closed_form_exponent(amax):
    """From the f32 bit pattern: amax = m 2^k with m in [1, 2) and 448 =
    1.75 * 2^8, so E = k - 8 when m <= 1.75 and k - 7 otherwise (a derivation
    independent of the oracle's counting)."""
    if amax == 0.0:
        return -127
    bits = int(np.array([amax], np.float32).view(np.uint32)[0])
    e, mant = (bits >> 23) & 0xFF, bits & 0x7FFFFF
    if e == 0:  # f32 subnormal: far below 448 * 2^-127
        return -127
    k = e - 127
    E = k - 8 if mant <= 0x600000 else k - 7
    return max(-127, min(127, E))


def block_rows(blocks):
    """One row of 18 blocks from a list of 18 arrays of 32 values."""
    return np.concatenate(blocks).astype(np.float32)[None, :]


def test_block_exponent_matches_the_closed_form():
    rng = np.random.default_rng(70)
    amaxes = list(np.float32(448.0) * np.float32(2.0) ** np.arange(-130, 121, 7).astype(np.float32))
    amaxes += [np.nextafter(np.float32(448.0), np.float32(np.inf)), np.float32(448.0),
               np.float32(447.99997), np.float32(1.0), np.float32(1e-40), np.float32(1e-45),
               np.float32(3.4e38), np.float32(0.0)]
    amaxes += list(np.exp(rng.uniform(-80, 80, 300)).astype(np.float32))
    for a in amaxes:
        x = np.zeros(D, np.float32)
        x[5] = a
        x[300] = -a
        _, e = oracle.quantize_rows_mx(x[None, :])
        want = closed_form_exponent(float(a))
        assert int(e[0, 0]) - 127 == want and int(e[0, 9]) - 127 == want, (a, e[0, 0])
        E = int(e[0, 0]) - 127
        if E > -127 and E < 127:  # minimal: 2^(E-1) would not do
            assert float(a) <= 448.0 * 2.0 ** E and float(a) > 448.0 * 2.0 ** (E - 1)


def test_representable_blocks_round_trip():
    rng = np.random.default_rng(71)
    vals = oracle.decode(np.arange(0x7F, dtype=np.uint8))
    for trial in range(20):
        blocks, want_e = [], []
        for b in range(18):
            j = int(rng.integers(-100, 100))
            c = rng.integers(0, 0x7F, 32)
            c[rng.integers(32)] = 0x7E                       # the block maximum is 448 2^j
            sign = np.where(rng.random(32) < 0.5, -1.0, 1.0)
            blocks.append(sign * vals[c] * 2.0 ** j)
            want_e.append(j)
        x = block_rows(blocks)
        codes, e = oracle.quantize_rows_mx(x)
        assert list(e[0].astype(int) - 127) == want_e
        back = oracle.dequantize_mx(codes, e)
        assert np.array_equal(back, x.astype(np.float64))


def test_power_of_two_equivariance_and_sign_symmetry():
    x = (np.random.default_rng(72).standard_normal((50, D)) * 3).astype(np.float32)
    c0, e0 = oracle.quantize_rows_mx(x)
    for j in (-40, -1, 1, 50):
        c1, e1 = oracle.quantize_rows_mx(x * np.float32(2.0 ** j))
        assert np.array_equal(c1, c0) and np.array_equal(e1.astype(int), e0.astype(int) + j)
    cn, en = oracle.quantize_rows_mx(-x)
    assert np.array_equal(cn, c0 ^ 0x80) and np.array_equal(en, e0)


def test_error_bound_and_block_maximum():
    x = np.random.default_rng(73).standard_t(3, (200, D)).astype(np.float32)
    codes, e = oracle.quantize_rows_mx(x)
    xhat = oracle.dequantize_mx(codes, e)
    E = np.repeat(e.astype(np.int64) - 127, 32, axis=1)
    err = np.abs(x - xhat)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** (E - 10)))
    mag = (codes & 0x7F).reshape(200, 18, 32).max(axis=2)
    assert np.all((mag >= 0x76) & (mag <= 0x7E))   # block maxima land in [224, 448] 2^E


def test_special_blocks():
    x = np.random.default_rng(74).standard_normal((1, D)).astype(np.float32)
    x[0, 0:32] = np.where(np.arange(32) % 2, np.float32(0.0), np.float32(-0.0))   # zero block
    x[0, 32:64] = np.float32(np.nan)                                              # all NaN
    x[0, 64 + 3] = np.float32(np.nan)                                            # a NaN entry
    x[0, 96 + 7] = np.float32(-np.inf)                                           # an inf entry
    x[0, 128:160] = np.float32(1e-41) * np.arange(32, dtype=np.float32)          # subnormal amax
    codes, e = oracle.quantize_rows_mx(x)
    assert e[0, 0] == 0 and np.array_equal(codes[0, 0:32], np.where(np.arange(32) % 2, 0x00, 0x80))
    assert e[0, 1] == 0 and not codes[0, 32:64].any()
    assert codes[0, 64 + 3] == 0x00
    fin = np.abs(x[0, 64:96][np.isfinite(x[0, 64:96])]).max()
    assert int(e[0, 2]) - 127 == closed_form_exponent(float(fin))
    assert codes[0, 96 + 7] == 0xFE
    assert int(e[0, 3]) - 127 == closed_form_exponent(float(np.abs(np.delete(x[0, 96:128], 7)).max()))
    assert e[0, 4] == 0
    want = oracle.encode(x[0, 128:160].astype(np.float64) * 2.0 ** 127)
    assert np.array_equal(codes[0, 128:160], want)


def test_attention_equals_attention_over_the_dequantized_rows():
    """orc_attention_mx is the plain attention over the dequantized rows (exact
    in f32 here), so it equals the f32-row attention of those values."""
    from fp8_e4m3_latent_amd import workloads
    w = workloads.tiny(seed=75, B=2, Q=2, H=16, T=150)
    codes, e = oracle.quantize_rows_mx(w.rows)
    xhat = oracle.dequantize_mx(codes, e).astype(np.float32)
    assert np.array_equal(xhat.astype(np.float64), oracle.dequantize_mx(codes, e))
    a = oracle.attention_mx(w.q_lat, w.q_rope, codes, e, w.kv_start, w.kv_len, Q=2)
    b = oracle.attention_f32rows(w.q_lat, w.q_rope, xhat, w.kv_start, w.kv_len, Q=2)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(b).max()
    s = oracle.attention_mx(w.q_lat, w.q_rope, codes, e, w.kv_start, w.kv_len, Q=2, num_splits=7)
    assert np.abs(a - s).max() <= 1e-12 * np.abs(a).max()


def test_bytes_per_token_layer():
    """576 codes + 18 exponent bytes = 594 B (8.25 bits per value) against the
    per-row variant's 584 B (8.11 bits)."""
    assert oracle.bytes_per_token_layer_mx(512, 64) == 594
    assert abs(8 * 594 / 576 - 8.25) < 1e-12
    assert abs(8 * oracle.bytes_per_token_layer(512, 64) / 576 - 8.111) < 1e-3
