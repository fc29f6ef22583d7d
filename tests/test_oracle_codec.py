"""Pins of the oracle's e4m3 codec (CPU only).

The codec is fixed by the OCP 8-bit floating point definition (E4M3: bias 7,
no infinities, NaN = S.1111.111, max finite 448, subnormals m * 2^-9) and by
the encoder rules of the page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA)
with .coli_kv v2" (colibri PR #299), commit message, kv_fp8.h item: round to
nearest even, saturate at +-448, keep the sign of zero, store NaN as 0; its
Tests item asks for an exhaustive round trip and RNE ties including the
binade-boundary mantissa carry.

Independent pins used here: closed-form spot values, PyTorch's float8_e4m3fn
conversion (a library routine with the same rounding inside +-464), a numpy
brute-force nearest search, and exhaustive sweeps (monotonicity, NaN, sign).
"""
import numpy as np
import pytest
import torch

import oracle

F32_MAX_FINITE = 0x7F7FFFFF


def f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def bits_of(x):
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


# (code, value) straight from the E4M3 formula: subnormal m*2^-9,
# normal (8+m)*2^(e-10).
SPOT = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x3F, 1.875), (0x40, 2.0), (0x57, 15.0), (0x58, 16.0),
    (0x7D, 416.0), (0x7E, 448.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
]


def test_decode_spot_values():
    for code, val in SPOT:
        assert oracle.decode(np.array([code], np.uint8))[0] == val, hex(code)
    neg0 = oracle.decode(np.array([0x80], np.uint8))[0]
    assert neg0 == 0.0 and np.signbit(neg0)
    nan = oracle.decode(np.array([0x7F, 0xFF], np.uint8))
    assert np.isnan(nan).all()


def test_decode_structure():
    v = oracle.decode(np.arange(256, dtype=np.uint8))
    finite = ~np.isnan(v)
    assert np.flatnonzero(~finite).tolist() == [0x7F, 0xFF]
    pos = v[:127]
    assert np.all(np.diff(pos) > 0), "non-negative codes must be strictly increasing"
    assert pos[0] == 0.0 and pos[126] == 448.0
    # sign symmetry
    assert np.array_equal(np.abs(v[128:255]), pos) and np.all(np.signbit(v[128:255]))
    # 8 subnormal values (incl. 0) on the 2^-9 grid, then 8 values per binade
    assert np.array_equal(pos[:8], np.arange(8) * 2.0 ** -9)
    for e in range(1, 16):
        seg = pos[8 * e: 8 * e + 8]
        lo = 2.0 ** (e - 7)
        expect = lo * (1 + np.arange(8) / 8)
        n = 7 if e == 15 else 8
        assert np.array_equal(seg[:n], expect[:n])


def test_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.decode(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    assert np.array_equal(ref[~both_nan], ours[~both_nan])
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(ours[~both_nan]))


def test_exhaustive_roundtrip():
    """E(decode(c)) == c for all 254 non-NaN codes; E(NaN) == 0x00."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.decode(codes).astype(np.float32)
    assert np.array_equal(oracle.encode(vals), codes)
    assert oracle.encode(np.array([np.nan], np.float32))[0] == 0


# Exact inputs on RNE ties.  Each value is the midpoint of two neighbouring
# e4m3 values; the even code wins.
TIES = [
    (1.0625, 0x38),             # between 1.0 (0x38) and 1.125 (0x39)
    (1.1875, 0x3A),             # between 1.125 (0x39) and 1.25 (0x3A)
    (1.9375, 0x40),             # between 1.875 (0x3F) and 2.0 (0x40): binade carry
    (15.5, 0x58),               # between 15 (0x57) and 16 (0x58): binade carry
    (432.0, 0x7E),              # between 416 (0x7D) and 448 (0x7E)
    (464.0, 0x7E),              # beyond 448: saturates
    (2.0 ** -10, 0x00),         # between 0 and 2^-9
    (-(2.0 ** -10), 0x80),      # negative tie to -0
    (3 * 2.0 ** -10, 0x02),     # between 1*2^-9 and 2*2^-9
    (15 * 2.0 ** -10, 0x08),    # between 7*2^-9 (0x07) and 2^-6 (0x08): subnormal->normal
    (-1.9375, 0xC0),
]


def test_rne_ties_and_carries():
    x = np.array([t for t, _ in TIES], dtype=np.float32)
    got = oracle.encode(x)
    assert got.tolist() == [c for _, c in TIES]
    # one ulp either side of a tie goes to the nearer neighbour
    for val, lo_code, hi_code in [(1.0625, 0x38, 0x39), (1.9375, 0x3F, 0x40),
                                  (15 * 2.0 ** -10, 0x07, 0x08), (432.0, 0x7D, 0x7E)]:
        b = bits_of(val)
        assert oracle.encode(np.array([f32(b - 1)], np.float32))[0] == lo_code
        assert oracle.encode(np.array([f32(b + 1)], np.float32))[0] == hi_code


def test_saturation_signed_zero():
    x = np.array([np.inf, -np.inf, 449.0, 1e30, -500.0, 448.0, 447.9, 3.4e38,
                  0.0, -0.0, -1e-30, 1e-30, f32(1), f32(0x80000001)], dtype=np.float32)
    expect = [0x7E, 0xFE, 0x7E, 0x7E, 0xFE, 0x7E, 0x7E, 0x7E,
              0x00, 0x80, 0x80, 0x00, 0x00, 0x80]
    assert oracle.encode(x).tolist() == expect


def test_every_nan_pattern_encodes_to_zero():
    n = (1 << 23) - 1
    pos = oracle.encode_bits_range(0x7F800001, n)
    neg = oracle.encode_bits_range(0xFF800001, n)
    assert not pos.any() and not neg.any()


def _midpoint_neighbourhood():
    v = oracle.decode(np.arange(127, dtype=np.uint8))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    b = mids.view(np.uint32).astype(np.int64)
    around = np.concatenate([b - 2, b - 1, b, b + 1, b + 2]).astype(np.uint32).view(np.float32)
    vals = v.astype(np.float32)
    vb = vals.view(np.uint32).astype(np.int64)
    near = np.concatenate([vb[1:] - 1, vb, vb + 1]).astype(np.uint32).view(np.float32)
    return np.concatenate([around, near])


def test_encoder_matches_torch_inside_range():
    """Inside |x| < 464 PyTorch's float8_e4m3fn cast rounds to nearest even
    exactly like the saturating encoder; NaN excluded."""
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([bits.view(np.float32), _midpoint_neighbourhood(),
                        -_midpoint_neighbourhood()])
    x = x[np.isfinite(x) & (np.abs(x) < 464)]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode(x), ref)


@pytest.mark.slow
def test_encoder_matches_torch_exhaustive_positive():
    """Every non-negative f32 below 464, in chunks."""
    end = bits_of(464.0)
    chunk = 1 << 26
    for first in range(0, end, chunk):
        cnt = min(chunk, end - first)
        ours = oracle.encode_bits_range(first, cnt)
        x = np.arange(first, first + cnt, dtype=np.uint32).view(np.float32)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, ref), hex(first)


def test_encoder_brute_force_nearest():
    """Independent nearest-value search in numpy over the 127 values of
    PyTorch's decode, ties to the even code, saturation beyond 448."""
    table = torch.arange(127, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()
    rng = np.random.default_rng(2)
    x = np.concatenate([
        (rng.standard_normal(200_000) * 10.0 ** rng.uniform(-12, 4, 200_000)),
        _midpoint_neighbourhood().astype(np.float64),
    ]).astype(np.float32)
    x = np.concatenate([x, -x])
    a = np.abs(x.astype(np.float64))
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes prefer the even one
    even = cand & (np.arange(127)[None, :] % 2 == 0)
    idx = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    idx = np.where(a >= 448.0, 126, idx)
    expect = (idx | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    assert np.array_equal(oracle.encode(x), expect)


@pytest.mark.slow
def test_encoder_monotone_and_sign_symmetric_exhaustive():
    """Over every non-negative finite f32 the code never decreases and never
    exceeds 0x7E; the negative half is the positive half with bit 7 set."""
    chunk = 1 << 26
    prev = 0
    for first in range(0, F32_MAX_FINITE + 1, chunk):
        cnt = min(chunk, F32_MAX_FINITE + 1 - first)
        c = oracle.encode_bits_range(first, cnt)
        assert c[0] >= prev
        assert np.all(np.diff(c.astype(np.int16)) >= 0), hex(first)
        assert c.max() <= 0x7E
        prev = int(c[-1])
        if first % (chunk * 8) == 0:  # sign symmetry on every 8th chunk
            n = oracle.encode_bits_range(first | 0x80000000, cnt)
            assert np.array_equal(n, c | 0x80)
    assert prev == 0x7E
