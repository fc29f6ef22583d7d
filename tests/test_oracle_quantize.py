"""Pins of the oracle's per-row quantizer (CPU only).

Rule being pinned (page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with
.coli_kv v2", colibri PR #299, commit message, kv_fp8.h item, and the PR
description): each token's Lc and Rc parts get one f32 scale amax/448 each;
the codes are the saturating RNE encoding of x * (448/amax); an amax so small
that 448/amax overflows to +inf is guarded (scale 0).

Pins: invariants that hold for any correct implementation (an amax entry
maps to +-448, power-of-two equivariance, sign symmetry, the error bound of a
4-significant-bit format, exact round trip of representable rows), the f32
overflow threshold of the guard computed independently in numpy, and the
defined outputs for NaN, inf and zero rows.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_e4m3_latent_amd import workloads

KL, KR = 512, 64


def dequant(codes, scales):
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    s = np.concatenate([np.repeat(scales[:, :1], KL, 1), np.repeat(scales[:, 1:], KR, 1)], 1)
    return v * s.astype(np.float64)


@pytest.fixture(scope="module")
def trows():
    rng = np.random.default_rng(5)
    n = 3000
    z = rng.standard_normal((n, KL + KR)).astype(np.float32)
    g = rng.standard_gamma(1.5, (n, KL + KR)).astype(np.float32)
    x = (np.float32(0.5) * z / np.sqrt(g * np.float32(2 / 3))).astype(np.float32)
    x[:500] *= np.float32(1e-3)  # a spread of magnitudes
    x[500:1000] *= np.float32(1e4)
    return x


def test_amax_entry_hits_448(trows):
    codes, scales = oracle.quantize_rows(trows)
    for seg, (a, b) in enumerate(((0, KL), (KL, KL + KR))):
        c = codes[:, a:b] & 0x7F
        assert np.all(c.max(axis=1) == 0x7E)
        am = np.abs(trows[:, a:b]).max(axis=1)
        # scale is the f32 quotient amax/448
        assert np.array_equal(scales[:, seg], (am / np.float32(448)).astype(np.float32))


def test_power_of_two_equivariance(trows):
    x = trows[1000:2000]
    c0, s0 = oracle.quantize_rows(x)
    for k in (-20, -3, 1, 7, 30):
        f = np.float32(2.0 ** k)
        c1, s1 = oracle.quantize_rows((x * f).astype(np.float32))
        assert np.array_equal(c1, c0), k
        assert np.array_equal(s1, (s0 * f).astype(np.float32)), k


def test_sign_symmetry(trows):
    c0, s0 = oracle.quantize_rows(trows)
    c1, s1 = oracle.quantize_rows(-trows)
    assert np.array_equal(c1, c0 ^ 0x80)
    assert np.array_equal(s1, s0)


def test_error_bound(trows):
    codes, scales = oracle.quantize_rows(trows)
    x = trows.astype(np.float64)
    err = np.abs(x - dequant(codes, scales))
    s = np.concatenate([np.repeat(scales[:, :1], KL, 1), np.repeat(scales[:, 1:], KR, 1)], 1)
    # half an ulp of a 4-significant-bit value, or half the subnormal step,
    # plus slack for the f32 scale and product roundings
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s.astype(np.float64) * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)


def test_representable_rows_roundtrip_exactly():
    rng = np.random.default_rng(6)
    vals = oracle.decode(np.arange(127, dtype=np.uint8))
    for k in (-30, -5, 0, 4, 40):
        c = rng.integers(0, 127, size=(50, KL + KR)).astype(np.uint8)
        c[:, 7] = 0x7E
        c[:, KL + 3] = 0x7E
        c |= np.where(rng.random(c.shape) < 0.5, 0x80, 0).astype(np.uint8)
        x = (np.where(c & 0x80, -1.0, 1.0) * vals[c & 0x7F] * 2.0 ** k).astype(np.float32)
        codes, scales = oracle.quantize_rows(x)
        assert np.array_equal(scales, np.full((50, 2), np.float32(2.0 ** k)))
        # -0 entries come back as 0x80, +0 as 0x00: compare through values + sign
        assert np.array_equal(codes, c)


def _guard_threshold_numpy():
    """Smallest f32 a with fl32(448 / a) finite, by bisection on the f32 grid."""
    lo = np.uint32(1)                      # 448 / tiny = inf
    hi = np.float32(1e-30).view(np.uint32)  # finite
    with np.errstate(over="ignore", divide="ignore"):
        while hi - lo > 1:
            mid = np.uint32((int(lo) + int(hi)) // 2)
            if np.isinf(np.float32(448) / mid.view(np.float32)):
                lo = mid
            else:
                hi = mid
    return hi.view(np.float32)


@pytest.mark.parametrize("amax,guarded", [
    (0.0, True), (1e-40, True), (1e-37, True), (1.3165e-36, True),
    (1.3166e-36, False), (2e-36, False), (1.0, False)])
def test_guard(amax, guarded):
    thr = _guard_threshold_numpy()
    assert 1.3165e-36 < thr <= 1.3166e-36
    x = np.zeros(KL, dtype=np.float32)
    x[3] = np.float32(amax)
    x[9] = -np.float32(amax) * np.float32(0.5)
    codes, s = oracle.quantize_segment(x)
    if guarded:
        assert s == 0.0 and not np.signbit(s)
        # x * 0: +0 -> 0x00, -finite -> 0x80 (sign kept)
        expect = np.where(np.signbit(x), 0x80, 0x00).astype(np.uint8)
        assert np.array_equal(codes, expect)
    else:
        assert s == np.float32(np.float32(amax) / np.float32(448))
        assert codes[3] == 0x7E
        if amax < 1e-35:
            assert s < np.finfo(np.float32).tiny  # a subnormal scale is kept


def test_nan_inf_zero_rows():
    x = np.linspace(-3, 3, KL + KR, dtype=np.float32)
    x[10] = np.nan
    x[11] = -np.nan
    x[12] = np.inf
    x[KL + 1] = -np.inf
    codes, scales = oracle.quantize_rows(x[None])
    assert codes[0, 10] == 0 and codes[0, 11] == 0
    assert codes[0, 12] == 0x7E and codes[0, KL + 1] == 0xFE
    # amax ignores NaN and inf
    assert scales[0, 0] == np.float32(np.float32(3.0) / np.float32(448))
    z = np.where(np.arange(KL + KR) % 2 == 0, np.float32(0.0), np.float32(-0.0))
    cz, sz = oracle.quantize_rows(z[None].astype(np.float32))
    assert np.array_equal(sz, np.zeros((1, 2), np.float32))
    assert np.array_equal(cz[0], np.where(np.arange(KL + KR) % 2 == 0, 0, 0x80))
    # guarded row with inf: inf * 0 is NaN -> 0x00
    g = np.zeros(KL + KR, dtype=np.float32)
    g[0] = np.inf
    cg, sg = oracle.quantize_rows(g[None])
    assert cg[0, 0] == 0x00 and sg[0, 0] == 0.0


def test_dst_rows_scatter():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((20, KL + KR)).astype(np.float32)
    dst = rng.permutation(50)[:20]
    c, s = oracle.quantize_rows(x, dst_rows=dst, n_cache_rows=50)
    c0, s0 = oracle.quantize_rows(x)
    assert np.array_equal(c[dst], c0) and np.array_equal(s[dst], s0)
    untouched = np.setdiff1d(np.arange(50), dst)
    assert not c[untouched].any() and not s[untouched].any()


def test_row_stride():
    rng = np.random.default_rng(8)
    big = rng.standard_normal((30, 600)).astype(np.float32)
    c1, s1 = oracle.quantize_rows(big[:, :KL + KR])
    c2, s2 = oracle.quantize_rows(np.ascontiguousarray(big[:, :KL + KR]))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_bulk_special_rows_small():
    """The planted special rows of the bulk-quantizer workload, at a small size,
    produce their defined outputs."""
    rows, idx = workloads.bulk_rows(seed=3, tokens=2048, layers=3, special_frac=0.01,
                                    guard_rows=4, threads=4)
    codes, scales = oracle.quantize_rows(rows)
    assert np.all(scales[idx["zero"]] == 0)
    assert np.all(scales[idx["subnormal_amax"]] == 0)
    for r in idx["zero"]:
        assert np.array_equal(codes[r], np.where(np.signbit(rows[r]), 0x80, 0))
    for r in idx["tie"]:
        k = scales[r]
        assert np.all(k > 0) and np.all(np.log2(k) == np.round(np.log2(k)))
        # every entry was a tie or the amax: codes are even mantissas, +-0x7E
        assert np.all((codes[r] & 1) == 0)
    for r in idx["inf"]:
        inf = np.isinf(rows[r])
        assert np.array_equal(codes[r][inf], np.where(rows[r][inf] > 0, 0x7E, 0xFE))
    for r in idx["nan"]:
        assert not codes[r][np.isnan(rows[r])].any()
    for amax in workloads.GUARD_AMAX:
        rr = idx["guard_%g" % amax]
        assert np.all((scales[rr] == 0) == (amax < 1.3166e-36))
    rr = idx["guard_subnormal_entries"]
    assert np.all(scales[rr] > 0)


def _torch_codes(x, via_inverse):
    """Codes of a plain per-segment reading built from numpy f32 arithmetic and
    torch's float8_e4m3fn cast (a library RNE conversion; every value here is
    finite and within 448 (1 + 2^-23), which the cast takes to at most 448)."""
    torch = pytest.importorskip("torch")
    out = np.empty(x.shape, np.uint8)
    for a, b in ((0, 512), (512, 576)):
        seg = x[:, a:b]
        amax = np.abs(seg).max(1, keepdims=True).astype(np.float32)
        if via_inverse:
            q = (seg * (np.float32(448.0) / amax).astype(np.float32)).astype(np.float32)
        else:
            q = (seg / (amax / np.float32(448.0)).astype(np.float32)).astype(np.float32)
        out[:, a:b] = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out


def test_codes_come_from_the_inverse_not_the_division():
    """Reading Q7 (the page's overflow guard forms 448/amax): each code is
    E(fl32(x * fl32(448/amax))).  On 20,000 Gaussian rows the oracle equals
    that reading through torch's e4m3 cast everywhere, and the other reading,
    E(fl32(x / fl32(amax/448))), differs from it on some codes (so this test
    tells the two apart)."""
    x = np.random.default_rng(77).standard_normal((20000, 576)).astype(np.float32)
    codes, _ = oracle.quantize_rows(x)
    inv_reading = _torch_codes(x, True)
    div_reading = _torch_codes(x, False)
    assert np.array_equal(codes, inv_reading)
    differ = np.argwhere(inv_reading != div_reading)
    assert len(differ) > 0
    for r, c in differ:
        assert codes[r, c] == inv_reading[r, c] != div_reading[r, c]
