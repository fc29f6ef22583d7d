"""GPU parity of the fp8 conversions and of kv8_quantize_rows against the oracle.

Bar: bit-exact codes and scales (the quantizer is integer/byte work once the
f32 divisions and products are fixed, and both sides take them in f32).
"""
import numpy as np
import pytest

import oracle
from fp8_e4m3_latent_amd import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

KL, KR, D = 512, 64, 576


@pytest.fixture(scope="module")
def kv8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_e4m3_latent_amd as m
    m.lib()
    return m


def say(msg):
    print(msg, flush=True)


def test_decode_all_codes_exact(kv8):
    say("decode_codes: all 256 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    bf, hf = kv8.decode_codes(codes)
    torch.cuda.synchronize()
    bf = bf.cpu().numpy().view(np.uint16)
    hf = hf.cpu().numpy().view(np.uint16)
    ref = oracle.decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue  # NaN codes: never produced by the encoder
        v = ref[c]
        # exact bf16 and fp16 patterns of the oracle value
        f32 = np.array([v], np.float32)
        assert f32.view(np.uint32)[0] & 0xFFFF == 0
        assert bf[c] == f32.view(np.uint32)[0] >> 16, hex(c)
        assert hf[c] == np.array([v], np.float16).view(np.uint16)[0], hex(c)
        assert np.float16(v) == v


def test_encoder_exhaustive_all_f32(kv8):
    """Every one of the 2^32 f32 bit patterns, vs the oracle: the encoder the
    quantizer uses (the gfx950 conversion behind the clamp, encoder 0) and the
    integer bit-math encoder (encoder 1)."""
    chunk = 1 << 28
    dev = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    ref = np.empty(chunk, dtype=np.uint8)
    for first in range(0, 1 << 32, chunk):
        oracle.encode_bits_range(first, chunk, out=ref)
        for enc in (0, 1):
            say("encode_bits: encoder %d first=0x%08x count=%d" % (enc, first, chunk))
            kv8.encode_bits(first, chunk, dev, encoder=enc)
            got = dev.cpu().numpy()
            if not np.array_equal(got, ref):
                bad = np.flatnonzero(got != ref)[:10]
                raise AssertionError("encoder %d: mismatch at bit patterns %s: gpu %s oracle %s" % (
                    enc, [hex(first + int(b)) for b in bad], got[bad].tolist(), ref[bad].tolist()))


def quantize_on_gpu(kv8, rows, n_cache=None, dst=None):
    n = rows.shape[0]
    nc = n if n_cache is None else n_cache
    src = torch.from_numpy(rows).cuda()
    codes = torch.full((nc, D), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((nc, 2), -7.0, dtype=torch.float32, device="cuda")
    d = None if dst is None else torch.from_numpy(np.ascontiguousarray(dst, np.int64)).cuda()
    kv8.quantize_rows(src, codes, scales, dst_rows=d)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def assert_same(codes, scales, rc, rs, what):
    if not np.array_equal(codes, rc):
        r, c = np.argwhere(codes != rc)[0]
        raise AssertionError("%s: code mismatch at row %d col %d: gpu %#x oracle %#x" % (
            what, r, c, codes[r, c], rc[r, c]))
    sb, rb = scales.view(np.uint32), rs.view(np.uint32)
    if not np.array_equal(sb, rb):
        r, c = np.argwhere(sb != rb)[0]
        raise AssertionError("%s: scale mismatch at row %d seg %d: gpu %r oracle %r" % (
            what, r, c, scales[r, c], rs[r, c]))


def test_quantize_bulk_rows_full_size(kv8):
    """32,768 tokens x 61 layers of Student-t rows with planted special rows."""
    say("quantize: bulk rows 32768 x 61 with planted specials")
    rows, idx = workloads.bulk_rows(seed=0)
    codes, scales = quantize_on_gpu(kv8, rows)
    rc, rs = oracle.quantize_rows(rows)
    assert_same(codes, scales, rc, rs, "bulk")
    # the planted rows produced their defined outputs on the GPU too
    assert np.all(scales[idx["zero"]] == 0) and np.all(scales[idx["subnormal_amax"]] == 0)
    assert np.all(scales[idx["guard_1.3166e-36"]] > 0)


def test_quantize_small_and_ragged_counts(kv8):
    rng = np.random.default_rng(3)
    for n in (1, 3, 4, 5, 63, 257):
        say("quantize: n_rows=%d" % n)
        rows = (rng.standard_normal((n, D)) * 10.0 ** rng.uniform(-3, 3, (n, 1))).astype(np.float32)
        codes, scales = quantize_on_gpu(kv8, rows)
        rc, rs = oracle.quantize_rows(rows)
        assert_same(codes, scales, rc, rs, "n=%d" % n)


def test_quantize_dst_rows_and_stride(kv8):
    rng = np.random.default_rng(4)
    n, nc = 300, 1000
    wide = rng.standard_normal((n, 640)).astype(np.float32)
    rows = wide[:, :D]                      # row stride 640 floats
    dst = rng.permutation(nc)[:n]
    say("quantize: scattered dst_rows, src stride 640")
    src = torch.from_numpy(wide).cuda()[:, :D]
    codes = torch.full((nc, D), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((nc, 2), -7.0, dtype=torch.float32, device="cuda")
    kv8.quantize_rows(src, codes, scales, dst_rows=torch.from_numpy(dst.astype(np.int64)).cuda())
    torch.cuda.synchronize()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    rc, rs = oracle.quantize_rows(np.ascontiguousarray(rows))
    assert_same(codes[dst], scales[dst], rc, rs, "scatter")
    untouched = np.setdiff1d(np.arange(nc), dst)
    assert np.all(codes[untouched] == 0xAB) and np.all(scales[untouched] == -7.0)


def test_quantize_deterministic_and_guard_band(kv8):
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((64, D)).astype(np.float32)
    for i, amax in enumerate([0.0, 1e-40, 1e-37, 1.3165e-36, 1.3166e-36, 2e-36, 3e38, 1e-30]):
        rows[i] = rng.uniform(-1, 1, D).astype(np.float32) * np.float32(amax)
        rows[i, 5] = np.float32(amax)
        rows[i, KL + 2] = -np.float32(amax)
    rows[10, :] = np.float32(-0.0)
    rows[11, 7] = np.nan
    rows[12, KL:] = np.inf
    say("quantize: guard band and special rows, twice")
    a = quantize_on_gpu(kv8, rows)
    b = quantize_on_gpu(kv8, rows)
    rc, rs = oracle.quantize_rows(rows)
    assert_same(*a, rc, rs, "guard")
    assert_same(*b, rc, rs, "guard (second run)")
    # the same rows in a batch of 8,320 (the many-rows launch shape; the 64
    # above use the few-rows one)
    say("quantize: guard band and special rows in a batch of 8320")
    big = np.tile(rows, (130, 1))
    c2, s2 = quantize_on_gpu(kv8, big)
    assert_same(c2, s2, np.tile(rc, (130, 1)), np.tile(rs, (130, 1)), "guard (8320 rows)")


def test_quantize_argument_errors(kv8):
    src = torch.zeros((4, D), dtype=torch.float32, device="cuda")
    codes = torch.zeros((4, D), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((4, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        kv8.quantize_rows(src[:, :500], codes, scales)
    L = kv8.lib()
    # misaligned source pointer
    rc = L.kv8_quantize_rows(src.data_ptr() + 4, D, 1, KL, KR, codes.data_ptr(),
                             scales.data_ptr(), None, None)
    assert rc == -1
    kv8.quantize_rows(src[:0], codes, scales)  # empty is a no-op
