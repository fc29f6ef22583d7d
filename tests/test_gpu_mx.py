"""GPU parity of the block-scaled (MX) variant against the oracle: the
quantizer kv8_quantize_rows_mx bit-exact (codes and ue8m0 exponents), and
kv8_absorb_decode_mx within max|d|/max|ref| <= 1e-3 of the oracle's f64
attention over the same codes and exponents.

Pages: "Phase 0 toward V4.1 on a 128 GB Mac: lossless mxfp8 residents and
kill-test tooling" (keep PR #3), mxfp8 residents paragraph (e4m3 bytes and
ue8m0 exponents per 32 values); "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA)
with .coli_kv v2" (colibri PR #299), commit message, attention_rows item.
"""
import numpy as np
import pytest

import oracle
from fp8_e4m3_latent_amd import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

KL, D, NB = 512, 576, 18
TOL = 1e-3


@pytest.fixture(scope="module")
def kv8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_e4m3_latent_amd as m
    m.lib()
    return m


def say(msg):
    print(msg, flush=True)


def mx_cache(kv8, rows, check=True):
    n = rows.shape[0]
    src = torch.from_numpy(np.ascontiguousarray(rows)).cuda()
    codes = torch.empty((n, D), dtype=torch.uint8, device="cuda")
    exps = torch.empty((n, NB), dtype=torch.uint8, device="cuda")
    kv8.quantize_rows_mx(src, codes, exps)
    torch.cuda.synchronize()
    del src
    c, e = codes.cpu().numpy(), exps.cpu().numpy()
    if check:
        rc, re_ = oracle.quantize_rows_mx(rows)
        if not np.array_equal(c, rc):
            r, k = np.argwhere(c != rc)[0]
            raise AssertionError("code mismatch at row %d col %d: gpu %#x oracle %#x (x = %r)" % (
                r, k, c[r, k], rc[r, k], rows[r, k]))
        if not np.array_equal(e, re_):
            r, k = np.argwhere(e != re_)[0]
            raise AssertionError("exponent mismatch at row %d block %d: gpu %d oracle %d" % (r, k, e[r, k], re_[r, k]))
    return codes, exps, c, e


def test_quantizer_bulk_rows_with_special_rows(kv8):
    """Student-t rows with planted zero, subnormal-amax, NaN, tie and inf rows
    and the guard-band rows (262,144 rows), bit-exact."""
    rows, _ = workloads.bulk_rows(seed=3, tokens=32768, layers=8)
    say("mx quantize: %d bulk rows" % rows.shape[0])
    mx_cache(kv8, rows)


def test_quantizer_scattered_rows_and_extreme_blocks(kv8):
    rng = np.random.default_rng(80)
    x = rng.standard_normal((300, D)).astype(np.float32)
    x[:, ::32] *= np.float32(1e30)                     # one huge value per block
    x[7] = np.float32(3e38) * np.sign(x[7])
    x[8] = np.float32(1e-44)
    x[9, 100:164] = np.float32(448.0) * np.float32(2.0) ** 60
    src = torch.from_numpy(x).cuda()
    codes = torch.full((700, D), 0xAB, dtype=torch.uint8, device="cuda")
    exps = torch.full((700, NB), 0xCD, dtype=torch.uint8, device="cuda")
    dst = np.random.default_rng(81).choice(700, 300, replace=False).astype(np.int64)
    kv8.quantize_rows_mx(src, codes, exps, dst_rows=torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    rc, re_ = oracle.quantize_rows_mx(x)
    assert np.array_equal(codes.cpu().numpy()[dst], rc) and np.array_equal(exps.cpu().numpy()[dst], re_)
    untouched = np.setdiff1d(np.arange(700), dst)
    assert (codes.cpu().numpy()[untouched] == 0xAB).all() and (exps.cpu().numpy()[untouched] == 0xCD).all()


def to_dev(w):
    ql = torch.from_numpy(w.q_lat.view(np.int16)).cuda().view(torch.bfloat16)
    qr = torch.from_numpy(w.q_rope.view(np.int16)).cuda().view(torch.bfloat16)
    return (ql, qr, torch.from_numpy(w.kv_start.astype(np.int64)).cuda(),
            torch.from_numpy(w.kv_len.astype(np.int32)).cuda())


def run_case(kv8, w, splits=1, sel=None, cache=None):
    say("mx decode: %s B=%d Q=%d H=%d max_len=%d splits=%d" % (w.name, w.B, w.Q, w.H, w.max_len, splits))
    codes, exps, c, e = cache if cache is not None else mx_cache(kv8, w.rows)
    ql, qr, st, ln = to_dev(w)
    out = kv8.absorb_decode_mx(ql, qr, codes, exps, st, ln, w.max_len, w.softmax_scale, num_splits=splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, KL)
    ref = oracle.attention_mx(w.q_lat, w.q_rope, c, e, w.kv_start, w.kv_len, Q=w.Q,
                              softmax_scale=w.softmax_scale, sel=sel).reshape(-1, KL)
    if sel is not None:
        got = got[sel]
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))
    say("  max|d|/max|ref| = %.3g" % err)
    assert err <= TOL, err
    return got, ref


def test_decode_tiny_with_outliers(kv8):
    run_case(kv8, workloads.tiny(seed=0))


@pytest.mark.parametrize("splits", [1, 3, 64])
def test_decode_splits(kv8, splits):
    run_case(kv8, workloads.tiny(seed=82, B=2, Q=1, H=128, T=5000, outlier_p=0.0), splits=splits)


def test_decode_ragged_causal_and_empty(kv8):
    w = workloads.tiny(seed=83, B=4, Q=4, H=32, T=1, outlier_p=0.0)
    lens = np.array([0, 2, 333, 1500], np.int32)
    w.kv_len = lens
    w.kv_start = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    w.rows = np.random.default_rng(84).standard_normal((int(lens.sum()), D)).astype(np.float32)
    got, _ = run_case(kv8, w)
    got = got.reshape(4, 4, 32, KL)
    assert not got[0].any() and not got[1, :2].any()


def test_decode_query_rows_of_any_magnitude(kv8):
    """Query rows scaled by 1e-37 … 1e36 over block-scaled rows scaled by the
    inverse (softmax scale 1, scores spread over several natural-log units),
    and query elements spread over 2^-40..1: the two e4m3 query terms of the
    scaled score MFMAs reproduce the bf16 queries (the same terms as the
    per-row path)."""
    T = 300
    mq = np.array([1e-37, 1e-30, 1e20, 1e36, 1.0])
    B = len(mq)
    w = workloads.tiny(seed=85, B=B, Q=1, H=32, T=T, outlier_p=0.0)
    ql = workloads.bf16_to_f32(w.q_lat).astype(np.float64)
    qr = workloads.bf16_to_f32(w.q_rope).astype(np.float64)
    rng = np.random.default_rng(86)
    for b in range(B):
        if b == B - 1:
            ql[b] = np.copysign(np.exp2(rng.uniform(-40.0, 0.0, size=ql[b].shape)), ql[b])
            qr[b] = np.copysign(np.exp2(rng.uniform(-40.0, 0.0, size=qr[b].shape)), qr[b])
            mr = 0.5
        else:
            ql[b] *= mq[b]
            qr[b] *= mq[b]
            mr = 3.0 / mq[b]
        w.rows[b * T:(b + 1) * T] *= np.float32(mr)
    w.q_lat = workloads.bf16_bits(ql.astype(np.float32))
    w.q_rope = workloads.bf16_bits(qr.astype(np.float32))
    assert np.all(np.isfinite(w.rows))
    w.softmax_scale = np.float32(1.0)
    cache = mx_cache(kv8, w.rows)
    run_case(kv8, w, cache=cache)
    run_case(kv8, w, splits=2, cache=cache)


def test_decode_rows_with_widely_spread_block_scales(kv8):
    """Blocks of one row 2^-40 .. 2^40 apart, rows of magnitude 1e-25 .. 1e20
    (every value finite in f32)."""
    w = workloads.tiny(seed=85, B=3, Q=1, H=32, T=400, outlier_p=0.0)
    rng = np.random.default_rng(86)
    w.rows *= (np.float32(2.0) ** rng.integers(-40, 41, (w.rows.shape[0], NB)).astype(np.float32)).repeat(32, axis=1)
    w.rows[:400] *= np.float32(1e-25)
    w.rows[800:] *= np.float32(1e20)
    assert np.all(np.isfinite(w.rows))
    run_case(kv8, w)
    run_case(kv8, w, splits=2)


def test_decode_batched_full_size_every_row(kv8):
    """B=32, T=8192, H=128 (the benchmark shape), all 4,096 output rows."""
    run_case(kv8, workloads.batched(seed=0), splits=8)
