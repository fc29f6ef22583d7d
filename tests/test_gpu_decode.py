"""GPU parity of kv8_absorb_decode / kv8_absorb_decode_splitT against the oracle.

The cache is built by the GPU quantizer and checked bit-exact against the
oracle's codes first; both sides then decode the SAME codes, scales and bf16
queries (the kernel is compared with a host reference on the dequantized
cache, not with unquantized attention).  Bar: max|gpu - oracle| /
max|oracle| <= 1e-3 over every compared output row.
"""
import numpy as np
import pytest

import oracle
from fp8_e4m3_latent_amd import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

KL, KR, D = 512, 64, 576
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


def build_cache(kv8, rows, check=True):
    """GPU-quantize rows into a device cache; optionally check bit-exactness."""
    n = rows.shape[0]
    src = torch.from_numpy(np.ascontiguousarray(rows)).cuda()
    codes = torch.empty((max(n, 1), D), dtype=torch.uint8, device="cuda")
    scales = torch.empty((max(n, 1), 2), dtype=torch.float32, device="cuda")
    kv8.quantize_rows(src, codes, scales)
    torch.cuda.synchronize()
    del src
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    if check and n:
        rc, rs = oracle.quantize_rows(rows)
        assert np.array_equal(c[:n], rc), "quantized codes differ from the oracle"
        assert np.array_equal(s[:n].view(np.uint32), rs.view(np.uint32)), "scales differ"
    return codes, scales, c, s


def to_dev(w):
    ql = torch.from_numpy(w.q_lat.view(np.int16)).cuda().view(torch.bfloat16)
    qr = torch.from_numpy(w.q_rope.view(np.int16)).cuda().view(torch.bfloat16)
    st = torch.from_numpy(w.kv_start.astype(np.int64)).cuda()
    ln = torch.from_numpy(w.kv_len.astype(np.int32)).cuda()
    return ql, qr, st, ln


def rel_err(got, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def run_case(kv8, w, splits=None, sel=None, check_cache=True, cache=None):
    say("decode: %s B=%d Q=%d H=%d max_len=%d splits=%s" % (
        w.name, w.B, w.Q, w.H, w.max_len, splits))
    codes, scales, c, s = cache if cache is not None else build_cache(kv8, w.rows, check_cache)
    ql, qr, st, ln = to_dev(w)
    if splits is None:
        out = kv8.absorb_decode(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale)
    else:
        out = kv8.absorb_decode_splitT(ql, qr, codes, scales, st, ln, w.max_len,
                                       w.softmax_scale, splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, KL)
    ref = oracle.attention(w.q_lat, w.q_rope, c, s, w.kv_start, w.kv_len, Q=w.Q,
                           softmax_scale=w.softmax_scale, sel=sel)
    if sel is not None:
        got = got[sel]
    ref = ref.reshape(-1, KL)
    assert np.all(np.isfinite(got))
    e = rel_err(got, ref)
    say("  max|d|/max|ref| = %.3g" % e)
    assert e <= TOL, e
    return got, ref


def test_tiny_workload(kv8):
    """B=1, H=16, T=1024, outlier rows (x50), every output row."""
    run_case(kv8, workloads.tiny(seed=0))


def test_ragged_causal_multi_query_small(kv8):
    """Q=4 causal queries, H=128 (four 128-row blocks), lengths with ragged tails."""
    w = workloads.batched(seed=1, B=3, T=1, H=128, Q=4)
    rng = np.random.default_rng(2)
    lens = np.array([37, 1000, 300], np.int32)
    w.kv_len = lens
    w.kv_start = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    w.rows = rng.standard_normal((int(lens.sum()), D)).astype(np.float32)
    w.name = "ragged-small"
    run_case(kv8, w)


def test_heads_not_multiple_of_block(kv8):
    """Q*H = 48 rows: one partly filled row block."""
    w = workloads.tiny(seed=3, B=2, Q=3, H=16, T=333)
    run_case(kv8, w)


@pytest.mark.parametrize("splits", [1, 3, 7, 64])
def test_splitT_small(kv8, splits):
    w = workloads.tiny(seed=4, B=2, Q=1, H=128, T=5000, outlier_p=0.0)
    run_case(kv8, w, splits=splits)


def test_empty_and_short_sequences(kv8):
    """kv_len 0 -> zeros; kv_len 2 with Q=4 -> the first two queries see nothing."""
    w = workloads.tiny(seed=5, B=3, Q=4, H=16, T=40)
    w.kv_len = np.array([0, 2, 40], np.int32)
    w.kv_start = np.array([0, 0, 40], np.int64)
    got, ref = run_case(kv8, w)
    got = got.reshape(3, 4, 16, KL)
    assert not got[0].any() and not got[1, :2].any() and got[1, 2:].any()


def test_extreme_row_scales(kv8):
    """Rows of every finite magnitude: sequences whose rows have amax near
    1e-30, 1, 1e30, 1e34 and 1e36, one row at amax 3e38, a sequence with
    queries times 1e30 over rows times 1e30 (scores far beyond the f32
    range), and guarded (all-zero) rows next to rows a thousand times larger
    than the rest.  Direct output and split partials; every output finite."""
    T = 200
    mult = np.array([1e-30, 1.0, 1e30, 1e34, 1e36, 1.0, 1e30], np.float32)
    B = len(mult)
    w = workloads.tiny(seed=6, B=B, Q=1, H=32, T=T, outlier_p=0.0)
    for b in range(B):
        w.rows[b * T:(b + 1) * T] *= mult[b]
    w.rows[210:215] = 0.0
    w.rows[220] *= np.float32(1e3)
    w.rows[390] *= np.float32(1e3)
    r = 5 * T + 77  # one row at amax 3e38 (it dominates its sequence)
    w.rows[r] *= np.float32(3e38) / np.abs(w.rows[r]).max()
    ql = workloads.bf16_to_f32(w.q_lat)
    ql[6] *= np.float32(1e30)
    w.q_lat = workloads.bf16_bits(ql)
    assert np.all(np.isfinite(w.rows))
    cache = build_cache(kv8, w.rows)
    run_case(kv8, w, cache=cache)
    run_case(kv8, w, splits=3, cache=cache)


def test_query_rows_of_any_magnitude(kv8):
    """Query rows of every bf16 magnitude.  The score MFMAs take each query
    element as two e4m3 terms after dividing its row by a power of two; the
    sum of the terms must reproduce the bf16 element (exactly for elements
    of at least 2^-9 of the row's largest, and for every element of rows
    below 2^-119, whose elements are then mostly bf16 subnormals).  Sequences
    whose queries are scaled by 1e-37, 1e-30, 1e-6, 1e20 and 1e36 attend rows
    scaled by the inverse, with softmax scale 1 so that the scores spread
    over several natural-log units (a query error of 2^-10 would show), and
    one sequence's query elements are 2^U(-40, 0) with random signs (most of
    them below 2^-9 of their row's largest)."""
    T = 300
    mq = np.array([1e-37, 1e-30, 1e-6, 1.0, 1e20, 1e36, 1.0])
    B = len(mq)
    w = workloads.tiny(seed=41, B=B, Q=1, H=32, T=T, outlier_p=0.0)
    ql = workloads.bf16_to_f32(w.q_lat).astype(np.float64)
    qr = workloads.bf16_to_f32(w.q_rope).astype(np.float64)
    rng = np.random.default_rng(42)
    for b in range(B):
        if b == B - 1:
            mag = np.exp2(rng.uniform(-40.0, 0.0, size=ql[b].shape))
            ql[b] = np.copysign(mag, ql[b])
            mag = np.exp2(rng.uniform(-40.0, 0.0, size=qr[b].shape))
            qr[b] = np.copysign(mag, qr[b])
            mr = 0.5
        else:
            ql[b] *= mq[b]
            qr[b] *= mq[b]
            mr = 3.0 / mq[b]  # score std ~ 3 before the softmax scale
        w.rows[b * T:(b + 1) * T] *= np.float32(mr)
    w.q_lat = workloads.bf16_bits(ql.astype(np.float32))
    w.q_rope = workloads.bf16_bits(qr.astype(np.float32))
    assert np.all(np.isfinite(w.rows))
    assert np.all(np.isfinite(workloads.bf16_to_f32(w.q_lat)))
    w.softmax_scale = np.float32(1.0)
    cache = build_cache(kv8, w.rows)
    run_case(kv8, w, cache=cache)
    run_case(kv8, w, splits=2, cache=cache)


def test_non_finite_query_elements(kv8):
    """A query row with one NaN, +inf or -inf element (latent or rope part)
    gives an all-NaN output row, as the oracle's; every other row of the
    same blocks matches the oracle.  Direct output and split partials."""
    w = workloads.tiny(seed=43, B=2, Q=1, H=32, T=300, outlier_p=0.0)
    ql = workloads.bf16_to_f32(w.q_lat)
    qr = workloads.bf16_to_f32(w.q_rope)
    bad = [(0, 3), (0, 9), (1, 4), (1, 31)]
    ql[0, 0, 3, 17] = np.nan
    ql[0, 0, 9, 500] = np.inf
    qr[1, 0, 4, 5] = -np.inf
    ql[1, 0, 31, 0] = np.nan
    w.q_lat = workloads.bf16_bits(ql)
    w.q_rope = workloads.bf16_bits(qr)
    cache = build_cache(kv8, w.rows)
    codes, scales, c, s = cache
    ql_d, qr_d, st, ln = to_dev(w)
    ref = oracle.attention(w.q_lat, w.q_rope, c, s, w.kv_start, w.kv_len, Q=w.Q,
                           softmax_scale=w.softmax_scale).reshape(w.B, w.H, KL)
    nan_rows = np.zeros((w.B, w.H), bool)
    for b, h in bad:
        nan_rows[b, h] = True
    assert np.all(np.isnan(ref[nan_rows])) and np.all(np.isfinite(ref[~nan_rows]))
    for splits in (None, 3):
        say("decode: non-finite query elements, splits=%s" % splits)
        if splits is None:
            out = kv8.absorb_decode(ql_d, qr_d, codes, scales, st, ln, w.max_len, w.softmax_scale)
        else:
            out = kv8.absorb_decode_splitT(ql_d, qr_d, codes, scales, st, ln, w.max_len,
                                           w.softmax_scale, splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(w.B, w.H, KL)
        assert np.all(np.isnan(got[nan_rows]))
        assert np.all(np.isfinite(got[~nan_rows]))
        e = rel_err(got[~nan_rows], ref[~nan_rows])
        say("  max|d|/max|ref| over the finite rows = %.3g" % e)
        assert e <= TOL, e


def _unit(v):
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def test_small_lc_scales_carry_the_weight(kv8):
    """Every row but one is 2^-20 times smaller than the remaining row, whose
    scores are about -200 for every head: the weight sits on rows whose Lc
    scale is ~2^-27 of the range's largest, far below the fp16 range of the
    probability operands unless they are shifted (watched range)."""
    w = workloads.tiny(seed=30, B=1, Q=1, H=16, T=300, outlier_p=0.0)
    w.rows *= np.float32(2.0 ** -20)
    q = workloads.bf16_to_f32(w.q_lat[0, 0])
    w.rows[150, :KL] = -5000.0 * _unit(q).sum(0)
    run_case(kv8, w)
    run_case(kv8, w, splits=2)


def test_dominant_row_with_small_lc_scale(kv8):
    """One row scores ~40 above every other row through its Rc part while its
    Lc scale is 2^-20 of the range's largest: its probability operand would
    be an fp16 subnormal without the shift."""
    w = workloads.tiny(seed=31, B=1, Q=1, H=16, T=300, outlier_p=0.0)
    qr = workloads.bf16_to_f32(w.q_rope)
    qr[0, 0, :] = qr[0, 0, 0]  # one rope direction for every head
    w.q_rope = workloads.bf16_bits(qr)
    d = 120
    w.rows[d, :KL] *= np.float32(2.0 ** -20)
    u = qr[0, 0, 0]
    w.rows[d, KL:] = (40.0 * 24.0 / np.linalg.norm(u)) * _unit(u)
    got, ref = run_case(kv8, w)
    # the result is the dominant row's (tiny) Lc, not zero
    assert np.abs(ref).max() < 1e-5 and np.abs(got).max() > 0.5 * np.abs(ref).max()
    run_case(kv8, w, splits=3)


def test_guarded_rows_as_reference(kv8):
    """All-zero (guarded, scale 0) rows score 0 while every other row scores
    about -15: the reference rows carry no Lc, and the rows that make the
    output have probability operands near 2^-22."""
    w = workloads.tiny(seed=32, B=1, Q=1, H=16, T=300, outlier_p=0.0)
    ql = workloads.bf16_to_f32(w.q_lat)
    ql[0, 0, :] = ql[0, 0, 0]
    w.q_lat = workloads.bf16_bits(ql)
    w.q_rope[:] = 0
    q = ql[0, 0, 0]
    rng = np.random.default_rng(33)
    w.rows[:, :KL] = -(15.0 * 24.0 / np.linalg.norm(q)) * _unit(q) + \
        0.1 * rng.standard_normal((w.rows.shape[0], KL)).astype(np.float32)
    w.rows[50:55] = 0.0
    run_case(kv8, w)
    run_case(kv8, w, splits=4)


def test_cancelling_ranges_within_the_partials_bound(kv8):
    """Cancellation across ranges, for the 16-bit partials: the rows are c_t U
    with c_t ~ U[0.9, 1.1] in the first half and U[-1.0, -0.8] in the second,
    under a uniform softmax (zero queries).  Every range's normalised context
    then points along dec(U), so its 16-bit codes (and their rounding) are the
    same in every range, while the merged output ~0.05 U is 20x smaller than
    each range's context: inside the partials' bound (65x for the 1e-3 bar).
    (The per-token fp16 rounding of the probability operands differs from row
    to row here, because the row scales differ, and averages out.)"""
    w = workloads.tiny(seed=34, B=1, Q=1, H=16, T=2048, outlier_p=0.0)
    w.q_lat[:] = 0
    w.q_rope[:] = 0
    rng = np.random.default_rng(35)
    u = rng.standard_normal(D).astype(np.float32)
    c = np.concatenate([rng.uniform(0.9, 1.1, 1024), rng.uniform(-1.0, -0.8, 1024)]).astype(np.float32)
    w.rows[:] = c[:, None] * u[None, :]
    got, ref = run_case(kv8, w, splits=2)
    ratio = np.abs(u[:KL]).max() / np.abs(ref).max()
    say("  range context / merged output: %.1f" % ratio)
    assert 10.0 < ratio < 65.0


@pytest.mark.parametrize("T", [64, 96, 3072, 3104])
def test_tile_counts_around_the_buffer_ring(kv8, T):
    """2, 3, 96 and 97 tiles of 32 rows: every residue of the tile count
    modulo the four raw tile buffers (the tile loop is unrolled by four; the
    last iterations re-copy the last tile, and one re-copy goes into the
    buffer the epilogue reuses): the direct output (B=128, H=256: 256 blocks,
    one range each) and the partials of one range merged."""
    w = workloads.tiny(seed=36, B=128, Q=1, H=256, T=T, outlier_p=0.0)
    cache = build_cache(kv8, w.rows, check=False)
    sel = sample_rows(w.B, w.Q, w.H, 256, 37)
    run_case(kv8, w, splits=1, sel=sel, cache=cache)
    codes, scales, c, s = cache
    ql, qr, st, ln = to_dev(w)
    part = torch.empty(kv8.partials_bytes(w.B, w.Q, w.H, 1) // 4, dtype=torch.float32, device="cuda")
    kv8.absorb_decode_partials(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale, 0, 1, part)
    out = kv8.lse_merge(part, w.B, w.Q, w.H, 1, w.softmax_scale)
    torch.cuda.synchronize()
    ref = oracle.attention(w.q_lat, w.q_rope, c, s, w.kv_start, w.kv_len, Q=w.Q,
                           softmax_scale=w.softmax_scale, sel=sel)
    e = rel_err(out.cpu().numpy().reshape(-1, KL)[sel], ref.reshape(-1, KL))
    say("  partials: max|d|/max|ref| = %.3g" % e)
    assert e <= TOL, e


def test_reference_raise_restart(kv8):
    """A late tile scores ~20 natural-log units above the first tiles, forcing
    the block to raise its reference maximum and run its range again."""
    w = workloads.tiny(seed=7, B=1, Q=1, H=32, T=900, outlier_p=0.0)
    ql = workloads.bf16_to_f32(w.q_lat[0, 0])
    unit = ql / np.linalg.norm(ql, axis=1, keepdims=True)
    for k, t in enumerate([700, 701, 850]):
        h = k % 32
        # score = (1/24) * q_h . Lc_t = 20 (natural-log units) for head h
        w.rows[t, :KL] = (20.0 * 24.0 / np.linalg.norm(ql[h])) * unit[h]
    run_case(kv8, w)


def test_negative_and_zero_softmax_scale(kv8):
    w = workloads.tiny(seed=8, B=2, Q=2, H=16, T=300)
    w.softmax_scale = np.float32(-1.0 / 24.0)
    run_case(kv8, w)
    w.softmax_scale = np.float32(0.0)
    run_case(kv8, w)


def test_deterministic(kv8):
    w = workloads.tiny(seed=9, B=2, Q=1, H=128, T=3000)
    codes, scales, c, s = build_cache(kv8, w.rows)
    ql, qr, st, ln = to_dev(w)
    a = kv8.absorb_decode(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale)
    b = kv8.absorb_decode(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_argument_errors(kv8):
    w = workloads.tiny(seed=10, B=1, Q=1, H=16, T=64)
    codes, scales, c, s = build_cache(kv8, w.rows)
    ql, qr, st, ln = to_dev(w)
    with pytest.raises(kv8.Kv8Error):
        kv8.absorb_decode_splitT(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale,
                                 num_splits=0)
    with pytest.raises(kv8.Kv8Error):
        kv8.absorb_decode(ql, qr, codes, scales, st, ln, w.max_len, float("nan"))
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(kv8.Kv8Error):
        kv8.absorb_decode_splitT(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale,
                                 num_splits=4, workspace=small)


# ---------------------------------------------------------------- full sizes

def sample_rows(B, Q, H, n, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(B * Q * H, size=min(n, B * Q * H), replace=False)).astype(np.int64)


def test_batched_full_size_every_row(kv8):
    """B=32, T=8192, H=128 (the benchmark launch), all 4,096 output rows."""
    w = workloads.batched(seed=0)
    run_case(kv8, w)


def test_long_context_splitT_full_size_every_row(kv8):
    """B=1, T=262144, H=128, 64 split ranges merged by log-sum-exp, with the
    planted strong matches (about 10 rows per head scoring ~3.5 natural-log
    units above the ordinary rows).  All 128 output rows."""
    w = workloads.long_context(seed=0)
    run_case(kv8, w, splits=64)


def ragged_subset(w, n=8):
    """Every output row (all Q positions and heads) of n sequences spread over
    the length range: the sequences at ranks 0, 8, ... of the sorted lengths."""
    order = np.argsort(w.kv_len, kind="stable")[:: max(1, w.B // n)][:n]
    seqs = np.sort(order)
    rows = [(b * w.Q + i) * w.H + h for b in seqs for i in range(w.Q) for h in range(w.H)]
    return seqs, np.array(rows, np.int64)


def test_ragged_full_size_subset_every_row(kv8):
    """B=64, lengths U[1k, 64k], Q=4 causal, whole cache quantized on the GPU;
    every row of 8 sequences spread over the length range (4,096 rows)."""
    w = workloads.ragged(seed=0)
    seqs, sel = ragged_subset(w)
    say("  ragged subset: sequences %s, lengths %s" % (list(seqs), list(w.kv_len[seqs])))
    run_case(kv8, w, sel=sel)


def test_two_stage_equals_single_call(kv8):
    """kv8_absorb_decode_partials + kv8_lse_merge with kv8_decode_plan's split
    reproduces kv8_absorb_decode bit for bit."""
    w = workloads.tiny(seed=21, B=4, Q=1, H=128, T=4000, outlier_p=0.0)
    codes, scales, c, s = build_cache(kv8, w.rows)
    ql, qr, st, ln = to_dev(w)
    a = kv8.absorb_decode(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale)
    k, n = kv8.decode_plan(w.B, w.Q, w.H, w.max_len)
    assert n > 1
    part = torch.empty(kv8.partials_bytes(w.B, w.Q, w.H, n) // 4, dtype=torch.float32,
                       device="cuda")
    kv8.absorb_decode_partials(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale, k, n,
                               part)
    b = kv8.lse_merge(part, w.B, w.Q, w.H, n, w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_partials_of_two_shards_merge(kv8):
    """Token ranges computed separately (as two devices holding halves of each
    sequence would) merge into the full decode."""
    w = workloads.tiny(seed=22, B=2, Q=1, H=32, T=3000, outlier_p=0.0)
    codes, scales, c, s = build_cache(kv8, w.rows)
    ql, qr, st, ln = to_dev(w)
    half = w.kv_len // 2
    shards = [(st, torch.from_numpy(half.astype(np.int32)).cuda()),
              (st + torch.from_numpy(half.astype(np.int64)).cuda(),
               torch.from_numpy((w.kv_len - half).astype(np.int32)).cuda())]
    R = w.Q * w.H
    parts = []
    for s0, l0 in shards:
        p = torch.empty(kv8.partials_bytes(w.B, w.Q, w.H, 1) // 4, dtype=torch.float32,
                        device="cuda")
        kv8.absorb_decode_partials(ql, qr, codes, scales, s0, l0, w.max_len, w.softmax_scale,
                                   0, 1, p)
        parts.append(p)
    n_o = w.B * R * KL // 2  # (int16 codes of O, in f32 units of the buffer)
    merged = torch.cat([parts[0][:n_o], parts[1][:n_o], parts[0][n_o:], parts[1][n_o:]])
    out = kv8.lse_merge(merged, w.B, w.Q, w.H, 2, w.softmax_scale)
    torch.cuda.synchronize()
    ref = oracle.attention(w.q_lat, w.q_rope, c, s, w.kv_start, w.kv_len, Q=w.Q,
                           softmax_scale=w.softmax_scale)
    e = rel_err(out.cpu().numpy().reshape(-1, KL), ref.reshape(-1, KL))
    assert e <= TOL, e


def test_step_graph_replay_matches_eager(kv8):
    """A decode step (append of one fresh row per sequence, split partials,
    merge) captured in a HIP graph and replayed three times, with eager steps
    and synchronisations between the replays, reproduces the eager step bit
    for bit on every replay; the eager step itself matches the oracle on the
    appended cache."""
    w = workloads.tiny(seed=23, B=4, Q=1, H=128, T=3000, outlier_p=0.0)
    codes, scales, _, _ = build_cache(kv8, w.rows)
    ql, qr, st, ln = to_dev(w)
    fresh_h = workloads.fresh_rows(24, w.B)
    fresh = torch.from_numpy(fresh_h).cuda()
    dst = st + (ln.to(torch.int64) - 1)
    k, n = kv8.decode_plan(w.B, w.Q, w.H, w.max_len)
    part = torch.empty(kv8.partials_bytes(w.B, w.Q, w.H, n) // 4, dtype=torch.float32,
                       device="cuda")
    out = torch.empty((w.B, w.Q, w.H, KL), dtype=torch.float32, device="cuda")

    def step():
        kv8.quantize_rows(fresh, codes, scales, dst_rows=dst)
        kv8.absorb_decode_partials(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale,
                                   k, n, part)
        kv8.lse_merge(part, w.B, w.Q, w.H, n, w.softmax_scale, out)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    o = oracle.attention(w.q_lat, w.q_rope, c, s, w.kv_start, w.kv_len, Q=w.Q,
                         softmax_scale=w.softmax_scale)
    assert rel_err(ref.cpu().numpy().reshape(-1, KL), o.reshape(-1, KL)) <= TOL

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        step()                      # eager work between the replays
        torch.cuda.synchronize()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("graph replay %d" % r)
        assert torch.equal(out, ref), "replay %d differs from the eager step" % r
