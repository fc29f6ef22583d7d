"""GPU parity of kv8_norm_rope_quantize_rows (the producer step fused with the
quantizer) against the oracle's norm_rope_rows followed by its quantizer.

Page: "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
(colibri PR #299), commit message, attention_rows item.

The kernel forms y in f32 (sum of squares reduced in f32, f32 sincos), the
oracle in f64, so a quantized code may differ by one e4m3 step where the
oracle's scaled value sits next to the midpoint between two codes.  The bar:
scales within a relative 2e-5; every differing code is a neighbour of the
oracle's code and the oracle's scaled value lies within a relative 1e-4 of
their midpoint, plus, times the segment's inverse scale, 8 f32 subnormal
steps of y (values the f32 products round among the subnormals) and for Rc
1e-6 of the source pair's norm (the rotation errs relative to the pair); at
most 1e-3 of the codes differ.  Rows whose result the f32
rounding cannot change (NaN, inf, zero rows) must match bit for bit.
"""
import numpy as np
import pytest

import oracle
from fp8_e4m3_latent_amd import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

KL, KR, D = 512, 64, 576
VALUES = None


@pytest.fixture(scope="module")
def kv8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_e4m3_latent_amd as m
    m.lib()
    return m


def say(msg):
    print(msg, flush=True)


def code_values():
    global VALUES
    if VALUES is None:
        VALUES = oracle.decode(np.arange(256, dtype=np.uint8))
    return VALUES


def inputs(seed, n, pos_max=262144):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, D)).astype(np.float32) * np.float32(2.0)
    w = g.uniform(0.25, 2.0, KL).astype(np.float32)
    pos = g.integers(0, pos_max, n).astype(np.int64)
    return x, w, pos


def gpu_run(kv8, x, w, eps, pos, theta, dst=None, n_cache=None):
    n = x.shape[0]
    rows = n if n_cache is None else n_cache
    codes = torch.zeros((max(rows, 1), D), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((max(rows, 1), 2), dtype=torch.float32, device="cuda")
    d = None if dst is None else torch.from_numpy(dst).cuda()
    kv8.norm_rope_quantize_rows(torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(), eps,
                                torch.from_numpy(pos).cuda(), theta, codes, scales, dst_rows=d)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def oracle_run(x, w, eps, pos, theta, dst=None, n_cache=None):
    y = oracle.norm_rope_rows(x, w, eps, pos, theta)
    c, s = oracle.quantize_rows(y, dst_rows=dst, n_cache_rows=n_cache)
    return y, c, s


def compare(x, y, gc, gs, oc, os_, exact=False):
    """The bar stated in the module docstring; x the source rows, y, oc, os_ the
    oracle's."""
    if exact:
        assert np.array_equal(gc, oc), "codes differ"
        assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"
        return 0
    np.testing.assert_allclose(gs, os_, rtol=2e-5, atol=0)
    bad = np.nonzero(gc != oc)
    if bad[0].size == 0:
        return 0
    assert bad[0].size <= 1e-3 * gc.size, "%d of %d codes differ" % (bad[0].size, gc.size)
    v = code_values()
    vg, vo = v[gc[bad]], v[oc[bad]]
    r, col = bad
    seg = (col >= KL).astype(np.int64)
    # the oracle's scaled value q = fl32(y * inv), inv = fl32(448 / amax)
    yy = y[r, col]
    amax = np.where(seg == 0, np.nanmax(np.where(np.isfinite(y[:, :KL]), np.abs(y[:, :KL]), 0), axis=1)[r],
                    np.nanmax(np.where(np.isfinite(y[:, KL:]), np.abs(y[:, KL:]), 0), axis=1)[r])
    inv = (np.float32(448.0) / amax.astype(np.float32)).astype(np.float32)
    q = (yy * inv).astype(np.float64)
    mid = (vg + vo) / 2
    lo = np.minimum(np.abs(vg), np.abs(vo))
    step = np.where(lo >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(lo, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(vg - vo) <= step * (1 + 1e-12)), "a differing code is not a neighbour"
    # relative 1e-4 of the midpoint, plus, scaled by inv: 8 f32 subnormal
    # steps of y (2^-149 each; f32 products that land among the subnormals
    # are rounded to an absolute step, the oracle's f64 values only once) and,
    # for Rc, 1e-6 of the source pair's norm (the f32 sincos and products err
    # relative to the pair, which a small rotated value does not show)
    p0 = np.where(seg == 1, KL + ((col - KL) & ~1), 0)
    pair = np.where(seg == 1, np.hypot(x[r, p0].astype(np.float64), x[r, p0 + 1].astype(np.float64)), 0.0)
    tol = 1e-4 * np.abs(mid) + (8.0 * 2.0 ** -149 + 1e-6 * pair) * inv.astype(np.float64)
    far = np.abs(q - mid) > tol
    assert not far.any(), "a differing code is not at a midpoint: row %s col %s y %s q %s mid %s" % (
        r[far][:4], col[far][:4], yy[far][:4], q[far][:4], mid[far][:4])
    return bad[0].size


@pytest.mark.parametrize("n", [1, 3, 37, 1000, 9000])
def test_producer_row_counts(kv8, n):
    """Row counts on both launch shapes (one row per wave below 8,192 rows,
    eight above), positions up to 2^18."""
    say("producer: n=%d" % n)
    x, w, pos = inputs(100 + n, n)
    gc, gs = gpu_run(kv8, x, w, 1e-6, pos, 10000.0)
    y, oc, os_ = oracle_run(x, w, 1e-6, pos, 10000.0)
    nd = compare(x, y, gc[:n], gs[:n], oc, os_)
    say("  codes differing by one step at a midpoint: %d of %d" % (nd, gc[:n].size))


def test_producer_scatter_and_stride(kv8):
    """dst_rows scatter into a larger cache and a source row stride above 576."""
    n, rows = 300, 1000
    x, w, pos = inputs(7, n)
    wide = np.zeros((n, D + 64), np.float32)
    wide[:, :D] = x
    dst = np.random.default_rng(8).permutation(rows)[:n].astype(np.int64)
    codes = torch.zeros((rows, D), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((rows, 2), dtype=torch.float32, device="cuda")
    kv8.norm_rope_quantize_rows(torch.from_numpy(wide).cuda(), torch.from_numpy(w).cuda(), 1e-6,
                                torch.from_numpy(pos).cuda(), 10000.0, codes, scales,
                                dst_rows=torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    y, oc, os_ = oracle_run(wide, w, 1e-6, pos, 10000.0, dst=dst, n_cache=rows)
    untouched = np.setdiff1d(np.arange(rows), dst)
    assert not gc[untouched].any() and not gs[untouched].any()
    compare(x, y, gc[dst], gs[dst], oc[dst], os_[dst])


def test_producer_special_rows_exact(kv8):
    """NaN, inf and zero rows, and eps = 0 on a zero row (0/0): the segments
    whose result the f32 rounding cannot change match bit for bit (an inf or
    NaN in Lc turns the whole segment into zeros or NaN; an inf in Rc
    saturates its own pair only)."""
    x, w, pos = inputs(9, 6)
    x[0, :] = 0.0
    x[1, 5] = np.nan
    x[2, 300] = np.inf
    x[3, KL + 3] = -np.inf
    x[4, KL:] = np.nan
    x[5, :KL] = -0.0
    for eps in (1e-6, 0.0):
        gc, gs = gpu_run(kv8, x, w, eps, pos, 10000.0)
        y, oc, os_ = oracle_run(x, w, eps, pos, 10000.0)
        for r in (0, 1, 2, 5):      # Lc segments
            assert np.array_equal(gc[r, :KL], oc[r, :KL]), (eps, r)
            assert gs[r, 0].view(np.uint32) == os_[r, 0].view(np.uint32), (eps, r)
        # Rc all NaN: codes 0, guarded scale 0
        assert not gc[4, KL:].any() and gs[4, 1] == 0 and not oc[4, KL:].any() and os_[4, 1] == 0
        # Rc with -inf in pair 1: that pair saturates; the other pairs (which set
        # the scale) are ordinary rotated values, compared to the general bar
        assert np.array_equal(gc[3, KL + 2:KL + 4], oc[3, KL + 2:KL + 4]), eps
        compare(x[3:4], y[3:4], gc[3:4], gs[3:4], oc[3:4], os_[3:4])


def test_producer_position_zero_equals_plain_quantizer_on_rc(kv8):
    """At position 0 the Rc codes and scale equal the plain quantizer's on the raw
    Rc values, bit for bit (the rotation is the identity)."""
    x, w, _ = inputs(10, 64)
    pos = np.zeros(64, np.int64)
    gc, gs = gpu_run(kv8, x, w, 1e-6, pos, 10000.0)
    oc, os_ = oracle.quantize_rows(x)
    assert np.array_equal(gc[:, KL:], oc[:, KL:])
    assert np.array_equal(gs[:, 1].view(np.uint32), os_[:, 1].view(np.uint32))


def test_producer_bulk_rows_sampled(kv8):
    """262,144 rows of the bulk distribution (Student-t with the planted special
    rows) through both launch shapes' bulk path."""
    rows, _ = workloads.bulk_rows(seed=0)
    x = np.ascontiguousarray(rows[:262144])
    del rows
    g = np.random.default_rng(11)
    w = g.uniform(0.25, 2.0, KL).astype(np.float32)
    pos = g.integers(0, 262144, x.shape[0]).astype(np.int64)
    say("producer: bulk %d rows" % x.shape[0])
    gc, gs = gpu_run(kv8, x, w, 1e-6, pos, 10000.0)
    y, oc, os_ = oracle_run(x, w, 1e-6, pos, 10000.0)
    nd = compare(x, y, gc, gs, oc, os_)
    say("  codes differing by one step at a midpoint: %d of %d" % (nd, gc.size))


def test_producer_argument_errors(kv8):
    x, w, pos = inputs(12, 4)
    codes = torch.zeros((4, D), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((4, 2), dtype=torch.float32, device="cuda")
    xs, ws, ps = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(), torch.from_numpy(pos).cuda()
    for eps, theta in ((-1.0, 10000.0), (float("nan"), 10000.0), (1e-6, 0.0), (1e-6, float("inf"))):
        with pytest.raises(kv8.Kv8Error):
            kv8.norm_rope_quantize_rows(xs, ws, eps, ps, theta, codes, scales)
    with pytest.raises(ValueError):
        kv8.norm_rope_quantize_rows(xs, ws[:100], 1e-6, ps, 10000.0, codes, scales)
    with pytest.raises(ValueError):
        kv8.norm_rope_quantize_rows(xs, ws, 1e-6, ps[:3], 10000.0, codes, scales)


def test_producer_append_then_decode(kv8):
    """One decode step as the page describes it: the producer normalises, rotates
    and quantizes each sequence's fresh row into the cache at the sequence's
    newest position, and the absorbed decode reads the updated cache.  The
    oracle runs the same two steps; the decode must match it within 1e-3 on the
    cache the GPU wrote (whose appended codes are checked to the producer's bar
    against the oracle's first)."""
    w = workloads.tiny(seed=31, B=4, Q=1, H=128, T=2000, outlier_p=0.0)
    src = torch.from_numpy(np.ascontiguousarray(w.rows)).cuda()
    codes = torch.empty((w.n_rows, D), dtype=torch.uint8, device="cuda")
    scales = torch.empty((w.n_rows, 2), dtype=torch.float32, device="cuda")
    kv8.quantize_rows(src, codes, scales)
    g = np.random.default_rng(32)
    fresh = (g.standard_normal((w.B, D)) * 3.0).astype(np.float32)
    wt = g.uniform(0.5, 1.5, KL).astype(np.float32)
    dst = (w.kv_start + w.kv_len - 1).astype(np.int64)
    pos = (w.kv_len - 1).astype(np.int64)
    kv8.norm_rope_quantize_rows(torch.from_numpy(fresh).cuda(), torch.from_numpy(wt).cuda(), 1e-6,
                                torch.from_numpy(pos).cuda(), 10000.0, codes, scales,
                                dst_rows=torch.from_numpy(dst).cuda())
    ql = torch.from_numpy(w.q_lat.view(np.int16)).cuda().view(torch.bfloat16)
    qr = torch.from_numpy(w.q_rope.view(np.int16)).cuda().view(torch.bfloat16)
    out = kv8.absorb_decode(ql, qr, codes, scales, torch.from_numpy(w.kv_start).cuda(),
                            torch.from_numpy(w.kv_len).cuda(), w.max_len, w.softmax_scale)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    # the oracle's cache: its quantizer on the rows, its producer on the fresh rows
    y, oc, os_ = oracle_run(fresh, wt, 1e-6, pos, 10000.0)
    compare(fresh, y, c[dst], s[dst], oc, os_)
    rc, rs = oracle.quantize_rows(w.rows)
    keep = np.setdiff1d(np.arange(w.n_rows), dst)
    assert np.array_equal(c[keep], rc[keep]) and np.array_equal(s[keep].view(np.uint32), rs[keep].view(np.uint32))
    ref = oracle.attention(w.q_lat, w.q_rope, c, s, w.kv_start, w.kv_len, Q=w.Q,
                           softmax_scale=w.softmax_scale)
    got = out.cpu().numpy().reshape(ref.shape)
    e = float(np.abs(got - ref).max() / np.abs(ref).max())
    say("  append + decode: max|d|/max|ref| = %.2e" % e)
    assert e <= 1e-3
