"""GPU parity of kv8_project_rows (non-absorbed projection of fp8 cache rows)
against the oracle's project_rows.

Page: "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2"
(colibri PR #299), commit message, attention_rows item.

The kernel sums bf16 x bf16 products in f32 (every e4m3 value is exact in
bf16) and scales the sum; the oracle sums in f64.  Bar per element: |gpu - ref|
<= e |ref| + 2^-20 s_Lc sum_k |dec(c_k)| |W_nk|, e = 2^-8 for the bf16 output
(one rounding to bf16) and 2^-23 for the f32 output (the rounding of the
scale's product), plus the f32 accumulation of 512 exact products.  The
dequantized Rc (one f32 product of exact values) must equal the oracle's
value rounded to f32, bit for bit.
"""
import numpy as np
import pytest

import oracle

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


def gpu_cache(kv8, n, seed):
    x = np.random.default_rng(seed).standard_normal((n, D)).astype(np.float32)
    x[::7, :KL] *= np.float32(30.0)            # rows of very different scales
    codes = torch.empty((n, D), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, 2), dtype=torch.float32, device="cuda")
    kv8.quantize_rows(torch.from_numpy(x).cuda(), codes, scales)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    rc, rs = oracle.quantize_rows(x)
    assert np.array_equal(c, rc) and np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    return codes, scales, c, s


def weights(N, seed):
    w = torch.from_numpy(np.random.default_rng(seed).standard_normal((N, KL)).astype(np.float32) * 0.05)
    wb = w.to(torch.bfloat16)
    return wb.cuda(), wb.view(torch.int16).numpy().view(np.uint16)


def check(c, s, wbits, rows, got, got_rope):
    ref, rref = oracle.project_rows(c[rows], s[rows], wbits)
    g = got.float().cpu().numpy().astype(np.float64)[rows] if got.shape[0] != len(rows) else got.float().cpu().numpy().astype(np.float64)
    x = np.abs(oracle.decode(c[rows, :KL])) * s[rows, :1].astype(np.float64)
    wv = np.abs((wbits.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    e = 2.0 ** -23 if got.dtype == torch.float32 else 2.0 ** -8
    bound = e * np.abs(ref) + 2.0 ** -20 * (x @ wv.T)
    err = np.abs(g - ref)
    assert np.all(err <= bound), "max err/bound %.3f" % float(np.max(err / np.maximum(bound, 1e-300)))
    if got_rope is not None:
        gr = got_rope.cpu().numpy()
        gr = gr[rows] if gr.shape[0] != len(rows) else gr
        assert np.array_equal(gr.view(np.uint32), rref.astype(np.float32).view(np.uint32))
    return float(np.max(err / np.maximum(np.abs(ref).max(), 1e-300)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,N", [(1, 128), (100, 256), (300, 384), (1000, 128), (513, 640)])
def test_project_small(kv8, n, N, dtype):
    """Row counts below, at and across the 256-row tile, several column tiles
    (N = 128 and 384 end in half a column tile)."""
    say("project: n=%d N=%d %s" % (n, N, dtype))
    codes, scales, c, s = gpu_cache(kv8, n, 40 + n)
    wb, wbits = weights(N, 41 + N)
    out, rope = kv8.project_rows(codes, scales, wb,
                                 out_dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    e = check(c, s, wbits, np.arange(n), out, rope)
    say("  max |err| / max |ref| = %.2e" % e)


def test_project_slice_of_cache_and_no_rope(kv8):
    """A slice starting at a nonzero cache row; no Rc output requested."""
    codes, scales, c, s = gpu_cache(kv8, 700, 50)
    wb, wbits = weights(256, 51)
    out, rope = kv8.project_rows(codes[200:530], scales[200:530], wb, with_rope=False)
    torch.cuda.synchronize()
    assert rope is None
    check(c[200:530], s[200:530], wbits, np.arange(330), out, None)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_project_full_size(kv8, dtype):
    """8,192 rows (one 8k-token sequence) x N = 32,768 (128 heads x (128 + 128)):
    every row of the first 128 columns, and 48 sampled rows over every
    column."""
    n, N = 8192, 32768
    say("project: full size n=%d N=%d %s" % (n, N, dtype))
    codes, scales, c, s = gpu_cache(kv8, n, 52)
    wb, wbits = weights(N, 53)
    out, rope = kv8.project_rows(codes, scales, wb,
                                 out_dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    e0 = check(c, s, wbits[:128], np.arange(n), out[:, :128], rope)
    say("  columns 0..127, every row: max |err| / max |ref| = %.2e" % e0)
    rows = np.sort(np.random.default_rng(54).choice(n, 48, replace=False))
    ot = out[torch.from_numpy(rows).cuda()]
    rt = rope[torch.from_numpy(rows).cuda()]
    e = check(c, s, wbits, rows, ot, rt)
    say("  48 rows, every column: max |err| / max |ref| = %.2e" % e)


def test_project_argument_errors(kv8):
    codes, scales, _, _ = gpu_cache(kv8, 4, 55)
    wb, _ = weights(100, 56)      # N not a multiple of 128
    with pytest.raises(kv8.Kv8Error):
        kv8.project_rows(codes, scales, wb)
    with pytest.raises(ValueError):
        kv8.project_rows(codes, scales[:3], weights(128, 57)[0])


def test_project_degenerate_rows_and_empty(kv8):
    """Rows the quantizer treats specially: all zero (both scales 0), zero Lc or
    zero Rc only, a subnormal amax (stored as scale 0), Lc scaled by 1e30 and
    by 1e-30, a NaN element (stored as code 0) and a constant row at the e4m3
    maximum.  Zero-scale parts must project to exact zeros; n = 0 is a no-op."""
    x = np.random.default_rng(60).standard_normal((8, D)).astype(np.float32)
    x[0] = 0.0
    x[1, :KL] = 0.0
    x[2, KL:] = 0.0
    x[3] = np.float32(1e-40) * np.sign(x[3])
    x[4, :KL] *= np.float32(1e30)
    x[5, 10] = np.nan
    x[6, :KL] = 448.0
    x[7, :KL] *= np.float32(1e-30)
    codes = torch.empty((8, D), dtype=torch.uint8, device="cuda")
    scales = torch.empty((8, 2), dtype=torch.float32, device="cuda")
    kv8.quantize_rows(torch.from_numpy(x).cuda(), codes, scales)
    wb, wbits = weights(256, 61)
    out, rope = kv8.project_rows(codes, scales, wb)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    rc, rs = oracle.quantize_rows(x)
    assert np.array_equal(c, rc) and np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    check(c, s, wbits, np.arange(8), out, rope)
    o = out.float().cpu().numpy()
    assert not np.any(np.isnan(o))
    assert np.all(o[[0, 1, 3]] == 0.0)
    assert np.all(rope.cpu().numpy()[[0, 2, 3]] == 0.0)
    e_out, e_rope = kv8.project_rows(codes[:0], scales[:0], wb)
    torch.cuda.synchronize()
    assert tuple(e_out.shape) == (0, 256) and tuple(e_rope.shape) == (0, 64)
