"""kv8_absorb_decode_noalloc (split partials in the library's static device
array, no allocation in the call) against kv8_absorb_decode, through the C
ABI: two calls in a row, the second with a smaller input, each equal to the
allocating entry point bit for bit (same split plan and kernels), plus the
size limit of the static array."""
import numpy as np
import pytest

from fp8_e4m3_latent_amd import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 576


@pytest.fixture(scope="module")
def kv8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_e4m3_latent_amd as m
    m.lib()
    return m


def say(msg):
    print(msg, flush=True)


def device_inputs(kv8, w):
    src = torch.from_numpy(w.rows).cuda()
    codes = torch.empty((w.n_rows, D), dtype=torch.uint8, device="cuda")
    scales = torch.empty((w.n_rows, 2), dtype=torch.float32, device="cuda")
    kv8.quantize_rows(src, codes, scales)
    del src
    ql = torch.from_numpy(w.q_lat.view(np.int16)).cuda().view(torch.bfloat16)
    qr = torch.from_numpy(w.q_rope.view(np.int16)).cuda().view(torch.bfloat16)
    st = torch.from_numpy(w.kv_start.astype(np.int64)).cuda()
    ln = torch.from_numpy(w.kv_len.astype(np.int32)).cuda()
    return ql, qr, codes, scales, st, ln


def test_noalloc_equals_absorb_decode_on_two_calls(kv8):
    cases = [workloads.batched(seed=0),                              # 8 ranges, 34 MB of partials
             workloads.tiny(seed=5, B=3, Q=2, H=64, T=3000, outlier_p=0.0)]  # smaller: 3 ranges
    for w in cases:
        k, n = kv8.decode_plan(w.B, w.Q, w.H, w.max_len)
        say("noalloc: %s B=%d Q=%d H=%d T=%d plan=%d x %d partials=%d bytes" % (
            w.name, w.B, w.Q, w.H, w.max_len, n, k, kv8.partials_bytes(w.B, w.Q, w.H, n)))
        assert n > 1 and kv8.partials_bytes(w.B, w.Q, w.H, n) <= kv8.NOALLOC_SCRATCH_BYTES
        ql, qr, codes, scales, st, ln = device_inputs(kv8, w)
        out = torch.full((w.B, w.Q, w.H, 512), float("nan"), dtype=torch.float32, device="cuda")
        kv8.absorb_decode_noalloc(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale, out=out)
        ref = kv8.absorb_decode(ql, qr, codes, scales, st, ln, w.max_len, w.softmax_scale)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        assert torch.equal(out, ref)


def test_noalloc_rejects_partials_beyond_the_static_array(kv8):
    """B=64, Q=4, H=128, max_len 65,536: 16 ranges of partials (545 MB) exceed
    the 64 MiB array, which is an argument error (no launch)."""
    B, Q, H, T = 64, 4, 128, 65536
    k, n = kv8.decode_plan(B, Q, H, T)
    assert kv8.partials_bytes(B, Q, H, n) > kv8.NOALLOC_SCRATCH_BYTES
    ql = torch.zeros((B, Q, H, 512), dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros((B, Q, H, 64), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((1, D), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((1, 2), dtype=torch.float32, device="cuda")
    st = torch.zeros(B, dtype=torch.int64, device="cuda")
    ln = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(kv8.Kv8Error) as ei:
        kv8.absorb_decode_noalloc(ql, qr, codes, scales, st, ln, T, 1.0 / 24)
    assert ei.value.status == -4
