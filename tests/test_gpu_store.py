"""The device slot pool of include/kv8_pool.h on the GPU: resume of an f32
store through the device quantizer (codes bit-exact with the oracle, file
untouched), the first save rewriting it in fp8, reload into another slot,
and a decode over pool slots against the oracle.

Page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2" (colibri
PR #299): commit message, first paragraph and .coli_kv v2 item.
"""
import hashlib

import numpy as np
import pytest

import oracle
from fp8_e4m3_latent_amd import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

L, W, KL = 2, 576, 512


@pytest.fixture(scope="module")
def kv8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_e4m3_latent_amd as m
    m.lib()
    return m


def say(msg):
    print(msg, flush=True)


def test_pool_resume_save_reload_and_decode(kv8, tmp_path):
    from fp8_e4m3_latent_amd import store
    p = str(tmp_path / "slot.kv8")
    n0, n1 = 5000, 700                      # tokens on disk (f32), tokens appended after resume
    rows = np.random.default_rng(60).standard_normal((n0 + n1, L, W)).astype(np.float32)
    rows[::97] *= np.float32(40.0)
    store.write_f32(p, rows[:n0])
    digest = hashlib.sha256(open(p, "rb").read()).hexdigest()

    pool = store.Pool(L, 3, 8192)
    try:
        assert pool.used_bytes() == store.pool_bytes(L, 3, 8192) == L * 3 * 8192 * 584
        say("pool: resume an f32 store of %d tokens into slot 1" % n0)
        with store.Store(p, L) as st:
            assert st.info() == (store.DTYPE_F32, n0)
            pool.load(1, st)
        torch.cuda.synchronize()
        assert pool.len(1) == n0
        assert hashlib.sha256(open(p, "rb").read()).hexdigest() == digest  # file untouched
        base = pool.slot_row(1)
        for l in range(L):
            c, s = pool.layer(l)
            rc, rs = oracle.quantize_rows(np.ascontiguousarray(rows[:n0, l]))
            assert np.array_equal(c[base:base + n0].cpu().numpy(), rc)
            assert np.array_equal(s[base:base + n0].cpu().numpy().view(np.uint32), rs.view(np.uint32))

        say("pool: append %d rows per layer with the quantizer, save (rewrites the store in fp8)" % n1)
        for l in range(L):
            c, s = pool.layer(l)
            dst = torch.arange(base + n0, base + n0 + n1, dtype=torch.int64, device="cuda")
            kv8.quantize_rows(torch.from_numpy(np.ascontiguousarray(rows[n0:, l])).cuda(), c, s, dst_rows=dst)
        torch.cuda.synchronize()
        pool.set_len(1, n0 + n1)
        with store.Store(p, L) as st:
            pool.save(1, st)
            assert st.info() == (store.DTYPE_E4M3, n0 + n1)
        with store.Store(p, L) as st:
            fc, fs = st.read()
        for l in range(L):
            rc, rs = oracle.quantize_rows(np.ascontiguousarray(rows[:, l]))
            assert np.array_equal(fc[:, l], rc) and np.array_equal(fs[:, l].view(np.uint32), rs.view(np.uint32))

        say("pool: reload the fp8 store into slot 2; append-only save of 0 new tokens")
        with store.Store(p, L) as st:
            pool.load(2, st)
            pool.save(2, st)                     # nothing new: no change
            assert st.info() == (store.DTYPE_E4M3, n0 + n1)
        b2 = pool.slot_row(2)
        for l in range(L):
            c, s = pool.layer(l)
            assert torch.equal(c[b2:b2 + n0 + n1], c[base:base + n0 + n1])
            assert torch.equal(s[b2:b2 + n0 + n1], s[base:base + n0 + n1])

        say("pool: decode over slots 1 and 2 of layer 1 (lengths %d, %d)" % (n0 + n1, n0 + 300))
        pool.set_len(2, n0 + 300)
        c, s = pool.layer(1)
        w = workloads.tiny(seed=61, B=2, Q=1, H=32, T=8, outlier_p=0.0)
        st_ = torch.tensor([base, b2], dtype=torch.int64, device="cuda")
        ln_ = torch.tensor([n0 + n1, n0 + 300], dtype=torch.int32, device="cuda")
        ql = torch.from_numpy(w.q_lat.view(np.int16)).cuda().view(torch.bfloat16)
        qr = torch.from_numpy(w.q_rope.view(np.int16)).cuda().view(torch.bfloat16)
        out = kv8.absorb_decode(ql, qr, c, s, st_, ln_, n0 + n1, w.softmax_scale)
        torch.cuda.synchronize()
        hc, hs = c.cpu().numpy(), s.cpu().numpy()
        ref = oracle.attention(w.q_lat, w.q_rope, hc, hs, np.array([base, b2], np.int64),
                               np.array([n0 + n1, n0 + 300], np.int32), Q=1, softmax_scale=w.softmax_scale)
        got = out.cpu().numpy().reshape(-1, KL)
        e = float(np.abs(got - ref.reshape(-1, KL)).max() / np.abs(ref).max())
        say("  max|d|/max|ref| = %.3g" % e)
        assert e <= 1e-3
    finally:
        pool.destroy()
