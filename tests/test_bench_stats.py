"""CPU check of the long-context workload statistics the bench reports
(largest softmax weight per head, weight on the head's own planted rows):
torch on the CPU against a direct f64 computation with the oracle's decode of
the same codes."""
import numpy as np
import pytest

import oracle
from fp8_e4m3_latent_amd import workloads

torch = pytest.importorskip("torch")


def test_long_context_stats_match_a_direct_softmax():
    import bench
    w = workloads.long_context(seed=3, T=4096, H=16)
    c, s = oracle.quantize_rows(w.rows)
    ql = torch.from_numpy(w.q_lat.view(np.int16)).view(torch.bfloat16)
    qr = torch.from_numpy(w.q_rope.view(np.int16)).view(torch.bfloat16)
    got = bench.long_context_stats(torch, w, torch.from_numpy(c), torch.from_numpy(s), ql, qr)

    x = oracle.decode(c).astype(np.float64)                      # [T, 576] e4m3 values
    lc = x[:, :512] * s[:, :1].astype(np.float64)
    rc = x[:, 512:] * s[:, 1:2].astype(np.float64)
    qlf = workloads.bf16_to_f32(w.q_lat).reshape(-1, 512).astype(np.float64)
    qrf = workloads.bf16_to_f32(w.q_rope).reshape(-1, 64).astype(np.float64)
    sc = float(w.softmax_scale) * (qlf @ lc.T + qrf @ rc.T)        # [H, T]
    p = np.exp(sc - sc.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    pos, heads = w.notes["planted_rows"], w.notes["planted_heads"]
    mass = np.zeros(w.H)
    np.add.at(mass, heads, p[heads, pos])
    maxp = p.max(axis=1)
    for key, ref in (("max_p", maxp), ("planted_mass", mass)):
        want = [ref.min(), np.median(ref), ref.max()]
        assert np.allclose(got[key], want, rtol=1e-4, atol=1e-9), (key, got[key], want)
    assert got["planted_rows"] == len(pos)
