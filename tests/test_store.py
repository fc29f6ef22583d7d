"""Byte accounting and the store file of include/kv8_pool.h, on the CPU (the
store never touches the GPU).

Page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with .coli_kv v2" (colibri
PR #299): commit message, first paragraph (kv_pool_bytes reports the fp8
pool), .coli_kv v2 item (magic and dtype in the header; appends through a
persistent handle; f32 files quantized on resume and kept intact until the
first append rewrites them; repair on open) and Tests item (round trip,
upgrade, reject, self-heal).  The quantized rows an upgrade needs come from
the oracle here (the device pool supplies them from the GPU quantizer; see
test_gpu_store.py).
"""
import hashlib
import os
import struct

import numpy as np
import pytest

import oracle
from fp8_e4m3_latent_amd import Kv8Error, store
from fp8_e4m3_latent_amd.store import DTYPE_E4M3, DTYPE_F32, Store

L, W = 3, 576
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "footprint_figures.txt")


def golden():
    vals = {}
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()[:2]
            vals[k] = float(v)
    return vals


def sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def fp8_records(n, seed):
    """Token-major E4M3 records from the oracle's quantization of random rows."""
    rows = np.random.default_rng(seed).standard_normal((n * L, W)).astype(np.float32)
    c, s = oracle.quantize_rows(rows)
    return c.reshape(n, L, W), s.reshape(n, L, 2), rows.reshape(n, L, W)


def test_pool_bytes_match_the_layout_and_the_page():
    """584 bytes per token and layer (576 codes + 2 f32 scales); the page's
    256k-token slot: 47.7 GB in f32 over 79 layers, and the fp8 pool 3.9x
    smaller (12.09 GB: the page's "~13 GB" is not reproduced, reading Q3)."""
    g = golden()
    per = oracle.bytes_per_token_layer(512, 64)
    assert store.pool_bytes(1, 1, 1) == per == 584
    assert store.pool_bytes(79, 1, 1, DTYPE_F32) == 79 * 2304
    slot = int(g["slot_tokens"])
    f32 = store.pool_bytes(79, 1, slot, DTYPE_F32)
    fp8 = store.pool_bytes(79, 1, slot)
    assert abs(f32 / 1e9 - g["slot_f32_gb"]) < 0.05
    assert abs(f32 / fp8 - g["kv_ram_reduction"]) < 0.05
    assert fp8 == 79 * 584 * 262144 == 12_094_275_584
    assert store.pool_bytes(61, 8, 4096) == 8 * 4096 * 61 * 584
    assert store.pool_bytes(1, 1, 1, dtype=7) == 0


def test_slot_capacity_for_a_budget():
    """The fp8 pool holds 3.9x the tokens of the f32 one in the same budget
    (sizing against the memory budget sees the smaller pool)."""
    budget = 288 * 10 ** 9 // 2
    t8 = store.slot_tokens_for(budget, 61, 16)
    t32 = store.slot_tokens_for(budget, 61, 16, DTYPE_F32)
    assert t8 % 32 == 0 and store.pool_bytes(61, 16, t8) <= budget < store.pool_bytes(61, 16, t8 + 32)
    assert store.pool_bytes(61, 16, t32, DTYPE_F32) <= budget
    assert 3.9 < t8 / t32 < 4.0
    assert store.slot_tokens_for(100, 61, 16) == 0


def test_round_trip_through_appends(tmp_path):
    p = str(tmp_path / "a.kv8")
    c, s, _ = fp8_records(70, 1)
    with Store(p, L) as st:
        assert st.info() == (DTYPE_E4M3, 0)
        st.append(c[:30], s[:30])
        st.append(c[30:31], s[30:31])
        st.append(c[31:], s[31:])
        assert st.info() == (DTYPE_E4M3, 70)
    assert os.path.getsize(p) == 64 + 70 * L * (W + 8)
    with Store(p, L) as st:
        rc, rs = st.read()
        assert np.array_equal(rc, c) and np.array_equal(rs.view(np.uint32), s.view(np.uint32))
        pc, ps = st.read(41, 5)
        assert np.array_equal(pc, c[41:46])


def test_f32_store_upgrades_on_first_append_and_stays_intact_until_then(tmp_path):
    p = str(tmp_path / "v1.kv8")
    c, s, rows = fp8_records(40, 2)
    store.write_f32(p, rows)
    digest = sha(p)
    with Store(p, L) as st:
        assert st.info() == (DTYPE_F32, 40)
        assert np.array_equal(st.read(), rows)
    assert sha(p) == digest                            # opening and reading change nothing
    nc, ns, _ = fp8_records(5, 3)
    with Store(p, L) as st:
        with pytest.raises(Kv8Error):                   # the quantized prior records are required
            st.append(nc, ns)
        assert sha(p) == digest
        st.append(nc, ns, prior_codes=c, prior_scales=s)
        assert st.info() == (DTYPE_E4M3, 45)
    assert not os.path.exists(p + ".kv8tmp")
    with Store(p, L) as st:
        rc, rs = st.read()
    assert np.array_equal(rc, np.concatenate([c, nc])) and np.array_equal(rs, np.concatenate([s, ns]))


def test_rejects_other_files_and_dimensions(tmp_path):
    p = str(tmp_path / "x.kv8")
    c, s, _ = fp8_records(4, 4)
    with Store(p, L) as st:
        st.append(c, s)
    for layers, kv_lora, rope in ((L + 1, 512, 64), (L, 256, 64), (L, 512, 32)):
        with pytest.raises(Kv8Error) as e:
            Store(p, layers, kv_lora, rope)
        assert e.value.status == -7
    raw = bytearray(open(p, "rb").read())
    bad = str(tmp_path / "bad.kv8")
    for mutate in (lambda b: b.__setitem__(0, ord("X")),          # magic
                   lambda b: b.__setitem__(33, b[33] ^ 1),        # torn count (check fails)
                   lambda b: b.__setitem__(12, 9)):               # unknown dtype
        b = bytearray(raw)
        mutate(b)
        open(bad, "wb").write(bytes(b))
        with pytest.raises(Kv8Error) as e:
            Store(bad, L)
        assert e.value.status == -7
    open(bad, "wb").write(bytes(raw[:40]))                         # truncated header
    with pytest.raises(Kv8Error):
        Store(bad, L)


def test_self_heal_on_open(tmp_path):
    p = str(tmp_path / "h.kv8")
    c, s, _ = fp8_records(10, 5)
    with Store(p, L) as st:
        st.append(c, s)
    good = open(p, "rb").read()
    # (1) a rewrite that never reached its rename: the leftover is removed
    open(p + ".kv8tmp", "wb").write(b"partial rewrite")
    with Store(p, L) as st:
        assert st.info() == (DTYPE_E4M3, 10)
    assert not os.path.exists(p + ".kv8tmp") and open(p, "rb").read() == good
    # (2) an append whose records landed but whose count update did not
    open(p, "ab").write(b"\x07" * (L * (W + 8) + 100))
    with Store(p, L) as st:
        assert st.info() == (DTYPE_E4M3, 10)
    assert open(p, "rb").read() == good
    # (3) a count above the records the file holds: lowered to the complete ones
    b = bytearray(good[: 64 + 7 * L * (W + 8) + 13])
    hdr = bytearray(b[:64])
    struct.pack_into("<Q", hdr, 32, 10)
    h = 0xcbf29ce484222325
    for x in bytes(hdr[:40]):  # (the header check the format defines: FNV-1a 64 of bytes 0-39)
        h = ((h ^ x) * 0x100000001b3) % (1 << 64)
    struct.pack_into("<Q", hdr, 40, h)
    b[:64] = hdr
    open(p, "wb").write(bytes(b))
    with Store(p, L) as st:
        assert st.info() == (DTYPE_E4M3, 7)
        rc, rs = st.read()
    assert np.array_equal(rc, c[:7]) and os.path.getsize(p) == 64 + 7 * L * (W + 8)


def test_an_interrupted_upgrade_leaves_the_f32_store(tmp_path):
    """A crash during the first append of an f32 store (the rewrite file
    written but not renamed) loses nothing: the f32 file is intact and the
    leftover is removed on the next open."""
    p = str(tmp_path / "u.kv8")
    _, _, rows = fp8_records(6, 6)
    store.write_f32(p, rows)
    digest = sha(p)
    open(p + ".kv8tmp", "wb").write(b"KV8STORE" + b"\x00" * 100)
    with Store(p, L) as st:
        assert st.info() == (DTYPE_F32, 6)
        assert np.array_equal(st.read(), rows)
    assert sha(p) == digest and not os.path.exists(p + ".kv8tmp")
