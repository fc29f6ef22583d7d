"""The C-ABI library loads and exports every function include/*.h declares
(CPU only: argument-error paths return before any GPU work)."""
import ctypes
import glob
import os
import re

import pytest

import fp8_e4m3_latent_amd as kv8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(kv8_\w+)\s*\(", text):
            names.add(m.group(1))
    return names


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kv8_quantize_rows", "kv8_absorb_decode", "kv8_absorb_decode_splitT"):
        assert required in names
    assert names == set(kv8.EXPORTS)


def test_library_exports_every_declared_symbol():
    if not os.path.exists(kv8.LIB_PATH):
        pytest.skip("libkv8.so not built")
    L = ctypes.CDLL(kv8.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_argument_errors_are_synchronous():
    if not os.path.exists(kv8.LIB_PATH):
        pytest.skip("libkv8.so not built")
    L = kv8.lib()
    assert L.kv8_status_string(0) == b"ok"
    assert L.kv8_status_string(-2).startswith(b"unsupported")
    # unsupported widths, negative sizes and null pointers never reach the GPU
    assert L.kv8_quantize_rows(None, 576, 4, 100, 64, None, None, None, None) == -2
    assert L.kv8_quantize_rows(None, 576, -1, 512, 64, None, None, None, None) == -1
    assert L.kv8_quantize_rows(None, 576, 4, 512, 64, None, None, None, None) == -1
    assert L.kv8_quantize_rows(None, 576, 0, 512, 64, None, None, None, None) == 0
    assert L.kv8_encode_bits(0, 0, 0, None, None) == 0
    assert L.kv8_encode_bits(5, 1 << 32, 0, 16, None) == -1
    assert L.kv8_encode_bits(0, 4, 2, 16, None) == -1
    assert L.kv8_decode_codes(None, -3, None, None, None) == -1


def test_new_entry_points_reject_bad_arguments_before_any_gpu_work():
    if not os.path.exists(kv8.LIB_PATH):
        pytest.skip("libkv8.so not built")
    L = kv8.lib()
    f32 = ctypes.c_float
    # producer: widths, eps, theta, null pointers; zero rows is a no-op
    nrq = L.kv8_norm_rope_quantize_rows
    assert nrq(None, 576, 4, 512, 32, None, f32(1e-6), None, f32(1e4), None, None, None, None) == -2
    assert nrq(None, 576, 4, 512, 64, None, f32(-1.0), None, f32(1e4), None, None, None, None) == -1
    assert nrq(None, 576, 4, 512, 64, None, f32(float("nan")), None, f32(1e4), None, None, None, None) == -1
    assert nrq(None, 576, 4, 512, 64, None, f32(1e-6), None, f32(0.0), None, None, None, None) == -1
    assert nrq(None, 576, 4, 512, 64, None, f32(1e-6), None, f32(1e4), None, None, None, None) == -1
    assert nrq(None, 576, 0, 512, 64, None, f32(1e-6), None, f32(1e4), None, None, None, None) == 0
    # projection: N must be a multiple of 128; null pointers; empty shapes
    pr = L.kv8_project_rows
    assert pr(None, None, 4, 512, 64, None, 100, None, None, None) == -2
    assert pr(None, None, 4, 512, 64, None, 128, None, None, None) == -1
    assert pr(None, None, 0, 512, 64, None, 128, None, None, None) == 0
    assert pr(None, None, -1, 512, 64, None, 128, None, None, None) == -1


def test_decode_plan():
    """The internal split plan (host arithmetic only): ranges fill 256 compute
    units, no range is longer than 4,096 tokens and none shorter than 1,024
    unless the sequence is."""
    if not os.path.exists(kv8.LIB_PATH):
        pytest.skip("libkv8.so not built")
    # B=32, H=128, T=8192: 32 row blocks -> 8 ranges of 1,024 tokens
    assert kv8.decode_plan(32, 1, 128, 8192) == (1024, 8)
    # one short sequence: no split
    assert kv8.decode_plan(1, 1, 16, 1024) == (1024, 1)
    # 256k tokens, one sequence: 256 ranges of 1,024
    assert kv8.decode_plan(1, 1, 128, 262144) == (1024, 256)
    # ragged B=64, Q=4: 256 row blocks already fill the GPU; the 4,096-token
    # cap cuts the longest (65,536) into 16 ranges
    assert kv8.decode_plan(64, 4, 128, 65536) == (4096, 16)
    for B, Q, H, T in ((3, 1, 16, 777), (8, 2, 64, 50000), (200, 1, 128, 3000), (1, 1, 128, 1)):
        k, n = kv8.decode_plan(B, Q, H, T)
        assert k % 32 == 0 or n == 1
        assert n * k >= T and (n - 1) * k < T
        assert n == 1 or k <= 4096


def test_two_stage_calls_check_sizes_before_any_gpu_work():
    """The merge rejects a partials buffer smaller than its shapes need, and a
    fixed-size split that does not cover max_len is an argument error (it
    would drop the tail rows)."""
    if not os.path.exists(kv8.LIB_PATH):
        pytest.skip("libkv8.so not built")
    L = kv8.lib()
    f32 = ctypes.c_float
    need = L.kv8_partials_bytes(2, 1, 128, 512, 8)
    assert need == 8 * 2 * 128 * (512 * 2 + 16)
    fake = ctypes.c_void_p(1 << 20)  # (never dereferenced: the checks come first)
    merge = L.kv8_lse_merge
    assert merge(fake, need - 1, 2, 1, 128, 512, 8, f32(0.04), fake, None) == -4
    assert merge(fake, need, 2, 1, 128, 500, 8, f32(0.04), fake, None) == -2
    assert merge(fake, need, 2, 1, 128, 512, 0, f32(0.04), fake, None) == -1
    assert merge(None, need, 2, 1, 128, 512, 8, f32(0.04), fake, None) == -1
    assert merge(fake, need, 2, 1, 128, 512, 8, f32(float("nan")), fake, None) == -1
    part = L.kv8_absorb_decode_partials
    args = [fake] * 6
    # 3 ranges of 1,024 rows cannot cover max_len 4,000
    assert part(*args, 4000, 2, 1, 128, 512, 64, f32(0.04), 1024, 3, fake,
                L.kv8_partials_bytes(2, 1, 128, 512, 3), None) == -1
    # too small a buffer for the ranges asked for
    assert part(*args, 4000, 2, 1, 128, 512, 64, f32(0.04), 1024, 4, fake,
                L.kv8_partials_bytes(2, 1, 128, 512, 3), None) == -4


def test_measurement_entry_points_reject_bad_arguments_before_any_gpu_work():
    if not os.path.exists(kv8.LIB_PATH):
        pytest.skip("libkv8.so not built")
    L = kv8.lib()
    mhz = ctypes.c_double()
    assert L.kv8_shader_clock_mhz(0, ctypes.byref(mhz), None) == -1
    assert L.kv8_shader_clock_mhz(100001, ctypes.byref(mhz), None) == -1
    assert L.kv8_shader_clock_mhz(1000, None, None) == -1
    # sizes must be multiples of 16 and non-empty ranges need aligned pointers
    assert L.kv8_stream_floor(None, 8, None, 0, None, 0, None) == -1
    assert L.kv8_stream_floor(None, 16, None, 0, None, 0, None) == -1
    assert L.kv8_stream_floor(ctypes.c_void_p(0x1008), 16, None, 0, None, 0, None) == -1
    assert L.kv8_stream_floor(None, 0, None, 0, ctypes.c_void_p(0x1000), 24, None) == -1
    assert L.kv8_stream_floor(None, 0, None, 0, None, 0, None) == 0
