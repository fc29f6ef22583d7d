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
    assert L.kv8_encode_bits(0, 0, None, None) == 0
    assert L.kv8_encode_bits(5, 1 << 32, 16, None) == -1
    assert L.kv8_decode_codes(None, -3, None, None, None) == -1
