"""ctypes wrapper of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and this
package imports nothing from the product package.

Arrays are numpy; bf16 values are passed as their uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def lib():
    """Load liboracle.so, building it first only if it does not exist."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # noqa: local build step
        _build.build_lib()
    L = ctypes.CDLL(_LIB_PATH)
    L.orc_decode.restype = ctypes.c_double
    L.orc_decode.argtypes = [ctypes.c_uint8]
    L.orc_encode.restype = ctypes.c_uint8
    L.orc_encode.argtypes = [ctypes.c_float]
    L.orc_encode_bits_range.restype = None
    L.orc_encode_bits_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64, _u8p, ctypes.c_int]
    L.orc_encode_array.restype = None
    L.orc_encode_array.argtypes = [_f32p, ctypes.c_int64, _u8p, ctypes.c_int]
    L.orc_quantize_segment.restype = ctypes.c_float
    L.orc_quantize_segment.argtypes = [_f32p, ctypes.c_int32, _u8p]
    L.orc_quantize_rows.restype = None
    L.orc_quantize_rows.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_int32, _u8p, _f32p, _i64p, ctypes.c_int]
    att = [_u16p, _u16p]
    tail = [_i64p, _i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_float, ctypes.c_int32, _i64p, ctypes.c_int64, _f64p,
            ctypes.c_int]
    L.orc_attention.restype = ctypes.c_int
    L.orc_attention.argtypes = att + [_u8p, _f32p] + tail
    L.orc_attention_f32rows.restype = ctypes.c_int
    L.orc_attention_f32rows.argtypes = att + [_f32p, ctypes.c_int64] + tail
    L.orc_norm_rope_rows.restype = None
    L.orc_norm_rope_rows.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_int32, _f32p, ctypes.c_float, _i64p, ctypes.c_float,
                                     _f32p, ctypes.c_int]
    L.orc_project_rows.restype = None
    L.orc_project_rows.argtypes = [_u8p, _f32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                   _u16p, ctypes.c_int32, _f64p, _f64p, ctypes.c_int]
    L.orc_quantize_rows_mx.restype = None
    L.orc_quantize_rows_mx.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, _u8p, _u8p, _i64p, ctypes.c_int]
    L.orc_attention_mx.restype = ctypes.c_int
    L.orc_attention_mx.argtypes = att + [_u8p, _u8p] + tail
    L.orc_bytes_per_token_layer_mx.restype = ctypes.c_int64
    L.orc_bytes_per_token_layer_mx.argtypes = [ctypes.c_int32, ctypes.c_int32]
    L.orc_bytes_per_token_layer.restype = ctypes.c_int64
    L.orc_bytes_per_token_layer.argtypes = [ctypes.c_int32, ctypes.c_int32]
    _lib = L
    return L


def default_threads():
    """Worker threads for the oracle: the CPUs this process may use, at most 16
    (the host share that goes with one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _p(a, t):
    return a.ctypes.data_as(t)


def _t(threads):
    return threads if threads and threads > 0 else default_threads()


def decode(codes):
    """f64 value of every e4m3 code in ``codes`` (uint8 array)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    L = lib()
    return np.array([L.orc_decode(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def encode(x, threads=0):
    """Saturating RNE e4m3 code of every f32 value in ``x``."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    lib().orc_encode_array(_p(a, _f32p), a.size, _p(out, _u8p), _t(threads))
    return out


def encode_bits_range(first, count, threads=0, out=None):
    """Codes of the f32 values with bit patterns first .. first+count-1."""
    if out is None:
        out = np.empty(count, dtype=np.uint8)
    lib().orc_encode_bits_range(first, count, _p(out, _u8p), _t(threads))
    return out


def quantize_segment(x):
    a = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(a.size, dtype=np.uint8)
    s = lib().orc_quantize_segment(_p(a, _f32p), a.size, _p(codes, _u8p))
    return codes, np.float32(s)


def quantize_rows(src, kv_lora=512, rope=64, dst_rows=None, n_cache_rows=None,
                  codes=None, scales=None, threads=0):
    """Quantize f32 token rows [n, >= kv_lora+rope] into (codes, scales).

    With dst_rows, row i is written to cache row dst_rows[i] of the given (or
    newly allocated, n_cache_rows long) cache arrays."""
    a = np.asarray(src, dtype=np.float32)
    assert a.ndim == 2 and a.strides[1] == 4
    n = a.shape[0]
    D = kv_lora + rope
    rows = n if n_cache_rows is None else n_cache_rows
    if codes is None:
        codes = np.zeros((rows, D), dtype=np.uint8)
    if scales is None:
        scales = np.zeros((rows, 2), dtype=np.float32)
    dp = None
    if dst_rows is not None:
        dst_rows = np.ascontiguousarray(dst_rows, dtype=np.int64)
        dp = _p(dst_rows, _i64p)
    lib().orc_quantize_rows(_p(a, _f32p), a.strides[0] // 4, n, kv_lora, rope,
                            _p(codes, _u8p), _p(scales, _f32p), dp, _t(threads))
    return codes, scales


def norm_rope_rows(src, norm_weight, eps, positions, rope_theta, kv_lora=512, rope=64,
                   threads=0):
    """The producer step: RMS-normalised Lc and rotary-embedded Rc of f32 rows
    [n, >= kv_lora+rope], computed in f64 and rounded to f32 -> [n, kv_lora+rope]."""
    a = np.asarray(src, dtype=np.float32)
    assert a.ndim == 2 and a.strides[1] == 4
    n = a.shape[0]
    w = np.ascontiguousarray(norm_weight, dtype=np.float32)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    assert w.size == kv_lora and pos.size == n
    out = np.empty((n, kv_lora + rope), dtype=np.float32)
    lib().orc_norm_rope_rows(_p(a, _f32p), a.strides[0] // 4, n, kv_lora, rope, _p(w, _f32p),
                             float(eps), _p(pos, _i64p), float(rope_theta), _p(out, _f32p),
                             _t(threads))
    return out


def project_rows(codes, scales, w_bf16, kv_lora=512, rope=64, threads=0):
    """Non-absorbed projection of cache rows: out f64 [n, N] = s_Lc * dec(Lc) @ W^T
    with W bf16 bits [N, kv_lora]; rope f64 [n, rope] = s_Rc * dec(Rc)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.float32)
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    n, N = c.shape[0], w.shape[0]
    assert c.shape[1] == kv_lora + rope and s.shape == (n, 2) and w.shape[1] == kv_lora
    out = np.empty((n, N), dtype=np.float64)
    rp = np.empty((n, rope), dtype=np.float64)
    lib().orc_project_rows(_p(c, _u8p), _p(s, _f32p), n, kv_lora, rope, _p(w, _u16p), N,
                           _p(out, _f64p), _p(rp, _f64p), _t(threads))
    return out, rp


def _attn_common(q_lat, q_rope, kv_start, kv_len, Q, sel):
    q_lat = np.ascontiguousarray(q_lat, dtype=np.uint16)
    q_rope = np.ascontiguousarray(q_rope, dtype=np.uint16)
    kv_start = np.ascontiguousarray(kv_start, dtype=np.int64)
    kv_len = np.ascontiguousarray(kv_len, dtype=np.int32)
    B = kv_start.size
    kv_lora = q_lat.shape[-1]
    rope = q_rope.shape[-1]
    H = q_lat.size // (B * Q * kv_lora)
    assert q_lat.size == B * Q * H * kv_lora and q_rope.size == B * Q * H * rope
    if sel is not None:
        sel = np.ascontiguousarray(sel, dtype=np.int64)
        out = np.zeros((sel.size, kv_lora), dtype=np.float64)
    else:
        out = np.zeros((B, Q, H, kv_lora), dtype=np.float64)
    return q_lat, q_rope, kv_start, kv_len, B, H, kv_lora, rope, sel, out


def attention(q_lat, q_rope, codes, scales, kv_start, kv_len, Q=1,
              softmax_scale=np.float32(1.0 / 24.0), num_splits=1, sel=None, threads=0):
    """Absorbed decode over dequantized fp8 rows in f64 (see kv8_oracle.h)."""
    q_lat, q_rope, kv_start, kv_len, B, H, kv_lora, rope, sel, out = _attn_common(
        q_lat, q_rope, kv_start, kv_len, Q, sel)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    assert codes.shape[-1] == kv_lora + rope
    rc = lib().orc_attention(_p(q_lat, _u16p), _p(q_rope, _u16p), _p(codes, _u8p),
                             _p(scales, _f32p), _p(kv_start, _i64p), _p(kv_len, _i32p),
                             B, Q, H, kv_lora, rope, float(softmax_scale), num_splits,
                             None if sel is None else _p(sel, _i64p),
                             0 if sel is None else sel.size, _p(out, _f64p), _t(threads))
    if rc != 0:
        raise ValueError("orc_attention: bad arguments")
    return out


def attention_f32rows(q_lat, q_rope, rows, kv_start, kv_len, Q=1,
                      softmax_scale=np.float32(1.0 / 24.0), num_splits=1, sel=None,
                      threads=0):
    """The same attention over raw f32 rows (no quantization)."""
    q_lat, q_rope, kv_start, kv_len, B, H, kv_lora, rope, sel, out = _attn_common(
        q_lat, q_rope, kv_start, kv_len, Q, sel)
    rows = np.asarray(rows, dtype=np.float32)
    assert rows.ndim == 2 and rows.strides[1] == 4
    rc = lib().orc_attention_f32rows(_p(q_lat, _u16p), _p(q_rope, _u16p), _p(rows, _f32p),
                                     rows.strides[0] // 4, _p(kv_start, _i64p),
                                     _p(kv_len, _i32p), B, Q, H, kv_lora, rope,
                                     float(softmax_scale), num_splits,
                                     None if sel is None else _p(sel, _i64p),
                                     0 if sel is None else sel.size, _p(out, _f64p), _t(threads))
    if rc != 0:
        raise ValueError("orc_attention_f32rows: bad arguments")
    return out


def bytes_per_token_layer(kv_lora=512, rope=64):
    return int(lib().orc_bytes_per_token_layer(kv_lora, rope))


def quantize_rows_mx(src, kv_lora=512, rope=64, dst_rows=None, n_cache_rows=None,
                     codes=None, exps=None, threads=0):
    """Block-scaled quantizer: f32 rows [n, >= kv_lora+rope] -> (codes uint8
    [rows, D], exps uint8 [rows, D/32]: ue8m0 bytes, scale 2^(byte-127))."""
    a = np.asarray(src, dtype=np.float32)
    assert a.ndim == 2 and a.strides[1] == 4
    n = a.shape[0]
    D = kv_lora + rope
    rows = n if n_cache_rows is None else n_cache_rows
    if codes is None:
        codes = np.zeros((rows, D), dtype=np.uint8)
    if exps is None:
        exps = np.zeros((rows, D // 32), dtype=np.uint8)
    dp = None
    if dst_rows is not None:
        dst_rows = np.ascontiguousarray(dst_rows, dtype=np.int64)
        dp = _p(dst_rows, _i64p)
    lib().orc_quantize_rows_mx(_p(a, _f32p), a.strides[0] // 4, n, kv_lora, rope,
                               _p(codes, _u8p), _p(exps, _u8p), dp, _t(threads))
    return codes, exps


def dequantize_mx(codes, exps):
    """f64 values of block-scaled rows: decode(code) * 2^(exp byte - 127)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    e = np.repeat(np.ascontiguousarray(exps, dtype=np.int64) - 127, 32, axis=-1)
    table = decode(np.arange(256, dtype=np.uint8))
    return np.ldexp(table[c], e)


def attention_mx(q_lat, q_rope, codes, exps, kv_start, kv_len, Q=1,
                 softmax_scale=np.float32(1.0 / 24.0), num_splits=1, sel=None, threads=0):
    """Absorbed decode over dequantized block-scaled rows, f64."""
    q_lat, q_rope, kv_start, kv_len, B, H, kv_lora, rope, sel, out = _attn_common(
        q_lat, q_rope, kv_start, kv_len, Q, sel)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    exps = np.ascontiguousarray(exps, dtype=np.uint8)
    assert codes.shape[-1] == kv_lora + rope and exps.shape[-1] == (kv_lora + rope) // 32
    rc = lib().orc_attention_mx(_p(q_lat, _u16p), _p(q_rope, _u16p), _p(codes, _u8p),
                                _p(exps, _u8p), _p(kv_start, _i64p), _p(kv_len, _i32p),
                                B, Q, H, kv_lora, rope, float(softmax_scale), num_splits,
                                None if sel is None else _p(sel, _i64p),
                                0 if sel is None else sel.size, _p(out, _f64p), _t(threads))
    if rc != 0:
        raise ValueError("orc_attention_mx: bad arguments")
    return out


def bytes_per_token_layer_mx(kv_lora=512, rope=64):
    return int(lib().orc_bytes_per_token_layer_mx(kv_lora, rope))
