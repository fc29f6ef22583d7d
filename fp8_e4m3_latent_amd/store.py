"""Binding of the slot pool, byte accounting and persistence of libkv8.so
(include/kv8_pool.h).  Argument marshalling only: the file format, the
repairs on open, the rewrite of f32 stores and the quantization on resume
all run in the library.

Host arrays are numpy (token-major: codes [n, layers, 576] uint8, scales
[n, layers, 2] float32, f32 rows [n, layers, 576]); pool memory is device
memory of the current device, reachable as torch tensors through
``Pool.layer()``.
"""
import ctypes
import os

import numpy as np

from . import KV_LORA, ROPE, ROW_BYTES, Kv8Error, lib

DTYPE_F32 = 0
DTYPE_E4M3 = 1
_vp, _i32, _i64, _u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
_ready = False


def _lib():
    global _ready
    L = lib()
    if not _ready:
        L.kv8_pool_bytes.restype = _u64
        L.kv8_pool_bytes.argtypes = [_i32, _i32, _i64, _i32, _i32, _i32]
        L.kv8_pool_slot_tokens_for.restype = _i64
        L.kv8_pool_slot_tokens_for.argtypes = [_u64, _i32, _i32, _i32, _i32, _i32]
        L.kv8_store_open.restype = ctypes.c_int
        L.kv8_store_open.argtypes = [ctypes.c_char_p, _i32, _i32, _i32, ctypes.POINTER(_vp)]
        L.kv8_store_info.restype = ctypes.c_int
        L.kv8_store_info.argtypes = [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_i64)]
        L.kv8_store_read.restype = ctypes.c_int
        L.kv8_store_read.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp]
        L.kv8_store_append.restype = ctypes.c_int
        L.kv8_store_append.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp]
        L.kv8_store_close.restype = ctypes.c_int
        L.kv8_store_close.argtypes = [_vp]
        L.kv8_store_write_f32.restype = ctypes.c_int
        L.kv8_store_write_f32.argtypes = [ctypes.c_char_p, _i32, _i32, _i32, _i64, _vp]
        L.kv8_pool_create.restype = ctypes.c_int
        L.kv8_pool_create.argtypes = [_i32, _i32, _i64, ctypes.POINTER(_vp)]
        L.kv8_pool_destroy.restype = ctypes.c_int
        L.kv8_pool_destroy.argtypes = [_vp]
        L.kv8_pool_used_bytes.restype = _u64
        L.kv8_pool_used_bytes.argtypes = [_vp]
        L.kv8_pool_layer.restype = ctypes.c_int
        L.kv8_pool_layer.argtypes = [_vp, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp)]
        L.kv8_pool_slot_row.restype = _i64
        L.kv8_pool_slot_row.argtypes = [_vp, _i32]
        L.kv8_pool_len.restype = _i64
        L.kv8_pool_len.argtypes = [_vp, _i32]
        L.kv8_pool_set_len.restype = ctypes.c_int
        L.kv8_pool_set_len.argtypes = [_vp, _i32, _i64]
        L.kv8_pool_load.restype = ctypes.c_int
        L.kv8_pool_load.argtypes = [_vp, _i32, _vp, _vp]
        L.kv8_pool_save.restype = ctypes.c_int
        L.kv8_pool_save.argtypes = [_vp, _i32, _vp, _vp]
        _ready = True
    return L


def _call(fn, *args):
    rc = getattr(_lib(), fn)(*args)
    if rc != 0:
        raise Kv8Error(fn, rc)


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def pool_bytes(n_layers, n_slots, slot_tokens, dtype=DTYPE_E4M3, kv_lora=KV_LORA, rope=ROPE):
    """Bytes of a pool of n_slots slots of slot_tokens tokens in n_layers layers."""
    return int(_lib().kv8_pool_bytes(n_layers, n_slots, slot_tokens, kv_lora, rope, dtype))


def slot_tokens_for(budget_bytes, n_layers, n_slots, dtype=DTYPE_E4M3, kv_lora=KV_LORA, rope=ROPE):
    """Largest slot capacity (a multiple of 32 tokens) whose pool fits the budget."""
    return int(_lib().kv8_pool_slot_tokens_for(budget_bytes, n_layers, n_slots, kv_lora, rope, dtype))


def write_f32(path, rows):
    """Write a store of f32 records: rows float32 [n, layers, kv_lora + rope]."""
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    n, layers, w = rows.shape
    _call("kv8_store_write_f32", os.fsencode(path), layers, KV_LORA, w - KV_LORA, n, _ptr(rows))


class Store:
    """A store file opened for reading and appending (repairs run on open)."""

    def __init__(self, path, n_layers, kv_lora=KV_LORA, rope=ROPE):
        h = _vp()
        _call("kv8_store_open", os.fsencode(path), n_layers, kv_lora, rope, ctypes.byref(h))
        self.handle, self.path = h, path
        self.n_layers, self.width = n_layers, kv_lora + rope

    def info(self):
        """(dtype on disk, number of token records)."""
        d, n = _i32(), _i64()
        _call("kv8_store_info", self.handle, ctypes.byref(d), ctypes.byref(n))
        return d.value, n.value

    def read(self, t0=0, n=None):
        """E4M3 store: (codes, scales); F32 store: rows."""
        dtype, total = self.info()
        n = total - t0 if n is None else n
        if dtype == DTYPE_E4M3:
            c = np.empty((n, self.n_layers, self.width), np.uint8)
            s = np.empty((n, self.n_layers, 2), np.float32)
            _call("kv8_store_read", self.handle, t0, n, _ptr(c), _ptr(s), None)
            return c, s
        r = np.empty((n, self.n_layers, self.width), np.float32)
        _call("kv8_store_read", self.handle, t0, n, None, None, _ptr(r))
        return r

    def append(self, codes, scales, prior_codes=None, prior_scales=None):
        codes = np.ascontiguousarray(codes, np.uint8)
        scales = np.ascontiguousarray(scales, np.float32)
        pc = None if prior_codes is None else np.ascontiguousarray(prior_codes, np.uint8)
        ps = None if prior_scales is None else np.ascontiguousarray(prior_scales, np.float32)
        _call("kv8_store_append", self.handle, codes.shape[0], _ptr(codes), _ptr(scales), _ptr(pc), _ptr(ps))

    def close(self):
        if self.handle:
            _call("kv8_store_close", self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class Pool:
    """Device slot pool of n_layers caches with n_slots slots of slot_tokens rows."""

    def __init__(self, n_layers, n_slots, slot_tokens):
        h = _vp()
        _call("kv8_pool_create", n_layers, n_slots, slot_tokens, ctypes.byref(h))
        self.handle = h
        self.n_layers, self.n_slots, self.slot_tokens = n_layers, n_slots, slot_tokens

    def used_bytes(self):
        return int(_lib().kv8_pool_used_bytes(self.handle))

    def layer(self, l):
        """(codes, scales) of layer l as torch tensors over the pool's memory."""
        import torch
        c, s = _vp(), _vp()
        _call("kv8_pool_layer", self.handle, l, ctypes.byref(c), ctypes.byref(s))
        rows = self.n_slots * self.slot_tokens
        return (_device_tensor(c.value, (rows, ROW_BYTES), torch.uint8),
                _device_tensor(s.value, (rows, 2), torch.float32))

    def slot_row(self, slot):
        return int(_lib().kv8_pool_slot_row(self.handle, slot))

    def len(self, slot):
        return int(_lib().kv8_pool_len(self.handle, slot))

    def set_len(self, slot, n):
        _call("kv8_pool_set_len", self.handle, slot, n)

    def load(self, slot, store, stream=None):
        from . import _stream
        _call("kv8_pool_load", self.handle, slot, store.handle, _stream(stream))

    def save(self, slot, store, stream=None):
        from . import _stream
        _call("kv8_pool_save", self.handle, slot, store.handle, _stream(stream))

    def destroy(self):
        if self.handle:
            _call("kv8_pool_destroy", self.handle)
            self.handle = None


def _device_tensor(ptr, shape, dtype):
    """A torch tensor viewing device memory owned by the pool (no copy)."""
    import torch
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()

    class _Mem:
        __cuda_array_interface__ = {
            "shape": (n,), "typestr": "|u1", "data": (ptr, False), "version": 3, "strides": None}

    return torch.as_tensor(_Mem(), device="cuda").view(dtype).view(*shape)
