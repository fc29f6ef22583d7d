"""fp8 e4m3 latent KV cache for MLA decode on MI355X (gfx950).

Thin Python binding of libkv8.so (include/kv8.h): it checks tensor dtypes,
devices, shapes and contiguity, passes raw device pointers and the current
HIP stream, and raises on a nonzero status.  Every step of the computation
runs in the HIP kernels; there is no fallback path.  PyTorch only provides
device memory and streams.

Cache layout: codes uint8 [rows, 576] (512 Lc codes, then 64 Rc codes),
scales float32 [rows, 2] (Lc scale, Rc scale).  bf16 queries are passed as
torch.bfloat16 tensors.
"""
import ctypes
import os

KV_LORA = 512
ROPE = 64
ROW_BYTES = KV_LORA + ROPE

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkv8.so")

_STATUS = {0: "KV8_OK", -1: "KV8_EINVAL", -2: "KV8_EUNSUPPORTED", -3: "KV8_ELAUNCH",
           -4: "KV8_EWORKSPACE", -5: "KV8_ENOMEM", -6: "KV8_EIO", -7: "KV8_EFORMAT"}

# every symbol include/kv8.h declares
EXPORTS = ("kv8_quantize_rows", "kv8_norm_rope_quantize_rows", "kv8_project_rows", "kv8_project_rows_f32", "kv8_absorb_decode", "kv8_splitT_workspace_bytes",
           "kv8_absorb_decode_splitT", "kv8_partials_bytes", "kv8_decode_plan",
           "kv8_absorb_decode_partials", "kv8_lse_merge", "kv8_status_string",
           "kv8_encode_bits", "kv8_decode_codes", "kv8_absorb_decode_noalloc",
           "kv8_quantize_rows_mx", "kv8_absorb_decode_mx", "kv8_mx_workspace_bytes",
           "kv8_shader_clock_mhz", "kv8_stream_floor",
           # include/kv8_pool.h (bound in store.py)
           "kv8_pool_bytes", "kv8_pool_slot_tokens_for", "kv8_store_open", "kv8_store_info",
           "kv8_store_read", "kv8_store_append", "kv8_store_close", "kv8_store_write_f32",
           "kv8_pool_create", "kv8_pool_destroy", "kv8_pool_used_bytes", "kv8_pool_layer",
           "kv8_pool_slot_row", "kv8_pool_len", "kv8_pool_set_len", "kv8_pool_load", "kv8_pool_save")
NOALLOC_SCRATCH_BYTES = 64 << 20  # KV8_NOALLOC_SCRATCH_BYTES

_lib = None


class Kv8Error(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().kv8_status_string(status).decode()
        super().__init__("%s failed: %s (%s)" % (fn, _STATUS.get(status, status), msg))
        self.status = status


def lib():
    """Load libkv8.so.  It must have been built (python -m fp8_e4m3_latent_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkv8.so is not built: run `python -m fp8_e4m3_latent_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32, u64, sz, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t,
                                       ctypes.c_float)
    L.kv8_stream_floor.restype = ctypes.c_int
    L.kv8_stream_floor.argtypes = [vp, u64, vp, u64, vp, u64, vp]
    L.kv8_shader_clock_mhz.restype = ctypes.c_int
    L.kv8_shader_clock_mhz.argtypes = [i32, ctypes.POINTER(ctypes.c_double), vp]
    L.kv8_status_string.restype = ctypes.c_char_p
    L.kv8_status_string.argtypes = [ctypes.c_int]
    L.kv8_quantize_rows.restype = ctypes.c_int
    L.kv8_quantize_rows.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp]
    L.kv8_quantize_rows_mx.restype = ctypes.c_int
    L.kv8_quantize_rows_mx.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp]
    L.kv8_project_rows.restype = ctypes.c_int
    L.kv8_project_rows.argtypes = [vp, vp, i64, i32, i32, vp, i32, vp, vp, vp]
    L.kv8_project_rows_f32.restype = ctypes.c_int
    L.kv8_project_rows_f32.argtypes = [vp, vp, i64, i32, i32, vp, i32, vp, vp, vp]
    L.kv8_norm_rope_quantize_rows.restype = ctypes.c_int
    L.kv8_norm_rope_quantize_rows.argtypes = [vp, i64, i64, i32, i32, vp, f32, vp, f32, vp, vp,
                                              vp, vp]
    dec = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp]
    L.kv8_absorb_decode.restype = ctypes.c_int
    L.kv8_absorb_decode.argtypes = dec + [vp]
    L.kv8_mx_workspace_bytes.restype = sz
    L.kv8_mx_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.kv8_absorb_decode_mx.restype = ctypes.c_int
    L.kv8_absorb_decode_mx.argtypes = dec + [i32, vp, sz, vp]
    L.kv8_absorb_decode_noalloc.restype = ctypes.c_int
    L.kv8_absorb_decode_noalloc.argtypes = dec + [vp]
    L.kv8_splitT_workspace_bytes.restype = sz
    L.kv8_splitT_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.kv8_absorb_decode_splitT.restype = ctypes.c_int
    L.kv8_absorb_decode_splitT.argtypes = dec + [i32, vp, sz, vp]
    L.kv8_partials_bytes.restype = sz
    L.kv8_partials_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.kv8_decode_plan.restype = ctypes.c_int
    L.kv8_decode_plan.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.kv8_absorb_decode_partials.restype = ctypes.c_int
    L.kv8_absorb_decode_partials.argtypes = dec[:-1] + [i32, i32, vp, sz, vp]
    L.kv8_lse_merge.restype = ctypes.c_int
    L.kv8_lse_merge.argtypes = [vp, sz, i32, i32, i32, i32, i32, f32, vp, vp]
    L.kv8_encode_bits.restype = ctypes.c_int
    L.kv8_encode_bits.argtypes = [u32, u64, i32, vp, vp]
    L.kv8_decode_codes.restype = ctypes.c_int
    L.kv8_decode_codes.argtypes = [vp, i64, vp, vp, vp]
    _lib = L
    return L


def _torch():
    import torch
    return torch


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype, ndim=None, contiguous=True):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor, got %s" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %s" % (name, ndim, tuple(t.shape)))
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _call(fn, *args):
    rc = getattr(lib(), fn)(*args)
    if rc != 0:
        raise Kv8Error(fn, rc)


def quantize_rows(src, codes, scales, dst_rows=None, stream=None):
    """Quantize f32 token rows src [n, >=576] (row stride may exceed 576) into
    the cache: row i -> cache row dst_rows[i] (int64 GPU tensor) or i."""
    torch = _torch()
    _check(src, "src", torch.float32, 2, contiguous=False)
    if src.stride(1) != 1:
        raise ValueError("src rows must be contiguous")
    if src.shape[1] < ROW_BYTES:
        raise ValueError("src rows must hold at least %d values" % ROW_BYTES)
    pc = _check(codes, "codes", torch.uint8, 2)
    ps = _check(scales, "scales", torch.float32, 2)
    if codes.shape[1] != ROW_BYTES or scales.shape[1] != 2 or scales.shape[0] != codes.shape[0]:
        raise ValueError("cache must be codes [rows, 576] uint8 and scales [rows, 2] f32")
    pd = None
    if dst_rows is not None:
        pd = _check(dst_rows, "dst_rows", torch.int64, 1)
        if dst_rows.numel() != src.shape[0]:
            raise ValueError("dst_rows must have one entry per source row")
    elif src.shape[0] > codes.shape[0]:
        raise ValueError("cache has fewer rows than src")
    _call("kv8_quantize_rows", ctypes.c_void_p(src.data_ptr()), src.stride(0), src.shape[0],
          KV_LORA, ROPE, pc, ps, pd, _stream(stream))


def quantize_rows_mx(src, codes, exps, dst_rows=None, stream=None):
    """Block-scaled quantizer: f32 rows src [n, >=576] -> codes uint8 [rows, 576]
    and ue8m0 block exponents exps uint8 [rows, 18] (row i -> dst_rows[i] or i)."""
    torch = _torch()
    _check(src, "src", torch.float32, 2, contiguous=False)
    if src.stride(1) != 1 or src.shape[1] < ROW_BYTES:
        raise ValueError("src rows must be contiguous and hold at least %d values" % ROW_BYTES)
    pc = _check(codes, "codes", torch.uint8, 2)
    pe = _check(exps, "exps", torch.uint8, 2)
    if codes.shape[1] != ROW_BYTES or exps.shape[1] != ROW_BYTES // 32 or exps.shape[0] != codes.shape[0]:
        raise ValueError("cache must be codes [rows, 576] and exps [rows, 18] uint8")
    pd = None
    if dst_rows is not None:
        pd = _check(dst_rows, "dst_rows", torch.int64, 1)
        if dst_rows.numel() != src.shape[0]:
            raise ValueError("dst_rows must have one entry per source row")
    elif src.shape[0] > codes.shape[0]:
        raise ValueError("cache has fewer rows than src")
    _call("kv8_quantize_rows_mx", ctypes.c_void_p(src.data_ptr()), src.stride(0), src.shape[0],
          KV_LORA, ROPE, pc, pe, pd, _stream(stream))


def norm_rope_quantize_rows(src, norm_weight, eps, positions, rope_theta, codes, scales,
                            dst_rows=None, stream=None):
    """The producer step fused with the quantizer: RMS-normalise the Lc part of
    each f32 row src [n, >=576] with norm_weight [512] and eps, rotate the Rc
    pairs by positions [n] (int64 GPU tensor) and rope_theta, and quantize the
    result into the cache (row i -> cache row dst_rows[i] or i)."""
    torch = _torch()
    _check(src, "src", torch.float32, 2, contiguous=False)
    if src.stride(1) != 1:
        raise ValueError("src rows must be contiguous")
    if src.shape[1] < ROW_BYTES:
        raise ValueError("src rows must hold at least %d values" % ROW_BYTES)
    pw = _check(norm_weight, "norm_weight", torch.float32, 1)
    if norm_weight.numel() != KV_LORA:
        raise ValueError("norm_weight must hold %d values" % KV_LORA)
    pp = _check(positions, "positions", torch.int64, 1)
    if positions.numel() != src.shape[0]:
        raise ValueError("positions must have one entry per source row")
    pc = _check(codes, "codes", torch.uint8, 2)
    ps = _check(scales, "scales", torch.float32, 2)
    if codes.shape[1] != ROW_BYTES or scales.shape[1] != 2 or scales.shape[0] != codes.shape[0]:
        raise ValueError("cache must be codes [rows, 576] uint8 and scales [rows, 2] f32")
    pd = None
    if dst_rows is not None:
        pd = _check(dst_rows, "dst_rows", torch.int64, 1)
        if dst_rows.numel() != src.shape[0]:
            raise ValueError("dst_rows must have one entry per source row")
    elif src.shape[0] > codes.shape[0]:
        raise ValueError("cache has fewer rows than src")
    _call("kv8_norm_rope_quantize_rows", ctypes.c_void_p(src.data_ptr()), src.stride(0),
          src.shape[0], KV_LORA, ROPE, pw, float(eps), pp, float(rope_theta), pc, ps, pd,
          _stream(stream))


def project_rows(codes, scales, w_kv_b, out=None, rope_out=None, with_rope=True, out_dtype=None,
                 stream=None):
    """Non-absorbed projection of the cache rows codes [n, 576] / scales [n, 2]
    (a contiguous slice of the cache): out [n, N] = s_Lc * dec(Lc) @ W^T for
    the bf16 weight w_kv_b [N, 512], in bf16 (default) or f32 (out_dtype, or
    the dtype of a given out); rope_out f32 [n, 64] = s_Rc * dec(Rc).
    Returns (out, rope_out) (rope_out None when with_rope is False)."""
    torch = _torch()
    pc = _check(codes, "codes", torch.uint8, 2)
    ps = _check(scales, "scales", torch.float32, 2)
    n = codes.shape[0]
    if codes.shape[1] != ROW_BYTES or tuple(scales.shape) != (n, 2):
        raise ValueError("codes must be [n, 576] uint8 and scales [n, 2] f32")
    pw = _check(w_kv_b, "w_kv_b", torch.bfloat16, 2)
    N = w_kv_b.shape[0]
    if w_kv_b.shape[1] != KV_LORA:
        raise ValueError("w_kv_b must be [N, 512]")
    if out is None:
        out = torch.empty((n, N), dtype=out_dtype or torch.bfloat16, device=codes.device)
    f32 = out.dtype == torch.float32
    po = _check(out, "out", torch.float32 if f32 else torch.bfloat16, 2)
    if tuple(out.shape) != (n, N):
        raise ValueError("out must be [n, N]")
    pr = None
    if with_rope:
        if rope_out is None:
            rope_out = torch.empty((n, ROPE), dtype=torch.float32, device=codes.device)
        pr = _check(rope_out, "rope_out", torch.float32, 2)
        if tuple(rope_out.shape) != (n, ROPE):
            raise ValueError("rope_out must be [n, 64]")
    else:
        rope_out = None
    _call("kv8_project_rows_f32" if f32 else "kv8_project_rows", pc, ps, n, KV_LORA, ROPE, pw, N, po, pr,
          _stream(stream))
    return out, rope_out


def _decode_args(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len, out, scales_dtype=None):
    torch = _torch()
    pql = _check(q_lat, "q_lat", torch.bfloat16, 4)
    pqr = _check(q_rope, "q_rope", torch.bfloat16, 4)
    B, Q, H, kl = q_lat.shape
    if kl != KV_LORA or tuple(q_rope.shape) != (B, Q, H, ROPE):
        raise ValueError("q_lat must be [B,Q,H,512] and q_rope [B,Q,H,64]")
    pc = _check(codes, "codes", torch.uint8, 2)
    ps = _check(scales, "scales", scales_dtype or torch.float32, 2)
    pst = _check(kv_start, "kv_start", torch.int64, 1)
    pln = _check(kv_len, "kv_len", torch.int32, 1)
    if kv_start.numel() != B or kv_len.numel() != B:
        raise ValueError("kv_start and kv_len need one entry per sequence")
    args = [pql, pqr, pc, ps, pst, pln, int(max_len), B, Q, H, KV_LORA, ROPE]
    if out is False:  # the call has no output tensor
        return args, None, None
    if out is None:
        out = torch.empty((B, Q, H, KV_LORA), dtype=torch.float32, device=q_lat.device)
    po = _check(out, "out", torch.float32, 4)
    if tuple(out.shape) != (B, Q, H, KV_LORA):
        raise ValueError("out must be [B,Q,H,512]")
    return args, out, po


def absorb_decode(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len, softmax_scale,
                  out=None, stream=None):
    """Absorbed-MLA decode over the fp8 cache; returns out f32 [B,Q,H,512]."""
    args, out, po = _decode_args(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len, out)
    _call("kv8_absorb_decode", *args, ctypes.c_float(softmax_scale), po, _stream(stream))
    return out


def absorb_decode_noalloc(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len,
                          softmax_scale, out=None, stream=None):
    """absorb_decode without any device allocation in the call: the split
    partials live in the library's static 64 MiB device array (shared by every
    call on the device; overlapping calls race).  Pass `out` to avoid the
    output allocation too."""
    args, out, po = _decode_args(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len, out)
    _call("kv8_absorb_decode_noalloc", *args, ctypes.c_float(softmax_scale), po, _stream(stream))
    return out


def splitT_workspace_bytes(B, Q, H, num_splits):
    return int(lib().kv8_splitT_workspace_bytes(B, Q, H, KV_LORA, num_splits))


def absorb_decode_splitT(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len,
                         softmax_scale, num_splits, workspace=None, out=None, stream=None):
    """Split-T decode with num_splits equal token ranges per sequence merged by
    log-sum-exp.  workspace: uint8 GPU tensor of splitT_workspace_bytes()."""
    torch = _torch()
    args, out, po = _decode_args(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len, out)
    B, Q, H = args[7], args[8], args[9]
    need = splitT_workspace_bytes(B, Q, H, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_lat.device)
    pw = _check(workspace, "workspace", torch.uint8, 1)
    _call("kv8_absorb_decode_splitT", *args, ctypes.c_float(softmax_scale), po,
          int(num_splits), pw, workspace.numel(), _stream(stream))
    return out


def absorb_decode_mx(q_lat, q_rope, codes, exps, kv_start, kv_len, max_len, softmax_scale,
                     num_splits=1, workspace=None, out=None, stream=None):
    """Absorbed decode over block-scaled rows (codes uint8 [rows, 576], exps
    uint8 [rows, 18], 4-byte aligned); num_splits equal ranges as in
    absorb_decode_splitT."""
    torch = _torch()
    pe = _check(exps, "exps", torch.uint8, 2)
    if exps.shape[1] != ROW_BYTES // 32 or exps.shape[0] != codes.shape[0]:
        raise ValueError("exps must be [rows, 18] uint8")
    args, out, po = _decode_args(q_lat, q_rope, codes, exps.view(torch.uint8), kv_start, kv_len,
                                 max_len, out, scales_dtype=torch.uint8)
    args[3] = pe
    B, Q, H = args[7], args[8], args[9]
    need = int(lib().kv8_mx_workspace_bytes(B, Q, H, KV_LORA, num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_lat.device)
    pw = _check(workspace, "workspace", torch.uint8, 1)
    _call("kv8_absorb_decode_mx", *args, ctypes.c_float(softmax_scale), po, int(num_splits), pw,
          workspace.numel(), _stream(stream))
    return out


def mx_workspace_bytes(B, Q, H, num_splits):
    return int(lib().kv8_mx_workspace_bytes(B, Q, H, KV_LORA, num_splits))


def decode_plan(B, Q, H, max_len):
    """(split_tokens, num_splits) that absorb_decode uses for these shapes."""
    a, n = ctypes.c_int32(), ctypes.c_int32()
    _call("kv8_decode_plan", B, Q, H, int(max_len), ctypes.byref(a), ctypes.byref(n))
    return a.value, n.value


def partials_bytes(B, Q, H, num_splits):
    return int(lib().kv8_partials_bytes(B, Q, H, KV_LORA, num_splits))


def absorb_decode_partials(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len,
                           softmax_scale, split_tokens, num_splits, partials, stream=None):
    """Stage 1 of the decode: one partial softmax per token range into
    `partials` (a 1-D f32 GPU tensor used as raw storage, partials_bytes()
    bytes: int16 codes of O, then f32 (m, l, o_scale, 0) per row)."""
    torch = _torch()
    args, _, _ = _decode_args(q_lat, q_rope, codes, scales, kv_start, kv_len, max_len, False)
    pp = _check(partials, "partials", torch.float32, 1)
    _call("kv8_absorb_decode_partials", *args, ctypes.c_float(softmax_scale),
          int(split_tokens), int(num_splits), pp, partials.numel() * 4, _stream(stream))


def lse_merge(partials, B, Q, H, num_splits, softmax_scale, out=None, stream=None):
    """Stage 2 of the decode: log-sum-exp merge of the partials into out."""
    torch = _torch()
    pp = _check(partials, "partials", torch.float32, 1)
    if out is None:
        out = torch.empty((B, Q, H, KV_LORA), dtype=torch.float32, device=partials.device)
    po = _check(out, "out", torch.float32, 4)
    _call("kv8_lse_merge", pp, partials.numel() * 4, B, Q, H, KV_LORA, int(num_splits),
          ctypes.c_float(softmax_scale), po, _stream(stream))
    return out


def encode_bits(first, count, out, encoder=0, stream=None):
    """out[k] = device code of the f32 with bit pattern first + k, from the
    quantizer's encoder (0) or the integer bit-math encoder (1)."""
    torch = _torch()
    po = _check(out, "out", torch.uint8, 1)
    if out.numel() < count:
        raise ValueError("out too small")
    _call("kv8_encode_bits", ctypes.c_uint32(first), ctypes.c_uint64(count), int(encoder), po,
          _stream(stream))


def decode_codes(codes, stream=None):
    """(bf16 bits, fp16 bits) of the device decode of every code (int16 tensors)."""
    torch = _torch()
    pc = _check(codes, "codes", torch.uint8, 1)
    bf = torch.empty(codes.numel(), dtype=torch.int16, device=codes.device)
    hf = torch.empty(codes.numel(), dtype=torch.int16, device=codes.device)
    _call("kv8_decode_codes", pc, codes.numel(), ctypes.c_void_p(bf.data_ptr()),
          ctypes.c_void_p(hf.data_ptr()), _stream(stream))
    return bf, hf


def shader_clock_mhz(busy_us=2000, stream=None):
    """Shader clock (MHz) of the current device with every SIMD running fp16
    MFMAs for about busy_us microseconds (synchronizes the stream)."""
    v = ctypes.c_double()
    _call("kv8_shader_clock_mhz", busy_us, ctypes.byref(v), _stream(stream))
    return v.value


def stream_floor(reads, write=None, stream=None):
    """One launch reading up to two device tensors and writing `write` (its
    content is overwritten) with plain 16-byte streaming loads and stores:
    the HBM floor for a kernel moving the same bytes."""
    ptrs = []
    for t in list(reads) + [None] * (2 - len(reads)):
        ptrs += [None, 0] if t is None else [ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size()]
    wp, wb = (None, 0) if write is None else (ctypes.c_void_p(write.data_ptr()), write.numel() * write.element_size())
    _call("kv8_stream_floor", *ptrs, wp, wb, _stream(stream))
