#!/usr/bin/env python3
"""Benchmark of the fp8 e4m3 latent KV cache on one MI355X.

    python bench.py [--steps K] [--warmup W] [--legs decode,quantize,splitT,ragged]

Headline step (one pass of the whole hot path): batched single-layer decode,
B=32 sequences x T=8192 cached tokens x H=128 heads, one query token each,
latent rows of 512 Lc + 64 Rc e4m3 codes with per-row f32 scales.  Each step
  1. appends one fresh f32 row per sequence with kv8_quantize_rows (written at
     the sequence's newest row), and
  2. decodes all 32 x 128 query rows with the two kernels kv8_absorb_decode
     runs (split partials, then the log-sum-exp merge), using the split plan
     kv8_decode_plan returns.
Three copies of the cache (3 x 153 MB, more than the 256 MB last-level cache)
are used in rotation so every step reads its KV from HBM.  Inputs are resident
in HBM before the timed region; times come from HIP events on the stream the
kernels run on.  The timed steps have nothing between their kernels; a
separate pass over the same number of steps, with events between the
kernels, gives the per-kernel breakdown (`kernel_ms`).

Settling: on this GPU, launch durations dip by up to 25% from about 1.5 ms to
about 30 ms after a sustained load starts, while the power controller
settles (the first dozen decode launches run at 91 us, then 109-116 us, then
83-85 us after ~30 ms). So before its W warmup steps every timed measurement
first makes untimed calls of its own step for SETTLE_MS of GPU time. The
record states how long the headline decode settled and how many calls that
took (`settle`), so the timed steps show the sustained-load rate.

Roofline of the decode kernel: its flops over its mean duration inside the
steps (HIP events around it on its stream).  Also recorded: the same launches
back to back (cold: caches in rotation; warm: one cache again and again), the
shader clock with every SIMD running MFMAs (kv8_shader_clock_mhz; the quoted
2.5 PFLOP/s assumes 2.4 GHz) and the fraction at that clock, and the HBM
floor of the kernel's bytes (kv8_stream_floor: one plain streaming launch
reading a cache copy and writing the partials' bytes).

Other legs (same JSON line, key "legs"): the fp8-vs-f32 gap on the tiny
workload (B=1, H=16, T=1024: the kernel's output against f32 attention over
the unquantized rows, computed in f64 with torch on the device), the bulk
quantizer (32,768 tokens x 61 layers of Student-t rows with planted special
rows; the same rows also through the producer step fused with the quantizer;
its HBM floor), the 256k-token split-T decode with 64 ranges, the non-absorbed
projection, the ragged Q=4 multi-query decode, and the block-scaled (MX)
variant on the headline shape.  Times are means with medians and bests.

The CPU baseline is the oracle (oracle/, test infrastructure) timed on this
host: a sample of the headline decode on the host's worker threads and on one
thread, the quantizer on a slice of the bulk rows, and samples of the 256k and
ragged workloads (each stated in its "sample").
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = ("fp8-KV absorbed-MLA decode KV GB/s & TFLOP/s (% peak); quantize rows/s")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
KL, KR, D = 512, 64, 576
FLOPS_PER_ROW_TOKEN = 2 * (KL + KR) + 2 * KL   # score 2*576 + context 2*512
KV_BYTES_PER_TOKEN = D + 8
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(name):
    p = os.path.join(ROOT, "fp8_e4m3_latent_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def counter_traffic(kernel, source):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current source of the kernel; else None."""
    try:
        data = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    rec = data.get(kernel)
    if not rec or rec.get("source_sha256_16") != source_hash(source):
        return None
    return rec.get("bytes_per_launch")


SETTLE_MS = 60.0


def settle(torch, fn, ms=SETTLE_MS, max_calls=20000):
    """Untimed calls fn(i) until `ms` of GPU time has passed since the first
    (the power controller's settling time, see the module docstring)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    n, el = 0, 0.0
    while n < max_calls:
        for _ in range(8):
            fn(n)
            n += 1
        e1.record()
        e1.synchronize()
        el = e0.elapsed_time(e1)
        if el >= ms:
            break
    return {"ms": el, "calls": n}


class Timer:
    """HIP events recorded on the current stream between launches."""

    def __init__(self, torch, n_marks, steps):
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_marks)]
                   for _ in range(steps)]

    def mark(self, step, i):
        self.ev[step][i].record()

    def intervals_ms(self):
        return np.array([[row[i].elapsed_time(row[i + 1]) for i in range(len(row) - 1)]
                         for row in self.ev])


# --------------------------------------------------------------------------
def leg_decode(torch, kv8, W, steps, warmup, cpu_sample_rows):
    B, T, H, Q = 32, 8192, 128, 1
    log("decode: generating %d x %d rows" % (B * T, D))
    w = W.batched(seed=0, B=B, T=T, H=H)
    dev = "cuda"
    rows = torch.from_numpy(w.rows).to(dev)
    n_copies = 3
    caches = []
    for k in range(n_copies):
        codes = torch.empty((B * T, D), dtype=torch.uint8, device=dev)
        scales = torch.empty((B * T, 2), dtype=torch.float32, device=dev)
        kv8.quantize_rows(rows, codes, scales)
        caches.append((codes, scales))
    del rows
    qs = []
    for k in range(n_copies):
        ql, qr = W.queries(100 + k, B, Q, H)
        qs.append((torch.from_numpy(ql.view(np.int16)).to(dev).view(torch.bfloat16),
                   torch.from_numpy(qr.view(np.int16)).to(dev).view(torch.bfloat16)))
    fresh = [torch.from_numpy(W.fresh_rows(200 + k, B)).to(dev) for k in range(n_copies)]
    kv_start = torch.from_numpy(w.kv_start).to(dev)
    kv_len = torch.from_numpy(w.kv_len).to(dev)
    dst = kv_start + (T - 1)                  # each sequence's newest row
    split_tokens, n_splits = kv8.decode_plan(B, Q, H, T)
    partials = torch.empty(kv8.partials_bytes(B, Q, H, n_splits) // 4, dtype=torch.float32,
                           device=dev)
    out = torch.empty((B, Q, H, KL), dtype=torch.float32, device=dev)
    sc = float(w.softmax_scale)

    def step(i, timer=None, t=None):
        c = i % n_copies
        codes, scales = caches[c]
        if timer: timer.mark(t, 0)
        kv8.quantize_rows(fresh[c], codes, scales, dst_rows=dst)
        if timer: timer.mark(t, 1)
        kv8.absorb_decode_partials(qs[c][0], qs[c][1], codes, scales, kv_start, kv_len, T, sc,
                                   split_tokens, n_splits, partials)
        if timer: timer.mark(t, 2)
        kv8.lse_merge(partials, B, Q, H, n_splits, sc, out)
        if timer: timer.mark(t, 3)

    settled = settle(torch, lambda i: step(i))
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # per-kernel breakdown: the same steps with HIP events between the kernels
    timer = Timer(torch, 4, steps)
    for t in range(steps):
        step(warmup + t, timer, t)
    torch.cuda.synchronize()
    iv = timer.intervals_ms()                 # [steps, 3]: append, decode, merge
    # the timed steps: nothing but the steps' kernels between the two events
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for t in range(steps):
        step(warmup + steps + t)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / steps
    flops = float(FLOPS_PER_ROW_TOKEN) * B * Q * H * T
    kv_bytes = float(KV_BYTES_PER_TOKEN) * B * T
    dec_ms = float(iv[:, 1].mean())
    res = {
        "B": B, "T": T, "H": H, "Q": Q, "split_tokens": split_tokens, "num_splits": n_splits,
        "ms_per_step": ms_step,
        "tflops_step": flops / (ms_step * 1e-3) / 1e12,
        "kv_gb_per_s_step": kv_bytes / (ms_step * 1e-3) / 1e9,
        "step_ms_with_events": spread(iv.sum(axis=1)),
        "kernel_ms": {"quantize_append": float(iv[:, 0].mean()),
                      "absorb_decode_kernel": dec_ms,
                      "lse_merge_kernel": float(iv[:, 2].mean()),
                      "absorb_decode_kernel_median": float(np.median(iv[:, 1])),
                      "absorb_decode_kernel_best": float(iv[:, 1].min()),
                      "lse_merge_kernel_best": float(iv[:, 2].min())},
        "flops_per_step": flops, "kv_bytes_per_step": kv_bytes,
        "settle": settled,
    }
    # duration of the decode kernel alone for the roofline: the same launches
    # back to back (the per-step events above also hold each launch's
    # dispatch gap behind the append kernel).  Cold: the three cache copies in
    # rotation (KV from HBM); warm: one copy again and again (KV in the
    # last-level cache after the first launch).
    b2b = 10
    base = warmup + 2 * steps

    def dec(c):
        kv8.absorb_decode_partials(qs[c][0], qs[c][1], caches[c][0], caches[c][1], kv_start, kv_len,
                                   T, sc, split_tokens, n_splits, partials)

    res["kernel_ms"]["absorb_decode_kernel_back_to_back"] = back_to_back_ms(
        torch, b2b, lambda i: dec((base + i) % n_copies))
    res["kernel_ms"]["absorb_decode_kernel_back_to_back_warm"] = back_to_back_ms(
        torch, b2b, lambda i: dec(0))
    # the one-call entry point, which takes stream-ordered memory for its
    # partials on every call, against the same decode and merge on a
    # caller-owned partials buffer
    out1 = torch.empty_like(out)

    def one_call(i):
        c = (base + i) % n_copies
        kv8.absorb_decode(qs[c][0], qs[c][1], caches[c][0], caches[c][1], kv_start, kv_len, T, sc, out=out1)

    def two_stage(i):
        dec((base + i) % n_copies)
        kv8.lse_merge(partials, B, Q, H, n_splits, sc, out1)

    one_call(0)
    res["kernel_ms"]["absorb_decode_call_allocating"] = back_to_back_ms(torch, b2b, one_call)
    res["kernel_ms"]["absorb_decode_partials_plus_merge"] = back_to_back_ms(torch, b2b, two_stage)
    res["decode_kernel_tflops"] = flops / (dec_ms * 1e-3) / 1e12
    res["decode_kernel_kv_gb_per_s"] = kv_bytes / (dec_ms * 1e-3) / 1e9
    # the HBM floor of the decode's traffic: one plain streaming launch that
    # reads a cache copy (codes and scales, copies in rotation) and writes
    # the partials' bytes
    rot = iter(range(10 ** 9))
    part_bytes = partials.numel() * partials.element_size()

    def floor_args():
        c = next(rot) % n_copies
        return list(caches[c]), partials

    res["loads_only_floor"] = floor_stats(torch, kv8, 20, floor_args, kv_bytes + part_bytes)
    # the shader clock under matrix-core load, right after the decode launches
    res["shader_clock_mhz"] = kv8.shader_clock_mhz(3000)
    cpu = None
    if cpu_sample_rows > 0:
        c = (warmup + steps - 1) % n_copies
        cpu = cpu_decode_baseline(torch, caches[c], qs[c], w, Q, sc, cpu_sample_rows)
    return res, cpu


def _host_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_passes(fn, budget_s, max_passes=8):
    """Run fn until about budget_s seconds have passed (at least once); median pass."""
    times = []
    while len(times) < max_passes and (not times or sum(times) < budget_s):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), times


def cpu_decode_baseline(torch, cache, q, w, Q, sc, sample_rows):
    """The oracle timed on the headline decode: a sample of query rows on the
    host's worker threads and a smaller sample on one thread."""
    import oracle
    codes, scales = cache
    c_h, s_h = codes.cpu().numpy(), scales.cpu().numpy()
    ql_h, qr_h = _host_bits(q[0]), _host_bits(q[1])
    rows = w.B * Q * w.H
    T = int(w.kv_len[0])
    cores = oracle.default_threads()
    out = {"unit": "TFLOP/s", "kind": "oracle", "cores": cores, "cpu_model": cpu_model(),
           "host_cpus": os.cpu_count()}
    for threads, n_sel, budget in ((cores, min(sample_rows, rows), 10.0),
                                   (1, min(max(sample_rows // 32, 16), rows), 3.0)):
        sel = np.linspace(0, rows - 1, n_sel).astype(np.int64)
        log("cpu baseline: oracle on %d of %d query rows, %d threads" % (sel.size, rows, threads))
        dt, times = _oracle_passes(
            lambda: oracle.attention(ql_h, qr_h, c_h, s_h, w.kv_start, w.kv_len, Q=Q,
                                     softmax_scale=sc, sel=sel, threads=threads), budget)
        v = float(FLOPS_PER_ROW_TOKEN) * T * sel.size / dt / 1e12
        sample = ("%d of %d query rows of the headline decode (T=%d, every sequence), f64; "
                  "median of %d passes, %.2f s each" % (sel.size, rows, T, len(times), dt))
        if threads == cores:
            out.update({"value": v, "sample": sample})
        else:
            out["threads_1"] = {"value": v, "sample": sample}
    return out


def cpu_quantize_baseline(W, cores):
    """The oracle's quantizer on a slice of the bulk rows (rows/s)."""
    import oracle
    rows_h, _ = W.bulk_rows(seed=0, tokens=8192, layers=8)
    out = {"unit": "rows/s", "kind": "oracle", "cores": cores}
    for threads, n in ((cores, rows_h.shape[0]), (1, rows_h.shape[0] // 4)):
        x = np.ascontiguousarray(rows_h[:n])
        dt, times = _oracle_passes(lambda: oracle.quantize_rows(x, threads=threads), 3.0)
        key = "value" if threads == cores else "threads_1"
        rec = {"value": n / dt, "gb_per_s": n * 2888 / dt / 1e9,  # 2,888 algorithmic bytes a row
               "sample": "%d Student-t bulk rows (8,192 tokens x 8 layers, special "
                         "rows planted), median of %d passes" % (n, len(times))}
        if threads == cores:
            out.update(rec)
        else:
            out[key] = rec
    return out


def cpu_workload_baseline(torch, kv8_cache, w, sel, what, cores):
    """The oracle on the query rows sel of a decode workload (TFLOP/s over the
    tokens those rows see)."""
    import oracle
    codes, scales = kv8_cache
    c_h, s_h = codes.cpu().numpy(), scales.cpu().numpy()
    ql, qr = w.q_lat, w.q_rope
    dt, times = _oracle_passes(
        lambda: oracle.attention(ql, qr, c_h, s_h, w.kv_start, w.kv_len, Q=w.Q,
                                 softmax_scale=w.softmax_scale, sel=sel, threads=cores), 4.0, 4)
    qh = w.Q * w.H
    seen = 0
    for r in sel:
        b, i = int(r) // qh, (int(r) % qh) // w.H
        seen += max(0, int(w.kv_len[b]) - (w.Q - 1) + i)
    return {"value": float(FLOPS_PER_ROW_TOKEN) * seen / dt / 1e12, "unit": "TFLOP/s",
            "kind": "oracle", "cores": cores,
            "sample": "%s; %d query rows, median of %d passes, %.2f s each" % (what, len(sel), len(times), dt)}


def leg_quantize(torch, kv8, W, steps):
    log("quantize: generating 32768 x 61 bulk rows")
    rows_h, _ = W.bulk_rows(seed=0)
    n = rows_h.shape[0]
    rows = torch.from_numpy(rows_h).to("cuda")
    del rows_h
    codes = torch.empty((n, D), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, 2), dtype=torch.float32, device="cuda")
    for _ in range(2):
        kv8.quantize_rows(rows, codes, scales)
    torch.cuda.synchronize()
    qst = timer_stats(torch, steps, lambda: kv8.quantize_rows(rows, codes, scales))
    ms = qst["ms"]
    nbytes = float(n) * (4 * D + D + 8)
    res = {"rows": n, **qst, "rows_per_s": n / (ms * 1e-3),
           "gb_per_s": nbytes / (ms * 1e-3) / 1e9, "bytes_per_launch": nbytes,
           "roofline": roofline_hbm(nbytes, ms, counter_traffic("quantize_rows_kernel",
                                                                "kv8_quantize.hip"))}
    # the producer step fused with the quantizer on the same rows: RMS norm of
    # Lc (seeded weight, eps 1e-6), rotation of the Rc pairs at the row's token
    # position (row index mod 32768, base 10000); 8 more bytes a row (position)
    g = np.random.default_rng(5)
    wgt = torch.from_numpy(g.uniform(0.25, 2.0, KL).astype(np.float32)).to("cuda")
    pos = torch.arange(n, dtype=torch.int64, device="cuda") % 32768
    prod = lambda: kv8.norm_rope_quantize_rows(rows, wgt, 1e-6, pos, 10000.0, codes, scales)
    for _ in range(2):
        prod()
    torch.cuda.synchronize()
    pst = timer_stats(torch, steps, prod)
    pms = pst["ms"]
    pbytes = float(n) * (4 * D + 8 + D + 8)
    res["producer"] = {"rows": n, **pst, "rows_per_s": n / (pms * 1e-3),
                       "gb_per_s": pbytes / (pms * 1e-3) / 1e9, "bytes_per_launch": pbytes,
                       "roofline": roofline_hbm(pbytes, pms, counter_traffic("norm_rope_quantize_rows",
                                                                            "kv8_quantize.hip"))}
    # the HBM floor: one plain streaming launch that reads the source rows and
    # writes as many bytes as the codes and scales
    sink = torch.empty(n * (D + 8), dtype=torch.uint8, device="cuda")
    res["loads_only_floor"] = floor_stats(torch, kv8, steps, lambda: ([rows], sink), nbytes)
    res["frac_of_floor"] = res["loads_only_floor"]["ms"] / ms
    del rows, codes, scales, pos, sink
    torch.cuda.empty_cache()
    return res


def long_context_stats(torch, w, codes, scales, ql, qr):
    """The softmax of the long-context workload over its dequantized cache, in
    f32 with plain torch on the device (a property of the workload, not a
    measurement of the kernels): per head, the largest weight and the weight
    on the head's own planted rows."""
    x = codes.view(torch.float8_e4m3fn).to(torch.float32)
    s = (ql.float().reshape(-1, KL) @ (x[:, :KL] * scales[:, :1]).T.contiguous()
         + qr.float().reshape(-1, KR) @ (x[:, KL:] * scales[:, 1:2]).T.contiguous())
    del x
    p = torch.softmax(s * float(w.softmax_scale), dim=1)
    del s
    pos = torch.from_numpy(w.notes["planted_rows"]).to(p.device)
    heads = torch.from_numpy(w.notes["planted_heads"]).to(p.device)
    mass = torch.zeros(w.H, dtype=torch.float64, device=p.device)
    mass.index_add_(0, heads, p[heads, pos].double())
    maxp = p.max(dim=1).values.double()
    q = lambda t: [float(t.min()), float(t.quantile(0.5)), float(t.max())]
    return {"what": "per head (min, median, max over the %d heads), softmax over the dequantized "
                    "cache; planted_mass is the weight on the head's own planted rows" % w.H,
            "planted_rows": int(len(w.notes["planted_rows"])),
            "max_p": q(maxp), "planted_mass": q(mass)}


def _decode_workload_leg(torch, kv8, w, steps, splits=None, cpu_sel=None, cpu_what="",
                         stats=None):
    dev = "cuda"
    rows = torch.from_numpy(w.rows).to(dev)
    n = w.n_rows
    codes = torch.empty((n, D), dtype=torch.uint8, device=dev)
    scales = torch.empty((n, 2), dtype=torch.float32, device=dev)
    kv8.quantize_rows(rows, codes, scales)
    torch.cuda.synchronize()
    qst = timer_stats(torch, steps, lambda: kv8.quantize_rows(rows, codes, scales))
    qt = qst["ms"]
    del rows
    ql = torch.from_numpy(w.q_lat.view(np.int16)).to(dev).view(torch.bfloat16)
    qr = torch.from_numpy(w.q_rope.view(np.int16)).to(dev).view(torch.bfloat16)
    st = torch.from_numpy(w.kv_start).to(dev)
    ln = torch.from_numpy(w.kv_len).to(dev)
    out = torch.empty((w.B, w.Q, w.H, KL), dtype=torch.float32, device=dev)
    sc = float(w.softmax_scale)
    if splits:
        ws = torch.empty(kv8.splitT_workspace_bytes(w.B, w.Q, w.H, splits), dtype=torch.uint8,
                         device=dev)
        fn = lambda: kv8.absorb_decode_splitT(ql, qr, codes, scales, st, ln, w.max_len, sc,
                                              splits, workspace=ws, out=out)
    else:
        fn = lambda: kv8.absorb_decode(ql, qr, codes, scales, st, ln, w.max_len, sc, out=out)
    fn()
    torch.cuda.synchronize()
    dst = timer_stats(torch, steps, fn)
    ms = dst["ms"]
    visible = sum(max(0, int(L) - (w.Q - 1) + i) for L in w.kv_len for i in range(w.Q))
    flops = float(FLOPS_PER_ROW_TOKEN) * w.H * visible
    kv_bytes = float(KV_BYTES_PER_TOKEN) * int(w.kv_len.sum())
    qbytes = float(n) * (4 * D + D + 8)
    res = {"B": w.B, "Q": w.Q, "H": w.H, "tokens": int(w.kv_len.sum()), **dst,
           "tflops": flops / (ms * 1e-3) / 1e12, "pct_peak_bf16": 100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "kv_gb_per_s": kv_bytes / (ms * 1e-3) / 1e9,
           "cache_build": {"rows": n, **qst, "rows_per_s": n / (qt * 1e-3),
                           "gb_per_s": qbytes / (qt * 1e-3) / 1e9}}
    if stats is not None:
        res["workload_stats"] = stats(torch, w, codes, scales, ql, qr)
    if cpu_sel is not None:
        import oracle
        log("cpu baseline: %s" % cpu_what)
        res["cpu_oracle"] = cpu_workload_baseline(torch, (codes, scales), w, cpu_sel, cpu_what,
                                                  oracle.default_threads())
    del codes, scales
    torch.cuda.empty_cache()
    return res


def leg_mx(torch, kv8, W, steps):
    """The block-scaled (MX) variant on the headline shape: B=32 x T=8192 x
    H=128 rows quantized to e4m3 codes with one ue8m0 exponent per 32 values
    (594 bytes a token), decoded with 8 ranges of 1,024 tokens per sequence
    (the e4m3 path's plan), plus the MX quantizer over the same rows."""
    B, T, H, Q = 32, 8192, 128, 1
    w = W.batched(seed=0, B=B, T=T, H=H)
    dev = "cuda"
    rows = torch.from_numpy(w.rows).to(dev)
    n = B * T
    codes = torch.empty((n, D), dtype=torch.uint8, device=dev)
    exps = torch.empty((n, D // 32), dtype=torch.uint8, device=dev)
    kv8.quantize_rows_mx(rows, codes, exps)
    torch.cuda.synchronize()
    qst = timer_stats(torch, steps, lambda: kv8.quantize_rows_mx(rows, codes, exps))
    del rows
    ql, qr = W.queries(100, B, Q, H)
    ql = torch.from_numpy(ql.view(np.int16)).to(dev).view(torch.bfloat16)
    qr = torch.from_numpy(qr.view(np.int16)).to(dev).view(torch.bfloat16)
    st = torch.from_numpy(w.kv_start).to(dev)
    ln = torch.from_numpy(w.kv_len).to(dev)
    _, splits = kv8.decode_plan(B, Q, H, T)
    ws = torch.empty(kv8.mx_workspace_bytes(B, Q, H, splits), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Q, H, KL), dtype=torch.float32, device=dev)
    fn = lambda: kv8.absorb_decode_mx(ql, qr, codes, exps, st, ln, T, float(w.softmax_scale),
                                      num_splits=splits, workspace=ws, out=out)
    fn()
    torch.cuda.synchronize()
    dst = timer_stats(torch, steps, fn)
    flops = float(FLOPS_PER_ROW_TOKEN) * B * Q * H * T
    qbytes = float(n) * (4 * D + D + D // 32)
    del codes, exps, ws
    torch.cuda.empty_cache()
    return {"B": B, "T": T, "H": H, "num_splits": splits, **dst,
            "tflops": flops / (dst["ms"] * 1e-3) / 1e12,
            "pct_peak_bf16": 100 * flops / (dst["ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "kv_gb_per_s": float(D + D // 32) * n / (dst["ms"] * 1e-3) / 1e9,
            "quantize": {"rows": n, **qst, "rows_per_s": n / (qst["ms"] * 1e-3),
                         "gb_per_s": qbytes / (qst["ms"] * 1e-3) / 1e9}}


def leg_kv8_gap(torch, kv8, W):
    """The tiny workload (B=1, H=16, T=1024, 1% outliers x50) decoded from the
    fp8 cache against f32 attention over the unquantized rows, in f64 with
    plain torch on the device: the difference the fp8 cache makes (the
    KV8=1 vs KV8=0 comparison), max|d| / max|ref|."""
    w = W.tiny(seed=0)
    dev = "cuda"
    rows = torch.from_numpy(w.rows).to(dev)
    codes = torch.empty((w.n_rows, D), dtype=torch.uint8, device=dev)
    scales = torch.empty((w.n_rows, 2), dtype=torch.float32, device=dev)
    kv8.quantize_rows(rows, codes, scales)
    ql = torch.from_numpy(w.q_lat.view(np.int16)).to(dev).view(torch.bfloat16)
    qr = torch.from_numpy(w.q_rope.view(np.int16)).to(dev).view(torch.bfloat16)
    out = kv8.absorb_decode(ql, qr, codes, scales, torch.from_numpy(w.kv_start).to(dev),
                            torch.from_numpy(w.kv_len).to(dev), w.max_len, float(w.softmax_scale))
    x = rows.double()
    s = (ql.double().reshape(-1, KL) @ x[:, :KL].T.contiguous()
         + qr.double().reshape(-1, KR) @ x[:, KL:].T.contiguous())
    p = torch.softmax(s * float(w.softmax_scale), dim=1)
    ref = p @ x[:, :KL]
    d = (out.double().reshape(-1, KL) - ref).abs().max() / ref.abs().max()
    return {"workload": "tiny: B=1, H=16, T=1024, rows N(0,1) with 1% of entries x50", "max_abs_rel": float(d)}


def leg_project(torch, kv8, steps):
    """Non-absorbed projection of one 8,192-token sequence's cache rows by a
    bf16 kv_b weight of N = 128 heads x (128 + 128) columns (random weights),
    with bf16 output and with f32 output."""
    n, N = 8192, 32768
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    rows = torch.randn((n, D), generator=g, device="cuda")
    codes = torch.empty((n, D), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, 2), dtype=torch.float32, device="cuda")
    kv8.quantize_rows(rows, codes, scales)
    del rows
    w = (torch.randn((N, KL), generator=g, device="cuda") * 0.05).to(torch.bfloat16)
    rope = torch.empty((n, KR), dtype=torch.float32, device="cuda")
    flops = 2.0 * n * KL * N
    res = {"rows": n, "N": N}
    for name, dt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        out = torch.empty((n, N), dtype=dt, device="cuda")
        fn = lambda: kv8.project_rows(codes, scales, w, out=out, rope_out=rope)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        st = timer_stats(torch, steps, fn)
        ms = st["ms"]
        nbytes = float(n) * (D + 8) + 2.0 * N * KL + out.element_size() * float(n) * N + 4.0 * n * KR
        ach = flops / (ms * 1e-3) / 1e12
        rec = {**st, "tflops": ach, "gb_per_s": nbytes / (ms * 1e-3) / 1e9,
               "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS, "traffic": None}}
        if name == "bf16":
            res.update(rec)
        else:
            res["f32_out"] = rec
        del out
    # context: the library bf16 GEMM (torch.matmul) of the same shape on bf16
    # operands, without the fp8 decode, row scale or Rc output
    a16 = torch.randn((n, KL), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((n, N), dtype=torch.bfloat16, device="cuda")
    fn = lambda: torch.matmul(a16, w.t(), out=out)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    st = timer_stats(torch, steps, fn)
    res["library_bf16_gemm"] = {
        **st, "tflops": flops / (st["ms"] * 1e-3) / 1e12,
        "what": "torch.matmul bf16 [8192, 512] x [512, 32768] -> bf16 (same shape, bf16 operands, "
                "no decode): the vendor GEMM as a reference for this K=512 shape"}
    del a16, out
    del codes, scales, w, rope
    torch.cuda.empty_cache()
    return res


def leg_copy(torch, steps):
    """Plain 1 GiB device copy: the reference for scaling HBM byte counters."""
    n = 1 << 28
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    ms = timer_call(torch, steps, lambda: y.copy_(x))
    del x, y
    torch.cuda.empty_cache()
    return {"bytes_read": 4 * n, "bytes_written": 4 * n, "ms": ms,
            "gb_per_s": 8.0 * n / (ms * 1e-3) / 1e9}


def timer_call(torch, steps, fn):
    """Mean ms of fn over steps launches, each bracketed by HIP events."""
    return timer_stats(torch, steps, fn)["ms"]


def timer_stats(torch, steps, fn):
    settle(torch, lambda i: fn())
    timer = Timer(torch, 2, steps)
    for t in range(steps):
        timer.mark(t, 0)
        fn()
        timer.mark(t, 1)
    torch.cuda.synchronize()
    return spread(timer.intervals_ms()[:, 0])


def spread(ms):
    ms = np.asarray(ms, dtype=np.float64)
    return {"ms": float(ms.mean()), "ms_median": float(np.median(ms)), "ms_best": float(ms.min())}


def back_to_back_ms(torch, n, fn):
    """Mean ms per launch of n launches of fn(i) with nothing between them."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def floor_stats(torch, kv8, steps, fn_reads_write, nbytes):
    """Time kv8_stream_floor over the same bytes as a kernel: fn_reads_write(i)
    returns (reads, write) for launch i."""
    fn = lambda: kv8.stream_floor(*fn_reads_write())
    fn()
    st = timer_stats(torch, steps, fn)
    st["bytes"] = nbytes
    st["gb_per_s"] = nbytes / (st["ms"] * 1e-3) / 1e9
    return st


def roofline_hbm(nbytes, ms, traffic):
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBPS, "traffic": traffic}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--legs", default="decode,quantize,splitT,project,ragged,mx",
                    help="comma list of quantize, splitT, project, ragged, mx, copy "
                         "(the headline decode always runs)")
    ap.add_argument("--cpu-sample-rows", type=int, default=4096,
                    help="query rows the oracle times for the CPU baseline (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    sys.path.insert(0, ROOT)
    import fp8_e4m3_latent_amd as kv8
    from fp8_e4m3_latent_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kv8.lib()  # fails loudly when the HIP library is missing
    legs = set(args.legs.split(","))

    res, cpu = leg_decode(torch, kv8, W, args.steps, args.warmup, args.cpu_sample_rows)
    flops = res["flops_per_step"]
    # the decode kernel's mean duration inside the steps (HIP events around it)
    dec_ms = res["kernel_ms"]["absorb_decode_kernel"]
    ach = flops / (dec_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": "absorb_decode_kernel", "kernel_ms": dec_ms,
            "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS,
            "traffic": counter_traffic("absorb_decode_kernel", "kv8_decode.hip")}
    clock = res["shader_clock_mhz"]
    roof["shader_clock_mhz"] = clock
    # the same peak at the clock the matrix cores ran at (the quoted peak
    # assumes the 2.4 GHz peak engine clock)
    roof["frac_at_measured_clock"] = ach / (PEAK_BF16_TFLOPS * clock / 2400.0)
    cpu_on = args.cpu_sample_rows > 0
    extra = {"kv8_gap_tiny": leg_kv8_gap(torch, kv8, W)}
    if "quantize" in legs:
        extra["bulk_quantize"] = leg_quantize(torch, kv8, W, max(5, args.steps // 2))
        if cpu_on:
            import oracle
            log("cpu baseline: oracle quantizer")
            cpu["quantize"] = cpu_quantize_baseline(W, oracle.default_threads())
    if "splitT" in legs:
        log("splitT: 256k-token slot, 64 ranges")
        sel = np.arange(0, 128, 8) if cpu_on else None
        extra["splitT_256k"] = _decode_workload_leg(
            torch, kv8, W.long_context(seed=0), max(5, args.steps // 2), splits=64, cpu_sel=sel,
            cpu_what="256k-token slot, every 8th of the 128 heads (16 rows), T=262,144",
            stats=long_context_stats)
    if "project" in legs:
        log("project: 8192 rows x N=32768")
        extra["project_8k"] = leg_project(torch, kv8, max(5, args.steps // 4))
    if "copy" in legs:
        extra["copy_1gib"] = leg_copy(torch, 3)
    if "ragged" in legs:
        log("ragged: B=64, lengths U[1k,64k], Q=4")
        # CPU subset: the first 8 sequences, all 4 query positions, every 16th head
        sel = (np.array([b * 512 + q * 128 + h for b in range(8) for q in range(4)
                         for h in range(0, 128, 16)]) if cpu_on else None)
        extra["ragged_q4"] = _decode_workload_leg(
            torch, kv8, W.ragged(seed=0), max(3, args.steps // 4), cpu_sel=sel,
            cpu_what="ragged Q=4: sequences 0-7, every query position, every 16th head")
    if "mx" in legs:
        log("mx: block-scaled variant, B=32 x T=8192 x H=128")
        extra["mx_decode"] = leg_mx(torch, kv8, W, max(5, args.steps // 4))
    line = {
        "metric": METRIC,
        "value": res["tflops_step"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3+f16",  # score MFMAs on e4m3 operands, context MFMAs on f16, f32 sums
        "data": "synthetic",
        "config": {"workload": "batched absorbed-MLA decode step: B=32 x T=8192 x H=128, Q=1, "
                               "latent 512+64 e4m3 with per-row f32 scales; append 1 row/sequence "
                               "+ decode; 3 rotating cache copies (cold)",
                   "B": 32, "T": 8192, "H": 128, "Q": 1, "kv_lora": KL, "rope": KR,
                   "split_tokens": res["split_tokens"], "num_splits": res["num_splits"]},
        "pct_peak_bf16": 100 * res["tflops_step"] / PEAK_BF16_TFLOPS,
        "kv_gb_per_s": res["kv_gb_per_s_step"],
        "kernel_ms": res["kernel_ms"],
        "settle": res["settle"],
        "step_ms_with_events": res["step_ms_with_events"],
        "decode_loads_only_floor": res["loads_only_floor"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "legs": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
