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
kernels, gives the per-kernel breakdown (`kernel_ms`).  The default 400 untimed steps (about 50 ms) bring the GPU to
its working clock first: with a handful of warmup steps the timed steps ran
about 15% slower.  The decode kernel's roofline uses its duration over launches
of that kernel alone, back to back on the same rotating caches (the per-step
events around it also hold its dispatch gap behind the append kernel).

Other legs (same JSON line, key "legs"): the bulk quantizer (32,768 tokens x
61 layers of Student-t rows with planted special rows; the same rows also
through the producer step fused with the quantizer), the 256k-token
split-T decode with 64 ranges, and the ragged Q=4 multi-query decode.

The CPU baseline is the oracle (oracle/, test infrastructure) timed on a
bounded sample of the headline decode on this host's cores.
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
        "kernel_ms": {"quantize_append": float(iv[:, 0].mean()),
                      "absorb_decode_kernel": dec_ms,
                      "lse_merge_kernel": float(iv[:, 2].mean()),
                      "absorb_decode_kernel_best": float(iv[:, 1].min())},
        "flops_per_step": flops, "kv_bytes_per_step": kv_bytes,
    }
    # duration of the decode kernel alone for the roofline: the same launches
    # back to back (the per-step events above also hold each launch's
    # dispatch gap behind the append kernel)
    b2b = max(steps, 10)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(b2b):
        c = (warmup + 2 * steps + i) % n_copies
        kv8.absorb_decode_partials(qs[c][0], qs[c][1], caches[c][0], caches[c][1], kv_start, kv_len,
                                   T, sc, split_tokens, n_splits, partials)
    e1.record()
    torch.cuda.synchronize()
    res["kernel_ms"]["absorb_decode_kernel_back_to_back"] = e0.elapsed_time(e1) / b2b
    res["decode_kernel_tflops"] = flops / (dec_ms * 1e-3) / 1e12
    res["decode_kernel_kv_gb_per_s"] = kv_bytes / (dec_ms * 1e-3) / 1e9
    # CPU baseline: the oracle on a bounded sample of the same decode
    cpu = None
    if cpu_sample_rows > 0:
        import oracle
        codes, scales = caches[(warmup + steps - 1) % n_copies]
        c_h, s_h = codes.cpu().numpy(), scales.cpu().numpy()
        ql_h = qs[(warmup + steps - 1) % n_copies][0].view(torch.int16).cpu().numpy().view(np.uint16)
        qr_h = qs[(warmup + steps - 1) % n_copies][1].view(torch.int16).cpu().numpy().view(np.uint16)
        cores = oracle.default_threads()
        n_sel = min(cpu_sample_rows, B * Q * H)
        sel = np.linspace(0, B * Q * H - 1, n_sel).astype(np.int64)
        log("cpu baseline: oracle on %d of %d query rows, %d threads" % (sel.size, B * Q * H, cores))
        # repeat the sample until about 10 s of CPU work (at most 8 times); median pass
        times = []
        while len(times) < 8 and sum(times) < 10.0:
            t0 = time.perf_counter()
            oracle.attention(ql_h, qr_h, c_h, s_h, w.kv_start, w.kv_len, Q=Q, softmax_scale=sc,
                             sel=sel, threads=cores)
            times.append(time.perf_counter() - t0)
        dt = float(np.median(times))
        sflops = float(FLOPS_PER_ROW_TOKEN) * T * sel.size
        cpu = {"value": sflops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": "%d of %d query rows of the headline decode (T=8192, every sequence), "
                         "f64; median of %d passes, %.2f s each, %.1f s in total"
                         % (sel.size, B * Q * H, len(times), dt, sum(times))}
    return res, cpu


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
    timer = Timer(torch, 2, steps)
    for t in range(steps):
        timer.mark(t, 0)
        kv8.quantize_rows(rows, codes, scales)
        timer.mark(t, 1)
    torch.cuda.synchronize()
    ms = float(timer.intervals_ms()[:, 0].mean())
    nbytes = float(n) * (4 * D + D + 8)
    res = {"rows": n, "ms": ms, "rows_per_s": n / (ms * 1e-3),
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
    pms = timer_call(torch, steps, prod)
    pbytes = float(n) * (4 * D + 8 + D + 8)
    res["producer"] = {"rows": n, "ms": pms, "rows_per_s": n / (pms * 1e-3),
                       "gb_per_s": pbytes / (pms * 1e-3) / 1e9, "bytes_per_launch": pbytes,
                       "roofline": roofline_hbm(pbytes, pms, counter_traffic("norm_rope_quantize_rows",
                                                                            "kv8_quantize.hip"))}
    del rows, codes, scales, pos
    torch.cuda.empty_cache()
    return res


def _decode_workload_leg(torch, kv8, w, steps, splits=None):
    dev = "cuda"
    rows = torch.from_numpy(w.rows).to(dev)
    n = w.n_rows
    codes = torch.empty((n, D), dtype=torch.uint8, device=dev)
    scales = torch.empty((n, 2), dtype=torch.float32, device=dev)
    kv8.quantize_rows(rows, codes, scales)
    torch.cuda.synchronize()
    qt = timer_call(torch, steps, lambda: kv8.quantize_rows(rows, codes, scales))
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
    ms = timer_call(torch, steps, fn)
    visible = sum(max(0, int(L) - (w.Q - 1) + i) for L in w.kv_len for i in range(w.Q))
    flops = float(FLOPS_PER_ROW_TOKEN) * w.H * visible
    kv_bytes = float(KV_BYTES_PER_TOKEN) * int(w.kv_len.sum())
    qbytes = float(n) * (4 * D + D + 8)
    return {"B": w.B, "Q": w.Q, "H": w.H, "tokens": int(w.kv_len.sum()), "ms": ms,
            "tflops": flops / (ms * 1e-3) / 1e12, "pct_peak_bf16": 100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "kv_gb_per_s": kv_bytes / (ms * 1e-3) / 1e9,
            "cache_build": {"rows": n, "ms": qt, "rows_per_s": n / (qt * 1e-3),
                            "gb_per_s": qbytes / (qt * 1e-3) / 1e9}}


def leg_project(torch, kv8, steps):
    """Non-absorbed projection of one 8,192-token sequence's cache rows by a
    bf16 kv_b weight of N = 128 heads x (128 + 128) columns (random weights)."""
    n, N = 8192, 32768
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    rows = torch.randn((n, D), generator=g, device="cuda")
    codes = torch.empty((n, D), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, 2), dtype=torch.float32, device="cuda")
    kv8.quantize_rows(rows, codes, scales)
    del rows
    w = (torch.randn((N, KL), generator=g, device="cuda") * 0.05).to(torch.bfloat16)
    out = torch.empty((n, N), dtype=torch.bfloat16, device="cuda")
    rope = torch.empty((n, KR), dtype=torch.float32, device="cuda")
    fn = lambda: kv8.project_rows(codes, scales, w, out=out, rope_out=rope)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ms = timer_call(torch, steps, fn)
    flops = 2.0 * n * KL * N
    nbytes = float(n) * (D + 8) + 2.0 * N * KL + 2.0 * n * N + 4.0 * n * KR
    ach = flops / (ms * 1e-3) / 1e12
    del codes, scales, w, out, rope
    torch.cuda.empty_cache()
    return {"rows": n, "N": N, "ms": ms, "tflops": ach, "gb_per_s": nbytes / (ms * 1e-3) / 1e9,
            "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS, "traffic": None}}


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
    timer = Timer(torch, 2, steps)
    for t in range(steps):
        timer.mark(t, 0)
        fn()
        timer.mark(t, 1)
    torch.cuda.synchronize()
    return float(timer.intervals_ms()[:, 0].mean())


def roofline_hbm(nbytes, ms, traffic):
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBPS, "traffic": traffic}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--legs", default="decode,quantize,splitT,project,ragged",
                    help="comma list of decode, quantize, splitT, project, ragged, copy")
    ap.add_argument("--cpu-sample-rows", type=int, default=4096,
                    help="query rows the oracle times for the CPU baseline (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
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
    dec_ms = res["kernel_ms"]["absorb_decode_kernel_back_to_back"]
    ach = flops / (dec_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": "absorb_decode_kernel", "kernel_ms": dec_ms,
            "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS,
            "traffic": counter_traffic("absorb_decode_kernel", "kv8_decode.hip")}
    extra = {}
    if "quantize" in legs:
        extra["bulk_quantize"] = leg_quantize(torch, kv8, W, max(5, args.steps // 2))
    if "splitT" in legs:
        log("splitT: 256k-token slot, 64 ranges")
        extra["splitT_256k"] = _decode_workload_leg(torch, kv8, W.long_context(seed=0),
                                                    max(5, args.steps // 2), splits=64)
    if "project" in legs:
        log("project: 8192 rows x N=32768")
        extra["project_8k"] = leg_project(torch, kv8, max(5, args.steps // 4))
    if "copy" in legs:
        extra["copy_1gib"] = leg_copy(torch, 3)
    if "ragged" in legs:
        log("ragged: B=64, lengths U[1k,64k], Q=4")
        extra["ragged_q4"] = _decode_workload_leg(torch, kv8, W.ragged(seed=0),
                                                  max(3, args.steps // 4))
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
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "batched absorbed-MLA decode step: B=32 x T=8192 x H=128, Q=1, "
                               "latent 512+64 e4m3 with per-row f32 scales; append 1 row/sequence "
                               "+ decode; 3 rotating cache copies (cold)",
                   "B": 32, "T": 8192, "H": 128, "Q": 1, "kv_lora": KL, "rope": KR,
                   "split_tokens": res["split_tokens"], "num_splits": res["num_splits"]},
        "pct_peak_bf16": 100 * res["tflops_step"] / PEAK_BF16_TFLOPS,
        "kv_gb_per_s": res["kv_gb_per_s_step"],
        "kernel_ms": res["kernel_ms"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "legs": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
