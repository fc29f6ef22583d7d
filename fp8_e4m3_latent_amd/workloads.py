"""Seeded synthetic workloads for the fp8 e4m3 latent KV cache.

This module only draws inputs: f32 latent rows, bf16 queries and the sequence
layout of the cache.  It holds none of the cache's arithmetic (no encoding,
decoding, scaling or attention); the tests feed the same arrays to the HIP
library and to the CPU oracle.

Conventions (all workloads):
  * numpy ``Generator(PCG64)``; ``SeedSequence(seed).spawn(k)`` gives one child
    stream per tensor, in a fixed order, so every tensor is reproducible on
    its own;
  * rows are f32, one row per token, ``kv_lora`` Lc values then ``rope`` Rc
    values (512 + 64 by default); the cache holds sequence b at rows
    ``kv_start[b] .. kv_start[b] + kv_len[b] - 1``;
  * queries are drawn in f32 with standard deviation 1/24 (= 1/sqrt(576)) and
    rounded to bf16 (round to nearest even), kept as uint16 bit patterns;
  * the softmax scale is the f32 value nearest 1/24.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

KV_LORA = 512
ROPE = 64
D = KV_LORA + ROPE
SOFTMAX_SCALE = np.float32(1.0 / 24.0)
Q_STD = np.float32(1.0 / 24.0)


def _streams(seed, n):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def bf16_bits(x):
    """Round f32 values to bf16 (nearest even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _queries(rng_lat, rng_rope, B, Q, H, kv_lora=KV_LORA, rope=ROPE):
    q_lat = rng_lat.standard_normal((B, Q, H, kv_lora), dtype=np.float32) * Q_STD
    q_rope = rng_rope.standard_normal((B, Q, H, rope), dtype=np.float32) * Q_STD
    return bf16_bits(q_lat), bf16_bits(q_rope)


def queries(seed, B, Q, H):
    """bf16 (q_lat, q_rope) of shape [B,Q,H,512] / [B,Q,H,64], std 1/24."""
    r_ql, r_qr = _streams(seed, 2)
    return _queries(r_ql, r_qr, B, Q, H)


def fresh_rows(seed, n):
    """n new f32 latent rows ~N(0,1) (the rows a decode step appends)."""
    (r,) = _streams(seed, 1)
    return r.standard_normal((n, D), dtype=np.float32)


@dataclass
class DecodeWorkload:
    """Inputs of one absorbed decode over a quantized latent cache."""
    name: str
    B: int
    Q: int
    H: int
    rows: np.ndarray            # f32 [n_rows, D]: the rows the cache is built from
    kv_start: np.ndarray        # int64 [B]
    kv_len: np.ndarray          # int32 [B]
    q_lat: np.ndarray           # uint16 (bf16) [B, Q, H, KV_LORA]
    q_rope: np.ndarray          # uint16 (bf16) [B, Q, H, ROPE]
    softmax_scale: np.float32 = SOFTMAX_SCALE
    num_splits: int = 1
    kv_lora: int = KV_LORA
    rope: int = ROPE
    notes: dict = field(default_factory=dict)

    @property
    def n_rows(self):
        return int(self.rows.shape[0])

    @property
    def max_len(self):
        return int(self.kv_len.max()) if self.B else 0


def tiny(seed=0, B=1, Q=1, H=16, T=1024, outlier_p=0.01, outlier_mul=50.0):
    """Tiny absorbed decode: rows ~N(0,1) with a Bernoulli(outlier_p) fraction of
    entries multiplied by outlier_mul (both segments), queries as above."""
    r_rows, r_mask, r_ql, r_qr = _streams(seed, 4)
    rows = r_rows.standard_normal((B * T, D), dtype=np.float32)
    mask = r_mask.random((B * T, D)) < outlier_p
    rows[mask] *= np.float32(outlier_mul)
    q_lat, q_rope = _queries(r_ql, r_qr, B, Q, H)
    kv_start = np.arange(B, dtype=np.int64) * T
    kv_len = np.full(B, T, dtype=np.int32)
    return DecodeWorkload("tiny", B, Q, H, rows, kv_start, kv_len, q_lat, q_rope)


def batched(seed=0, B=32, T=8192, H=128, Q=1):
    """Batched single-layer decode: B sequences of T tokens, rows ~N(0,1)."""
    r_rows, r_ql, r_qr = _streams(seed, 3)
    rows = r_rows.standard_normal((B * T, D), dtype=np.float32)
    q_lat, q_rope = _queries(r_ql, r_qr, B, Q, H)
    kv_start = np.arange(B, dtype=np.int64) * T
    kv_len = np.full(B, T, dtype=np.int32)
    return DecodeWorkload("batched", B, Q, H, rows, kv_start, kv_len, q_lat, q_rope)


def long_context(seed=0, T=262144, H=128, num_splits=64, planted_frac=0.005,
                 match_rms=4.0):
    """One long sequence with planted strong matches.

    A planted_frac share of the token rows (at seeded distinct positions) get,
    for the k-th planted row, an Lc part pointing along the Lc query of head
    k mod H with root-mean-square match_rms (so a planted row scores far above
    the ~N(0, 1/24^2) scores of ordinary rows and the softmax is peaked);
    their Rc part stays ~N(0,1)."""
    r_rows, r_pos, r_ql, r_qr = _streams(seed, 4)
    rows = r_rows.standard_normal((T, D), dtype=np.float32)
    q_lat, q_rope = _queries(r_ql, r_qr, 1, 1, H)
    n_plant = int(round(planted_frac * T))
    pos = np.sort(r_pos.choice(T, size=n_plant, replace=False))
    ql = bf16_to_f32(q_lat[0, 0]).astype(np.float64)          # [H, KV_LORA]
    unit = ql / np.linalg.norm(ql, axis=1, keepdims=True)
    heads = np.arange(n_plant) % H
    rows[pos, :KV_LORA] = (match_rms * np.sqrt(KV_LORA) * unit[heads]).astype(np.float32)
    w = DecodeWorkload("long_context", 1, 1, H, rows, np.zeros(1, np.int64),
                       np.full(1, T, np.int32), q_lat, q_rope, num_splits=num_splits)
    w.notes["planted_rows"] = pos
    w.notes["planted_heads"] = heads
    return w


def ragged(seed=0, B=64, H=128, Q=4, len_lo=1024, len_hi=65536):
    """Ragged multi-query decode: lengths uniform on [len_lo, len_hi] (inclusive),
    Q causal query positions per sequence, rows ~N(0,1) packed back to back."""
    r_len, r_rows, r_ql, r_qr = _streams(seed, 4)
    kv_len = r_len.integers(len_lo, len_hi, size=B, endpoint=True).astype(np.int32)
    kv_start = np.zeros(B, dtype=np.int64)
    kv_start[1:] = np.cumsum(kv_len[:-1], dtype=np.int64)
    n = int(kv_len.sum(dtype=np.int64))
    rows = _normal_rows_threaded(r_rows, n)
    q_lat, q_rope = _queries(r_ql, r_qr, B, Q, H)
    return DecodeWorkload("ragged", B, Q, H, rows, kv_start, kv_len, q_lat, q_rope)


def _normal_rows_threaded(rng, n, chunk=32768, threads=None):
    seeds = rng.bit_generator.seed_seq.spawn((n + chunk - 1) // chunk)
    out = np.empty((n, D), dtype=np.float32)

    def fill(i):
        g = np.random.Generator(np.random.PCG64(seeds[i]))
        b = i * chunk
        e = min(n, b + chunk)
        out[b:e] = g.standard_normal((e - b, D), dtype=np.float32)

    with ThreadPoolExecutor(threads or min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(len(seeds))))
    return out


# ---------------------------------------------------------------------------
# Bulk rows for the quantizer, with planted special rows
# ---------------------------------------------------------------------------

def tie_midpoints():
    """The 126 points halfway between consecutive non-negative e4m3 values below
    448, listed from the format's grid: in the subnormal step 2^-9 the points
    (2m+1) 2^-10, m = 0..7; in each binade [2^E, 2^(E+1)), E = -6..7, the points
    (1 + (2m+1)/16) 2^E, m = 0..7; in the top binade (E = 8) m = 0..5 only."""
    pts = [(2 * m + 1) * 2.0 ** -10 for m in range(8)]
    for E in range(-6, 8):
        pts += [(1 + (2 * m + 1) / 16) * 2.0 ** E for m in range(8)]
    pts += [(1 + (2 * m + 1) / 16) * 2.0 ** 8 for m in range(6)]
    return np.array(pts, dtype=np.float32)


SPECIAL_KINDS = ("zero", "subnormal_amax", "nan", "tie", "inf")
GUARD_AMAX = (1e-37, 1.3165e-36, 1.3166e-36, 2e-36)


def bulk_rows(seed=0, tokens=32768, layers=61, special_frac=0.001, guard_rows=16,
              threads=None):
    """tokens x layers rows of Student-t(3) x 0.5 values (drawn as
    Z / sqrt(2 G / 3), Z ~ N(0,1), G ~ Gamma(3/2)), one child stream per layer.

    Planted at distinct seeded rows, round(special_frac * n) rows of each kind,
    every special in both segments:
      zero            all entries +-0 (random signs);
      subnormal_amax  entries 1e-40 * U(-1,1), one entry exactly +-1e-40;
      nan             1..8 entries per segment NaN (random sign and payload);
      tie             k = 2^j, j ~ U{-20..20}: one entry +-448k, the rest
                      +-k * (a random e4m3 tie midpoint), so every scaled entry
                      sits exactly halfway between two codes;
      inf             1..4 entries per segment +-inf.
    Plus guard_rows rows for each amax in GUARD_AMAX (entries amax * U(-1,1),
    one entry exactly +-amax) and guard_rows rows whose entries are f32
    subnormals under an amax of 2e-36.
    Returns (rows f32 [tokens*layers, D], dict kind -> row indices)."""
    n = tokens * layers
    ss = np.random.SeedSequence(seed)
    layer_seeds = ss.spawn(layers)
    r_pos, r_special = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(2)]
    rows = np.empty((n, D), dtype=np.float32)
    c23 = np.float32(2.0 / 3.0)

    def fill(i):
        g = np.random.Generator(np.random.PCG64(layer_seeds[i]))
        z = g.standard_normal((tokens, D), dtype=np.float32)
        gam = g.standard_gamma(1.5, size=(tokens, D), dtype=np.float32)
        rows[i * tokens:(i + 1) * tokens] = np.float32(0.5) * z / np.sqrt(gam * c23)

    with ThreadPoolExecutor(threads or min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(layers)))

    n_spec = int(round(special_frac * n))
    n_guard = guard_rows * (len(GUARD_AMAX) + 1)
    picks = r_pos.choice(n, size=n_spec * len(SPECIAL_KINDS) + n_guard, replace=False)
    index = {}
    for k, kind in enumerate(SPECIAL_KINDS):
        index[kind] = np.sort(picks[k * n_spec:(k + 1) * n_spec])
    gpos = picks[n_spec * len(SPECIAL_KINDS):]
    for k, a in enumerate(GUARD_AMAX):
        index["guard_%g" % a] = np.sort(gpos[k * guard_rows:(k + 1) * guard_rows])
    index["guard_subnormal_entries"] = np.sort(gpos[len(GUARD_AMAX) * guard_rows:])

    segs = ((0, KV_LORA), (KV_LORA, D))
    rs = r_special
    mids = tie_midpoints()

    def signs(size):
        return np.where(rs.random(size) < 0.5, np.float32(1), np.float32(-1))

    for r in index["zero"]:
        rows[r] = np.where(rs.random(D) < 0.5, np.float32(0.0), np.float32(-0.0))
    for r in index["subnormal_amax"]:
        for a, b in segs:
            v = (np.float32(1e-40) * rs.uniform(-1, 1, b - a).astype(np.float32)).astype(np.float32)
            v[rs.integers(b - a)] = np.float32(1e-40) * signs(1)[0]
            rows[r, a:b] = v
    for r in index["nan"]:
        for a, b in segs:
            k = rs.integers(1, 9)
            cols = a + rs.choice(b - a, size=k, replace=False)
            payload = rs.integers(1, 1 << 23, size=k).astype(np.uint32)
            sign = (rs.random(k) < 0.5).astype(np.uint32) << 31
            rows[r, cols] = (sign | np.uint32(0x7F800000) | payload).view(np.float32)
    for r in index["tie"]:
        for a, b in segs:
            kk = np.float32(2.0 ** int(rs.integers(-20, 21)))
            v = mids[rs.integers(len(mids), size=b - a)] * kk * signs(b - a)
            v[rs.integers(b - a)] = np.float32(448.0) * kk * signs(1)[0]
            rows[r, a:b] = v
    for r in index["inf"]:
        for a, b in segs:
            k = rs.integers(1, 5)
            cols = a + rs.choice(b - a, size=k, replace=False)
            rows[r, cols] = np.float32(np.inf) * signs(k)
    for k, amax in enumerate(GUARD_AMAX):
        am = np.float32(amax)
        for r in index["guard_%g" % amax]:
            for a, b in segs:
                v = (am * rs.uniform(-1, 1, b - a).astype(np.float32)).astype(np.float32)
                v[rs.integers(b - a)] = am * signs(1)[0]
                rows[r, a:b] = v
    am = np.float32(2e-36)
    for r in index["guard_subnormal_entries"]:
        for a, b in segs:
            # f32 subnormals (below 2^-126) under a normal amax
            v = (np.float32(1e-39) * rs.uniform(-1, 1, b - a).astype(np.float32)).astype(np.float32)
            v[rs.integers(b - a)] = am * signs(1)[0]
            rows[r, a:b] = v
    return rows, index
