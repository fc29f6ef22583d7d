"""The oracle built with AddressSanitizer + UndefinedBehaviorSanitizer runs its
self-test cleanly (page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with
.coli_kv v2", colibri PR #299, commit message, Validation: ASan/UBSan clean)."""
import subprocess

from oracle import build


def test_oracle_selftest_under_asan_ubsan():
    exe = build.build_selftest()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle selftest ok" in r.stdout
