"""Build the CPU oracle (test infrastructure only) with the host C++ compiler.

    python oracle/build.py            # -> oracle/liboracle.so
    python oracle/build.py --selftest # also builds and runs the sanitizer self-test

The oracle is compiled without fast-math and with FP contraction off, so each
float operation in it is a single IEEE operation rounded to nearest-even.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kv8_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")
SELFTEST_SRC = os.path.join(HERE, "selftest.cpp")
SELFTEST_BIN = os.path.join(HERE, "selftest_san")

CXX = os.environ.get("CXX", "g++")
FLAGS = ["-std=c++17", "-O2", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
         "-Wall", "-Wextra", "-pthread"]


def build_lib():
    tmp = LIB + ".tmp"
    cmd = [CXX, *FLAGS, "-shared", SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def build_selftest():
    """ASan + UBSan build of the oracle together with its C++ self-test."""
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
           "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           SRC, SELFTEST_SRC, "-o", SELFTEST_BIN]
    subprocess.run(cmd, check=True)
    return SELFTEST_BIN


if __name__ == "__main__":
    print(build_lib())
    if "--selftest" in sys.argv:
        exe = build_selftest()
        subprocess.run([exe], check=True)
