"""The kernels' exact division (paged_kv_gqa_03_amd/csrc/fastdiv.hpp) checked
on the CPU: the header is plain C++, compiled here with g++ and run over
every 32-bit numerator for divisors that earlier magic-number division got
wrong (block sizes 1000 and 3000 from slot 6.1M on), powers of two, 1, and
the largest divisors, then over random (numerator, divisor) pairs."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "fastdiv_check.cpp")
INC = os.path.join(ROOT, "paged_kv_gqa_03_amd", "csrc")


def test_exact_division_every_32bit_numerator(tmp_path):
    exe = str(tmp_path / "fastdiv_check")
    subprocess.run(["g++", "-O2", "-fopenmp", "-std=c++17", "-I" + INC, SRC, "-o", exe], check=True)
    divisors = ["1", "2", "3", "7", "16", "1000", "3000", "65537", "2147483647", "2147483648", "4294967295"]
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([exe] + divisors, capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
