"""The library's host rules (csrc/walker.h and csrc/host_rules.h: ownership walk, argument
checks, work-item targets, workspace layout) built with a host compiler under address and
undefined-behaviour sanitizers, every finding fatal.  CPU only.

tests/host_rules_check.cpp holds the checks: the walker against brute force on small
sequences, against every position below 2^31 - 1 for three (C, I) pairs and against
invariants at the 2^31 bounds; the argument checks against the documented contract
rewritten in 128-bit arithmetic over 800,000 drawn argument sets (extreme values
included); the workspace layout's alignment and section sizes.  Here the walker's counts
and positions are also compared with the oracle's plain filter over positions."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import dcp_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CXX = shutil.which("g++") or shutil.which("clang++")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
INC = ["-I", os.path.join(ROOT, "include"), "-I",
       os.path.join(ROOT, "decode_attention_context_amd", "csrc"), "-I", "/opt/rocm/include",
       "-D__HIP_PLATFORM_AMD__"]

pytestmark = pytest.mark.skipif(CXX is None or not os.path.isdir("/opt/rocm/include"),
                                reason="needs a host C++ compiler and the ROCm headers")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("host_rules") / "host_rules_check")
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror"] + SAN + INC + \
        [os.path.join(ROOT, "tests", "host_rules_check.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _run(args, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run(args, capture_output=True, text=True, timeout=timeout, env=env)


def test_sanitizers_are_live(tmp_path):
    """The same flags turn a signed overflow into a failing run (so a silent pass below
    means no finding, not a disabled sanitizer)."""
    src = tmp_path / "ovf.cpp"
    src.write_text("#include <climits>\n#include <cstdlib>\n"
                   "int main(int c, char**) { int x = INT_MAX - 1 + c; x += 1; "
                   "return x == 0 ? 3 : 0; }\n")
    exe = str(tmp_path / "ovf")
    subprocess.run([CXX, "-std=c++17", "-O1"] + SAN + [str(src), "-o", exe], check=True)
    r = _run([exe])
    assert r.returncode != 0 and "runtime error" in r.stderr, (r.returncode, r.stderr)


def test_host_rules_self_checks(checker):
    r = _run([checker, "self"])
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


POSITION_CASES = [(0, 0, 1, 1), (1, 0, 2, 1), (1, 1, 2, 1), (1000, 1, 2, 128), (4097, 3, 8, 64),
                  (10000, 2, 3, 100), (12345, 0, 4, 1), (65536, 7, 8, 64), (70000, 5, 7, 13),
                  (200000, 3, 4, 128), (99991, 0, 1, 16)]


@pytest.mark.parametrize("L,rank,C,I", POSITION_CASES)
def test_walker_positions_match_oracle(checker, L, rank, C, I):
    r = _run([checker, "positions", str(L), str(rank), str(C), str(I)])
    assert r.returncode == 0, r.stderr
    lines = r.stdout.split()
    n64, n32 = int(lines[0]), int(lines[1])
    got = np.array([int(x) for x in lines[2:]], dtype=np.int64)
    ref = orc.owned_tokens(L, rank, C, I)
    assert n64 == n32 == ref.size
    assert np.array_equal(got, ref)


COUNT_CASES = [(1 << 24, 3, 8, 64), ((1 << 24) + 77, 7, 8, 64), (16777259, 1, 3, 1),
               (20000000, 15, 16, 1000), (20000000, 0, 1, 1), (9999999, 2, 5, 1 << 20)]


@pytest.mark.parametrize("L,rank,C,I", COUNT_CASES)
def test_walker_counts_match_oracle(checker, L, rank, C, I):
    r = _run([checker, "count", str(L), str(rank), str(C), str(I)])
    assert r.returncode == 0, r.stderr
    n64, n32 = (int(x) for x in r.stdout.split()[:2])
    assert n64 == n32 == orc.owned_count(L, rank, C, I)
