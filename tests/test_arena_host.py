"""The work-list arena's range logic (decode_kv_cache_amd/csrc/kvx_arena.h)
on the CPU: tests/cpp/arena_test.cpp drives it with random allocations and
releases over made-up chunk addresses and checks, after every operation,
that live ranges never overlap and stay inside chunks, that free and live
bytes add up to the chunk bytes, that a failing chunk allocation is passed
back, and that releasing everything leaves each chunk whole (never merged
with an adjacent chunk)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="no C++ compiler")


def test_arena_random_operations(tmp_path):
    exe = str(tmp_path / "arena_test")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror",
                        f"-I{os.path.join(ROOT, 'decode_kv_cache_amd', 'csrc')}",
                        os.path.join(ROOT, "tests", "cpp", "arena_test.cpp"), "-o", exe, "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
