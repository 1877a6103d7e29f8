"""The C ABI from C: include/kvx.h and include/kvx_xfer.h compile as strict
C99 (-pedantic -Werror), and two C programs linked against the in-tree
libkvx.so check cases worked by hand (host-only: no device memory is
touched): tests/c_abi/plan_from_c.c plans a transfer and checks its runs,
triples, byte counts and error classes; tests/c_abi/xfer_from_c.c drives
the transfer state machine through prefill-first deferral, a failed write
with its recompute list, and a deferral timeout; tests/c_abi/xfer_threads_from_c.c
shares one state machine between eight threads.  On a GPU,
tests/c_abi/push_from_c.c runs the device calls from C."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_kv_cache_amd")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
FLAGS = ["-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
         "-isystem", ROCM_INCLUDE, "-D__HIP_PLATFORM_AMD__=1"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")


def test_headers_compile_as_c99():
    for h in ("kvx.h", "kvx_xfer.h"):
        r = subprocess.run(["gcc"] + FLAGS + ["-fsyntax-only", "-x", "c", os.path.join(ROOT, "include", h)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


@pytest.mark.parametrize("prog", ["plan_from_c", "xfer_from_c", "xfer_threads_from_c"])
def test_c_program(prog, tmp_path):
    lib = os.path.join(PKG, "libkvx.so")
    assert os.path.exists(lib), "build libkvx.so first (python -m decode_kv_cache_amd.build)"
    exe = str(tmp_path / prog)
    r = subprocess.run(["gcc"] + FLAGS + [os.path.join(ROOT, "tests", "c_abi", prog + ".c"), f"-L{PKG}", "-lkvx",
                                          f"-Wl,-rpath,{PKG}", "-lpthread", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.gpu
def test_device_calls_from_c(tmp_path):
    """tests/c_abi/push_from_c.c: device pools allocated from C, then
    kvx_push_layer, kvx_pack + kvx_unpack, kvx_push_many, the write queue
    behind another stream's events, and kvx_copy_heads_layers into a one-head
    HND pool, each checked byte for byte against the per-token definition
    written in the program."""
    lib = os.path.join(PKG, "libkvx.so")
    assert os.path.exists(lib), "build libkvx.so first (python -m decode_kv_cache_amd.build)"
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    exe = str(tmp_path / "push_from_c")
    r = subprocess.run(["gcc"] + FLAGS + [os.path.join(ROOT, "tests", "c_abi", "push_from_c.c"), f"-L{PKG}", "-lkvx",
                                          f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{PKG}",
                                          f"-Wl,-rpath,{rocm_lib}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    print("running", exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
