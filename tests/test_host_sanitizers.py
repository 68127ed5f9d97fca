"""The C-ABI host layer (argument validation, status strings, the host-side
metadata and prefix-group checkers) built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side, then the whole CPU ABI test
file run against that build in a child process with the sanitizer runtime
preloaded.  Any out-of-bounds access, use after free or undefined behaviour
on those paths aborts the child.  CPU only: no call here reaches a device.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_gqa_attention_neox_amd")
HIPCC = "/opt/rocm/bin/hipcc"
# sanitizers on the host pass only (each -fsanitize right after -Xarch_host)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]
KERNEL_OBJS = ["rope_cache.o", "decode.o", "prefill.o", "attn_generic.o"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not available")
    objs = [os.path.join(PKG, "_build", o) for o in KERNEL_OBJS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (run the package build first)")
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libqwen2attn_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", *SAN, "-x", "hip", "-c",
                    os.path.join(PKG, "csrc", "qwen2_attn_api.cpp"), "-o", api_o],
                   check=True, capture_output=True, text=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *SAN,
                    api_o, *objs, "-o", lib], check=True, capture_output=True, text=True)
    undef = subprocess.run(["nm", "-u", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in undef and "__ubsan_handle" in undef, "build is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "from paged_gqa_attention_neox_amd import binding as B\n"
        "B.LIB_PATH = %r\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r,"
        " '-k', 'not exported_dynamic_symbols']))\n"
    ) % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail
    assert "runtime error" not in tail, tail
