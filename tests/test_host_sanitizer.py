"""Host-side validation, planning and the block pool under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed).

A copy of the library is built with the sanitizers on its host code only
(each -fsanitize behind -Xarch_host; the gfx950 device code is unchanged) into
_build/sanitize/, rebuilt when a source changes, and the CPU tests of the C
ABI, the block pool, the latent-cache ABI and the threaded calls run against it in a child
process that preloads the ASan runtime. Any report aborts the child.
"""

import glob
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
TESTS = ["tests/test_abi_cpu.py", "tests/test_block_pool.py", "tests/test_mla_abi_cpu.py", "tests/test_threads_cpu.py"]
HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
              "-shared-libasan"]


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def sources_digest(build_mod):
    h = hashlib.sha256()
    for path in sorted(build_mod.SOURCES + glob.glob(os.path.join(build_mod.PKG_DIR, "csrc", "*.h"))
                       + glob.glob(os.path.join(ROOT, "include", "*.h"))):
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(HOST_FLAGS + build_mod.HIP_FLAGS).encode())
    return h.hexdigest()[:16]


@pytest.fixture(scope="module")
def sanitized_lib():
    import __graft_entry__
    b = __graft_entry__._build_module()
    os.makedirs(OUT_DIR, exist_ok=True)
    lib = os.path.join(OUT_DIR, f"libpa_decode_asan_{sources_digest(b)}.so")
    if not os.path.exists(lib):
        for old in glob.glob(os.path.join(OUT_DIR, "libpa_decode_asan_*.so")):
            os.unlink(old)
        b.build(out_path=lib, host_flags=HOST_FLAGS)
    return lib


@pytest.mark.skipif(asan_runtime() is None, reason="clang ASan runtime not installed")
def test_host_code_is_clean_under_address_and_ub_sanitizers(sanitized_lib):
    out = subprocess.run(["nm", "-D", sanitized_lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out      # the copy is instrumented
    env = dict(os.environ, LD_PRELOAD=asan_runtime(), PA_DECODE_LIB=sanitized_lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *TESTS],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail
