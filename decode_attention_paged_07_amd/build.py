"""Compile the HIP sources into the in-tree shared library libpa_decode.so.

Each source is compiled for gfx950 by its own hipcc process (in parallel,
objects in a temporary directory), then one hipcc link writes the library
next to this file; it is replaced atomically so a running process never
loads a half-written library.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_NAME = "libpa_decode.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = [os.path.join(PKG_DIR, "csrc", f)
           for f in ("pa_kernels.hip", "pa_shared.hip", "pa_append.hip", "pa_mla.hip", "pa_mla_wide.hip", "pa_probe.hip",
                     "pa_noalloc.hip", "pa_api.cpp",
                     "pa_blocks.cpp")]
INCLUDE = os.path.join(ROOT, "include")

# Packed-fp32 VALU instructions stay disabled in device code: plain float
# arithmetic is emitted as scalar-per-lane VALU ops.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]

# MFMA results go to ordinary VGPRs (amdgpu-mfma-vgpr-form) in every source
# but pa_mla_wide.hip. By default the backend gives a kernel whose launch
# bounds allow more than 256 registers per lane the accumulator-register (AGPR)
# form of every MFMA; the decode loop's output accumulators then live in
# AGPRs, and since VALU code cannot operate on AGPRs they are copied out and
# back around every block (about 40 % of the loop's VALU instructions at head
# size 128). With the VGPR form those copies disappear, each decode kernel
# needs fewer registers (bf16 at head size 128: 218 instead of 236 per lane;
# the shared-prefix kernel: 314 instead of 442), and outputs are
# bit-identical. Measured on MI355X: the shared-prefix call 3-5 % faster, the
# decode workloads equal within 1 %. The 32-heads-per-wave latent-cache kernel
# needs both register files (256 output accumulators beside 144 registers of
# queries), which only the AGPR form provides; its VALU code touches the
# accumulators only to rescale them, rarely, and at the end.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
SOURCE_FLAGS = {"pa_mla_wide.hip": []}


def source_flags(src: str):
    return SOURCE_FLAGS.get(os.path.basename(src), VGPR_FORM)


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libpa_decode.so")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; drop that notice.
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    return res.returncode, msgs


def build(verbose: bool = False, extra_flags=None, out_path: str = LIB_PATH, host_flags=None) -> str:
    """Compile every source and link ``out_path`` (default: the in-tree library).

    extra_flags go to every compile; host_flags (e.g. sanitizer options, each
    behind -Xarch_host) to every compile and to the link."""
    tmp = out_path + f".tmp{os.getpid()}"
    flags = [*HIP_FLAGS, *(extra_flags or []), *(host_flags or [])]
    with tempfile.TemporaryDirectory(prefix="pa_build_") as objdir:
        def compile_one(src):
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            rc, msgs = _run([hipcc(), *flags, *source_flags(src), "-I", INCLUDE, "-I", os.path.join(PKG_DIR, "csrc"),
                             "-c", src, "-o", obj], verbose)
            return src, obj, rc, msgs

        jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8"))))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, SOURCES))
        failed = [(src, rc, msgs) for src, _, rc, msgs in results if rc != 0]
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(f"{src} ({rc}):\n{msgs}" for src, rc, msgs in failed))
        if verbose:
            for _, _, _, msgs in results:
                if msgs.strip():
                    print(msgs, file=sys.stderr)
        rc, msgs = _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *(host_flags or []),
                         "-o", tmp, *[obj for _, obj, _, _ in results]], verbose)
        if rc != 0:
            if os.path.exists(tmp):
                os.unlink(tmp)
            raise RuntimeError(f"hipcc link failed ({rc}):\n{msgs}")
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
