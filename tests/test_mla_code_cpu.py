"""Checks on the built latent-cache (MLA) kernel's gfx950 code, no GPU needed.

* The tile reads (ds_read_b128) are an asm block whose outputs are
  early-clobber: no read may write a register that a later read of the same
  block uses as its address, or the returning data would redirect the later
  reads (the compiler treats an asm block's outputs as written at once).
* Residency of the persistent grid: each workgroup (one to four waves, one
  per 16-head group) uses 36 KiB of LDS and each wave more than 256 registers
  per lane, so a compute unit holds four waves (one per SIMD), the number the
  launch plan sizes the grid by; no scratch.
"""

import os
import re
import struct
import subprocess
import tempfile

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
LDS_PER_CU = 160 * 1024
REGISTERS_PER_SIMD_LANE = 512


@pytest.fixture(scope="module")
def lib_path():
    import __graft_entry__
    b = __graft_entry__._build_module()
    if not os.path.exists(b.LIB_PATH):
        b.build()
    return b.LIB_PATH


def gfx950_code_objects(path):
    with open(path, "rb") as f:
        data = f.read()
    base = data.find(b"__CLANG_OFFLOAD_BUNDLE__")
    while base >= 0:
        n = struct.unpack_from("<Q", data, base + 24)[0]
        off = base + 32
        for _ in range(n):
            o, size, tlen = struct.unpack_from("<QQQ", data, off)
            triple = data[off + 24:off + 24 + tlen].decode()
            off += 24 + tlen
            if triple.endswith("gfx950"):
                yield data[base + o:base + o + size]
        base = data.find(b"__CLANG_OFFLOAD_BUNDLE__", base + 1)


def mla_kernel_asm(path):
    for elf in gfx950_code_objects(path):
        if b"pa_mla_streamk_kernel" not in elf:
            continue
        with tempfile.NamedTemporaryFile(suffix=".co") as f:
            f.write(elf)
            f.flush()
            text = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", f.name], capture_output=True, text=True,
                                  check=True).stdout
        bodies = re.findall(r"<_ZN2pa21pa_mla_streamk_kernel[^>]*>:\n(.*?)(?:\n\n|\Z)", text, flags=re.S)
        assert bodies, "pa_mla_streamk_kernel not found in the disassembly"
        return "\n\n".join(bodies)        # every instantiation, groups kept apart
    raise AssertionError("no gfx950 code object holds pa_mla_streamk_kernel")


def read_groups(asm, op):
    """Runs of consecutive `op` reads: (first dest reg, last dest reg, address reg) each."""
    groups, cur = [], []
    for line in asm.splitlines():
        m = re.search(op + r" v\[(\d+):(\d+)\], v(\d+)", line)
        if m:
            cur.append(tuple(int(x) for x in m.groups()))
        elif cur:
            groups.append(cur)
            cur = []
    if cur:
        groups.append(cur)
    return groups


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not installed")
@pytest.mark.parametrize("op", ["ds_read_b128"])
def test_tile_reads_never_overwrite_their_address(lib_path, op):
    # 18 reads per bf16 tile, 9 per fp8 tile
    groups = [g for g in read_groups(mla_kernel_asm(lib_path), op) if len(g) >= 9]
    assert sum(len(g) >= 16 for g in groups) and sum(len(g) == 9 for g in groups), \
        f"expected asm groups of 18 and of 9 {op}"
    for g in groups:
        for i, (lo, hi, _) in enumerate(g):
            later = {a for _, _, a in g[i + 1:]}
            assert not any(lo <= a <= hi for a in later), f"{op} into v[{lo}:{hi}] clobbers a later address"


def test_persistent_grid_is_resident(lib_path):
    k = {name: r for name, r in bench.code_object_kernels(lib_path).items() if "pa_mla_streamk_kernel" in name}
    assert len(k) == 8                  # one to four head-group waves per workgroup, bf16 and fp8 cache
    for res in k.values():
        check_resident(res)


def test_wide_kernel_is_resident(lib_path):
    """The 32-heads-per-wave kernel: one workgroup (one wave per SIMD) per
    compute unit, so its LDS (two 36 KiB tile buffers and the accumulator
    staging, plus two 18 KiB code buffers with an fp8 cache) fits one compute
    unit's, each wave fits a SIMD's 512 registers per lane, and nothing spills
    to scratch."""
    k = {name: r for name, r in bench.code_object_kernels(lib_path).items() if "pa_mla_wide_kernel" in name}
    assert len(k) == 4                  # three or four 32-head waves per workgroup, bf16 and fp8 cache
    for name, res in k.items():
        assert res["scratch"] == 0
        low = (72 + 36 if "true>" in name else 72) * 1024
        assert low <= res["lds"] <= LDS_PER_CU, (name, res["lds"])
        assert (res["alloc"] or res["vgpr"]) <= REGISTERS_PER_SIMD_LANE


def test_bench_knows_which_kernel_runs():
    src = open(os.path.join(ROOT, "decode_attention_paged_07_amd", "csrc", "pa_api.cpp")).read()
    assert int(re.search(r"#define PA_MLA_WIDE_MIN_HEADS (\d+)", src).group(1)) == bench.MLA_WIDE_MIN_HEADS


def check_resident(res):
    assert res["scratch"] == 0
    assert res["lds"] <= 36 * 1024 + 1024
    # worst case: one-wave workgroups, each with its own tile buffers
    csrc = os.path.join(ROOT, "decode_attention_paged_07_amd", "csrc")
    knobs = open(os.path.join(csrc, "pa_kernels.h")).read() + open(os.path.join(csrc, "pa_api.cpp")).read()
    waves_per_cu = max(int(x) for x in re.findall(r"#define PA_MLA_(?:FP8_)?WAVES_PER_CU\w* (\d+)", knobs))
    assert waves_per_cu * res["lds"] <= LDS_PER_CU
    per_simd = math_ceil_div(waves_per_cu, 4)
    assert per_simd * (res["alloc"] or res["vgpr"]) <= REGISTERS_PER_SIMD_LANE


def math_ceil_div(a, b):
    return -(-a // b)
