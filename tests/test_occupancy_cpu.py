"""Residency of the persistent decode grid, checked on the built library.

The stream-K launch sizes its grid as waves per compute unit times the number
of compute units, one wave per SIMD per four-wave workgroup, and every wave
takes an equal share of the batch. All of its workgroups must be resident at
once: a kernel that needs more registers than that many waves per SIMD allow
runs its last workgroups only after others finish, in a second round. The
hardware allocation comes from each kernel's descriptor in the gfx950 code
object (512 registers per lane per SIMD on gfx950), the waves per compute
unit from the knobs the launch plan reads.
"""

import math
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KNOBS_HEADER = os.path.join(ROOT, "decode_attention_paged_07_amd", "csrc", "pa_kernels.h")
REGISTERS_PER_SIMD_LANE = 512
# (policy, block size) -> the knob the launch plan uses for it
KNOB = {("PolicyBf16", 16): "BF16", ("PolicyBf16", 32): "BS32_BF16",
        ("PolicyFp8", 16): "FP8", ("PolicyFp8", 32): "BS32_FP8",
        ("PolicyFp8Mx", 16): "FP8MX", ("PolicyFp8Mx", 32): "BS32_FP8MX",
        ("PolicyF32", 16): "F32", ("PolicyF32", 32): "BS32_F32"}


@pytest.fixture(scope="module")
def kernels():
    import __graft_entry__
    b = __graft_entry__._build_module()
    if not os.path.exists(b.LIB_PATH):
        b.build()
    return bench.code_object_kernels(b.LIB_PATH)


def knobs():
    with open(KNOBS_HEADER) as f:
        raw = dict(re.findall(r"#define (PA_SK_WAVES_PER_CU_\w+) (\w+)", f.read()))

    def value(name):
        v = raw[name]
        return value(v) if v in raw else float(v)
    return {k[len("PA_SK_WAVES_PER_CU_"):]: value(k) for k in raw}


def test_every_streamk_kernel_fits_its_persistent_grid(kernels):
    kn = knobs()
    checked = 0
    for name, r in kernels.items():
        m = re.search(r"pa_streamk_kernel<pa::(Policy\w+)<(\d+), (\d+)>", name)
        if not m:
            continue
        per_cu = kn[KNOB[(m.group(1), int(m.group(3)))]]
        per_simd = math.ceil(per_cu / 4)
        assert r["alloc"] is not None, name
        assert r["alloc"] * per_simd <= REGISTERS_PER_SIMD_LANE, \
            f"{name}: {r['alloc']} registers per lane x {per_simd} waves per SIMD"
        assert r["scratch"] == 0, f"{name} spills {r['scratch']} bytes per lane"
        checked += 1
    # 4 element-type policies x 3 head sizes x 2 block sizes x ALiBi on/off
    assert checked == 48


def test_descriptor_allocation_covers_the_registers_used(kernels):
    for name, r in kernels.items():
        assert r["alloc"] is not None and r["alloc"] % 8 == 0, name
        assert r["alloc"] >= r["vgpr"], f"{name}: allocates {r['alloc']}, uses {r['vgpr']}"


def test_no_kernel_spills_to_scratch(kernels):
    spilling = {name: r["scratch"] for name, r in kernels.items() if r["scratch"]}
    assert not spilling, spilling
