"""GPU parity with 32-token cache blocks (through the C ABI) against the fp64
oracle, which reads any block size from the cache shapes: plain decode on
both schedulers, the shared-prefix decode, and the KV append. The kernels
take a 32-token block as one tile of two 16-row sub-tiles that interleave in
runs of 8 tokens, so the cases put lengths on both sides of every run and
block boundary."""

import numpy as np
import pytest
import torch

import workloads
from tests import _run
from tests import test_gpu_append as app
from tests import test_gpu_shared_prefix as shp

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def check(case, split_tokens=0, seqs=None, what=""):
    cfg = case.cfg
    print(f"[case] {what}: bs={cfg.block_size} S={cfg.num_seqs} H={cfg.num_heads} Hkv={cfg.num_kv_heads} "
          f"D={cfg.head_size} q={cfg.q_dtype} kv={cfg.kv_dtype} split={split_tokens}", flush=True)
    out = _run.run_hip(case, split_tokens=split_tokens)
    torch.cuda.synchronize()
    ref = _run.run_oracle(case, seqs)
    return out, _run.compare(out, ref, cfg.q_dtype, seqs=seqs, what=what)


SMALL = {
    "gqa": workloads.GQA.with_(num_seqs=10, pool_blocks=512, seq_lens=("uniform", 1, 1500), block_size=32),
    "fp8": workloads.FP8.with_(num_seqs=10, pool_blocks=512, seq_lens=("lognormal", 300, 1.0, 1800),
                               block_size=32),
    "mha": workloads.MHA.with_(num_seqs=6, pool_blocks=256, seq_lens=("uniform", 1, 1100), block_size=32),
    "long-alibi": workloads.LONG.with_(num_seqs=2, pool_blocks=256, seq_lens=("const", 3000), block_size=32),
    "f32-d128": workloads.TINY.with_(head_size=128, num_seqs=5, num_heads=8, num_kv_heads=2, pool_blocks=64,
                                     seq_lens=("uniform", 1, 700), block_size=32),
}


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("split", [0, 256, 512])
def test_small_workloads_block32(name, split):
    check(workloads.make_case(SMALL[name], device=DEV), split_tokens=split, what=f"{name}-bs32")


@pytest.mark.parametrize("name", ["gqa", "fp8", "f32-d128"])
@pytest.mark.parametrize("d", [64, 32])
def test_small_head_sizes_block32(name, d):
    cfg = SMALL[name].with_(head_size=d)
    check(workloads.make_case(cfg, device=DEV), what=f"{name}-d{d}-bs32")


EDGE_LENS = (1, 7, 8, 9, 15, 16, 17, 23, 24, 25, 31, 32, 33, 48, 63, 64, 65, 255, 256, 257, 511, 512, 513, 2)


@pytest.mark.parametrize("kv,q", [("auto", "bf16"), ("fp8_e4m3", "bf16"), ("auto", "f32")])
def test_edge_lengths_with_nan_poison_block32(kv, q):
    """Tail slots of the last block (including a whole unused 16-token half),
    unused blocks and unused table entries hold NaN; never read."""
    cfg = workloads.GQA.with_(num_seqs=len(EDGE_LENS), num_heads=16, num_kv_heads=4, pool_blocks=128,
                              seq_lens=("fixed", EDGE_LENS), kv_dtype=kv, q_dtype=q, block_size=32)
    for split in (0, 256):
        case = workloads.make_case(cfg, device=DEV, poison=True, max_seq_len=900)
        out, _ = check(case, split_tokens=split, what=f"edge-poison-bs32-{kv}-{q}-{split}")
        assert torch.isfinite(out.float()).all()


def test_full_size_gqa_block32_sampled():
    """The GQA workload's shapes (128 sequences, lengths U[1, 8192]) with the
    same token capacity in 32-token blocks, in the automatic launch plan."""
    cfg = workloads.GQA.with_(block_size=32, pool_blocks=workloads.GQA.pool_blocks // 2)
    case = workloads.make_case(cfg, device=DEV)
    lens = case.meta.seq_lens
    rng = np.random.default_rng(cfg.seed)
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens))} |
                  set(int(i) for i in rng.choice(len(lens), 4, replace=False)))
    out, (mabs, mrel) = check(case, seqs=seqs, what="gqa-full-bs32")
    print(f"[full] gqa bs32: sampled seqs {seqs} max_abs={mabs:.2e} max_rel={mrel:.2e}", flush=True)
    assert torch.isfinite(out.float()).all()


SHARED = {
    "gqa8-group8": shp.SMALL["gqa8-group8"].with_(block_size=32, pool_blocks=512),
    "gqa8-group11": shp.SMALL["gqa8-group11"].with_(block_size=32, pool_blocks=512),
    "fp8-group8": shp.SMALL["fp8-group8"].with_(block_size=32, pool_blocks=512),
    "alibi-g4-group6": shp.SMALL["alibi-g4-group6"].with_(block_size=32, pool_blocks=512),
    "f32-d64-group4": shp.SMALL["f32-d64-group4"].with_(block_size=32, pool_blocks=128),
    "f32-d128-group5": shp.SMALL["f32-d128-group5"].with_(block_size=32, pool_blocks=256),
    "gqa8-d32-group8": shp.SMALL["gqa8-group8"].with_(block_size=32, pool_blocks=512, head_size=32),
    "fp8-d32-group8": shp.SMALL["fp8-group8"].with_(block_size=32, pool_blocks=512, head_size=32),
}


@pytest.mark.parametrize("name", sorted(SHARED))
def test_shared_prefix_block32(name):
    case = workloads.make_case(SHARED[name], device=DEV)
    shp.check(case, f"{name}-bs32")


@pytest.mark.parametrize("in_kind,kv_kind,d", [("bf16", "bf16", 128), ("f32", "f32", 64),
                                               ("bf16", "e4m3fn", 128), ("f32", "e4m3fn", 64),
                                               ("bf16", "bf16", 32), ("bf16", "e4m3fn", 32)])
@pytest.mark.parametrize("T", [1, 5, 32, 45])
def test_append_block32(in_kind, kv_kind, d, T):
    ks, vs = (0.021, 0.037) if kv_kind == "e4m3fn" else (None, None)
    c = app.make(in_kind, kv_kind, S=6, T=T, hkv=4, d=d, pool=48, seed=T * 5 + d, k_scale=ks, v_scale=vs, bs=32)
    app.check(c, in_kind, kv_kind, f"bs32 T={T}")


def test_append_edge_positions_block32():
    pos = [0, 15, 16, 31, 32, 63, 6 * 32 - 2, -1, 6 * 32 - 1]
    c = app.make("bf16", "bf16", S=len(pos), T=2, hkv=2, d=128, pool=54, seed=4, positions=pos, bs=32)
    app.check(c, "bf16", "bf16", "bs32 edge positions")
