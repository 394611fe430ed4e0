"""Seeded random configurations against the oracle: cache type (f32, bf16,
fp8, fp8 arithmetic), head size, block size, group size, lengths (zeros and
block edges included), ALiBi, scheduler and split size, max_seq_len slack.
Each case is small; together they cover combinations the targeted tests do
not list one by one."""

import numpy as np
import pytest
import torch

import workloads
from tests import _fp8tol, _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    kind = ["f32", "bf16", "fp8", "fp8c"][seed % 4]
    d = int(rng.choice([32, 64, 128]))
    bs = int(rng.choice([16, 32]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    s = int(rng.integers(1, 13))
    edges = [0, 1, bs - 1, bs, bs + 1, 2 * bs, 255, 256, 257]
    lens = [int(rng.choice(edges)) if rng.random() < 0.4 else int(rng.integers(0, 1500)) for _ in range(s)]
    if max(lens) == 0:
        lens[0] = 1
    split = int(rng.choice([0, 0, 256, 512, 1024]))
    slack = int(rng.choice([0, 0, 37, 300]))
    base = workloads.FP8 if kind.startswith("fp8") else workloads.GQA
    cfg = base.with_(name=f"rand{seed}", num_seqs=s, num_heads=hkv * group, num_kv_heads=hkv, head_size=d,
                     block_size=bs, seq_lens=("fixed", tuple(lens)), alibi=bool(rng.random() < 0.3),
                     q_dtype="f32" if kind == "f32" else "bf16",
                     pool_blocks=sum(-(-n // bs) for n in lens) + 8 + 2 * (max(lens) + slack) // bs,
                     seed=seed, compute="fp8" if kind == "fp8c" else "auto")
    return cfg, split, max(lens) + slack


@pytest.mark.parametrize("seed", range(40))
def test_random_config(seed):
    cfg, split, max_len = draw(seed)
    print(f"[case] seed {seed}: {cfg.q_dtype}/{cfg.kv_dtype}/{cfg.compute} D={cfg.head_size} bs={cfg.block_size} "
          f"H={cfg.num_heads} Hkv={cfg.num_kv_heads} lens={cfg.seq_lens[1]} alibi={cfg.alibi} split={split} "
          f"max_seq_len={max_len}", flush=True)
    case = workloads.make_case(cfg, device=DEV, max_seq_len=max_len, poison=True)
    out = _run.run_hip(case, split_tokens=split, compute=cfg.compute)
    torch.cuda.synchronize()
    extra = None
    if cfg.compute == "fp8":
        ref = _run.run_oracle_fp8(case)
        extra = _fp8tol.row_bounds(workloads.host_arrays(case))
    else:
        ref = _run.run_oracle(case)
    _run.compare(out, ref, cfg.q_dtype, what=f"random seed {seed}", extra=extra)
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("kind,bs,alibi", [("bf16", 16, True), ("bf16", 32, False), ("fp8", 16, False),
                                           ("fp8", 32, True), ("f32", 16, True), ("fp8c", 16, True)])
def test_many_short_sequences(kind, bs, alibi):
    # 600 short sequences over about 1024 stream-K waves: each wave's share
    # runs through several (sequence, kv head) pairs, so the pipeline's
    # prefetched next pair (q rows, ALiBi slope, first table entries and first
    # block) is exercised for every cache type.
    rng = np.random.default_rng(7 + bs + 100 * alibi)
    lens = rng.integers(1, 71, 600)
    lens[rng.random(600) < 0.15] = 0
    base = workloads.FP8 if kind.startswith("fp8") else workloads.GQA
    cfg = base.with_(name=f"short_{kind}", num_seqs=600, num_heads=8, num_kv_heads=2, head_size=128, block_size=bs,
                     seq_lens=("fixed", tuple(int(x) for x in lens)), alibi=alibi,
                     q_dtype="f32" if kind == "f32" else "bf16", pool_blocks=4096 * 16 // bs, seed=bs,
                     compute="fp8" if kind == "fp8c" else "auto")
    print(f"[case] {kind} bs={bs} alibi={alibi}: 600 sequences, {int((lens == 0).sum())} empty", flush=True)
    case = workloads.make_case(cfg, device=DEV, poison=True)
    out = _run.run_hip(case, compute=cfg.compute)
    torch.cuda.synchronize()
    extra = None
    if cfg.compute == "fp8":
        ref = _run.run_oracle_fp8(case)
        extra = _fp8tol.row_bounds(workloads.host_arrays(case))
    else:
        ref = _run.run_oracle(case)
    _run.compare(out, ref, cfg.q_dtype, what=f"600 short sequences, {kind}", extra=extra)
