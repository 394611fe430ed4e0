"""Seeded random latent-cache (MLA) decodes against the fp64 oracle.

Each case draws the cache type (bf16 or fp8 codes), the block size (16 or
32), the head count (1..128: both kernels, every head-group count and partial
groups), 1..39 sequences of 0..5000 tokens (about a tenth empty), and a
max_seq_len above the longest; unused slots and table entries are NaN-poisoned.
Element-wise |gpu - oracle| <= 1e-2 + 1e-2 |oracle|."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


@pytest.mark.parametrize("seed", range(24))
def test_random_latent_decode(seed):
    import decode_attention_paged_07_amd as pa
    rng = np.random.default_rng(60000 + seed)
    kind = "fp8" if rng.random() < 0.5 else "bf16"
    bs = 32 if rng.random() < 0.5 else 16
    heads = int(rng.integers(1, 129))
    n = int(rng.integers(1, 40))
    lens = rng.integers(0, 5001, n)
    lens[rng.random(n) < 0.1] = 0
    need = sum(-(-int(L) // bs) for L in lens)
    base = workloads.MLA_FP8 if kind == "fp8" else workloads.MLA
    cfg = base.with_(num_seqs=n, num_heads=heads, block_size=bs, pool_blocks=need + 8)
    case = workloads.make_mla_case(cfg, seed=seed, device=DEV, seq_lens=lens.tolist(), poison=True,
                                   max_seq_len=int(lens.max()) + int(rng.integers(0, 64)))
    print(f"[case] random latent decode {seed}: {kind} bs={bs} H={heads} S={n}", flush=True)
    out = torch.full((n, heads, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens,
                  case.max_seq_len, kv_scale=case.kv_scale)
    torch.cuda.synchronize()
    h = workloads.mla_host_arrays(case)
    ref = oracle.mla_decode(h["query"], h["latent_cache"], h["block_tables"], h["seq_lens"], h["scale"], 512,
                            q_kind="bf16", kv_kind=h["kv_kind"], kv_scale=h["kv_scale"])
    _run.compare(out, ref, "bf16", what=f"random latent decode {seed}")
