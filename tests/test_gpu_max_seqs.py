"""The largest batch the C ABI accepts: PA_MAX_SEQS (65535) sequences.

At that size the stream-K start-up scan runs through all 64 of its batches
(1024 sequences each, the last one partial), the merge grids have num_seqs
rows, and the 256-token split grid has as many. Lengths are short (a few
blocks), about a fifth of the sequences are empty. Every empty sequence's row
must be zero, every output finite, and a sample of sequences (every batch
boundary and 300 more) is compared with the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
MAX_SEQS = 65535


def lengths(seed, hi):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, hi, MAX_SEQS)
    lens[rng.random(MAX_SEQS) < 0.2] = 0
    return lens


def sample(lens, seed):
    rng = np.random.default_rng(seed + 1)
    edges = [0, 1, 63, 64, 127, 128, 129, MAX_SEQS - 1]
    edges += [b * 1024 + d for b in range(1, 64) for d in (-1, 0)]
    seqs = np.unique(np.concatenate([edges, rng.choice(MAX_SEQS, 300, replace=False)]))
    return [int(s) for s in seqs if s < MAX_SEQS]


def check_rows(out, lens, ref, seqs, what):
    empty = torch.from_numpy(np.flatnonzero(lens == 0)).to(DEV)
    assert not out.index_select(0, empty).any(), f"{what}: an empty sequence's row is not zero"
    assert torch.isfinite(out.float()).all(), f"{what}: non-finite output"
    _run.compare(out, ref, "bf16", seqs=seqs, what=what)


@pytest.mark.parametrize("kind,split", [("bf16", 0), ("bf16", 256), ("fp8", 0)])
def test_max_sequences_decode(kind, split):
    lens = lengths(41, 50)
    base = workloads.FP8 if kind == "fp8" else workloads.GQA
    cfg = base.with_(name=f"max_seqs_{kind}", num_seqs=MAX_SEQS, num_heads=8, num_kv_heads=2,
                     pool_blocks=4 * MAX_SEQS, seq_lens=("fixed", tuple(int(x) for x in lens)))
    case = workloads.make_case(cfg, device=DEV)
    print(f"[case] {MAX_SEQS} sequences, {kind}, split={split}, {int((lens == 0).sum())} empty", flush=True)
    out = torch.full_like(case.query, float("nan"))
    _run.run_hip(case, split_tokens=split, out=out)
    torch.cuda.synchronize()
    seqs = sample(lens, 41)
    check_rows(out, lens, _run.run_oracle(case, seqs), seqs, f"{MAX_SEQS} sequences {kind} split={split}")


@pytest.mark.parametrize("kind,heads", [("bf16", 16), ("bf16", 72), ("fp8", 72)])
def test_max_sequences_latent_decode(kind, heads):
    import decode_attention_paged_07_amd as pa
    lens = lengths(42, 40)
    cfg = workloads.MLA.with_(num_seqs=MAX_SEQS, num_heads=heads, pool_blocks=3 * MAX_SEQS,
                              kv_dtype="fp8_e4m3" if kind == "fp8" else "auto")
    case = workloads.make_mla_case(cfg, seed=42, device=DEV, seq_lens=[int(x) for x in lens])
    print(f"[case] {MAX_SEQS} sequences, latent {kind}, {heads} heads", flush=True)
    out = torch.full((MAX_SEQS, heads, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens,
                  case.max_seq_len, kv_scale=case.kv_scale)
    torch.cuda.synchronize()
    seqs = sample(lens, 42)
    h = workloads.mla_host_arrays(case, seqs)
    ref = oracle.mla_decode(h["query"], h["latent_cache"], h["block_tables"], h["seq_lens"], h["scale"], 512,
                            q_kind="bf16", kv_kind=h["kv_kind"], kv_scale=h["kv_scale"])
    check_rows(out, lens, ref, seqs, f"{MAX_SEQS} sequences latent {kind} H={heads}")
