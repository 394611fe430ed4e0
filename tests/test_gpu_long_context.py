"""One very long context beside short ones: a 300,001-token sequence (18,751
blocks, the last holding one token) with a one-token and an empty sequence.

The long sequence alone holds nearly all the work, so every stream-K share is a
piece of it: each of its (sequence, kv head) pairs is merged from about a
hundred segments, and the 256-token split grid has 1,172 partitions. Compared
with the fp64 oracle element by element."""

import pytest
import torch

import oracle
import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
LENS = (300_001, 1, 0, 4099)


@pytest.mark.parametrize("kind,split", [("bf16", 0), ("bf16", 256), ("alibi", 0), ("fp8", 0)])
def test_long_context_decode(kind, split):
    base = {"bf16": workloads.GQA, "alibi": workloads.LONG, "fp8": workloads.FP8}[kind]
    cfg = base.with_(name=f"ctx_{kind}", num_seqs=len(LENS), pool_blocks=19_500, seq_lens=("fixed", LENS))
    case = workloads.make_case(cfg, device=DEV, poison=True)
    print(f"[case] long context {kind}, split={split}, lens {LENS}", flush=True)
    out = _run.run_hip(case, split_tokens=split)
    torch.cuda.synchronize()
    assert not out[2].any()
    _run.compare(out, _run.run_oracle(case), "bf16", what=f"long context {kind} split={split}")


@pytest.mark.parametrize("kind,heads", [("bf16", 16), ("bf16", 128), ("fp8", 128)])
def test_long_context_latent_decode(kind, heads):
    import decode_attention_paged_07_amd as pa
    lens = [300_001, 3, 0]
    cfg = workloads.MLA.with_(num_seqs=3, num_heads=heads, pool_blocks=19_000,
                              kv_dtype="fp8_e4m3" if kind == "fp8" else "auto")
    case = workloads.make_mla_case(cfg, seed=43, device=DEV, seq_lens=lens, poison=True)
    print(f"[case] long context latent {kind}, {heads} heads, lens {lens}", flush=True)
    out = torch.full((3, heads, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens,
                  case.max_seq_len, kv_scale=case.kv_scale)
    torch.cuda.synchronize()
    assert not out[2].any()
    h = workloads.mla_host_arrays(case)
    ref = oracle.mla_decode(h["query"], h["latent_cache"], h["block_tables"], h["seq_lens"], h["scale"], 512,
                            q_kind="bf16", kv_kind=h["kv_kind"], kv_scale=h["kv_scale"])
    _run.compare(out, ref, "bf16", what=f"long context latent {kind} H={heads}")
