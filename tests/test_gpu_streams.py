"""Decode calls on three HIP streams at once (default priority): a bf16 GQA
batch, an fp8 batch and a latent-cache batch, launched interleaved five times
each, end bitwise equal to the same calls made one at a time on the default
stream. The binding keeps one workspace per (device, stream), and the
kernels are deterministic."""

import pytest
import torch

import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def test_three_streams_match_serial_calls():
    import decode_attention_paged_07_amd as pa
    gqa = workloads.make_case(workloads.GQA.with_(num_seqs=12, pool_blocks=2000,
                                                  seq_lens=("uniform", 1, 2000)), device=DEV)
    fp8 = workloads.make_case(workloads.FP8.with_(num_seqs=10, pool_blocks=2000,
                                                  seq_lens=("uniform", 1, 2500)), device=DEV)
    mcfg = workloads.MLA.with_(num_seqs=6, num_heads=128, pool_blocks=800)
    mla = workloads.make_mla_case(mcfg, seed=3, device=DEV, seq_lens=[700, 1, 3000, 64, 900, 2047])

    def run_mla(out):
        pa.mla_decode(out, mla.query, mla.latent_cache, mla.scale, mla.block_tables, mla.seq_lens,
                      mla.max_seq_len)
        return out

    print("[case] three streams", flush=True)
    ref_g = _run.run_hip(gqa)
    ref_f = _run.run_hip(fp8)
    ref_m = run_mla(torch.empty(6, 128, 512, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()

    outs = [torch.full_like(ref_g, float("nan")), torch.full_like(ref_f, float("nan")),
            torch.full_like(ref_m, float("nan"))]
    streams = [torch.cuda.Stream(device=DEV) for _ in range(3)]
    torch.cuda.synchronize()
    for _ in range(5):
        with torch.cuda.stream(streams[0]):
            _run.run_hip(gqa, out=outs[0])
        with torch.cuda.stream(streams[1]):
            _run.run_hip(fp8, out=outs[1])
        with torch.cuda.stream(streams[2]):
            run_mla(outs[2])
    torch.cuda.synchronize()
    for got, ref, name in zip(outs, (ref_g, ref_f, ref_m), ("gqa", "fp8", "mla")):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), name
