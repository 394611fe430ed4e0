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


def test_growing_batch_replaces_the_workspace_a_few_times():
    """Forty calls on a batch that grows by one sequence per call, launched
    without a synchronisation between them, each needing more workspace than
    the last: the stream's cached buffer is replaced only a few times (it grows
    by half at least), outgrown buffers are dropped once the work queued before
    them is done, and every call's output agrees with the oracle."""
    import decode_attention_paged_07_amd as pa
    n = 40
    case = workloads.make_case(workloads.GQA.with_(num_seqs=n, pool_blocks=3000,
                                                   seq_lens=("uniform", 1, 1200)), device=DEV)
    cfg = case.cfg
    ref = _run.run_oracle(case)
    outs = [torch.full((k,) + tuple(case.query.shape[1:]), float("nan"), dtype=case.query.dtype, device=DEV)
            for k in range(1, n + 1)]
    stream = torch.cuda.Stream(device=DEV)
    key = (DEV, stream.cuda_stream)
    torch.cuda.synchronize()
    pa._workspaces.pop(key, None)               # torch reuses pooled streams: start this one's entry empty
    sizes = []
    print("[case] growing batch on one stream", flush=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for k in range(1, n + 1):
            pa.paged_attention_decode(outs[k - 1], case.query[:k], case.key_cache, case.value_cache,
                                      cfg.num_kv_heads, case.scale, case.block_tables[:k], case.seq_lens[:k],
                                      cfg.block_size, case.max_seq_len)
            ws = pa._workspaces[key]
            if not sizes or ws.numel() != sizes[-1]:
                sizes.append(ws.numel())
    torch.cuda.synchronize()
    assert len(sizes) >= 2, "the workload should outgrow its first workspace"
    assert all(b >= a + a // 2 for a, b in zip(sizes, sizes[1:])), sizes
    assert len(sizes) <= 8, sizes
    for k in range(1, n + 1):
        _run.compare(outs[k - 1], ref[:k], cfg.q_dtype, what=f"first {k} sequences")
    with torch.cuda.stream(stream):             # every retired buffer's work is done: the next call drops it
        pa.paged_attention_decode(outs[-1], case.query, case.key_cache, case.value_cache, cfg.num_kv_heads,
                                  case.scale, case.block_tables, case.seq_lens, cfg.block_size, case.max_seq_len)
    torch.cuda.synchronize()
    assert pa._retired == []
    del pa._workspaces[key]
