"""The decode step under HIP graph capture: the library allocates nothing,
records no memset and keeps no per-call state, so an append + decode step
captured once replays correctly. Each replay follows eager work that changes
the inputs, and must equal an eager call on the same inputs bit for bit (the
kernels are deterministic for a fixed launch configuration)."""

import pytest
import torch

import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _step(pa, case, out, key, value, pos, scales, compute="auto"):
    cfg = case.cfg
    kv = "auto" if cfg.kv_dtype == "auto" else "fp8"
    ks, vs = scales
    pa.kv_cache_append(case.key_cache, case.value_cache, key, value, case.block_tables, pos,
                       kv_cache_dtype=kv, k_scale=ks, v_scale=vs)
    pa.paged_attention_decode(out, case.query, case.key_cache, case.value_cache, cfg.num_kv_heads, case.scale,
                              case.block_tables, case.seq_lens, cfg.block_size, case.max_seq_len,
                              alibi_slopes=case.alibi_slopes, kv_cache_dtype=cfg.kv_dtype, k_scale=ks,
                              v_scale=vs, compute=compute)


@pytest.mark.parametrize("name,compute", [("gqa", "auto"), ("fp8", "auto"), ("fp8", "fp8")])
def test_captured_step_replays_like_eager(name, compute):
    import decode_attention_paged_07_amd as pa
    base = {"gqa": workloads.GQA, "fp8": workloads.FP8}[name]
    cfg = base.with_(num_seqs=8, pool_blocks=1024, seq_lens=("uniform", 1, 900))
    case = workloads.make_case(cfg, device=DEV, max_seq_len=1024)
    lens = case.meta.seq_lens
    # one free slot after every sequence: write the new token into a fresh block
    # when the last one is full (as the block allocator would)
    table = case.block_tables.cpu().numpy()
    used = set(case.meta.used_blocks.tolist())
    free = (b for b in range(cfg.pool_blocks) if b not in used)
    for s, n in enumerate(lens.tolist()):
        if n % cfg.block_size == 0:
            table[s, n // cfg.block_size] = next(free)
    case.block_tables = torch.from_numpy(table).to(DEV)
    pos = case.seq_lens.clone()
    case.seq_lens += 1                                     # attend over the appended token too
    case.meta.seq_lens = case.meta.seq_lens + 1
    scales = (torch.tensor([case.k_scale], dtype=torch.float32, device=DEV),
              torch.tensor([case.v_scale], dtype=torch.float32, device=DEV))
    g = torch.Generator(device=DEV)
    g.manual_seed(17)
    shape = (cfg.num_seqs, cfg.num_kv_heads, cfg.head_size)
    key = torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)
    value = torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)
    out = torch.empty_like(case.query)
    print(f"[case] graph {name} compute={compute}", flush=True)
    _step(pa, case, out, key, value, pos, scales, compute)          # warm-up: allocates the workspace
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(pa, case, out, key, value, pos, scales, compute)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: new query, new token, and a write to out
        case.query.copy_(torch.randn(case.query.shape, generator=g, device=DEV).to(case.query.dtype))
        key.copy_(torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16))
        value.copy_(torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = torch.empty_like(out)
        _step(pa, case, eager, key, value, pos, scales, compute)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                           eager.view(torch.int16) if eager.dtype == torch.bfloat16 else eager), f"replay {rep}"
    # and the last replay is the attention the oracle defines
    if compute == "auto":
        ref = _run.run_oracle(case)
        _run.compare(got, ref, cfg.q_dtype, what=f"graph {name}")
