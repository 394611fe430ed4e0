"""GPU parity of the latent-cache (MLA) decode against the fp64 MLA oracle.

The HIP path runs through the C ABI (pa_mla_decode via the binding). Inputs
are bf16 with fp32 accumulation and bf16 output: element-wise
|gpu - oracle| <= 1e-2 + 1e-2 * |oracle|.
"""

import numpy as np
import pytest
import torch

import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def run_mla(case, out=None):
    import decode_attention_paged_07_amd as pa
    if out is None:
        out = torch.empty(case.cfg.num_seqs, case.cfg.num_heads, 512, dtype=torch.bfloat16, device=DEV)
    pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens,
                  case.max_seq_len)
    return out


def oracle_mla(case, seqs=None):
    import oracle
    h = workloads.mla_host_arrays(case, seqs)
    return oracle.mla_decode(h["query"], h["latent_cache"], h["block_tables"], h["seq_lens"], h["scale"], 512,
                             q_kind="bf16", kv_kind="bf16")


def check(case, seqs=None, what=""):
    print(f"[case] mla {what} S={case.cfg.num_seqs} H={case.cfg.num_heads} "
          f"lens={case.meta.seq_lens[:8].tolist()}", flush=True)
    out = run_mla(case)
    torch.cuda.synchronize()
    ref = oracle_mla(case, seqs)
    return out, _run.compare(out, ref, "bf16", seqs=seqs, what=what)


def small(lens, heads=16, seed=11, poison=True, pool=None):
    lens = list(lens)
    need = sum(-(-n // 16) for n in lens)
    cfg = workloads.MLA.with_(num_seqs=len(lens), num_heads=heads, pool_blocks=pool or need + 8)
    return workloads.make_mla_case(cfg, seed=seed, device=DEV, seq_lens=lens, poison=poison)


@pytest.mark.parametrize("lens", [[1], [16], [17, 40, 3], [255, 256, 257], [1000, 31, 512]])
def test_ragged_lengths_poisoned_tails(lens):
    check(small(lens), what=f"lens {lens}")


@pytest.mark.parametrize("heads", [1, 8, 15, 17, 40, 64, 100, 128])
def test_head_counts(heads):
    check(small([70, 300, 5, 129], heads=heads, seed=heads), what=f"H={heads}")


def test_zero_length_sequences_give_zero_rows():
    case = small([0, 5, 0, 33], poison=True)
    out, _ = check(case, what="zero lengths")
    assert not out[0].any() and not out[2].any()


def test_long_sequences_cut_into_many_segments():
    # 8192 + 3000 tokens = 700 blocks over ~1000 shares: every share holds a
    # block or none, so both sequences are merged from hundreds of segments.
    check(small([8192, 3000]), what="segments")


def test_long_sequences_many_heads():
    check(small([6000, 2500, 17], heads=128, seed=5), what="segments H=128")


def test_many_short_sequences():
    rng = np.random.default_rng(8)
    lens = rng.integers(1, 65, 300).tolist()
    check(small(lens, seed=8, poison=False), what="300 short")


def test_deterministic_run_to_run():
    case = small([4000, 123, 77], seed=3)
    a = run_mla(case)
    b = run_mla(case)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_oversized_max_seq_len_and_table():
    # The table is wider than the longest sequence and max_seq_len exceeds it.
    lens = [40, 100]
    cfg = workloads.MLA.with_(num_seqs=2, pool_blocks=20)
    case = workloads.make_mla_case(cfg, seed=9, device=DEV, seq_lens=lens, max_seq_len=400, poison=True)
    check(case, what="wide table")


@pytest.mark.parametrize("name", ["mla", "mla128"])
def test_full_size_workload_every_sequence(name):
    """Both full-size latent-cache workloads (256 sequences of U[1, 8192]
    tokens, 16 and 128 query heads) in the launch configuration the benchmark
    times, every sequence against the oracle."""
    cfg = workloads.MLA_CONFIGS[name]
    case = workloads.make_mla_case(cfg, device=DEV)
    out, (max_abs, max_rel) = check(case, what=f"{name} full size, all {cfg.num_seqs} sequences")
    print(f"[{name}] all sequences max_abs={max_abs:.3e} max_rel={max_rel:.3e}", flush=True)
    assert torch.isfinite(out.float()).all()
    del case
    torch.cuda.empty_cache()


def test_captured_call_replays_like_eager():
    """The latent-cache call allocates nothing and keeps no per-call state:
    captured once in a HIP graph, each replay (after eager work that changes
    the query and the cache and poisons the output) equals an eager call bit
    for bit, and the last one matches the oracle."""
    cfg = workloads.MLA.with_(num_seqs=6, pool_blocks=600)
    case = workloads.make_mla_case(cfg, seed=21, device=DEV, seq_lens=[1, 300, 1200, 17, 2500, 640])
    out = run_mla(case)                                   # warm-up: allocates the workspace
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_mla(case, out)
    torch.cuda.synchronize()
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    for rep in range(3):
        case.query.copy_(torch.randn(case.query.shape, generator=g, device=DEV).to(torch.bfloat16))
        case.latent_cache[: 300].copy_(torch.randn((300,) + tuple(case.latent_cache.shape[1:]), generator=g,
                                                   device=DEV).to(torch.bfloat16))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = run_mla(case)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
    _run.compare(got, oracle_mla(case), "bf16", what="graph mla")


def test_replay_after_a_larger_eager_call():
    """A call captured in a graph keeps a workspace of its own: a larger eager
    call made after the capture (which outgrows the binding's cached workspace
    and replaces it) does not disturb the replays, which still match the
    oracle."""
    cfg = workloads.MLA.with_(num_seqs=4, pool_blocks=400)
    case = workloads.make_mla_case(cfg, seed=31, device=DEV, seq_lens=[1500, 20, 900, 700])
    out = run_mla(case)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_mla(case, out)
    torch.cuda.synchronize()
    big_cfg = workloads.MLA.with_(num_seqs=48, num_heads=128, pool_blocks=3200)
    big = workloads.make_mla_case(big_cfg, seed=32, device=DEV,
                                  seq_lens=np.random.default_rng(32).integers(1, 1000, 48).tolist())
    print("[case] graph replay after a larger eager call", flush=True)
    for rep in range(2):
        big_out = run_mla(big)
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        _run.compare(out, oracle_mla(case), "bf16", what=f"replay {rep} after a larger eager call")
    _run.compare(big_out, oracle_mla(big, [0, 47]), "bf16", seqs=[0, 47], what="the larger eager call")


def test_shared_physical_blocks():
    # Later sequences map their first 20 blocks to sequence 0's (read-only
    # sharing of a prompt's blocks); each result is still per sequence.
    cfg = workloads.MLA.with_(num_seqs=4, pool_blocks=200)
    # No NaN poison here: a shorter sequence's partial last block can be a
    # block that a longer one uses in full.
    case = workloads.make_mla_case(cfg, seed=23, device=DEV, seq_lens=[700, 500, 900, 100],
                                   share_prefix_blocks=20)
    tbl = case.block_tables.cpu().numpy()
    assert (tbl[1, :20] == tbl[0, :20]).all() and (tbl[2, :20] == tbl[0, :20]).all()
    check(case, what="shared blocks")


@pytest.mark.parametrize("scale", [0.0, 1.0])
def test_scale_edge_values(scale):
    # scale 0: every token weighs the same (the mean of the c_kv rows); scale 1
    # (about 14x the workload's): a sharply peaked softmax.
    case = small([37, 400, 1], seed=29)
    case.scale = scale
    check(case, what=f"scale {scale}")


@pytest.mark.parametrize("seed", range(12))
def test_random_configurations(seed):
    # Seeded random head counts (1..128: one to eight head groups, so one to
    # four waves per workgroup and one or two workgroups per share), batch
    # sizes and lengths (zero-length sequences included), NaN-poisoned tails.
    rng = np.random.default_rng(1000 + seed)
    heads = int(rng.integers(1, 129))
    n = int(rng.integers(1, 41))
    lens = rng.integers(0, 3001, n)
    lens[rng.random(n) < 0.1] = 0
    lens[0] = max(int(lens[0]), 1)
    case = small(lens.tolist(), heads=heads, seed=seed)
    check(case, what=f"random seed {seed}: H={heads} S={n}")
