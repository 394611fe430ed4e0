"""GPU parity of the latent-cache calls with 32-token cache blocks
([num_blocks, 576/x, 32, x]): decode (bf16 and fp8 cache, both kernels)
against the fp64 MLA oracle at the bf16 tolerance, and the appends against
the oracle's append_latent bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
WIDTH = 576
BASE = {"bf16": workloads.MLA, "fp8": workloads.MLA_FP8}


def host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def small(lens, heads=16, kind="bf16", seed=11, poison=True, extra=8):
    lens = list(lens)
    need = sum(-(-n // 32) for n in lens)
    cfg = BASE[kind].with_(num_seqs=len(lens), num_heads=heads, block_size=32, pool_blocks=need + extra)
    return workloads.make_mla_case(cfg, seed=seed, device=DEV, seq_lens=lens, poison=poison)


def check(case, seqs=None, what=""):
    import decode_attention_paged_07_amd as pa
    cfg = case.cfg
    print(f"[case] mla bs32 {what} kv={cfg.kv_dtype} S={cfg.num_seqs} H={cfg.num_heads} "
          f"lens={case.meta.seq_lens[:8].tolist()}", flush=True)
    assert case.latent_cache.shape[2] == 32
    out = torch.empty(cfg.num_seqs, cfg.num_heads, 512, dtype=torch.bfloat16, device=DEV)
    pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens,
                  case.max_seq_len, kv_scale=case.kv_scale)
    torch.cuda.synchronize()
    h = workloads.mla_host_arrays(case, seqs)
    ref = oracle.mla_decode(h["query"], h["latent_cache"], h["block_tables"], h["seq_lens"], h["scale"], 512,
                            q_kind="bf16", kv_kind=h["kv_kind"], kv_scale=h["kv_scale"])
    return out, _run.compare(out, ref, "bf16", seqs=seqs, what=what)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("lens", [[1], [16], [31, 32, 33], [17, 255, 257, 1000]])
def test_ragged_lengths_poisoned_tails(kind, lens):
    check(small(lens, kind=kind), what=f"lens {lens}")


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("heads", [1, 16, 40, 64, 65, 100, 128])
def test_head_counts(kind, heads):
    check(small([70, 300, 5, 129], heads=heads, kind=kind, seed=heads), what=f"H={heads}")


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("heads", [16, 128])
def test_long_sequences_cut_into_many_segments(kind, heads):
    check(small([8192, 3000, 17], heads=heads, kind=kind, seed=5), what=f"segments H={heads}")


def test_zero_length_sequences_give_zero_rows():
    out, _ = check(small([0, 5, 0, 33]), what="zero lengths")
    assert not out[0].any() and not out[2].any()


@pytest.mark.parametrize("seed", range(4))
def test_random_configurations(seed):
    rng = np.random.default_rng(3000 + seed)
    heads = int(rng.integers(1, 129))
    n = int(rng.integers(1, 30))
    lens = rng.integers(0, 3001, n)
    lens[rng.random(n) < 0.1] = 0
    kind = "fp8" if seed % 2 else "bf16"
    check(small(lens.tolist(), heads=heads, kind=kind, seed=seed), what=f"random {seed}: H={heads}")


@pytest.mark.parametrize("kind,heads", [("bf16", 16), ("bf16", 128), ("fp8", 16), ("fp8", 128)])
def test_full_size_workload(kind, heads):
    """The MLA workload's batch (256 sequences of U[1, 8192] tokens) in
    32-token blocks: every sequence at 16 heads, every 8th at 128."""
    cfg = BASE[kind].with_(num_heads=heads, block_size=32, pool_blocks=65536)
    case = workloads.make_mla_case(cfg, device=DEV)
    seqs = None if heads <= 16 else list(range(0, cfg.num_seqs, 8))
    out, (max_abs, max_rel) = check(case, seqs=seqs, what=f"full size {kind} H={heads}")
    print(f"[bs32 {kind} H={heads}] max_abs={max_abs:.3e} max_rel={max_rel:.3e}", flush=True)
    del case
    torch.cuda.empty_cache()


# --- appends ------------------------------------------------------------------

def make_append(S, T, pool, seed, fp8, positions=None):
    import decode_attention_paged_07_amd as pa
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    rng = np.random.default_rng(seed)
    shape = pa.mla_cache_shape(pool, 32, fp8)
    if fp8:
        cache = torch.randint(0, 256, shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    else:
        cache = torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)
    max_blocks = pool // S
    table = rng.permutation(pool)[:S * max_blocks].reshape(S, max_blocks).astype(np.int32)
    if positions is None:
        positions = rng.integers(-1, max_blocks * 32 - T + 1, S).astype(np.int32)
    rows = (torch.randn((S, T, WIDTH), generator=g, device=DEV) * 3).to(torch.bfloat16)
    return dict(cache=cache, table=torch.from_numpy(table).to(DEV),
                positions=torch.from_numpy(np.asarray(positions, np.int32)).to(DEV), rows=rows)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("T", [1, 3, 32, 35])
def test_append_matches_oracle(fp8, T):
    import decode_attention_paged_07_amd as pa
    c = make_append(S=6, T=T, pool=30, seed=T * 5 + fp8, fp8=fp8)
    print(f"[case] mla bs32 append T={T} fp8={fp8}", flush=True)
    before = host(c["cache"])
    scale = 0.05 if fp8 else 1.0
    pa.mla_cache_append(c["cache"], c["rows"], c["table"], c["positions"], kv_scale=scale)
    torch.cuda.synchronize()
    ref = oracle.append_latent(before, host(c["rows"]), host(c["table"]), host(c["positions"]),
                               kv_kind="e4m3fn" if fp8 else None, kv_scale=float(np.float32(scale)))
    bad = np.argwhere(host(c["cache"]) != ref)
    assert bad.size == 0, f"cache differs in {len(bad)} elements, first {bad[:4].tolist()}"


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_append_then_decode(kind):
    import decode_attention_paged_07_amd as pa
    lens = [1, 31, 32, 33, 300, 704]
    need = sum(-(-n // 32) for n in lens) + len(lens)
    cfg = BASE[kind].with_(num_seqs=len(lens), num_heads=16, block_size=32, pool_blocks=need + 8)
    case = workloads.make_mla_case(cfg, seed=44, device=DEV, seq_lens=lens, max_seq_len=736)
    used = set(case.meta.used_blocks.tolist())
    free = (b for b in range(cfg.pool_blocks) if b not in used)
    table = case.block_tables.cpu().numpy()
    for s, n in enumerate(lens):
        if n % 32 == 0:
            table[s, n // 32] = next(free)
    case.block_tables = torch.from_numpy(table).to(DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    rows = torch.randn((len(lens), WIDTH), generator=g, device=DEV).to(torch.bfloat16)
    pos = case.seq_lens.clone()
    before = host(case.latent_cache)
    print(f"[case] mla bs32 append then decode {kind}", flush=True)
    pa.mla_cache_append(case.latent_cache, rows, case.block_tables, pos, kv_scale=case.kv_scale)
    case.seq_lens += 1
    out = torch.empty(len(lens), 16, 512, dtype=torch.bfloat16, device=DEV)
    pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens, 736,
                  kv_scale=case.kv_scale)
    torch.cuda.synchronize()
    fp8 = kind == "fp8"
    ks = float(np.float32(case.kv_scale))
    grown = oracle.append_latent(before, host(rows)[:, None], host(case.block_tables), host(pos),
                                 kv_kind="e4m3fn" if fp8 else None, kv_scale=ks)
    ref = oracle.mla_decode(host(case.query), grown, host(case.block_tables), host(case.seq_lens), case.scale,
                            512, q_kind="bf16", kv_kind="e4m3fn" if fp8 else "bf16", kv_scale=ks if fp8 else 1.0)
    _run.compare(out, ref, "bf16", what=f"bs32 append then decode {kind}")
