"""GPU parity of the latent-row append (pa_mla_cache_append, through the C ABI)
against the oracle's append_latent: whole latent caches compared bit for bit,
and the MLA decode of the grown cache against the oracle decode."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
WIDTH = 576


def host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def make(S, T, pool, seed, positions=None):
    """Random latent cache (values in every slot), a scattered table of
    pool // S blocks per sequence, T new rows per sequence."""
    import decode_attention_paged_07_amd as pa
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    rng = np.random.default_rng(seed)
    cache = torch.randn(pa.mla_cache_shape(pool), generator=g, device=DEV).to(torch.bfloat16)
    max_blocks = pool // S
    table = rng.permutation(pool)[:S * max_blocks].reshape(S, max_blocks).astype(np.int32)
    if positions is None:
        positions = rng.integers(-1, max_blocks * 16 - T + 1, S).astype(np.int32)
    rows = (torch.randn((S, T, WIDTH), generator=g, device=DEV) * 3).to(torch.bfloat16)
    return dict(cache=cache, table=torch.from_numpy(table).to(DEV),
                positions=torch.from_numpy(np.asarray(positions, np.int32)).to(DEV), rows=rows)


def check(c, what):
    import decode_attention_paged_07_amd as pa
    print(f"[case] mla append {what}: rows={tuple(c['rows'].shape)} pool={c['cache'].shape[0]}", flush=True)
    before = host(c["cache"])
    pa.mla_cache_append(c["cache"], c["rows"], c["table"], c["positions"])
    torch.cuda.synchronize()
    ref = oracle.append_latent(before, host(c["rows"]), host(c["table"]), host(c["positions"]))
    bad = np.argwhere(host(c["cache"]) != ref)
    assert bad.size == 0, f"{what}: latent cache differs in {len(bad)} elements, first {bad[:4].tolist()}"


@pytest.mark.parametrize("T", [1, 2, 3, 15, 16, 17, 19, 40])
def test_append_matches_oracle(T):
    c = make(S=6, T=T, pool=48, seed=T * 13 + 1)
    check(c, f"T={T}")


def test_two_dimensional_rows_are_one_token():
    c = make(S=5, T=1, pool=40, seed=2)
    c["rows"] = c["rows"][:, 0].contiguous()
    import decode_attention_paged_07_amd as pa
    before = host(c["cache"])
    pa.mla_cache_append(c["cache"], c["rows"], c["table"], c["positions"])
    torch.cuda.synchronize()
    ref = oracle.append_latent(before, host(c["rows"])[:, None], host(c["table"]), host(c["positions"]))
    assert np.array_equal(host(c["cache"]), ref)


def test_edge_positions():
    """First slot, last slot of a block, block boundary, last slot of the table,
    skipped sequences, positions running past the table."""
    pos = [0, 15, 16, 31, 8 * 16 - 2, -1, 8 * 16 - 1, -100]
    c = make(S=8, T=2, pool=64, seed=3, positions=pos)
    check(c, "edge positions")


def test_table_entries_outside_pool_are_skipped():
    c = make(S=4, T=3, pool=16, seed=9, positions=[0, 14, 33, 5])
    t = c["table"].cpu()
    t[0, 0] = 10 ** 6
    t[1, 1] = -3          # sequence 1 writes slots 14, 15 of its block 0 only
    t[2, 2] = 16          # one past the pool
    c["table"] = t.to(DEV)
    check(c, "bad table entries")


def grow_tables(case):
    """A fresh unused block for every sequence whose next token opens one."""
    meta = case.meta
    used = set(meta.used_blocks.tolist())
    free = (b for b in range(case.cfg.pool_blocks) if b not in used)
    table = case.block_tables.cpu().numpy()
    for s, n in enumerate(meta.seq_lens.tolist()):
        if n % 16 == 0:
            assert n // 16 < table.shape[1], "table has no room for the next block"
            table[s, n // 16] = next(free)
    case.block_tables = torch.from_numpy(table).to(DEV)
    meta.block_tables = table


@pytest.mark.parametrize("heads", [16, 128])
def test_append_then_decode_reads_the_new_rows(heads):
    """Append one row per sequence with the HIP kernel, decode the grown cache
    with the HIP kernel, compare with the oracle decode of the oracle-appended
    cache (tolerance as for the MLA decode parity)."""
    import decode_attention_paged_07_amd as pa
    lens = [1, 15, 16, 17, 300, 704]
    need = sum(-(-n // 16) for n in lens) + len(lens)
    cfg = workloads.MLA.with_(num_seqs=len(lens), num_heads=heads, pool_blocks=need + 8)
    case = workloads.make_mla_case(cfg, seed=heads, device=DEV, seq_lens=lens, max_seq_len=720)
    grow_tables(case)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    rows = torch.randn((len(lens), WIDTH), generator=g, device=DEV).to(torch.bfloat16)
    pos = case.seq_lens.clone()
    before = host(case.latent_cache)
    print(f"[case] mla append then decode H={heads}", flush=True)
    pa.mla_cache_append(case.latent_cache, rows, case.block_tables, pos)
    case.seq_lens += 1
    case.meta.seq_lens = case.meta.seq_lens + 1
    out = torch.empty(len(lens), heads, 512, dtype=torch.bfloat16, device=DEV)
    pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens, 720)
    torch.cuda.synchronize()
    grown = oracle.append_latent(before, host(rows)[:, None], host(case.block_tables), host(pos))
    ref = oracle.mla_decode(host(case.query), grown, host(case.block_tables), host(case.seq_lens), case.scale,
                            512, q_kind="bf16", kv_kind="bf16")
    _run.compare(out, ref, "bf16", what=f"mla append then decode H={heads}")


def test_full_size_decode_step_append():
    """The MLA workload's shapes (256 sequences of U[1, 8192] tokens, 128K-block
    pool): one new row per sequence after its last token. Every written slot
    equals its row, and nothing else in the 2.4 GB cache changed."""
    import decode_attention_paged_07_amd as pa
    cfg = workloads.MLA
    case = workloads.make_mla_case(cfg, device=DEV, max_seq_len=8192 + 16)
    grow_tables(case)
    S = cfg.num_seqs
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    rows = torch.randn((S, WIDTH), generator=g, device=DEV).to(torch.bfloat16)
    pos = case.seq_lens.clone()
    before = case.latent_cache.clone()
    print(f"[case] full-size mla append S={S}", flush=True)
    pa.mla_cache_append(case.latent_cache, rows, case.block_tables, pos)
    torch.cuda.synchronize()
    lens = case.meta.seq_lens.astype(np.int64)
    blocks = [int(case.meta.block_tables[s, lens[s] // 16]) for s in range(S)]
    slots = [int(lens[s] % 16) for s in range(S)]
    got = host(case.latent_cache[torch.tensor(blocks, device=DEV), :, torch.tensor(slots, device=DEV), :])
    assert np.array_equal(got.reshape(S, WIDTH), host(rows))
    changed = (case.latent_cache.view(torch.int16) != before.view(torch.int16)).any(dim=3).any(dim=1)
    where = torch.nonzero(changed).cpu().numpy()
    written = {(b, o) for b, o in zip(blocks, slots)}
    assert {(int(b), int(o)) for b, o in where} <= written


@pytest.mark.parametrize("seed", range(30))
def test_random_appends(seed):
    """Seeded random appends: bf16 or fp8 cache, 16- or 32-token blocks, 1-69
    tokens per sequence, distinct table blocks with some entries outside the
    pool, positions from negative to past the table, several value ranges and
    scales; the whole cache compared bit for bit with the oracle."""
    import decode_attention_paged_07_amd as pa
    rng = np.random.default_rng(70000 + seed)
    fp8 = bool(rng.random() < 0.5)
    bs = 32 if rng.random() < 0.5 else 16
    S, T, mb = int(rng.integers(1, 20)), int(rng.integers(1, 70)), int(rng.integers(1, 12))
    pool = S * mb + int(rng.integers(0, 10))
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    shape = pa.mla_cache_shape(pool, bs, fp8)
    if fp8:
        cache = torch.randint(0, 256, shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    else:
        cache = torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)
    table = rng.permutation(pool)[:S * mb].reshape(S, mb).astype(np.int32)
    off = rng.random((S, mb)) < 0.1
    table[off] = rng.choice([-2, -1, pool, pool + 1], int(off.sum()))
    pos = rng.integers(-3, mb * bs + 5, S).astype(np.int32)
    rows = (torch.randn((S, T, WIDTH), generator=g, device=DEV) * float(rng.choice([0.5, 3.0, 40.0])))
    rows = rows.to(torch.bfloat16)
    scale = float(np.float32(rng.choice([1.0, 0.02, 0.3])))
    print(f"[case] random append {seed}: fp8={fp8} bs={bs} S={S} T={T} mb={mb} pool={pool}", flush=True)
    before = host(cache)
    pa.mla_cache_append(cache, rows, torch.from_numpy(table).to(DEV), torch.from_numpy(pos).to(DEV), kv_scale=scale)
    torch.cuda.synchronize()
    ref = oracle.append_latent(before, host(rows), table, pos, kv_kind="e4m3fn" if fp8 else None, kv_scale=scale)
    bad = np.argwhere(host(cache) != ref)
    assert bad.size == 0, f"cache differs in {len(bad)} elements, first {bad[:4].tolist()}"
