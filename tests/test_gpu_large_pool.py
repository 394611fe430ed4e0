"""Caches larger than 4 GiB, used only through blocks that lie past their
first 4 GiB.

Each case is built small, then its blocks are placed one to one at block
numbers whose byte offset is at least 4 GiB in a cache of more than 4 GiB (the
last block of the cache always among them); every other block holds NaN. A
block address formed in 32 bits would read a NaN block, or one before the
cache, and a wrapped store would change a NaN block: the outputs are compared
with the oracle, and after the writing calls every block outside the case is
checked to be unchanged. Paths covered: the bf16 and fp8 decodes (stream-K,
the 256-token split grid, the fp8 arithmetic), the shared-prefix decode, the
K/V append, the block copy, and the latent-cache decode (16 and 128 heads,
bf16 and fp8 caches, 16- and 32-token blocks) and latent append."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _fp8tol, _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
GIB4 = 1 << 32
# NaN bit patterns by element size: bf16, e4m3fn codes, fp32.
NAN_BITS = {2: (torch.int16, 0x7FC0), 1: (torch.uint8, 0x7F), 4: (torch.int32, 0x7FC00000)}


def block_bytes(cache):
    return cache[0].numel() * cache.element_size()


def high_ids(table, pool, first, rng):
    """Distinct block numbers in [first, pool) for the distinct entries of
    table, the first entry's block mapped to pool - 1. Returns (ids, new)."""
    ids = np.unique(table)
    assert pool - first >= ids.size, "the pool has too few blocks past 4 GiB"
    new = first + rng.permutation(pool - first)[:ids.size]
    k0 = int(np.searchsorted(ids, table[0, 0]))
    top = np.flatnonzero(new == pool - 1)
    if top.size:
        new[top[0]], new[k0] = new[k0], new[top[0]]
    else:
        new[k0] = pool - 1
    return ids, new


def embed(cache, ids, new, pool):
    """A NaN-filled cache of pool blocks holding cache[ids[i]] at block new[i]."""
    big = torch.empty((pool,) + tuple(cache.shape[1:]), dtype=cache.dtype, device=DEV)
    dt, bits = NAN_BITS[cache.element_size()]
    big.view(dt).fill_(bits)
    big[torch.from_numpy(new.astype(np.int64)).to(DEV)] = cache[torch.from_numpy(ids.astype(np.int64)).to(DEV)]
    return big


def relocate(case, caches, pool, seed):
    """Moves the case's blocks past 4 GiB of a pool-block cache (caches: the
    attribute names of its cache tensors); returns the block numbers used."""
    rng = np.random.default_rng(seed)
    table = case.block_tables.cpu().numpy()
    bb = block_bytes(getattr(case, caches[0]))
    first = -(-GIB4 // bb)
    ids, new = high_ids(table, pool, first, rng)
    for name in caches:
        setattr(case, name, embed(getattr(case, name), ids, new, pool))
    moved = new[np.searchsorted(ids, table)].astype(np.int32)
    assert int(moved.min()) * bb >= GIB4 and int(moved.max()) == pool - 1
    assert pool * bb > GIB4
    case.block_tables = torch.from_numpy(moved).to(DEV)
    case.meta.block_tables = moved
    torch.cuda.synchronize()
    return np.unique(moved)


def others_unchanged(cache, used, what):
    """Every block outside ``used`` still holds the NaN pattern."""
    dt, bits = NAN_BITS[cache.element_size()]
    keep = torch.ones(cache.shape[0], dtype=torch.bool, device=DEV)
    keep[torch.from_numpy(used.astype(np.int64)).to(DEV)] = False
    flat = cache.view(dt).reshape(cache.shape[0], -1)
    changed = int((flat[keep] != bits).any(dim=1).sum())
    assert changed == 0, f"{what}: {changed} blocks outside the case were written"


def own_block_positions(seq_lens, bs, T):
    """Append positions whose T tokens stay inside each sequence's own blocks
    (the table entries past a sequence all name one pad block, which several
    sequences writing at once would leave with either write): the sequence
    end, moved back as far as needed."""
    lens = np.maximum(seq_lens.astype(np.int64), 1)
    room = -(-lens // bs) * bs
    assert T <= bs
    return np.minimum(lens, room - T).astype(np.int32)


def host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ---- K/V decode ---------------------------------------------------------------

@pytest.fixture(scope="module")
def bf16_case():
    cfg = workloads.GQA.with_(num_seqs=6, pool_blocks=1500, seq_lens=("uniform", 1, 3000))
    case = workloads.make_case(cfg, seed=31, device=DEV)
    used = relocate(case, ("key_cache", "value_cache"), 140_000, 31)
    return case, used


@pytest.fixture(scope="module")
def fp8_case():
    cfg = workloads.FP8.with_(num_seqs=6, pool_blocks=1500, seq_lens=("uniform", 1, 3000))
    case = workloads.make_case(cfg, seed=32, device=DEV)
    used = relocate(case, ("key_cache", "value_cache"), 270_000, 32)
    return case, used


@pytest.mark.parametrize("split", [0, 256])
def test_bf16_decode_past_4gib(bf16_case, split):
    case, _ = bf16_case
    print(f"[case] bf16 decode, blocks past 4 GiB, split={split}", flush=True)
    out = _run.run_hip(case, split_tokens=split)
    torch.cuda.synchronize()
    _run.compare(out, _run.run_oracle(case), "bf16", what=f"bf16 past 4 GiB split={split}")


@pytest.mark.parametrize("split", [0, 256])
def test_fp8_decode_past_4gib(fp8_case, split):
    case, _ = fp8_case
    print(f"[case] fp8 cache decode, blocks past 4 GiB, split={split}", flush=True)
    out = _run.run_hip(case, split_tokens=split)
    torch.cuda.synchronize()
    _run.compare(out, _run.run_oracle(case), "bf16", what=f"fp8 past 4 GiB split={split}")


def test_fp8_arithmetic_past_4gib(fp8_case):
    case, _ = fp8_case
    print("[case] fp8 arithmetic, blocks past 4 GiB", flush=True)
    out = _run.run_hip(case, compute="fp8")
    torch.cuda.synchronize()
    extra = _fp8tol.row_bounds(workloads.host_arrays(case))
    _run.compare(out, _run.run_oracle_fp8(case), "bf16", what="fp8 arithmetic past 4 GiB", extra=extra)


def test_shared_prefix_decode_past_4gib():
    import decode_attention_paged_07_amd as pa
    cfg = workloads.GQA.with_(num_seqs=12, pool_blocks=1500, seq_lens=("uniform", 1, 600),
                              prefix_groups=(6, 320))
    case = workloads.make_case(cfg, seed=33, device=DEV)
    relocate(case, ("key_cache", "value_cache"), 140_000, 33)
    groups = pa.find_prefix_groups(case.meta.block_tables, case.meta.seq_lens, cfg.block_size)
    assert groups, "the case has no shared prefix"
    print("[case] shared-prefix decode, blocks past 4 GiB", flush=True)
    out = torch.empty_like(case.query)
    pa.paged_attention_decode_shared(out, case.query, case.key_cache, case.value_cache, cfg.num_kv_heads,
                                     case.scale, case.block_tables, case.seq_lens, cfg.block_size,
                                     case.max_seq_len, pa.prefix_groups(groups, cfg.num_seqs, DEV))
    torch.cuda.synchronize()
    _run.compare(out, _run.run_oracle(case), "bf16", what="shared prefix past 4 GiB")


# ---- writes into the cache ----------------------------------------------------

@pytest.mark.parametrize("which", ["bf16", "fp8"])
def test_kv_append_past_4gib(bf16_case, fp8_case, which):
    """Runs last among the K/V tests of its case: it changes the cache."""
    import decode_attention_paged_07_amd as pa
    case, used = bf16_case if which == "bf16" else fp8_case
    cfg = case.cfg
    S, T = cfg.num_seqs, 5
    g = torch.Generator(device=DEV)
    g.manual_seed(34)
    key = (torch.randn((S, T, cfg.num_kv_heads, cfg.head_size), generator=g, device=DEV) * 2).to(torch.bfloat16)
    value = (torch.randn((S, T, cfg.num_kv_heads, cfg.head_size), generator=g, device=DEV) * 2).to(torch.bfloat16)
    table = case.meta.block_tables
    positions = own_block_positions(case.meta.seq_lens, cfg.block_size, T)
    positions[1] = -1                                          # skipped
    idx = torch.from_numpy(used.astype(np.int64)).to(DEV)
    k0, v0 = host(case.key_cache.index_select(0, idx)), host(case.value_cache.index_select(0, idx))
    compact = np.searchsorted(used, table).astype(np.int32)
    kind = "e4m3fn" if which == "fp8" else "bf16"
    print(f"[case] {which} K/V append, blocks past 4 GiB", flush=True)
    pa.kv_cache_append(case.key_cache, case.value_cache, key, value, case.block_tables,
                       torch.from_numpy(positions).to(DEV), kv_cache_dtype="fp8" if which == "fp8" else "auto",
                       k_scale=case.k_scale, v_scale=case.v_scale)
    torch.cuda.synchronize()
    ks32, vs32 = float(np.float32(case.k_scale)), float(np.float32(case.v_scale))
    rk, rv = oracle.append_tokens(k0, v0, host(key), host(value), compact, positions, in_kind="bf16",
                                  kv_kind=kind, k_scale=ks32 if which == "fp8" else 1.0,
                                  v_scale=vs32 if which == "fp8" else 1.0)
    gk, gv = host(case.key_cache.index_select(0, idx)), host(case.value_cache.index_select(0, idx))
    for nm, got, ref in (("K", gk, rk), ("V", gv, rv)):
        bad = np.argwhere(got.view(np.uint8) != ref.view(np.uint8))
        assert bad.size == 0, f"{which} {nm}: {len(bad)} bytes differ, first {bad[:4].tolist()}"
    others_unchanged(case.key_cache, used, f"{which} K append")
    others_unchanged(case.value_cache, used, f"{which} V append")


def test_block_copy_past_4gib(bf16_case):
    import decode_attention_paged_07_amd as pa
    case, used = bf16_case
    pool = case.key_cache.shape[0]
    rng = np.random.default_rng(35)
    free = np.setdiff1d(np.arange(-(-GIB4 // block_bytes(case.key_cache)), pool), used)
    src = rng.choice(used, 8, replace=False).astype(np.int32)
    dst = rng.choice(free, 8, replace=False).astype(np.int32)
    print("[case] block copy, blocks past 4 GiB", flush=True)
    pa.copy_blocks(case.key_cache, case.value_cache, torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV))
    torch.cuda.synchronize()
    for c in (case.key_cache, case.value_cache):
        s, d = torch.from_numpy(src.astype(np.int64)).to(DEV), torch.from_numpy(dst.astype(np.int64)).to(DEV)
        assert torch.equal(c.index_select(0, s).view(torch.int16), c.index_select(0, d).view(torch.int16))
        others_unchanged(c, np.concatenate([used, dst]), "block copy")


# ---- latent cache ---------------------------------------------------------------

MLA_POOLS = {   # (pool blocks, block size, fp8): each cache over 4 GiB
    "bf16": (250_000, 16, False),
    "fp8": (480_000, 16, True),
    "bf16-bs32": (120_000, 32, False),
}


@pytest.fixture(scope="module", params=sorted(MLA_POOLS))
def mla_pool(request):
    pool, bs, fp8 = MLA_POOLS[request.param]
    cfg = workloads.MLA.with_(num_seqs=5, num_heads=128, pool_blocks=1200, block_size=bs,
                              kv_dtype="fp8_e4m3" if fp8 else "auto")
    case = workloads.make_mla_case(cfg, seed=36, device=DEV, seq_lens=[2500, 1, 700, 1777, 64])
    used = relocate(case, ("latent_cache",), pool, 36)
    return request.param, case, used


def mla_oracle(case, heads):
    h = workloads.mla_host_arrays(case)
    return oracle.mla_decode(h["query"][:, :heads], h["latent_cache"], h["block_tables"], h["seq_lens"], h["scale"],
                             512, q_kind="bf16", kv_kind=h["kv_kind"], kv_scale=h["kv_scale"])


@pytest.mark.parametrize("heads", [16, 128])
def test_mla_decode_past_4gib(mla_pool, heads):
    import decode_attention_paged_07_amd as pa
    name, case, _ = mla_pool
    print(f"[case] latent decode {name}, {heads} heads, blocks past 4 GiB", flush=True)
    q = case.query[:, :heads].contiguous()
    out = torch.empty(q.shape[0], heads, 512, dtype=torch.bfloat16, device=DEV)
    pa.mla_decode(out, q, case.latent_cache, case.scale, case.block_tables, case.seq_lens, case.max_seq_len,
                  kv_scale=case.kv_scale)
    torch.cuda.synchronize()
    _run.compare(out, mla_oracle(case, heads), "bf16", what=f"latent {name} H={heads} past 4 GiB")


def test_mla_append_past_4gib(mla_pool):
    """Runs after the decodes of its pool: it changes the cache."""
    import decode_attention_paged_07_amd as pa
    name, case, used = mla_pool
    S, T = case.cfg.num_seqs, 3
    g = torch.Generator(device=DEV)
    g.manual_seed(37)
    rows = (torch.randn((S, T, 576), generator=g, device=DEV) * 0.5).to(torch.bfloat16)
    table = case.meta.block_tables
    positions = own_block_positions(case.meta.seq_lens, case.cfg.block_size, T)
    idx = torch.from_numpy(used.astype(np.int64)).to(DEV)
    before = host(case.latent_cache.index_select(0, idx))
    compact = np.searchsorted(used, table).astype(np.int32)
    fp8 = MLA_POOLS[name][2]
    print(f"[case] latent append {name}, blocks past 4 GiB", flush=True)
    pa.mla_cache_append(case.latent_cache, rows, case.block_tables, torch.from_numpy(positions).to(DEV),
                        kv_scale=case.kv_scale)
    torch.cuda.synchronize()
    ref = oracle.append_latent(before, host(rows), compact, positions, kv_kind="e4m3fn" if fp8 else None,
                               kv_scale=float(np.float32(case.kv_scale)))
    got = host(case.latent_cache.index_select(0, idx))
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"latent append {name}: {len(bad)} elements differ, first {bad[:4].tolist()}"
    others_unchanged(case.latent_cache, used, f"latent append {name}")
