"""GPU parity of the KV-cache append kernel (through the C ABI) against the
CPU oracle: whole caches compared bit for bit after the append."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3fn": torch.uint8}


def host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def make(in_kind, kv_kind, S, T, hkv, d, pool, seed, positions=None, k_scale=None, v_scale=None, bs=16):
    """Random caches (garbage in every slot) of bs-token blocks, a scattered
    table, new tokens."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    rng = np.random.default_rng(seed)
    elem = kv_kind if kv_kind != "e4m3fn" else "fp8_e4m3"
    x = 16 // workloads.generate.ELEM_BYTES[elem]
    kshape, vshape = (pool, hkv, d // x, bs, x), (pool, hkv, d, bs)
    if kv_kind == "e4m3fn":
        kc = torch.randint(0, 256, kshape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
        vc = torch.randint(0, 256, vshape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    else:
        kc = torch.randn(kshape, generator=g, device=DEV).to(TORCH[kv_kind])
        vc = torch.randn(vshape, generator=g, device=DEV).to(TORCH[kv_kind])
    max_blocks = pool // S
    table = rng.permutation(pool)[:S * max_blocks].reshape(S, max_blocks).astype(np.int32)
    if positions is None:
        positions = rng.integers(-1, max_blocks * bs - T + 1, S).astype(np.int32)
    key = (torch.randn((S, T, hkv, d), generator=g, device=DEV) * 3).to(TORCH[in_kind])
    value = (torch.randn((S, T, hkv, d), generator=g, device=DEV) * 3).to(TORCH[in_kind])
    return dict(kc=kc, vc=vc, table=torch.from_numpy(table).to(DEV),
                positions=torch.from_numpy(np.asarray(positions, np.int32)).to(DEV), key=key, value=value,
                k_scale=k_scale, v_scale=v_scale)


def check(c, in_kind, kv_kind, what):
    import decode_attention_paged_07_amd as pa
    print(f"[case] {what}: in={in_kind} kv={kv_kind} key={tuple(c['key'].shape)} pool={c['kc'].shape[0]}",
          flush=True)
    kc0, vc0 = host(c["kc"]), host(c["vc"])
    name = "fp8" if kv_kind == "e4m3fn" else "auto"
    ks = 1.0 if c["k_scale"] is None else c["k_scale"]
    vs = 1.0 if c["v_scale"] is None else c["v_scale"]
    pa.kv_cache_append(c["kc"], c["vc"], c["key"], c["value"], c["table"], c["positions"],
                       kv_cache_dtype=name, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    # the oracle's quotient uses the same float32 scale values the kernel reads
    ks32, vs32 = float(np.float32(ks)), float(np.float32(vs))
    rk, rv = oracle.append_tokens(kc0, vc0, host(c["key"]), host(c["value"]), host(c["table"]),
                                  host(c["positions"]), in_kind=in_kind, kv_kind=kv_kind,
                                  k_scale=ks32, v_scale=vs32)
    gk, gv = host(c["kc"]), host(c["vc"])
    for nm, got, ref in (("K", gk, rk), ("V", gv, rv)):
        gb = got.view(np.uint8) if got.dtype != np.uint8 else got
        rb = ref.view(np.uint8) if ref.dtype != np.uint8 else ref
        bad = np.argwhere(gb != rb)
        assert bad.size == 0, f"{what}: {nm} cache differs in {len(bad)} bytes, first {bad[:4].tolist()}"


@pytest.mark.parametrize("in_kind,kv_kind,d", [("bf16", "bf16", 128), ("bf16", "bf16", 64),
                                               ("f32", "f32", 64), ("f32", "f32", 128),
                                               ("bf16", "e4m3fn", 128), ("bf16", "e4m3fn", 64),
                                               ("f32", "e4m3fn", 128), ("bf16", "bf16", 32),
                                               ("f32", "f32", 32), ("bf16", "e4m3fn", 32)])
@pytest.mark.parametrize("T", [1, 3, 16, 19])
def test_append_matches_oracle(in_kind, kv_kind, d, T):
    ks, vs = (0.021, 0.037) if kv_kind == "e4m3fn" else (None, None)
    c = make(in_kind, kv_kind, S=6, T=T, hkv=4, d=d, pool=48, seed=T * 7 + d, k_scale=ks, v_scale=vs)
    check(c, in_kind, kv_kind, f"T={T}")


def test_append_edge_positions():
    """First slot, last slot of a block, block boundary, last slot of the table,
    skipped sequences, positions running past the table."""
    S, T = 8, 2
    pos = [0, 15, 16, 31, 8 * 16 - 2, -1, 8 * 16 - 1, -100]
    c = make("bf16", "bf16", S=S, T=T, hkv=2, d=128, pool=64, seed=3, positions=pos)
    check(c, "bf16", "bf16", "edge positions")


def test_append_table_entries_outside_pool_are_skipped():
    c = make("bf16", "e4m3fn", S=4, T=1, hkv=2, d=128, pool=16, seed=9, positions=[0, 16, 33, 5],
             k_scale=0.05, v_scale=0.05)
    t = c["table"].cpu()
    t[0, 0] = 10 ** 6
    t[2, 2] = -3
    c["table"] = t.to(DEV)
    check(c, "bf16", "e4m3fn", "bad table entries")


@pytest.mark.parametrize("scale", [1.0, 0.3, 7.5, 2.0 ** -4])
def test_quantiser_on_every_bf16_pattern(scale):
    """All 65536 bf16 bit patterns (NaN, +-0, subnormals, huge values) through
    the fp8 append: every code equals the oracle's, bit for bit."""
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    S, hkv, d = 64, 8, 128                                       # 64 * 8 * 128 = 65536
    c = make("bf16", "e4m3fn", S=S, T=1, hkv=hkv, d=d, pool=64, seed=1, positions=[5] * S,
             k_scale=scale, v_scale=scale)
    c["key"] = bits.reshape(S, 1, hkv, d).to(DEV)
    c["value"] = bits.flip(0).reshape(S, 1, hkv, d).to(DEV).contiguous()
    check(c, "bf16", "e4m3fn", f"every bf16 pattern, scale {scale}")


def grow_tables(case):
    """Give every sequence whose next token starts a new block a fresh,
    unused physical block (what the block allocator does before the append)."""
    meta = case.meta
    bs = case.cfg.block_size
    used = set(meta.used_blocks.tolist())
    free = (b for b in range(case.cfg.pool_blocks) if b not in used)
    table = case.block_tables.cpu().numpy()
    for s, n in enumerate(meta.seq_lens.tolist()):
        if n % bs == 0:
            assert n // bs < table.shape[1], "table has no room for the next block"
            table[s, n // bs] = next(free)
    case.block_tables = torch.from_numpy(table).to(DEV)
    meta.block_tables = table


def test_append_then_decode_reads_the_new_tokens():
    """Integration: append one token to every sequence of a small GQA batch with
    the HIP kernel, decode with the HIP kernel, compare with the oracle decode of
    the oracle-appended caches."""
    import decode_attention_paged_07_amd as pa
    from tests import _run
    cfg = workloads.GQA.with_(num_seqs=6, pool_blocks=512, seq_lens=("fixed", (1, 15, 16, 17, 300, 704)))
    case = workloads.make_case(cfg, device=DEV, max_seq_len=720)
    grow_tables(case)
    S, hkv, d = cfg.num_seqs, cfg.num_kv_heads, cfg.head_size
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    key = torch.randn((S, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    value = torch.randn((S, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    pos = case.seq_lens.clone()                                  # the new token goes after the last one
    kc0, vc0 = host(case.key_cache), host(case.value_cache)
    print("[case] append then decode", flush=True)
    pa.kv_cache_append(case.key_cache, case.value_cache, key, value, case.block_tables, pos)
    case.seq_lens += 1
    case.meta.seq_lens = case.meta.seq_lens + 1
    out = _run.run_hip(case)
    torch.cuda.synchronize()
    rk, rv = oracle.append_tokens(kc0, vc0, host(key)[:, None], host(value)[:, None], host(case.block_tables),
                                  host(pos), in_kind="bf16", kv_kind="bf16")
    ref = oracle.paged_decode(host(case.query), rk, rv, host(case.block_tables), host(case.seq_lens),
                              case.scale, q_kind="bf16", kv_kind="bf16")
    _run.compare(out, ref, "bf16", what="append then decode")


def test_full_size_decode_step_append():
    """The fp8 workload's shapes: one new token per sequence for 256 sequences,
    written after each sequence's last token; every written slot checked."""
    import decode_attention_paged_07_amd as pa
    cfg = workloads.FP8
    case = workloads.make_case(cfg, device=DEV, max_seq_len=16384 + 16)
    grow_tables(case)
    S, hkv, d = cfg.num_seqs, cfg.num_kv_heads, cfg.head_size
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    key = torch.randn((S, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    value = torch.randn((S, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    pos = case.seq_lens.clone()
    print(f"[case] full-size fp8 append S={S}", flush=True)
    pa.kv_cache_append(case.key_cache, case.value_cache, key, value, case.block_tables, pos,
                       kv_cache_dtype="fp8", k_scale=case.k_scale, v_scale=case.v_scale)
    torch.cuda.synchronize()
    kq = oracle.quantise_e4m3fn(oracle.bf16_bits_to_f64(host(key)).astype(np.float32),
                                float(np.float32(case.k_scale)))
    vq = oracle.quantise_e4m3fn(oracle.bf16_bits_to_f64(host(value)).astype(np.float32),
                                float(np.float32(case.v_scale)))
    lens = case.meta.seq_lens.astype(np.int64)
    blocks = torch.tensor([int(case.meta.block_tables[s, lens[s] // 16]) for s in range(S)], device=DEV)
    kb = host(case.key_cache.index_select(0, blocks))          # [S, hkv, d/16, 16, 16]
    vb = host(case.value_cache.index_select(0, blocks))        # [S, hkv, d, 16]
    for s in range(S):
        o = int(lens[s] % 16)
        assert np.array_equal(kb[s, :, :, o, :].reshape(hkv, d), kq[s]), s
        assert np.array_equal(vb[s, :, :, o], vq[s]), s
