"""Oracle against the golden fixtures; seeded generators against the recipe."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _golden


@pytest.mark.parametrize("alibi", [False, True])
def test_oracle_worked_example(alibi):
    ex = _golden.worked_example(alibi)
    got = oracle.paged_decode(ex["query"], ex["key_cache"], ex["value_cache"],
                              ex["block_tables"], ex["seq_lens"], ex["scale"],
                              q_kind="f32", kv_kind="f32", alibi_slopes=ex["alibi_slopes"])
    np.testing.assert_allclose(got, ex["expect"], rtol=1e-15, atol=1e-15)


def test_partition_count_fixture_matches_oracle_partitions():
    rng = np.random.default_rng(0)
    for max_len, parts in _golden.partition_counts():
        if max_len > 4096:
            continue   # keep the CPU tier fast; the formula is the same
        d, bs, x = 4, 16, 4
        nblk = -(-max_len // bs)
        kp = rng.standard_normal((nblk, 1, d // x, bs, x)).astype(np.float32)
        vp = rng.standard_normal((nblk, 1, d, bs)).astype(np.float32)
        table = np.arange(nblk, dtype=np.int32)[None]
        q = rng.standard_normal((1, 1, d)).astype(np.float32)
        _, tmp, _, _ = oracle.paged_decode_partitioned(
            q, kp, vp, table, np.array([max_len], np.int32), 0.5, q_kind="f32", kv_kind="f32")
        assert tmp.shape[2] == parts == math.ceil(max_len / 256)


def test_e4m3fn_fixture():
    t = oracle.e4m3fn_table()
    for code, val in _golden.e4m3fn_codes():
        if math.isnan(val):
            assert math.isnan(t[code])
        else:
            assert t[code] == val and math.copysign(1, t[code]) == math.copysign(1, val)


# ---------------------------------------------------------------------------
# Generators.
# ---------------------------------------------------------------------------

def test_realised_draws_of_the_recipe():
    m = workloads.make_metadata(workloads.GQA)
    lens = m.seq_lens.astype(np.int64)
    assert lens.sum() == 542507
    assert (lens * 8 * 128 * 2 * 2).sum() == 2222108672
    assert sum(-(-int(n) // 16) for n in lens) == 33967 == m.used_blocks.size
    m = workloads.make_metadata(workloads.FP8)
    lens = m.seq_lens.astype(np.int64)
    assert lens.sum() == 1565815
    assert sum(-(-int(n) // 16) for n in lens) == 97982 == m.used_blocks.size
    assert lens.max() == 16384 and lens.min() >= 1


@pytest.mark.parametrize("name", ["tiny", "mha", "gqa", "long", "fp8"])
def test_tables_draw_without_replacement(name):
    cfg = workloads.CONFIGS[name]
    m = workloads.make_metadata(cfg)
    assert m.block_tables.dtype == np.int32
    ids = np.concatenate([m.block_tables[s, :-(-int(n) // 16)] for s, n in enumerate(m.seq_lens)])
    assert np.unique(ids).size == ids.size
    assert ids.min() >= 0 and ids.max() < cfg.pool_blocks
    assert m.block_tables.shape == (cfg.num_seqs, -(-m.max_seq_len // 16))


def test_generator_is_deterministic_and_seeded():
    a = workloads.make_case(workloads.TINY)
    b = workloads.make_case(workloads.TINY)
    c = workloads.make_case(workloads.TINY, seed=5)
    for f in ("query", "key_cache", "value_cache", "block_tables"):
        assert torch.equal(getattr(a, f), getattr(b, f))
    assert not torch.equal(a.key_cache, c.key_cache)
    assert a.meta.seq_lens.tolist() == [17, 40]
    assert a.key_cache.shape == (16, 4, 16, 16, 4) and a.value_cache.shape == (16, 4, 64, 16)


def test_fp8_quantisation_recipe():
    cfg = workloads.FP8.with_(num_seqs=4, pool_blocks=64, seq_lens=("fixed", (1, 17, 100, 256)))
    c = workloads.make_case(cfg)
    assert c.key_cache.dtype == torch.uint8 and c.key_cache.shape[-1] == 16
    assert c.k_scale == c.v_scale > 0
    lut = oracle.e4m3fn_table()
    kv = np.concatenate([lut[c.key_cache.numpy().ravel()], lut[c.value_cache.numpy().ravel()]])
    assert not np.isnan(kv).any()
    assert np.abs(kv).max() == 448.0      # the amax element maps to the largest code


def test_poison_marks_every_unused_slot():
    cfg = workloads.GQA.with_(num_seqs=3, pool_blocks=40, seq_lens=("fixed", (17, 1, 48)))
    c = workloads.make_case(cfg, poison=True, max_seq_len=80)
    kc = c.key_cache.float()
    t = c.block_tables.numpy()
    used = set()
    for s, n in enumerate([17, 1, 48]):
        nb = -(-n // 16)
        used.update(t[s, :nb].tolist())
        last = t[s, nb - 1]
        tail = n % 16
        if tail:
            assert torch.isnan(kc[last, :, :, tail:, :]).all()
            assert not torch.isnan(kc[last, :, :, :tail, :]).any()
        for e in t[s, nb:]:
            assert torch.isnan(kc[e]).all()
    for b in range(40):
        if b not in used:
            assert torch.isnan(kc[b]).all()


def test_shared_prefix_blocks():
    cfg = workloads.GQA.with_(num_seqs=3, pool_blocks=40, seq_lens=("fixed", (64, 40, 8)))
    m = workloads.make_metadata(cfg, share_prefix_blocks=2)
    assert m.block_tables[1, :2].tolist() == m.block_tables[0, :2].tolist()
    assert m.block_tables[2, 0] == m.block_tables[0, 0]


def test_host_arrays_compaction_is_a_relabelling():
    cfg = workloads.GQA.with_(num_seqs=5, num_heads=8, num_kv_heads=2, head_size=64,
                              pool_blocks=200, seq_lens=("fixed", (3, 70, 16, 33, 1)))
    c = workloads.make_case(cfg)
    full = {
        "query": c.query.view(torch.int16).numpy().view(np.uint16),
        "key_cache": c.key_cache.view(torch.int16).numpy().view(np.uint16),
        "value_cache": c.value_cache.view(torch.int16).numpy().view(np.uint16),
    }
    ref = oracle.paged_decode(full["query"], full["key_cache"], full["value_cache"],
                              c.block_tables.numpy(), c.meta.seq_lens, c.scale,
                              q_kind="bf16", kv_kind="bf16")
    h = workloads.host_arrays(c, seqs=[1, 3])
    got = oracle.paged_decode(h["query"], h["key_cache"], h["value_cache"], h["block_tables"],
                              h["seq_lens"], h["scale"], q_kind="bf16", kv_kind="bf16")
    assert np.array_equal(got, ref[[1, 3]])
