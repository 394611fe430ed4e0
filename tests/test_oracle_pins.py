"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test checks the oracle against something it does not share code with: a
library routine (torch's fp8/bf16 conversions, torch SDPA in float64), brute
force on contiguous tensors scattered element by element, closed forms, or
invariants of the mathematics (block relabelling, softmax shift invariance).
"""

import math

import numpy as np
import pytest
import torch

import oracle



# ---------------------------------------------------------------------------
# Helpers local to the tests: contiguous K/V and an element-by-element scatter.
# ---------------------------------------------------------------------------

def scatter_to_pool(k_list, v_list, pool_blocks, bs, x, rng, dtype=np.float32):
    """Place per-sequence contiguous K/V [L, Hkv, D] into a random pool.

    Writes one element at a time with the layout definitions
    K_pool[b, k, d // x, o, d % x] and V_pool[b, k, d, o] for token t in
    logical block i = t // bs at slot o = t % bs, b = table[i].
    """
    hkv, d = k_list[0].shape[1:]
    k_pool = rng.standard_normal((pool_blocks, hkv, d // x, bs, x)).astype(dtype)
    v_pool = rng.standard_normal((pool_blocks, hkv, d, bs)).astype(dtype)
    lens = [k.shape[0] for k in k_list]
    max_blocks = max(1, max(-(-n // bs) for n in lens))
    perm = rng.permutation(pool_blocks)
    table = np.zeros((len(k_list), max_blocks), dtype=np.int32)
    pos = 0
    for s, (kk, vv) in enumerate(zip(k_list, v_list)):
        n = kk.shape[0]
        for i in range(-(-n // bs)):
            table[s, i] = perm[pos]
            pos += 1
        for t in range(n):
            b = table[s, t // bs]
            o = t % bs
            for k in range(hkv):
                for dd in range(d):
                    k_pool[b, k, dd // x, o, dd % x] = kk[t, k, dd]
                    v_pool[b, k, dd, o] = vv[t, k, dd]
    return k_pool, v_pool, table


def dense_sdpa(q, k_list, v_list, scale, slopes=None, shift_to_end=True):
    """Dense reference through torch.nn.functional.scaled_dot_product_attention
    in float64 on the CPU. q [S, H, D]; k_list[s], v_list[s] [L, Hkv, D]."""
    s_count, h, d = q.shape
    out = np.zeros((s_count, h, d))
    for s in range(s_count):
        kk = torch.from_numpy(np.asarray(k_list[s], np.float64))
        vv = torch.from_numpy(np.asarray(v_list[s], np.float64))
        n, hkv, _ = kk.shape
        if n == 0:
            continue
        g = h // hkv
        kk = kk.permute(1, 0, 2).repeat_interleave(g, dim=0).unsqueeze(0)  # [1,H,L,D]
        vv = vv.permute(1, 0, 2).repeat_interleave(g, dim=0).unsqueeze(0)
        qq = torch.from_numpy(np.asarray(q[s], np.float64)).reshape(1, h, 1, d)
        mask = None
        if slopes is not None:
            t = torch.arange(n, dtype=torch.float64)
            pos = t - (n - 1) if shift_to_end else t
            mask = (torch.from_numpy(np.asarray(slopes, np.float64)).reshape(h, 1)
                    * pos.reshape(1, n)).reshape(1, h, 1, n)
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=mask, scale=scale)
        out[s] = o.reshape(h, d).numpy()
    return out


def run_oracle(q, kp, vp, table, lens, scale, slopes=None, kind="f32", **kw):
    return oracle.paged_decode(q, kp, vp, table, np.asarray(lens, np.int32), scale,
                               q_kind=kind, kv_kind=kind, alibi_slopes=slopes, **kw)


def random_problem(rng, lens, h, hkv, d, bs=16, x=4, extra_blocks=3):
    k_list = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lens]
    v_list = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lens]
    pool = sum(-(-n // bs) for n in lens) + extra_blocks
    kp, vp, table = scatter_to_pool(k_list, v_list, pool, bs, x, rng)
    q = rng.standard_normal((len(lens), h, d)).astype(np.float32)
    return q, k_list, v_list, kp, vp, table


# ---------------------------------------------------------------------------
# Element decoding.
# ---------------------------------------------------------------------------

def test_e4m3fn_table_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    mine = oracle.e4m3fn_table()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_e4m3fn_spot_values():
    t = oracle.e4m3fn_table()
    assert t[0x7E] == 448.0 == oracle.E4M3FN_MAX
    assert t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x38] == 1.0                # exponent 7 = bias
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2      # no infinities, only two NaN codes


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32)
    ref = ref.numpy().astype(np.float64)  # NaN payloads stay NaN
    mine = oracle.bf16_bits_to_f64(bits)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def test_decode_rejects_scale_on_16bit():
    with pytest.raises(ValueError):
        oracle.decode_cache_values(np.zeros(2, np.float32), "f32", 2.0)


# ---------------------------------------------------------------------------
# Gather and attention against dense references.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("h,hkv", [(4, 4), (8, 2), (6, 1)])
def test_brute_force_vs_dense_sdpa(h, hkv):
    rng = np.random.default_rng(11)
    lens = [1, 15, 16, 17, 40]
    d, x = 8, 4
    q, k_list, v_list, kp, vp, table = random_problem(rng, lens, h, hkv, d, x=x)
    got = run_oracle(q, kp, vp, table, lens, 0.37)
    ref = dense_sdpa(q, k_list, v_list, 0.37)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_brute_force_with_alibi_vs_dense_sdpa():
    rng = np.random.default_rng(12)
    lens = [3, 33, 50]
    h, hkv, d = 4, 2, 8
    q, k_list, v_list, kp, vp, table = random_problem(rng, lens, h, hkv, d)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625], np.float32)
    got = run_oracle(q, kp, vp, table, lens, 0.3, slopes=slopes)
    ref = dense_sdpa(q, k_list, v_list, 0.3, slopes=slopes)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # softmax shift invariance: slope*t (not anchored at the last token) gives
    # the same output, so only max_logits depends on the anchor.
    ref2 = dense_sdpa(q, k_list, v_list, 0.3, slopes=slopes, shift_to_end=False)
    np.testing.assert_allclose(got, ref2, rtol=1e-12, atol=1e-12)


def test_brute_force_loops_vs_oracle():
    """Naive per-token loops (no numpy matmul) on a tiny case."""
    rng = np.random.default_rng(13)
    lens = [5, 19]
    h, hkv, d = 2, 1, 4
    q, k_list, v_list, kp, vp, table = random_problem(rng, lens, h, hkv, d)
    scale = 0.7
    got = run_oracle(q, kp, vp, table, lens, scale)
    for s, n in enumerate(lens):
        for hh in range(h):
            logits = []
            for t in range(n):
                acc = 0.0
                for dd in range(d):
                    acc += float(q[s, hh, dd]) * float(k_list[s][t, hh // (h // hkv), dd])
                logits.append(scale * acc)
            m = max(logits)
            e = [math.exp(v - m) for v in logits]
            z = sum(e)
            for dd in range(d):
                val = sum(e[t] * float(v_list[s][t, hh // (h // hkv), dd]) for t in range(n)) / z
                assert abs(val - got[s, hh, dd]) < 1e-12


@pytest.mark.parametrize("x", [1, 2, 4, 8, 16, 64])
def test_result_independent_of_x(x):
    rng = np.random.default_rng(14)
    lens = [30, 7]
    h, hkv, d = 4, 2, 64
    k_list = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lens]
    v_list = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lens]
    q = rng.standard_normal((2, h, d)).astype(np.float32)
    base = dense_sdpa(q, k_list, v_list, 0.125)
    kp, vp, table = scatter_to_pool(k_list, v_list, 6, 16, x, np.random.default_rng(1))
    got = run_oracle(q, kp, vp, table, lens, 0.125)
    np.testing.assert_allclose(got, base, rtol=1e-12, atol=1e-12)


def test_block_relabelling_is_bitwise_invariant():
    rng = np.random.default_rng(15)
    lens = [40, 17, 64]
    q, _, _, kp, vp, table = random_problem(rng, lens, 4, 2, 16, extra_blocks=5)
    ref = run_oracle(q, kp, vp, table, lens, 0.25)
    perm = rng.permutation(kp.shape[0])        # new id of old block b is perm[b]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    table2 = perm[table].astype(np.int32)
    got = run_oracle(q, kp2, vp2, table2, lens, 0.25)
    assert np.array_equal(got, ref)


def test_unused_slots_and_entries_never_read():
    rng = np.random.default_rng(16)
    lens = [17, 40]
    q, k_list, v_list, kp, vp, table = random_problem(rng, lens, 2, 2, 8, extra_blocks=2)
    ref = dense_sdpa(q, k_list, v_list, 0.5)
    used = set()
    for s, n in enumerate(lens):
        for i in range(-(-n // 16)):
            used.add(int(table[s, i]))
    nan_block = [b for b in range(kp.shape[0]) if b not in used][0]
    kp = kp.copy()
    vp = vp.copy()
    kp[nan_block] = np.nan
    vp[nan_block] = np.nan
    table = np.concatenate([table, np.full((2, 3), nan_block, np.int32)], axis=1)
    for s, n in enumerate(lens):
        last = table[s, (n - 1) // 16]
        kp[last, :, :, n % 16 or 16:, :] = np.nan
        vp[last, :, :, n % 16 or 16:] = np.nan
    got = run_oracle(q, kp, vp, table, lens, 0.5)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Softmax closed forms and special cases.
# ---------------------------------------------------------------------------

def test_weights_sum_to_one():
    rng = np.random.default_rng(17)
    for n in (1, 2, 255, 1000):
        w = oracle.attention_weights(rng.standard_normal(n) * 30)
        assert abs(w.sum() - 1.0) <= 1e-12
        assert np.all(w >= 0)


def test_seq_len_one_returns_that_v_row():
    rng = np.random.default_rng(18)
    q, k_list, v_list, kp, vp, table = random_problem(rng, [1], 4, 2, 16)
    got = run_oracle(q, kp, vp, table, [1], 3.0)
    for hh in range(4):
        assert np.array_equal(got[0, hh], v_list[0][0, hh // 2].astype(np.float64))


def test_constant_v_returns_constant():
    rng = np.random.default_rng(19)
    lens = [37]
    h, hkv, d = 2, 1, 8
    k_list = [rng.standard_normal((37, hkv, d)).astype(np.float32)]
    row = rng.standard_normal(d).astype(np.float32)
    v_list = [np.tile(row, (37, hkv, 1))]
    kp, vp, table = scatter_to_pool(k_list, v_list, 4, 16, 4, rng)
    q = rng.standard_normal((1, h, d)).astype(np.float32)
    got = run_oracle(q, kp, vp, table, lens, 1.0)
    np.testing.assert_allclose(got[0], np.tile(row.astype(np.float64), (h, 1)), rtol=0, atol=1e-12)


def test_zero_scale_returns_mean_of_v():
    rng = np.random.default_rng(20)
    q, k_list, v_list, kp, vp, table = random_problem(rng, [29], 2, 2, 8)
    got = run_oracle(q, kp, vp, table, [29], 0.0)
    mean = v_list[0].astype(np.float64).mean(axis=0)          # [Hkv, D]
    np.testing.assert_allclose(got[0], mean, rtol=0, atol=1e-12)


def test_seq_len_zero_gives_zeros():
    rng = np.random.default_rng(21)
    q, k_list, v_list, kp, vp, table = random_problem(rng, [5, 9], 2, 2, 8)
    got = run_oracle(q, kp, vp, table, [0, 9], 0.5)
    assert np.array_equal(got[0], np.zeros((2, 8)))
    ref = dense_sdpa(q[1:], [k_list[1]], [v_list[1]], 0.5)
    np.testing.assert_allclose(got[1:], ref, rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(22)
    lens = [20, 33]
    h, hkv, d = 8, 2, 16
    g = h // hkv
    k_list = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lens]
    v_list = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lens]
    q = rng.standard_normal((2, h, d)).astype(np.float32)
    kp, vp, table = scatter_to_pool(k_list, v_list, 8, 16, 4, np.random.default_rng(2))
    gqa = run_oracle(q, kp, vp, table, lens, 0.2)
    k_rep = [np.repeat(k, g, axis=1) for k in k_list]
    v_rep = [np.repeat(v, g, axis=1) for v in v_list]
    kp2, vp2, table2 = scatter_to_pool(k_rep, v_rep, 8, 16, 4, np.random.default_rng(3))
    mha = run_oracle(q, kp2, vp2, table2, lens, 0.2)
    assert np.array_equal(gqa, mha)


def test_alibi_zero_slope_and_limits():
    rng = np.random.default_rng(23)
    lens = [45]
    q, k_list, v_list, kp, vp, table = random_problem(rng, lens, 2, 2, 8)
    plain = run_oracle(q, kp, vp, table, lens, 0.5)
    zero = run_oracle(q, kp, vp, table, lens, 0.5, slopes=np.zeros(2, np.float32))
    assert np.array_equal(plain, zero)
    # A huge positive slope puts all weight on the newest token.
    huge = run_oracle(q, kp, vp, table, lens, 0.5, slopes=np.full(2, 1e4, np.float32))
    np.testing.assert_allclose(huge[0], v_list[0][-1].astype(np.float64), rtol=0, atol=1e-12)


def test_fp8_cache_decoding_and_scales():
    """fp8 path = f32 path on the decoded values times the scales."""
    rng = np.random.default_rng(24)
    lens = [21, 3]
    h, hkv, d, bs, x = 4, 2, 32, 16, 16
    codes_k = rng.integers(0, 256, (4, hkv, d // x, bs, x)).astype(np.uint8)
    codes_v = rng.integers(0, 256, (4, hkv, d, bs)).astype(np.uint8)
    # keep NaN codes out of the valid tokens
    codes_k[codes_k & 0x7F == 0x7F] = 0x30
    codes_v[codes_v & 0x7F == 0x7F] = 0x31
    table = np.array([[2, 0], [3, 1]], np.int32)
    q = rng.standard_normal((2, h, d)).astype(np.float32)
    got = oracle.paged_decode(q, codes_k, codes_v, table, np.array(lens, np.int32), 0.1,
                              q_kind="f32", kv_kind="e4m3fn", k_scale=0.5, v_scale=3.0)
    lut = oracle.e4m3fn_table()
    ref = oracle.paged_decode(q, (lut[codes_k] * 0.5).astype(np.float64),
                              (lut[codes_v] * 3.0).astype(np.float64), table,
                              np.array(lens, np.int32), 0.1, q_kind="f32", kv_kind="f32")
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Partitions and their merge.
# ---------------------------------------------------------------------------

def test_merge_closed_form_two_partitions():
    # Partition a: logits {0, ln 2}; partition b: logit {ln 3}. Whole-sequence
    # weights are 1/6, 2/6, 3/6.
    va = np.array([[1.0, 0.0], [0.0, 1.0]])
    vb = np.array([[2.0, 2.0]])
    m_a, s_a = math.log(2), 1.5                        # exp(-ln2)+exp(0)
    o_a = (0.5 * va[0] + 1.0 * va[1]) / s_a
    m_b, s_b = math.log(3), 1.0
    o_b = vb[0]
    got = oracle.merge_partitions(np.array([m_a, m_b]), np.array([s_a, s_b]),
                                  np.stack([o_a, o_b]))
    expect = (1 / 6) * va[0] + (2 / 6) * va[1] + (3 / 6) * vb[0]
    np.testing.assert_allclose(got, expect, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("seq_len", [1, 255, 256, 257, 700])
def test_partitioned_equals_direct(seq_len):
    rng = np.random.default_rng(25 + seq_len)
    lens = [seq_len, max(1, seq_len // 3)]
    h, hkv, d = 4, 2, 8
    q = rng.standard_normal((2, h, d)).astype(np.float32)
    bs, x = 16, 4
    nblk = sum(-(-n // bs) for n in lens) + 1
    kp = rng.standard_normal((nblk, hkv, d // x, bs, x)).astype(np.float32)
    vp = rng.standard_normal((nblk, hkv, d, bs)).astype(np.float32)
    table = np.zeros((2, -(-max(lens) // bs)), np.int32)
    perm = rng.permutation(nblk)
    pos = 0
    for s, n in enumerate(lens):
        for i in range(-(-n // bs)):
            table[s, i] = perm[pos]
            pos += 1
    slopes = np.array([0.1, 0.2, 0.3, 0.4], np.float32)
    direct = run_oracle(q, kp, vp, table, lens, 0.3, slopes=slopes)
    out, tmp, mx, es = oracle.paged_decode_partitioned(
        q, kp, vp, table, np.array(lens, np.int32), 0.3, q_kind="f32", kv_kind="f32",
        alibi_slopes=slopes)
    np.testing.assert_allclose(out, direct, rtol=1e-12, atol=1e-13)
    assert tmp.shape[2] == math.ceil(max(lens) / 256)
    # each partition's stats against a dense softmax on its own token range
    k_rows, v_rows = oracle.gather_sequence(kp, vp, table[0], lens[0])
    k_rows = k_rows.astype(np.float64)
    v_rows = v_rows.astype(np.float64)
    for hh in range(h):
        logits = oracle.head_logits(q[0, hh].astype(np.float64), k_rows[:, hh // 2], 0.3,
                                    float(slopes[hh]))
        for p in range(math.ceil(lens[0] / 256)):
            seg = logits[p * 256:(p + 1) * 256]
            assert mx[0, hh, p] == seg.max()
            np.testing.assert_allclose(es[0, hh, p], np.exp(seg - seg.max()).sum(), rtol=1e-14)
            w = np.exp(seg - seg.max())
            np.testing.assert_allclose(tmp[0, hh, p], w @ v_rows[p * 256:(p + 1) * 256, hh // 2]
                                       / w.sum(), rtol=1e-12, atol=1e-14)
    # partitions past the end are not written
    if tmp.shape[2] > math.ceil(lens[1] / 256):
        assert np.isnan(mx[1, 0, -1])


def test_alibi_anchor_of_partition_max_logits():
    """tests/golden/alibi_partitions.txt: a hand-derived two-partition case in
    which every logit is the ALiBi term alone. The per-partition maxima are
    -5.5 and 0 only if the term is anchored at the newest token,
    slope * (t - (L - 1)); the exp-sums, partial outputs and merged output are
    the closed forms of the fixture."""
    from tests import _golden
    ex = _golden.alibi_partitions()
    out, tmp, mx, es = oracle.paged_decode_partitioned(
        ex["query"], ex["key_cache"], ex["value_cache"], ex["block_tables"], ex["seq_lens"], ex["scale"],
        q_kind="f32", kv_kind="f32", alibi_slopes=ex["alibi_slopes"])
    assert mx.shape == (1, 1, 2)
    np.testing.assert_array_equal(mx[0, 0], ex["m"])
    np.testing.assert_allclose(es[0, 0], ex["s"], rtol=1e-14)
    np.testing.assert_allclose(tmp[0, 0], ex["tmp"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(out, ex["expect"], rtol=1e-14, atol=1e-15)
    direct = oracle.paged_decode(ex["query"], ex["key_cache"], ex["value_cache"], ex["block_tables"],
                                 ex["seq_lens"], ex["scale"], q_kind="f32", kv_kind="f32",
                                 alibi_slopes=ex["alibi_slopes"])
    np.testing.assert_allclose(direct, ex["expect"], rtol=1e-14, atol=1e-15)


def test_oracle_declares_a_pin_for_every_function():
    public = {"e4m3fn_table", "bf16_bits_to_f64", "gather_sequence", "head_logits",
              "attention_weights", "paged_decode", "paged_decode_partitioned",
              "merge_partitions"}
    assert public <= set(oracle.PINS)
