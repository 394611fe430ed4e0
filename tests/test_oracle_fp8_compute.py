"""Pins of the fp8-arithmetic oracle (oracle/decode_fp8_compute.py) against
what the definition and the mathematics fix: closed forms, invariants, an
independent rounding routine, a hand-worked example."""

import numpy as np
import pytest
import torch

import oracle
from oracle import decode_fp8_compute as f8
from tests import _golden


def all_float32_probe_values():
    """Every e4m3 value, the float32 midpoints between neighbours and the float32
    numbers adjacent to those midpoints, both signs."""
    vals = oracle.e4m3fn_table()[:0x7F].astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    m32 = mids.astype(np.float32)
    out = [vals, mids, np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(-np.inf)),
           np.array([448.0, 449.0, 464.0, 465.0, 1e9, 2.0 ** -10, 2.0 ** -11, 0.0])]
    v = np.concatenate([np.asarray(o, np.float64) for o in out])
    return np.concatenate([v, -v]).astype(np.float32)


def test_rounding_matches_the_float32_quantiser_on_float32_inputs():
    v = all_float32_probe_values()
    rng = np.random.default_rng(0)
    r = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 10, 20000))).astype(np.float32)
    for x in (v, r):
        assert np.array_equal(f8.round_to_e4m3fn(x.astype(np.float64)), oracle.quantise_e4m3fn(x, 1.0))


def test_rounding_uses_full_precision_and_ties_to_even():
    # 1.0625 is the midpoint of 1.0 (0x38, even) and 1.125 (0x39): tie -> 0x38.
    assert f8.round_to_e4m3fn(1.0625) == 0x38
    # 1.1875 is the midpoint of 1.125 (0x39) and 1.25 (0x3A): tie -> 0x3A.
    assert f8.round_to_e4m3fn(1.1875) == 0x3A
    # Just above a midpoint in float64 (not representable in float32): up.
    assert f8.round_to_e4m3fn(1.0625 + 1e-12) == 0x39
    assert f8.round_to_e4m3fn(-(1.0625 + 1e-12)) == 0xB9
    # Saturation and NaN.
    assert f8.round_to_e4m3fn(1e30) == 0x7E and f8.round_to_e4m3fn(-1e30) == 0xFE
    assert f8.round_to_e4m3fn(np.nan) == 0x7F
    # Smallest subnormal 2^-9 and the tie below it (2^-10 -> even code 0).
    assert f8.round_to_e4m3fn(2.0 ** -9) == 0x01 and f8.round_to_e4m3fn(2.0 ** -10) == 0x00
    assert f8.round_to_e4m3fn(1.5 * 2.0 ** -9) == 0x02


@pytest.mark.parametrize("k", [-20, -3, 0, 1, 7])
def test_mx_closed_forms(k):
    x = np.zeros(32)
    x[5] = 2.0 ** k
    codes, xe = f8.mx_quantise_e4m3(x)
    assert xe.tolist() == [k - 8] and codes[5] == 0x78 and np.count_nonzero(codes) == 1
    x[5] = 1.75 * 2.0 ** k                       # 448 * 2^(k-8): the largest code
    codes, xe = f8.mx_quantise_e4m3(x)
    assert xe.tolist() == [k - 8] and codes[5] == 0x7E
    x[5] = -1.9 * 2.0 ** k                       # 486.4 * 2^(k-8) saturates
    codes, xe = f8.mx_quantise_e4m3(x)
    assert codes[5] == 0xFE


def test_mx_zero_block_equivariance_and_error():
    codes, xe = f8.mx_quantise_e4m3(np.zeros(64))
    assert xe.tolist() == [-127, -127] and not codes.any()
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 128)) * np.exp2(rng.integers(-5, 5, (50, 1)))
    codes, xe = f8.mx_quantise_e4m3(x)
    for j in (-3, 4):
        c2, x2 = f8.mx_quantise_e4m3(np.ldexp(x, j))
        assert np.array_equal(c2, codes) and np.array_equal(x2, xe + j)
    cn, xn = f8.mx_quantise_e4m3(-x)
    assert np.array_equal(cn, codes ^ 0x80) and np.array_equal(xn, xe)
    deq = f8.mx_dequantise(codes, xe)
    scaled = np.abs(np.ldexp(x, -np.repeat(xe, 32, axis=-1)))
    normal = (scaled >= 2.0 ** -6) & (scaled <= 448.0)
    rel = np.abs(deq - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4 + 1e-15
    # Block maxima in (448, 512) * 2^X saturate: 448 * 2^X, under 1/8 relative error.
    sat = scaled > 448.0
    assert sat.any()
    np.testing.assert_array_equal(np.abs(deq[sat]), np.ldexp(448.0, np.repeat(xe, 32, axis=-1)[sat]))
    assert (np.abs(deq - x)[sat] / np.abs(x)[sat]).max() < 2.0 ** -3
    # Every block's largest element lands in the top binade [256, 448].
    top = np.max(np.abs(oracle.e4m3fn_table()[codes]).reshape(50, 4, 32), axis=-1)
    assert (top >= 256).all() and (top <= 448).all()


def test_golden_example():
    ex = _golden.fp8_compute_example()
    codes, xe = f8.mx_quantise_e4m3(oracle.bf16_bits_to_f64(ex["query"]))
    assert codes[0, 0, 0] == ex["q_code"] and xe[0, 0, 0] == -8
    out = f8.paged_decode_fp8_compute(ex["query"], ex["key_cache"], ex["value_cache"], ex["block_tables"],
                                      ex["seq_lens"], ex["scale"])
    np.testing.assert_allclose(out, ex["expect"], rtol=0, atol=1e-15)


def rand_case(rng, s=3, h=4, hkv=2, d=64, bs=16, lens=(1, 40, 70), pool=24, spread=None):
    q = torch.randn(s, h, d).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kc = oracle.quantise_e4m3fn(rng.standard_normal((pool, hkv, d // 16, bs, 16)).astype(np.float32), 0.5)
    vc = oracle.quantise_e4m3fn(rng.standard_normal((pool, hkv, d, bs)).astype(np.float32), 0.5)
    if spread is not None:                       # per-block key magnitudes far apart
        kc = oracle.quantise_e4m3fn((oracle.e4m3fn_table()[kc] * spread[:, None, None, None, None])
                                    .astype(np.float32), 1.0)
    table = rng.permutation(pool)[: s * 5].reshape(s, 5).astype(np.int32)
    return q, kc, vc, table, np.array(lens, np.int32)


def test_single_token_and_identical_keys():
    rng = np.random.default_rng(5)
    torch.manual_seed(5)
    q, kc, vc, table, _ = rand_case(rng)
    out = f8.paged_decode_fp8_compute(q, kc, vc, table, np.array([1, 1, 1], np.int32), 0.1,
                                      k_scale=0.7, v_scale=0.3)
    for s in range(3):
        v0 = oracle.e4m3fn_table()[vc[table[s, 0], :, :, 0]] * 0.3          # [hkv, d]
        np.testing.assert_allclose(out[s], np.repeat(v0, 2, axis=0), rtol=1e-14, atol=0)
    # Identical keys everywhere: every token has the same p, so out = mean of V.
    kc[:] = kc[0, 0, 0, 0, 0]
    lens = np.array([5, 40, 70], np.int32)
    out = f8.paged_decode_fp8_compute(q, kc, vc, table, lens, 0.1, v_scale=0.3)
    for s in range(3):
        _, v_raw = oracle.gather_sequence(kc, vc, table[s], int(lens[s]))
        mean = oracle.e4m3fn_table()[v_raw].mean(axis=0) * 0.3             # [hkv, d]
        np.testing.assert_allclose(out[s], np.repeat(mean, 2, axis=0), rtol=1e-12, atol=1e-14)


def test_physical_permutation_invariance():
    rng = np.random.default_rng(8)
    torch.manual_seed(8)
    q, kc, vc, table, lens = rand_case(rng)
    out = f8.paged_decode_fp8_compute(q, kc, vc, table, lens, 0.125, k_scale=0.9, v_scale=1.1)
    perm = rng.permutation(kc.shape[0])
    inv = np.argsort(perm)
    out2 = f8.paged_decode_fp8_compute(q, kc[perm], vc[perm], inv[table].astype(np.int32), lens, 0.125,
                                       k_scale=0.9, v_scale=1.1)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("alibi", [False, True])
def test_within_p_quantisation_bound_of_exact_attention(alibi):
    """Against exact softmax attention over the same MX-quantised q: only P's
    e4m3 rounding separates them. Each p has relative error <= 2^-4 (or an
    absolute 2^-10 below 2^-6) against 2^(z - c_b) <= 1, so
    |out - exact| <= max_t |v_t - exact| * (sum of those errors) / (sum p - errors).
    Blocks with very different key magnitudes make the 2^c_b factors matter."""
    rng = np.random.default_rng(11)
    torch.manual_seed(11)
    spread = np.exp2(rng.integers(-2, 3, 24)).astype(np.float64)
    q, kc, vc, table, lens = rand_case(rng, spread=spread, lens=(17, 64, 80))
    slopes = np.array([0.5, 0.25, 0.125, 0.0625]) if alibi else None
    out = f8.paged_decode_fp8_compute(q, kc, vc, table, lens, 0.2, k_scale=1.3, v_scale=0.8,
                                      alibi_slopes=slopes)
    codes, xe = f8.mx_quantise_e4m3(oracle.bf16_bits_to_f64(q))
    qt = f8.mx_dequantise(codes, xe)
    tab = oracle.e4m3fn_table()
    worst = 0.0
    for s in range(3):
        k_raw, v_raw = oracle.gather_sequence(kc, vc, table[s], int(lens[s]))
        for h in range(4):
            kv = h // 2
            logits = oracle.head_logits(qt[s, h], tab[k_raw[:, kv]] * 1.3, 0.2,
                                        None if slopes is None else slopes[h])
            w = oracle.attention_weights(logits)
            v = tab[v_raw[:, kv]] * 0.8
            exact = w @ v
            z = logits / np.log(2.0)
            p_hat = np.concatenate([np.exp2(z[b:b + 16] - np.ceil(z[b:b + 16].max()))
                                    for b in range(0, len(z), 16)])
            c = np.concatenate([np.full(min(16, len(z) - b), np.ceil(z[b:b + 16].max()))
                                for b in range(0, len(z), 16)])
            err = np.maximum(2.0 ** -4 * p_hat, 2.0 ** -10) * np.exp2(c)
            bound = np.max(np.abs(v - exact), axis=0) * err.sum() / (np.sum(p_hat * np.exp2(c)) - err.sum())
            dev = np.abs(out[s, h] - exact)
            assert (dev <= bound + 1e-12).all()
            worst = max(worst, float((dev / np.maximum(bound, 1e-300)).max()))
    assert worst > 0.0


def test_block_reference_is_the_ceiling():
    """z = (0.5, -9) in one block: with c = ceil(0.5) = 1 the second p is
    2^-10, the tie between 0 and 2^-9, which rounds to the even code 0, so out
    is exactly V[0]; a floor reference (c = 0) would keep 2^-9 of V[1]."""
    ex = _golden.fp8_compute_example()
    kc = ex["key_cache"].copy()
    kc[2, 0, 0, 0, 0] = 0x30                       # K[0] = 0.5
    kc[2, 0, 0, 1, 0] = 0xD1                       # K[1] = -9 = -1.125 * 2^3
    assert oracle.e4m3fn_table()[0xD1] == -9.0
    out = f8.paged_decode_fp8_compute(ex["query"], kc, ex["value_cache"], ex["block_tables"], ex["seq_lens"],
                                      ex["scale"])
    v0 = oracle.e4m3fn_table()[ex["value_cache"][2, 0, :, 0]]
    np.testing.assert_allclose(out[0, 0], v0, rtol=1e-15, atol=0)


@pytest.mark.parametrize("alibi", [False, True])
def test_exact_attention_bound_holds_for_the_oracle(alibi):
    """tests/_fp8tol.exact_attention_bound (q quantisation plus P quantisation)
    bounds the fp8-arithmetic oracle's distance from exact attention of the
    unquantised bf16 queries, on random caches with spread key magnitudes."""
    from tests import _fp8tol
    rng = np.random.default_rng(17)
    torch.manual_seed(17)
    spread = np.exp2(rng.integers(-2, 3, 24)).astype(np.float64)
    q, kc, vc, table, lens = rand_case(rng, spread=spread, lens=(17, 64, 80))
    slopes = np.array([0.5, 0.25, 0.125, 0.0625], np.float32) if alibi else None
    h = dict(query=q, key_cache=kc, value_cache=vc, block_tables=table, seq_lens=lens, scale=0.2, k_scale=1.3,
             v_scale=0.8, alibi_slopes=slopes)
    out = f8.paged_decode_fp8_compute(q, kc, vc, table, lens, 0.2, k_scale=1.3, v_scale=0.8, alibi_slopes=slopes)
    exact, bound = _fp8tol.exact_attention_bound(h)
    direct = oracle.paged_decode(q, kc, vc, table, lens, 0.2, q_kind="bf16", kv_kind="e4m3fn",
                                 alibi_slopes=slopes, k_scale=1.3, v_scale=0.8)
    np.testing.assert_allclose(exact, direct, rtol=1e-12, atol=1e-13)
    dev = np.abs(out - exact)
    assert (dev <= bound + 1e-12).all()
    assert dev.max() > 0 and (dev / np.maximum(bound, 1e-300)).max() > 1e-3   # not vacuous
