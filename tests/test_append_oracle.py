"""Pins of the KV-append oracle (fp8 quantiser and slot writes) against facts
fixed outside it: torch's float8_e4m3fn conversion, hand-derived rounding
cases, exact round trips, and read-back through the decode oracle's gather."""

import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import decode_fp64

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e4m3fn_rounding.txt")
ka = sys.modules["oracle.kv_append"]


def golden_rounding():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                x, s, c = line.split()
                rows.append((float(x), float(s), int(c, 16)))
    return rows


def torch_codes(y_f32):
    """Reference codes: torch's float32 -> float8_e4m3fn conversion of the
    quotient clamped to +-448 (torch has no saturating mode)."""
    t = torch.from_numpy(np.clip(y_f32, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_golden_rounding_cases():
    rows = golden_rounding()
    assert len(rows) >= 15
    for x, s, code in rows:
        got = int(oracle.quantise_e4m3fn(np.array([x], np.float32), s)[0])
        assert got == code, (x, s, hex(got), hex(code))


@pytest.mark.parametrize("scale", [1.0, 0.3, 7.5, 2.0 ** -4, 1.0 / 448.0 * 4.2])
def test_quantiser_matches_torch_on_every_bf16_input(scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = decode_fp64.bf16_bits_to_f64(bits).astype(np.float32)
    with np.errstate(over="ignore"):
        y = x / np.float32(scale)
    mine = oracle.quantise_e4m3fn(x, scale)
    ref = torch_codes(y)
    nan = np.isnan(y)
    assert np.all(mine[nan] == 0x7F)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_quantiser_matches_torch_on_random_f32():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(200000) * 10 ** rng.uniform(-4, 3, 200000),
                        rng.uniform(-600, 600, 20000)]).astype(np.float32)
    for scale in (1.0, 0.0123):
        assert np.array_equal(oracle.quantise_e4m3fn(x, scale), torch_codes(x / np.float32(scale)))


def test_every_finite_code_round_trips():
    table = oracle.e4m3fn_table()
    codes = np.array([c for c in range(256) if not math.isnan(table[c])], np.uint8)
    for scale in (1.0, 0.25, 8.0):           # powers of two keep value*scale exact
        vals = (table[codes] * scale).astype(np.float32)
        assert np.array_equal(oracle.quantise_e4m3fn(vals, scale), codes)


# ---------------------------------------------------------------------------
# Slot writes.
# ---------------------------------------------------------------------------

def _problem(rng, kind, x, T=3, S=4, hkv=2, d=32, bs=16, pool=24):
    shape_k = (pool, hkv, d // x, bs, x)
    shape_v = (pool, hkv, d, bs)
    if kind == "e4m3fn":
        kc = rng.integers(0, 0x7F, shape_k, dtype=np.uint8)
        vc = rng.integers(0, 0x7F, shape_v, dtype=np.uint8)
    else:
        kc = rng.standard_normal(shape_k).astype(np.float32)
        vc = rng.standard_normal(shape_v).astype(np.float32)
    perm = rng.permutation(pool)
    table = perm[:S * 5].reshape(S, 5).astype(np.int32)          # 5 blocks = 80 slots per sequence
    positions = np.array([0, 15, 17, 60][:S], np.int32)
    key = rng.standard_normal((S, T, hkv, d)).astype(np.float32)
    value = rng.standard_normal((S, T, hkv, d)).astype(np.float32)
    return kc, vc, key, value, table, positions


@pytest.mark.parametrize("kind,x", [("f32", 4), ("e4m3fn", 16), ("f32", 1)])
def test_read_back_through_the_decode_gather(kind, x):
    rng = np.random.default_rng(3)
    kc, vc, key, value, table, positions = _problem(rng, kind, x)
    ks, vs = 0.02, 0.05
    kc2, vc2 = oracle.append_tokens(kc, vc, key, value, table, positions, in_kind="f32",
                                    kv_kind=kind, k_scale=ks, v_scale=vs)
    T = key.shape[1]
    for s in range(len(positions)):
        p0 = int(positions[s])
        n = p0 + T
        k_old, v_old = oracle.gather_sequence(kc, vc, table[s], n)
        k_new, v_new = oracle.gather_sequence(kc2, vc2, table[s], n)
        assert np.array_equal(k_new[:p0], k_old[:p0]) and np.array_equal(v_new[:p0], v_old[:p0])
        if kind == "e4m3fn":
            k_dec = oracle.decode_cache_values(k_new[p0:], "e4m3fn", ks)
            v_dec = oracle.decode_cache_values(v_new[p0:], "e4m3fn", vs)
            # the stored value is the nearest code: within half a code step (<= 1/16 relative
            # for normal values, 2^-10 absolute below 2^-6) times the scale
            for dec, src, sc in ((k_dec, key[s], ks), (v_dec, value[s], vs)):
                err = np.abs(dec - src)
                bound = np.maximum(np.abs(src) / 16.0, 2.0 ** -10 * sc) + 1e-12
                assert np.all(err <= bound)
        else:
            assert np.array_equal(k_new[p0:], key[s]) and np.array_equal(v_new[p0:], value[s])


def test_untouched_slots_are_bitwise_unchanged():
    rng = np.random.default_rng(4)
    kc, vc, key, value, table, positions = _problem(rng, "f32", 4)
    positions[1] = -1                                             # skipped sequence
    kc2, vc2 = oracle.append_tokens(kc, vc, key, value, table, positions, in_kind="f32", kv_kind="f32")
    bs, T = 16, key.shape[1]
    touched = np.zeros((kc.shape[0], bs), bool)
    for s, p0 in enumerate(positions):
        if p0 < 0:
            continue
        for j in range(T):
            p = p0 + j
            touched[table[s, p // bs], p % bs] = True
    for b in range(kc.shape[0]):
        for o in range(bs):
            if not touched[b, o]:
                assert np.array_equal(kc2[b, :, :, o, :], kc[b, :, :, o, :])
                assert np.array_equal(vc2[b, :, :, o], vc[b, :, :, o])


def test_element_scatter_brute_force():
    """Element-by-element writes from the layout definitions."""
    rng = np.random.default_rng(6)
    kc, vc, key, value, table, positions = _problem(rng, "f32", 4, T=2, d=8)
    kc2, vc2 = oracle.append_tokens(kc, vc, key, value, table, positions, in_kind="f32", kv_kind="f32")
    ref_k, ref_v = kc.copy(), vc.copy()
    _, hkv, dx, bs, x = kc.shape
    for s in range(len(positions)):
        for j in range(key.shape[1]):
            p = int(positions[s]) + j
            b = int(table[s][p // bs])
            for k in range(hkv):
                for dd in range(dx * x):
                    ref_k[b, k, dd // x, p % bs, dd % x] = key[s, j, k, dd]
                    ref_v[b, k, dd, p % bs] = value[s, j, k, dd]
    assert np.array_equal(kc2, ref_k) and np.array_equal(vc2, ref_v)


def test_positions_past_the_table_and_bad_entries_are_not_written():
    rng = np.random.default_rng(8)
    kc, vc, key, value, table, positions = _problem(rng, "f32", 4, T=3)
    positions[:] = [78, -5, 0, 0]                                 # 78, 79 fit; 80 is past 5 blocks
    table[2, 0] = 10 ** 6                                          # outside the pool
    table[3, 0] = -7
    kc2, vc2 = oracle.append_tokens(kc, vc, key, value, table, positions, in_kind="f32", kv_kind="f32")
    k_new, _ = oracle.gather_sequence(kc2, vc2, table[0], 80)
    assert np.array_equal(k_new[78:80], key[0, :2])
    changed = (kc2 != kc).any(axis=(1, 2, 4))                      # [block, slot]
    assert changed.sum() == 2


# ---------------------------------------------------------------------------
# Planted mistakes must be caught.
# ---------------------------------------------------------------------------

def test_pins_catch_ties_away_from_zero(monkeypatch):
    def q_bad(x, scale):
        with np.errstate(over="ignore"):
            y = np.asarray(x, np.float32) / np.float32(scale)
        table = oracle.e4m3fn_table()[:0x7F]
        mag = np.minimum(np.abs(y.astype(np.float64)), 448.0)
        hi = np.minimum(np.searchsorted(table, mag), 0x7E)
        lo = np.maximum(hi - 1, 0)
        code = np.where(mag - table[lo] < table[hi] - mag, lo, hi).astype(np.uint8)
        return np.where(np.isnan(y), 0x7F, code | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)
    monkeypatch.setattr(oracle, "quantise_e4m3fn", q_bad)
    with pytest.raises(AssertionError):
        test_golden_rounding_cases()


def test_pins_catch_dropped_scale(monkeypatch):
    orig = ka.quantise_e4m3fn
    monkeypatch.setattr(oracle, "quantise_e4m3fn", lambda x, s: orig(x, 1.0))
    with pytest.raises(AssertionError):
        test_quantiser_matches_torch_on_every_bf16_input(0.3)


def test_pins_catch_swapped_chunk_and_slot(monkeypatch):
    orig = ka.append_tokens

    def bad(kc, vc, *a, **kw):
        # writes K as if the block were [d/x, x, bs] instead of [d/x, bs, x]
        nb, hkv, dx, bs, x = kc.shape
        k2, v2 = orig(kc.reshape(nb, hkv, dx, x, bs).swapaxes(3, 4).copy(), vc, *a, **kw)
        return k2.swapaxes(3, 4).reshape(nb, hkv, dx, bs, x).copy(), v2
    monkeypatch.setattr(oracle, "append_tokens", bad)
    with pytest.raises(AssertionError):
        test_element_scatter_brute_force()
