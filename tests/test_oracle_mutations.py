"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each mutant replaces one oracle function with a plausible wrong version; the
same independent reference the pin tests use must then disagree.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_pins import dense_sdpa, random_problem, run_oracle

ofp = sys.modules["oracle.decode_fp64"]


def _gather_swapped_slot_and_chunk(key_cache, value_cache, table_row, seq_len):
    # wrong: reads the K block as [bs, d/x, x] instead of [d/x, bs, x]
    nb, hkv, dx, bs, x = key_cache.shape
    k_bad = key_cache.reshape(nb, hkv, bs, dx, x).transpose(0, 1, 3, 2, 4)
    return ofp._orig_gather(np.ascontiguousarray(k_bad), value_cache, table_row, seq_len)


def _logits_no_scale(q_h, k_rows, scale, slope):
    return ofp._orig_logits(q_h, k_rows, 1.0, slope)


def _logits_alibi_sign(q_h, k_rows, scale, slope):
    return ofp._orig_logits(q_h, k_rows, scale, None if slope is None else -slope)


def _merge_ignores_exp_sums(max_logits, exp_sums, outs):
    return ofp._orig_merge(max_logits, np.ones_like(exp_sums), outs)


@pytest.fixture(autouse=True)
def _keep_originals():
    ofp._orig_gather = ofp.gather_sequence
    ofp._orig_logits = ofp.head_logits
    ofp._orig_merge = ofp.merge_partitions
    yield


def _problem(alibi=False):
    rng = np.random.default_rng(99)
    lens = [17, 40]
    h, hkv, d = 4, 2, 16
    q, k_list, v_list, kp, vp, table = random_problem(rng, lens, h, hkv, d)
    slopes = np.array([0.3, 0.2, 0.1, 0.05], np.float32) if alibi else None
    ref = dense_sdpa(q, k_list, v_list, 0.25, slopes=slopes)
    return q, kp, vp, table, lens, slopes, ref


@pytest.mark.parametrize("target,mutant", [
    ("gather_sequence", _gather_swapped_slot_and_chunk),
    ("head_logits", _logits_no_scale),
    ("head_logits", _logits_alibi_sign),
])
def test_dense_reference_catches(monkeypatch, target, mutant):
    q, kp, vp, table, lens, slopes, ref = _problem(alibi=True)
    good = run_oracle(q, kp, vp, table, lens, 0.25, slopes=slopes)
    np.testing.assert_allclose(good, ref, rtol=1e-12, atol=1e-12)
    monkeypatch.setattr(ofp, target, mutant)
    bad = run_oracle(q, kp, vp, table, lens, 0.25, slopes=slopes)
    assert np.max(np.abs(bad - ref)) > 1e-3


def test_gqa_pin_catches_modulo_head_mapping():
    rng = np.random.default_rng(5)
    lens = [20]
    h, hkv, d = 4, 2, 8
    q, k_list, v_list, kp, vp, table = random_problem(rng, lens, h, hkv, d)
    ref = dense_sdpa(q, k_list, v_list, 0.5)        # repeat_interleave grouping

    good = run_oracle(q, kp, vp, table, lens, 0.5)
    np.testing.assert_allclose(good, ref, rtol=1e-12, atol=1e-12)
    # Build the wrongly grouped result directly: head i takes kv i % hkv.
    bad = np.zeros_like(good)
    k_rows, v_rows = oracle.gather_sequence(kp, vp, table[0], lens[0])
    for i in range(h):
        w = oracle.attention_weights(oracle.head_logits(q[0, i].astype(np.float64),
                                                        k_rows[:, i % hkv].astype(np.float64),
                                                        0.5, None))
        bad[0, i] = w @ v_rows[:, i % hkv].astype(np.float64)
    assert np.max(np.abs(bad - ref)) > 1e-3


def test_partition_pin_catches_unweighted_merge(monkeypatch):
    rng = np.random.default_rng(6)
    q, _, _, kp, vp, table = random_problem(rng, [600], 2, 2, 8)
    direct = run_oracle(q, kp, vp, table, [600], 0.5)
    monkeypatch.setattr(ofp, "merge_partitions", _merge_ignores_exp_sums)
    out, *_ = oracle.paged_decode_partitioned(q, kp, vp, table, np.array([600], np.int32), 0.5,
                                              q_kind="f32", kv_kind="f32")
    assert np.max(np.abs(out - direct)) > 1e-4


def test_fp8_pin_catches_wrong_bias(monkeypatch):
    def bias8():
        t = ofp._orig_table()
        return t / 2.0                  # exponent bias 8 instead of 7
    ofp._orig_table = ofp.e4m3fn_table
    monkeypatch.setattr(ofp, "e4m3fn_table", bias8)
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    mine = ofp.e4m3fn_table()
    ok = ~np.isnan(ref)
    assert not np.array_equal(mine[ok], ref[ok])


def _logits_alibi_unanchored(q_h, k_rows, scale, slope):
    # wrong: ALiBi term slope * t, not zero on the newest token
    logits = ofp._orig_logits(q_h, k_rows, scale, None)
    if slope is not None:
        logits = logits + np.float64(slope) * np.arange(k_rows.shape[0], dtype=np.float64)
    return logits


def test_alibi_anchor_pin_catches_unanchored_bias(monkeypatch):
    """Softmax is shift-invariant, so the dense reference cannot see where the
    ALiBi term is anchored; the hand-derived partition maxima can."""
    from tests import _golden
    ex = _golden.alibi_partitions()
    args = (ex["query"], ex["key_cache"], ex["value_cache"], ex["block_tables"], ex["seq_lens"], ex["scale"])
    monkeypatch.setattr(ofp, "head_logits", _logits_alibi_unanchored)
    out, _, mx, _ = oracle.paged_decode_partitioned(*args, q_kind="f32", kv_kind="f32",
                                                    alibi_slopes=ex["alibi_slopes"])
    np.testing.assert_allclose(out, ex["expect"], rtol=1e-12, atol=1e-12)   # output unchanged
    assert not np.allclose(mx[0, 0], ex["m"])                               # the maxima are not
