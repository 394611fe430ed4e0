"""Readers for the text fixtures under tests/golden/ (shared by CPU and GPU tests)."""

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def partition_counts():
    return [(int(a), int(b)) for a, b in _rows("partition_counts.txt")]


def e4m3fn_codes():
    return [(int(a, 16), float(b)) for a, b in _rows("e4m3fn_codes.txt")]


def worked_example(alibi=False):
    """Inputs (pages' layouts, fp32, x = 4) and the closed-form output of the
    hand-derived example in worked_example.txt."""
    kv = {k: v for k, v in _rows("worked_example.txt")}
    n, d, scale, phys = int(kv["seq_len"]), int(kv["head_size"]), float(kv["scale"]), int(kv["table"])
    bs, x, pool = 16, 4, 8
    k_pool = np.zeros((pool, 1, d // x, bs, x), np.float32)
    v_pool = np.zeros((pool, 1, d, bs), np.float32)
    v_rows = [(1.0, 0.0, 2.0), (0.0, 1.0, 2.0), (0.0, 0.0, 2.0)]
    for t in range(n):
        k_pool[phys, 0, 0, t, 0] = float(t)           # K[t] = t * e0
        for dd, val in enumerate(v_rows[t]):
            v_pool[phys, 0, dd, t] = val
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 8.0
    e = math.e
    expect = np.zeros((1, 1, d))
    if alibi:
        w = np.array([e ** -2, 1.0, e ** 2]) / (e ** -2 + 1.0 + e ** 2)
    else:
        w = np.array([1.0, e, e * e]) / (1.0 + e + e * e)
    expect[0, 0, 0] = w[0]
    expect[0, 0, 1] = w[1]
    expect[0, 0, 2] = 2.0
    slopes = np.ones(1, np.float32) if alibi else None
    return {
        "query": q, "key_cache": k_pool, "value_cache": v_pool,
        "block_tables": np.array([[phys]], np.int32), "seq_lens": np.array([n], np.int32),
        "scale": scale, "alibi_slopes": slopes, "expect": expect,
    }


def alibi_partitions():
    """Inputs (pages' layouts, fp32, x = 4) and the closed-form per-partition
    statistics and output of the hand-derived example in alibi_partitions.txt.
    Returns the input arrays plus m [2], s [2], tmp [2, D] and expect [1, 1, D]."""
    kv = {k: v for k, v in _rows("alibi_partitions.txt")}
    n, d = int(kv["seq_len"]), int(kv["head_size"])
    scale, slope = float(kv["scale"]), float(kv["slope"])
    pool, mult, add = int(kv["pool"]), int(kv["table_mult"]), int(kv["table_add"])
    bs, x = 16, 4
    nblk = -(-n // bs)
    table = np.array([[(mult * i + add) % pool for i in range(nblk)]], np.int32)
    k_pool = np.zeros((pool, 1, d // x, bs, x), np.float32)
    v_pool = np.zeros((pool, 1, d, bs), np.float32)
    for t in range(n):
        phys, slot = table[0, t // bs], t % bs
        for dd in range(d):
            k_pool[phys, 0, dd // x, slot, dd % x] = float((t + dd) % 7 - 3)
        v_pool[phys, 0, 0, slot] = 1.0
        v_pool[phys, 0, 1, slot] = 1.0 if t >= 256 else 0.0
        v_pool[phys, 0, 2, slot] = 1.0 if t == n - 1 else 0.0
    r = math.exp(-slope)
    m = np.array([(255 - (n - 1)) * slope, 0.0])
    s = np.array([(1 - r ** 256) / (1 - r), (1 - r ** (n - 256)) / (1 - r)])
    tmp = np.zeros((2, d))
    tmp[0, 0] = 1.0
    tmp[1, 0], tmp[1, 1], tmp[1, 2] = 1.0, 1.0, 1.0 / s[1]
    z = s[0] * math.exp(m[0]) + s[1]
    expect = np.zeros((1, 1, d))
    expect[0, 0, 0], expect[0, 0, 1], expect[0, 0, 2] = 1.0, s[1] / z, 1.0 / z
    return {
        "query": np.zeros((1, 1, d), np.float32), "key_cache": k_pool, "value_cache": v_pool,
        "block_tables": table, "seq_lens": np.array([n], np.int32), "scale": scale,
        "alibi_slopes": np.array([slope], np.float32), "m": m, "s": s, "tmp": tmp, "expect": expect,
    }


def fp8_compute_example():
    """Inputs (bf16 q bits, e4m3 caches in the pages' layouts, x = 16) and the
    closed-form output of the hand-derived fp8-arithmetic example."""
    rows = {r[0]: r[1:] for r in _rows("fp8_compute_example.txt")}
    d, bs = int(rows["head_size"][0]), int(rows["block_size"][0])
    scale = float(rows["scale"][0])
    x, pool, phys = 16, 4, 2
    k_pool = np.zeros((pool, 1, d // x, bs, x), np.uint8)
    v_pool = np.zeros((pool, 1, d, bs), np.uint8)
    k_pool[phys, 0, 0, 0, 0] = int(rows["k0"][0])
    k_pool[phys, 0, 0, 1, 0] = int(rows["k1"][0])
    for t, key in enumerate(("v0", "v1")):
        for dd, code in enumerate(rows[key]):
            v_pool[phys, 0, dd, t] = int(code)
    q = np.zeros((1, 1, d), np.uint16)
    q[0, 0, 0] = 0x3F80                                  # bf16 1.0
    expect = np.zeros((1, 1, d))
    expect[0, 0, 0] = float(rows["out0"][0])
    expect[0, 0, 1] = float(rows["out1"][0])
    return dict(query=q, key_cache=k_pool, value_cache=v_pool,
                block_tables=np.array([[phys]], np.int32), seq_lens=np.array([2], np.int32),
                scale=scale, q_code=int(rows["q_code_block0"][0]), expect=expect)
