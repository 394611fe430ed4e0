"""Plain fp64 definition of paged decode attention (oracle; test infrastructure).

Nothing here is blocked, fused or reordered beyond what the definition states:
each sequence's K/V rows are gathered through its block table into logical
token order, decoded exactly to float64, and one softmax-weighted sum is taken
per query head. Slow and obviously correct is the point.

Readings of points the pages leave open (each also listed in the design notes):
  * The attention formula itself did not survive extraction on the 10100.com
    article (§2). It is taken as out = softmax(scale * q.K^T + alibi) . V over
    the sequence's valid tokens, the standard decode-attention definition that
    the rest of the pages (a scale argument, an optional alibi_slopes argument,
    softmax in fp32) supports.
  * ``x`` in the K layout [num_blocks, num_kv_heads, head_size/x, block_size, x]
    is not defined on the pages; it is read from the array's last axis, and the
    result must not depend on it.
  * Query head h reads kv head h // (num_heads // num_kv_heads) (contiguous
    groups); the pages only show a separate num_kv_heads argument.
  * ALiBi bias for token t of a sequence of length L is slope_h * (t - (L - 1)):
    zero on the newest token, more negative for older ones. Softmax is
    shift-invariant, so only max_logits (not the output) depends on this choice.
  * Tail slots t >= L of the last block and table entries past ceil(L/bs) are
    never read.
  * seq_len == 0 gives an all-zero output row.
  * The fp8 cache is OCP E4M3 "fn" (no infinities, max 448, 0x7F/0xFF NaN);
    the pages only say "e4m3". A decoded value is code_value * scale, with one
    fp32 scale for K and one for V (the pages dereference a single k_scale).
  * Partitions are 256 consecutive logical tokens (the benchmark's
    PARTITION_SIZE_ROCM); the merge of per-partition (max, exp-sum, normalised
    output) triples is the standard log-sum-exp merge, which the pages do not
    show.

PINS maps each function to what pins it (tests/test_oracle_*.py).
"""

from __future__ import annotations

import math

import numpy as np

# Largest finite OCP E4M3FN magnitude: exponent field 1111, mantissa 110.
E4M3FN_MAX = 448.0

PINS = {
    "e4m3fn_table": "all 256 codes vs torch.float8_e4m3fn -> float32 (library "
                    "routine); spot values 0x7E=448, 0x08=2^-6, 0x01=2^-9",
    "bf16_bits_to_f64": "all 65536 patterns vs torch.bfloat16 -> float32",
    "gather_sequence": "brute force vs contiguous K/V scattered element by "
                       "element through a random table; x-invariance",
    "head_logits": "brute force vs torch scaled_dot_product_attention (fp64) "
                   "with the ALiBi bias as an additive mask; slope sign/limit",
    "attention_weights": "weights sum to 1; seq_len=1; constant V; scale=0 mean",
    "paged_decode": "dense attention two ways (numpy loops, torch SDPA fp64); "
                    "physical-block permutation invariance (bitwise); GQA = MHA "
                    "with repeat_interleave'd kv heads; hand-derived golden",
    "paged_decode_partitioned": "partitioned = direct within 1e-12 for "
                                "L in {1,255,256,257,...}; per-partition "
                                "stats vs dense softmax on each token range",
    "merge_partitions": "closed form on two partitions; equals direct softmax",
}


# ---------------------------------------------------------------------------
# Exact decoding of stored element types to float64.
# ---------------------------------------------------------------------------

def e4m3fn_table() -> np.ndarray:
    """Value of each of the 256 OCP E4M3FN codes as float64.

    Format (OCP 8-bit floating point specification, E4M3 variant "fn"):
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    is subnormal (value (m/8) * 2^-6); exponent 1111 with mantissa 111 is NaN
    and there are no infinities, so 1111_110 = 448 is the largest finite value.
    The 10100.com article (§4) only states that the cache holds e4m3 values
    that are converted on load with a scale.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if (code >> 7) & 1 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            table[code] = np.nan
        elif exp_field == 0:
            table[code] = sign * (mant / 8.0) * 2.0 ** (-6)
        else:
            table[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return table


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    bfloat16 is the upper half of an IEEE binary32, so placing the 16 bits in
    the high half of a 32-bit word gives the same value as a float32.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 values are passed as their uint16 bit patterns")
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_cache_values(raw: np.ndarray, kind: str, scale: float = 1.0) -> np.ndarray:
    """Decode stored values of ``kind`` ("f32", "bf16", "e4m3fn") to float64.

    For "e4m3fn" each code is looked up in the closed-form table and multiplied
    by the per-tensor ``scale`` (the scaled conversion of the 10100.com article,
    §4). For the 16/32-bit kinds the values are used as stored and ``scale``
    must be 1.
    """
    if kind == "f32":
        if scale != 1.0:
            raise ValueError("scale applies to the fp8 cache only")
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if kind == "bf16":
        if scale != 1.0:
            raise ValueError("scale applies to the fp8 cache only")
        return bf16_bits_to_f64(raw)
    if kind == "e4m3fn":
        raw = np.asarray(raw)
        if raw.dtype != np.uint8:
            raise TypeError("e4m3fn codes are passed as uint8")
        return e4m3fn_table()[raw] * np.float64(scale)
    raise ValueError(f"unknown element kind {kind!r}")


# ---------------------------------------------------------------------------
# Gather through the block table.
# ---------------------------------------------------------------------------

def gather_sequence(key_cache: np.ndarray, value_cache: np.ndarray,
                    table_row: np.ndarray, seq_len: int):
    """Logical-order K and V rows of one sequence, still in stored form.

    Block-table indexing (10100.com article, §1): the sequence's row of the
    int32 table maps its logical block i to physical block table_row[i];
    logical token t lives in logical block t // block_size at slot
    t % block_size. Layouts (same article, §2):
      K cache [num_blocks, num_kv_heads, head_size/x, block_size, x]
      V cache [num_blocks, num_kv_heads, head_size, block_size]
    so K[t, k, d] = K_cache[table_row[t // bs], k, d // x, t % bs, d % x] and
    V[t, k, d] = V_cache[table_row[t // bs], k, d, t % bs].

    Returns (K, V), each [seq_len, num_kv_heads, head_size], same dtype as the
    caches (decoding happens afterwards, only on the gathered rows).
    """
    _, hkv, dx, bs, x = key_cache.shape
    d = dx * x
    if value_cache.shape[1:] != (hkv, d, bs):
        raise ValueError("V cache shape does not match the K cache")
    k_rows = np.empty((seq_len, hkv, d), dtype=key_cache.dtype)
    v_rows = np.empty((seq_len, hkv, d), dtype=value_cache.dtype)
    n_blocks = -(-seq_len // bs)
    for i in range(n_blocks):
        phys = int(np.int64(table_row[i]))
        t0 = i * bs
        t1 = min(seq_len, t0 + bs)
        n = t1 - t0
        # K block [hkv, d/x, bs, x] -> [bs, hkv, d/x, x] -> [bs, hkv, d]
        kb = key_cache[phys].transpose(2, 0, 1, 3).reshape(bs, hkv, d)
        # V block [hkv, d, bs] -> [bs, hkv, d]
        vb = value_cache[phys].transpose(2, 0, 1)
        k_rows[t0:t1] = kb[:n]
        v_rows[t0:t1] = vb[:n]
    return k_rows, v_rows


# ---------------------------------------------------------------------------
# The attention itself, one sequence and one query head at a time.
# ---------------------------------------------------------------------------

def head_logits(q_h: np.ndarray, k_rows: np.ndarray, scale: float,
                slope: float | None) -> np.ndarray:
    """Logits of one query head over the sequence's tokens (float64).

    logit[t] = scale * (q . K[t]) + slope * (t - (L - 1)), the ALiBi term only
    when a slope is given.
    """
    seq_len = k_rows.shape[0]
    logits = np.float64(scale) * (k_rows @ q_h)
    if slope is not None:
        t = np.arange(seq_len, dtype=np.float64)
        logits = logits + np.float64(slope) * (t - (seq_len - 1))
    return logits


def attention_weights(logits: np.ndarray) -> np.ndarray:
    """Softmax over the tokens, shifted by the maximum for range safety."""
    m = np.max(logits)
    w = np.exp(logits - m)
    return w / np.sum(w)


def _decoded_sequence(key_cache, value_cache, table_row, seq_len, kv_kind,
                      k_scale, v_scale):
    k_raw, v_raw = gather_sequence(key_cache, value_cache, table_row, seq_len)
    k_rows = decode_cache_values(k_raw, kv_kind, k_scale)
    v_rows = decode_cache_values(v_raw, kv_kind, v_scale)
    return k_rows, v_rows


def _check_shapes(query, key_cache, value_cache, block_tables, seq_lens):
    s, h, d = query.shape
    _, hkv, dx, bs, x = key_cache.shape
    if dx * x != d:
        raise ValueError("head_size of query and K cache differ")
    if h % hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    if block_tables.shape[0] != s or seq_lens.shape[0] != s:
        raise ValueError("block_tables / seq_lens do not match num_seqs")
    return s, h, hkv, d, bs


def paged_decode(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                 block_tables: np.ndarray, seq_lens: np.ndarray, scale: float, *,
                 q_kind: str, kv_kind: str, alibi_slopes: np.ndarray | None = None,
                 k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """out[s, h, :] = softmax_t(scale*q[s,h].K[t] + alibi) . V[t], in float64.

    query [S, H, D] (stored form, ``q_kind`` "f32" or "bf16" bit patterns);
    caches in the pages' layouts (see ``gather_sequence``), stored form
    ``kv_kind``; block_tables int32 [S, max_blocks]; seq_lens int [S];
    alibi_slopes [H] (fp32 values) or None; k_scale/v_scale multiply decoded
    fp8 codes. Returns float64 [S, H, D].
    """
    s_count, h_count, hkv, d, _ = _check_shapes(query, key_cache, value_cache,
                                                block_tables, seq_lens)
    group = h_count // hkv
    q = decode_cache_values(query, q_kind)
    out = np.zeros((s_count, h_count, d), dtype=np.float64)
    for s in range(s_count):
        seq_len = int(seq_lens[s])
        if seq_len == 0:
            continue
        k_rows, v_rows = _decoded_sequence(key_cache, value_cache, block_tables[s],
                                           seq_len, kv_kind, k_scale, v_scale)
        for h in range(h_count):
            kv = h // group
            slope = None if alibi_slopes is None else float(alibi_slopes[h])
            logits = head_logits(q[s, h], k_rows[:, kv, :], scale, slope)
            w = attention_weights(logits)
            out[s, h] = w @ v_rows[:, kv, :]
    return out


# ---------------------------------------------------------------------------
# Partitioned form: per-partition statistics and their merge.
# ---------------------------------------------------------------------------

def merge_partitions(max_logits: np.ndarray, exp_sums: np.ndarray,
                     outs: np.ndarray) -> np.ndarray:
    """Merge per-partition (m_p, s_p, o_p) into one softmax-weighted output.

    m_p = max logit in partition p, s_p = sum_t exp(logit_t - m_p) over it,
    o_p = (sum_t exp(logit_t - m_p) V_t) / s_p. With M = max_p m_p the whole-
    sequence softmax weight of partition p is s_p exp(m_p - M), so
    out = sum_p s_p exp(m_p - M) o_p / sum_p s_p exp(m_p - M).
    """
    big_m = np.max(max_logits)
    w = exp_sums * np.exp(max_logits - big_m)
    return (w @ outs) / np.sum(w)


def paged_decode_partitioned(query, key_cache, value_cache, block_tables, seq_lens,
                             scale, *, q_kind, kv_kind, alibi_slopes=None,
                             k_scale=1.0, v_scale=1.0, partition_tokens=256):
    """Same result as ``paged_decode`` computed through fixed-size partitions.

    The benchmark and test snippets of the PR #47361 report allocate, per
    (sequence, query head, partition), a normalised partial output, an fp32
    exp-sum and an fp32 max-logit, with
    num_partitions = ceil(max_seq_len / 256). Partition p of a sequence covers
    logical tokens [p*256, min((p+1)*256, L)); partitions that start at or
    past L hold no tokens and are left as NaN here.

    Returns (out [S,H,D], tmp_out [S,H,P,D], max_logits [S,H,P],
    exp_sums [S,H,P]), float64; P from the largest seq_len.
    """
    s_count, h_count, hkv, d, _ = _check_shapes(query, key_cache, value_cache,
                                                block_tables, seq_lens)
    group = h_count // hkv
    q = decode_cache_values(query, q_kind)
    max_len = int(np.max(seq_lens)) if s_count else 0
    n_parts = max(1, math.ceil(max_len / partition_tokens))
    out = np.zeros((s_count, h_count, d))
    tmp_out = np.full((s_count, h_count, n_parts, d), np.nan)
    max_logits = np.full((s_count, h_count, n_parts), np.nan)
    exp_sums = np.full((s_count, h_count, n_parts), np.nan)
    for s in range(s_count):
        seq_len = int(seq_lens[s])
        if seq_len == 0:
            continue
        k_rows, v_rows = _decoded_sequence(key_cache, value_cache, block_tables[s],
                                           seq_len, kv_kind, k_scale, v_scale)
        used = math.ceil(seq_len / partition_tokens)
        for h in range(h_count):
            kv = h // group
            slope = None if alibi_slopes is None else float(alibi_slopes[h])
            logits = head_logits(q[s, h], k_rows[:, kv, :], scale, slope)
            for p in range(used):
                t0 = p * partition_tokens
                t1 = min(seq_len, t0 + partition_tokens)
                m_p = np.max(logits[t0:t1])
                e = np.exp(logits[t0:t1] - m_p)
                s_p = np.sum(e)
                max_logits[s, h, p] = m_p
                exp_sums[s, h, p] = s_p
                tmp_out[s, h, p] = (e @ v_rows[t0:t1, kv, :]) / s_p
            out[s, h] = merge_partitions(max_logits[s, h, :used], exp_sums[s, h, :used],
                                         tmp_out[s, h, :used])
    return out, tmp_out, max_logits, exp_sums
