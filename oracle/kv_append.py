"""Plain CPU definition of appending new tokens' K/V to the paged cache
(oracle; test infrastructure).

Each decode step stores the new token's key and value in the cache before
attention reads it: the cache grows one token at a time, and a sequence's
logical token p lives in physical block block_tables[s, p // block_size] at
slot p % block_size ("vLLM 0.25.0 解读：PagedAttention 退场，MRv2 接管", §1,
logical blocks mapped to non-contiguous physical ones; 10100.com retirement
article, §1, the per-sequence int32 table). With an fp8 cache the stored
element is an e4m3 code whose value times the per-tensor scale stands for the
original (10100.com article, §4, where loads multiply by *k_scale).

Readings of points the pages leave open (also listed in the design notes):
  * Tokens to store come as key/value [num_seqs, T, num_kv_heads, head_size]
    (T new tokens per sequence; T = 1 in a decode step); token j of sequence s
    goes to logical position positions[s] + j. positions[s] < 0 skips the
    sequence. Positions past the table, and table entries outside the pool,
    are not written.
  * 16- and 32-bit caches hold the input values unchanged (same element type).
  * fp8 codes: y = x / scale computed in float32 (the precision the kernel
    decides in), then the OCP E4M3FN value nearest to y, ties to the code with
    an even mantissa, |y| > 448 saturating to +-448, NaN giving code 0x7F; the
    sign of y (also of a zero) is kept in the sign bit.
"""

from __future__ import annotations

import numpy as np

from .decode_fp64 import E4M3FN_MAX, bf16_bits_to_f64, e4m3fn_table

PINS = {
    "quantise_e4m3fn": "codes of every bfloat16 input at several scales vs torch.float8_e4m3fn "
                       "conversion of the clamped fp32 quotient (library routine); "
                       "hand-derived ties and saturation cases (tests/golden/e4m3fn_rounding.txt); "
                       "every finite code round-trips",
    "append_tokens": "read-back through the decode oracle's table gather returns the new "
                     "tokens at their positions and the old tokens unchanged; every slot not "
                     "named by a position is bitwise unchanged; brute-force element scatter",
}


def quantise_e4m3fn(x, scale: float) -> np.ndarray:
    """E4M3FN code (uint8) of x / scale, per the reading in the module docstring.

    The quotient is formed in float32. Among the 127 non-negative finite codes
    (0x00..0x7E, whose values increase with the code) the nearest value to
    |y| is chosen, ties going to the even code; the sign bit of y is then set.
    """
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.asarray(x, dtype=np.float32) / np.float32(scale)    # overflow -> inf -> saturates
    table = e4m3fn_table()
    pos_vals = table[:0x7F]                       # codes 0x00 .. 0x7E, ascending values
    mag = np.minimum(np.abs(y.astype(np.float64)), E4M3FN_MAX)
    hi = np.searchsorted(pos_vals, mag, side="left")      # first value >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = pos_vals[hi] - mag
    d_lo = mag - pos_vals[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0) & (lo != hi))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = code | (np.signbit(y).astype(np.uint8) << 7)
    code = np.where(np.isnan(y), np.uint8(0x7F), code)
    return code.astype(np.uint8)


def _input_values(raw, in_kind):
    if in_kind == "f32":
        return np.asarray(raw, dtype=np.float32)
    if in_kind == "bf16":
        return bf16_bits_to_f64(raw).astype(np.float32)    # exact
    raise ValueError(f"unknown input kind {in_kind!r}")


def append_tokens(key_cache: np.ndarray, value_cache: np.ndarray, key: np.ndarray,
                  value: np.ndarray, block_tables: np.ndarray, positions: np.ndarray, *,
                  in_kind: str, kv_kind: str, k_scale: float = 1.0, v_scale: float = 1.0):
    """Copies of (key_cache, value_cache) with the new tokens stored.

    Caches in the pages' layouts, K [num_blocks, num_kv_heads, head_size/x,
    block_size, x] and V [num_blocks, num_kv_heads, head_size, block_size]
    (10100.com article, §2), so token p of kv head k at dimension d is
    K[b, k, d // x, p % bs, d % x] and V[b, k, d, p % bs] with
    b = block_tables[s, p // bs].
    key/value: [S, T, Hkv, D] in stored form (float32, or bfloat16 bit patterns
    as uint16). kv_kind: "f32" / "bf16" (same as in_kind: stored unchanged) or
    "e4m3fn" (uint8 codes from quantise_e4m3fn with k_scale / v_scale).
    """
    kc = key_cache.copy()
    vc = value_cache.copy()
    num_blocks, hkv, dx, bs, x = kc.shape
    d = dx * x
    s_count, t_count = key.shape[:2]
    if key.shape != (s_count, t_count, hkv, d) or value.shape != key.shape:
        raise ValueError("key/value must be [num_seqs, T, num_kv_heads, head_size]")
    if kv_kind == "e4m3fn":
        k_new = quantise_e4m3fn(_input_values(key, in_kind), k_scale)
        v_new = quantise_e4m3fn(_input_values(value, in_kind), v_scale)
    elif kv_kind == in_kind:
        k_new, v_new = key, value
    else:
        raise ValueError("a 16/32-bit cache stores the input element type unchanged")
    max_pos = block_tables.shape[1] * bs
    for s in range(s_count):
        p0 = int(positions[s])
        if p0 < 0:
            continue
        for j in range(t_count):
            p = p0 + j
            if p >= max_pos:
                continue
            b = int(block_tables[s, p // bs])
            if b < 0 or b >= num_blocks:
                continue
            o = p % bs
            for k in range(hkv):
                kc[b, k, :, o, :] = k_new[s, j, k].reshape(dx, x)
                vc[b, k, :, o] = v_new[s, j, k]
    return kc, vc
