"""fp8-arithmetic paged decode attention, in plain float64 (oracle; test
infrastructure only, like the rest of this package).

The 10100.com article (§4) contrasts the PagedAttention fp8 path, which only
stores K/V as e4m3 and widens them to fp16/bf16 for the products, with newer
kernels that run the whole decode on fp8 operands and convert once at the
output. The page gives no formula for that variant. The plainest reading that
gfx950's block-scaled fp8 matrix instructions support, taken here:

  1. q is quantised to MX fp8: each block of 32 consecutive head dims shares
     a power-of-two scale 2^X, X = floor(log2 max|q|) - 8 (8 being e4m3's
     largest exponent), clamped to [-127, 127] (-127 for an all-zero block,
     127 for an infinite maximum); each element becomes the nearest e4m3 value
     of q / 2^X, ties to even, magnitude saturated at 448.
  2. logit l_t = scale * k_scale * sum_d q~_d K_d with q~ the dequantised MX
     values and K_d the e4m3 code values (every product is exact).
  3. z_t = log2(e) * (l_t + slope * (t - (L - 1))), the log2-domain logit.
  4. For each cache block b of the sequence (tokens b*bs .. min(L, (b+1)*bs)-1):
     c_b = ceil(max_t z_t) and p_t = e4m3(2^(z_t - c_b)), nearest, ties to
     even (so every p_t <= 1).
  5. out = v_scale * sum_b 2^c_b sum_t p_t V_t / sum_b 2^c_b sum_t p_t, with
     V_t the e4m3 code values.

Nothing is blocked or reordered beyond what these steps state. Pins: PINS.
"""

from __future__ import annotations

import numpy as np

from .decode_fp64 import E4M3FN_MAX, bf16_bits_to_f64, e4m3fn_table, gather_sequence

MX_BLOCK = 32
E4M3_EMAX = 8          # largest power of two among e4m3fn values (256 <= 448 < 512)

PINS = {
    "round_to_e4m3fn": "equals quantise_e4m3fn (the append oracle's float32 rounding) on every "
                       "float32 midpoint and neighbour of each code and on random float32 "
                       "samples; float64 inputs just off a midpoint round by their side "
                       "(no double rounding); ties to even by hand",
    "mx_quantise_e4m3": "closed forms: block max 2^k -> X = k - 8 and code 0x78; 1.75*2^k -> "
                        "0x7E; 1.9*2^k saturates to 0x7E; zero block -> X = -127, codes 0; "
                        "power-of-two equivariance; dequantised error <= 2^-4 relative in "
                        "the normal range; sign symmetry",
    "paged_decode_fp8_compute": "one token -> v_scale * V exactly; identical keys -> mean of V; "
                                "physical-block permutation invariance (bitwise); hand-worked "
                                "golden example (tests/golden/fp8_compute_example.txt); the "
                                "block reference is the ceiling (a 2^-10 tie rounds to 0); within "
                                "the P-quantisation bound of exact attention over the same "
                                "MX-quantised q on adversarial block maxima",
}


def round_to_e4m3fn(y) -> np.ndarray:
    """E4M3FN code (uint8) nearest to each float64 value y, ties to the even
    code, magnitude saturated at 448, NaN -> 0x7F, sign kept.

    Unlike quantise_e4m3fn (which forms a float32 quotient first), y is used
    at full float64 precision, so no intermediate rounding can move it across
    a midpoint.
    """
    y = np.asarray(y, dtype=np.float64)
    pos_vals = e4m3fn_table()[:0x7F]              # codes 0x00 .. 0x7E, ascending
    mag = np.minimum(np.abs(y), E4M3FN_MAX)
    with np.errstate(invalid="ignore"):
        hi = np.searchsorted(pos_vals, np.where(np.isnan(mag), 0.0, mag), side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = pos_vals[hi] - mag
    d_lo = mag - pos_vals[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0) & (lo != hi))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = code | (np.signbit(y).astype(np.uint8) << 7)
    return np.where(np.isnan(y), np.uint8(0x7F), code).astype(np.uint8)


def mx_exponents(x: np.ndarray) -> np.ndarray:
    """Shared exponent X of each MX block (last axis in blocks of 32)."""
    x = np.asarray(x, dtype=np.float64)
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.where(np.isnan(blocks), 0.0, np.abs(blocks)), axis=-1)
    _, e = np.frexp(amax)                         # amax = m * 2^e, m in [0.5, 1)
    x_exp = e.astype(np.int64) - 1 - E4M3_EMAX    # floor(log2 amax) - 8
    x_exp = np.clip(x_exp, -127, 127)
    x_exp = np.where(amax == 0.0, -127, x_exp)
    x_exp = np.where(np.isinf(amax), 127, x_exp)
    return x_exp


def mx_quantise_e4m3(x: np.ndarray):
    """MX e4m3 quantisation along the last axis (a multiple of 32).

    Returns (codes uint8, same shape as x; exponents int64, one per block).
    The dequantised value of element i is e4m3(codes[i]) * 2^exponents[i // 32].
    """
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % MX_BLOCK:
        raise ValueError("the last axis must be a multiple of 32")
    x_exp = mx_exponents(x)
    per_elem = np.repeat(x_exp, MX_BLOCK, axis=-1)
    codes = round_to_e4m3fn(np.ldexp(x, -per_elem))
    return codes, x_exp


def mx_dequantise(codes: np.ndarray, x_exp: np.ndarray) -> np.ndarray:
    per_elem = np.repeat(np.asarray(x_exp), MX_BLOCK, axis=-1)
    return np.ldexp(e4m3fn_table()[codes], per_elem)


def head_output_fp8(q_tilde: np.ndarray, k_vals: np.ndarray, v_vals: np.ndarray, block_size: int,
                    scale: float, k_scale: float, v_scale: float, slope: float | None) -> np.ndarray:
    """Steps 2-5 for one query head over one sequence's decoded rows.

    q_tilde [D] dequantised MX values; k_vals / v_vals [L, D] e4m3 code values
    (without k_scale / v_scale).
    """
    seq_len = k_vals.shape[0]
    logits = np.float64(scale) * np.float64(k_scale) * (k_vals @ q_tilde)
    if slope is not None:
        logits = logits + np.float64(slope) * (np.arange(seq_len, dtype=np.float64) - (seq_len - 1))
    z = logits / np.log(2.0)                       # log2(e) * logit
    num = np.zeros(v_vals.shape[1])
    den = 0.0
    for b0 in range(0, seq_len, block_size):
        zb = z[b0:b0 + block_size]
        c_b = np.ceil(np.max(zb))
        p = e4m3fn_table()[round_to_e4m3fn(np.exp2(zb - c_b))]
        num += np.ldexp(p @ v_vals[b0:b0 + block_size], int(c_b))
        den += np.ldexp(np.sum(p), int(c_b))
    return np.float64(v_scale) * num / den


def paged_decode_fp8_compute(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                             block_tables: np.ndarray, seq_lens: np.ndarray, scale: float, *,
                             k_scale: float = 1.0, v_scale: float = 1.0,
                             alibi_slopes: np.ndarray | None = None) -> np.ndarray:
    """Steps 1-5 for every (sequence, query head), float64 [S, H, D].

    query: bf16 bit patterns [S, H, D]; caches: e4m3fn codes (uint8) in the
    pages' layouts (10100.com article, §2), gathered through the block table
    as in the plain oracle (§1); seq_len 0 gives a zero row.
    """
    s_count, h_count, d = query.shape
    _, hkv, dx, bs, x = key_cache.shape
    if dx * x != d or h_count % hkv:
        raise ValueError("shapes do not match")
    group = h_count // hkv
    codes, x_exp = mx_quantise_e4m3(bf16_bits_to_f64(query))
    q_tilde = mx_dequantise(codes, x_exp)
    table = e4m3fn_table()
    out = np.zeros((s_count, h_count, d))
    for s in range(s_count):
        seq_len = int(seq_lens[s])
        if seq_len == 0:
            continue
        k_raw, v_raw = gather_sequence(key_cache, value_cache, block_tables[s], seq_len)
        k_vals, v_vals = table[k_raw], table[v_raw]
        for h in range(h_count):
            kv = h // group
            slope = None if alibi_slopes is None else float(alibi_slopes[h])
            out[s, h] = head_output_fp8(q_tilde[s, h], k_vals[:, kv, :], v_vals[:, kv, :], bs, scale,
                                        k_scale, v_scale, slope)
    return out
