"""Comparison bound for the fp8-arithmetic decode against its oracle.

Both sides round computed values to e4m3: p = e4m3(2^(z - c)) with
c = ceil(block max z). The kernel forms z from an MFMA sum of exact fp8
products plus float32 ALiBi terms, and 2^x with the hardware exp2; the oracle
in float64. Where 2^(z - c) lies within the kernel's error of an e4m3
rounding midpoint, or a block max within it of an integer, the two sides may
legitimately pick neighbouring codes. This module bounds what such picks can
move each output element; elsewhere the two must agree to the usual bf16
output tolerance.

Error model (log2 units), with a margin of two over what was measured. The
MFMA figure is empirical, not derived: no accuracy of the block-scaled fp8
MFMA's internal summation is published, so the allowance is calibrated on the
hardware. That instruction summed its products with a relative error of at
most 2^-12 of sum |terms| (the largest seen over 200 random one-wave trials on
gfx950), so
|dz| <= 2^-11 * |c| * sum_d |q~_d K_d| + 2^-20 * (|slope2| * (L + 32) + 1),
and 2^x carries a further relative 2^-21. Within a block the P.V product
carries the same 2^-12 relative error; that is far inside the bf16 output
tolerance and needs no allowance.
"""

from __future__ import annotations

import numpy as np

import oracle


def _neighbours(p):
    """Adjacent e4m3fn values lo <= p <= hi (p >= 0)."""
    vals = oracle.e4m3fn_table()[:0x7F]
    hi_i = np.clip(np.searchsorted(vals, p, side="left"), 1, 0x7E)
    return vals[hi_i - 1], vals[hi_i]


def row_bounds(h) -> np.ndarray:
    """Per-element bound [S, H, D] for host arrays ``h`` (workloads.host_arrays)."""
    q, kc, vc = h["query"], h["key_cache"], h["value_cache"]
    s_count, h_count, d = q.shape
    hkv, bs = kc.shape[1], kc.shape[3]
    group = h_count // hkv
    codes, x_exp = oracle.mx_quantise_e4m3(oracle.bf16_bits_to_f64(q))
    qt = oracle.mx_dequantise(codes, x_exp)
    tab = oracle.e4m3fn_table()
    c_mult = float(h["scale"]) * float(h["k_scale"]) / np.log(2.0)
    out = np.zeros((s_count, h_count, d))
    for s in range(s_count):
        seq_len = int(h["seq_lens"][s])
        if seq_len == 0:
            continue
        k_raw, v_raw = oracle.gather_sequence(kc, vc, h["block_tables"][s], seq_len)
        t = np.arange(seq_len, dtype=np.float64)
        for hh in range(h_count):
            kv = hh // group
            k = tab[k_raw[:, kv]]
            v = tab[v_raw[:, kv]] * float(h["v_scale"])
            slope2 = 0.0 if h["alibi_slopes"] is None else float(h["alibi_slopes"][hh]) / np.log(2.0)
            z = c_mult * (k @ qt[s, hh]) + slope2 * (t - (seq_len - 1))
            dz = 2.0 ** -11 * abs(c_mult) * (np.abs(k) @ np.abs(qt[s, hh])) \
                + 2.0 ** -20 * (abs(slope2) * (seq_len + 32) + 1.0)
            delta = np.zeros(seq_len)                     # possible |change| of each p
            weight = np.zeros(seq_len)                    # 2^c of its block
            num = np.zeros(d)
            den = 0.0
            for b0 in range(0, seq_len, bs):
                sl = slice(b0, min(seq_len, b0 + bs))
                zb = z[sl]
                zmax = zb.max()
                c = np.ceil(zmax)
                p_hat = np.exp2(zb - c)
                p = tab[oracle.round_to_e4m3fn(p_hat)]
                lo, hi = _neighbours(p_hat)
                rel = np.log(2.0) * dz[sl] + 2.0 ** -21
                near_mid = np.abs(p_hat - (lo + hi) / 2) <= rel * p_hat
                delta[sl] = np.where(near_mid, hi - lo, 0.0)
                if abs(zmax - np.round(zmax)) <= dz[sl].max():
                    # c may differ by one: normal codes only rescale by 2, small ones re-round
                    delta[sl] = np.maximum(delta[sl], np.where(p_hat < 2.0 ** -5, 2.0 ** -8, 0.0))
                weight[sl] = 2.0 ** c
                num += 2.0 ** c * (p @ v[sl])
                den += 2.0 ** c * p.sum()
            ref = num / den
            moved = weight * delta
            out[s, hh] = (moved @ np.abs(v - ref)) / max(den - moved.sum(), 1e-300)
    return out


def exact_attention_bound(h):
    """(exact [S, H, D], bound [S, H, D]): exact softmax attention of the
    unquantised bf16 queries over the decoded fp8 cache, and a derived bound on
    how far the fp8-arithmetic result (the oracle's) may lie from it.

    Two quantisations separate them:
      * q -> MX fp8 moves each logit by d_t = scale * k_scale * K_t . (q~ - q);
        with |d_t| <= delta, every softmax weight changes by a factor within
        e^(+-2 delta), so the output moves by at most
        max_t |v_t - exact| * (e^(2 delta) - 1);
      * P -> e4m3 (relative 2^-4, or absolute 2^-10 below 2^-6, against
        2^(z - c_b) <= 1 with c_b = ceil(block max z)) moves it by at most
        max_t |v_t - exact~| * E / (sum_t p_t 2^c_b - E), E = sum_t err_t 2^c_b
        (the bound pinned on the CPU in test_oracle_fp8_compute), where exact~
        is exact attention over q~, itself within the first bound of exact.
    """
    q, kc, vc = h["query"], h["key_cache"], h["value_cache"]
    s_count, h_count, d = q.shape
    hkv, bs = kc.shape[1], kc.shape[3]
    group = h_count // hkv
    q64 = oracle.bf16_bits_to_f64(q)
    codes, x_exp = oracle.mx_quantise_e4m3(q64)
    qt = oracle.mx_dequantise(codes, x_exp)
    tab = oracle.e4m3fn_table()
    ks, vsc, scale = float(h["k_scale"]), float(h["v_scale"]), float(h["scale"])
    exact = np.zeros((s_count, h_count, d))
    bound = np.zeros((s_count, h_count, d))
    for s in range(s_count):
        seq_len = int(h["seq_lens"][s])
        if seq_len == 0:
            continue
        k_raw, v_raw = oracle.gather_sequence(kc, vc, h["block_tables"][s], seq_len)
        nb = -(-seq_len // bs)
        for hh in range(h_count):
            kv = hh // group
            k = tab[k_raw[:, kv]] * ks
            v = tab[v_raw[:, kv]] * vsc
            slope = None if h["alibi_slopes"] is None else float(h["alibi_slopes"][hh])
            l_exact = oracle.head_logits(q64[s, hh], k, scale, slope)
            l_q = oracle.head_logits(qt[s, hh], k, scale, slope)
            w = oracle.attention_weights(l_exact)
            ex = w @ v
            exact[s, hh] = ex
            spread = np.max(np.abs(v - ex), axis=0)
            b_q = spread * np.expm1(2.0 * np.max(np.abs(l_q - l_exact)))
            z = l_q / np.log(2.0)
            zp = np.full(nb * bs, -np.inf)
            zp[:seq_len] = z
            c = np.ceil(zp.reshape(nb, bs).max(axis=1))
            cz = np.repeat(c, bs)[:seq_len]
            p_hat = np.exp2(z - cz)
            err = np.maximum(2.0 ** -4 * p_hat, 2.0 ** -10) * np.exp2(cz)
            e_sum = err.sum()
            b_p = (spread + b_q) * e_sum / max(np.sum(p_hat * np.exp2(cz)) - e_sum, 1e-300)
            bound[s, hh] = b_q + b_p
    return exact, bound
