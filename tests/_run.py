"""Helpers shared by GPU tests, smoke() and bench.py: run the HIP path on a
workload Case, run the oracle on the same inputs, compare element-wise."""

from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 1e-2)}   # (atol, rtol) by output dtype


def run_hip(case, split_tokens=0, workspace=None, out=None, compute="auto"):
    import decode_attention_paged_07_amd as pa
    if out is None:
        out = torch.empty_like(case.query)
    pa.paged_attention_decode(
        out, case.query, case.key_cache, case.value_cache, case.cfg.num_kv_heads, case.scale,
        case.block_tables, case.seq_lens, case.cfg.block_size, case.max_seq_len,
        alibi_slopes=case.alibi_slopes, kv_cache_dtype=case.cfg.kv_dtype,
        k_scale=case.k_scale, v_scale=case.v_scale, workspace=workspace,
        split_tokens=split_tokens, compute=compute)
    return out


def run_oracle_fp8(case, seqs=None):
    """The fp8-arithmetic oracle on the same inputs (fp8 cache, bf16 q)."""
    import oracle
    import workloads
    h = workloads.host_arrays(case, seqs)
    return oracle.paged_decode_fp8_compute(h["query"], h["key_cache"], h["value_cache"], h["block_tables"],
                                           h["seq_lens"], h["scale"], k_scale=h["k_scale"],
                                           v_scale=h["v_scale"], alibi_slopes=h["alibi_slopes"])


def run_oracle(case, seqs=None):
    import oracle
    import workloads
    h = workloads.host_arrays(case, seqs)
    return oracle.paged_decode(h["query"], h["key_cache"], h["value_cache"], h["block_tables"],
                               h["seq_lens"], h["scale"], q_kind=h["q_kind"], kv_kind=h["kv_kind"],
                               alibi_slopes=h["alibi_slopes"], k_scale=h["k_scale"],
                               v_scale=h["v_scale"])


def compare(gpu: torch.Tensor, ref: np.ndarray, dtype: str, seqs=None, what="", extra=None):
    """Element-wise |gpu - ref| <= atol + rtol*|ref| (+ extra, an element-wise
    allowance); returns (max_abs, max_rel)."""
    atol, rtol = TOL[dtype]
    g = gpu.float().cpu().numpy().astype(np.float64)
    if seqs is not None:
        g = g[list(seqs)]
    assert g.shape == ref.shape, (g.shape, ref.shape)
    err = np.abs(g - ref)
    bound = atol + rtol * np.abs(ref)
    if extra is not None:
        bound = bound + extra
    bad = ~(err <= bound)             # NaN counts as a failure
    max_abs = float(np.nanmax(err)) if err.size else 0.0
    sig = np.abs(ref) > 1e-3
    max_rel = float(np.nanmax(err[sig] / np.abs(ref[sig]))) if sig.any() else 0.0
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside "
                             f"atol={atol} rtol={rtol}; max_abs={max_abs:.3e} max_rel={max_rel:.3e}; "
                             f"first bad (s,h,d) {idx}: gpu {[g[tuple(i)] for i in idx]} "
                             f"ref {[ref[tuple(i)] for i in idx]}")
    return max_abs, max_rel
