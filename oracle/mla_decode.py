"""Plain fp64 definition of paged MLA (latent-cache) decode (oracle; test infrastructure).

Multi-head latent attention, as the 10100.com article on the retirement of
vLLM's PagedAttention kernels describes it (§2): instead of separate K and V
tensors, every token stores one compressed representation [c_kv, k_rope], and
the PagedAttention kernels have no path that turns it back into K and V.

Readings of points the pages leave open (each also listed in the design notes):
  * The dimensions did not survive extraction. The latent width d_c and the
    rope width d_r are parameters; the workloads take DeepSeek-V2's published
    512 and 64 (the model the article names).
  * Decode runs in the absorbed form: query head h arrives as
    [q_nope_h W_UK_h, q_rope_h] (width d_c + d_r), its logit over token t is
    scale * (q_h . [c_kv_t, k_rope_t]), and its output is the softmax-weighted
    sum of c_kv_t (width d_c). The up-projection W_UV_h and everything after
    it are outside the attention. This equals standard multi-head attention
    over the decompressed K_h = [W_UK_h c_kv, k_rope] and V_h = W_UV_h c_kv
    once the output is multiplied by W_UV_h (pinned by that identity).
  * All query heads read the one latent row (one kv head).
  * The latent cache is paged like the pages' K cache with one kv head:
    [num_blocks, (d_c + d_r)/x, block_size, x]; block-table indexing as in §1.
  * Tail slots t >= L and table entries past ceil(L / bs) are never read;
    seq_len == 0 gives an all-zero output row.
  * Appending latent rows follows the K/V append (kv_append.py): the row of
    new token j of sequence s goes to logical position positions[s] + j,
    stored unchanged (the cache holds the input's bf16 patterns); a negative
    position skips the sequence, and positions past the table or table
    entries outside the pool are not written.
  * An fp8 latent cache follows the pages' scaled fp8 storage (§4) with one
    per-tensor scale for the whole row, since the row is both key and value:
    the stored E4M3FN code times kv_scale stands for the element, and the
    append stores the code nearest to element / kv_scale (quantise_e4m3fn).
    The layout is the same K layout with x = 16.

PINS maps each function to what pins it (tests/test_oracle_mla.py).
"""

from __future__ import annotations

import numpy as np

from .decode_fp64 import bf16_bits_to_f64, decode_cache_values
from .kv_append import quantise_e4m3fn

PINS = {
    "gather_latent": "brute force vs contiguous latent rows scattered element "
                     "by element through a random table; x-invariance",
    "mla_decode": "dense attention with K = [c_kv, k_rope], V = c_kv via torch "
                  "scaled_dot_product_attention (fp64, library routine); the "
                  "decompression identity against the paged MHA oracle and "
                  "SDPA on K_h = [W_UK_h c, k_rope], V_h = W_UV_h c; physical "
                  "permutation invariance (bitwise); seq_len=1; constant c_kv; "
                  "q=0 mean; rope-only logits",
    "append_latent": "read-back through gather_latent returns the new rows at their "
                     "positions and the old rows unchanged; every slot not named by a "
                     "position is bitwise unchanged; brute-force element scatter; "
                     "skip rules; decode after append vs dense SDPA on the grown rows; "
                     "fp8 codes vs torch.float8_e4m3fn conversion of the clamped quotient",
}


def gather_latent(latent_cache: np.ndarray, table_row: np.ndarray, seq_len: int) -> np.ndarray:
    """Logical-order latent rows [seq_len, d_c + d_r] of one sequence, stored form.

    Logical token t lives in physical block table_row[t // bs] at slot t % bs
    (10100.com article, §1). Within a block the row is split into x-element
    chunks: element e of token slot o is latent_cache[b, e // x, o, e % x]
    (the pages' K layout, §2, with one kv head).
    """
    _, dx, bs, x = latent_cache.shape
    width = dx * x
    rows = np.empty((seq_len, width), dtype=latent_cache.dtype)
    for t in range(seq_len):
        phys = int(np.int64(table_row[t // bs]))
        slot = t % bs
        rows[t] = latent_cache[phys, :, slot, :].reshape(width)   # chunk-major: e = c*x + i
    return rows


def mla_decode(query: np.ndarray, latent_cache: np.ndarray, block_tables: np.ndarray,
               seq_lens: np.ndarray, scale: float, latent_dim: int, *,
               q_kind: str, kv_kind: str, kv_scale: float = 1.0) -> np.ndarray:
    """out[s, h, :] = sum_t softmax_t(scale * q[s,h] . row_t) * row_t[:latent_dim].

    query [S, H, d_c + d_r] (stored form ``q_kind``), latent cache
    [num_blocks, (d_c + d_r)/x, bs, x] (stored form ``kv_kind``; for
    "e4m3fn" the rows are the codes' values times ``kv_scale``), block_tables
    int32 [S, max_blocks], seq_lens [S], latent_dim = d_c. Returns float64
    [S, H, d_c].
    """
    s_count, h_count, width = query.shape
    _, dx, _, x = latent_cache.shape
    if dx * x != width:
        raise ValueError("query width differs from the latent row width")
    if not 0 < latent_dim <= width:
        raise ValueError("latent_dim must be in (0, row width]")
    q = decode_cache_values(query, q_kind)
    out = np.zeros((s_count, h_count, latent_dim), dtype=np.float64)
    for s in range(s_count):
        seq_len = int(seq_lens[s])
        if seq_len == 0:
            continue
        rows = decode_cache_values(gather_latent(latent_cache, block_tables[s], seq_len), kv_kind, kv_scale)
        c_kv = rows[:, :latent_dim]
        for h in range(h_count):
            logits = np.float64(scale) * (rows @ q[s, h])
            w = np.exp(logits - np.max(logits))
            w = w / np.sum(w)
            out[s, h] = w @ c_kv
    return out


def append_latent(latent_cache: np.ndarray, rows: np.ndarray, block_tables: np.ndarray,
                  positions: np.ndarray, *, kv_kind: str | None = None,
                  kv_scale: float = 1.0) -> np.ndarray:
    """Copy of latent_cache with the new tokens' latent rows stored.

    rows [S, T, d_c + d_r]; token j of sequence s lands at logical position
    p = positions[s] + j, physical block block_tables[s, p // bs], slot
    p % bs (10100.com article, §1), element e of the row at
    [b, e // x, p % bs, e % x] (the pages' K layout, §2, with one kv head).
    kv_kind None stores the rows as given (the cache's own stored form);
    "e4m3fn" takes bf16 rows (uint16 bit patterns) and stores the uint8 codes
    of element / kv_scale (§4). Skip rules as in the module docstring.
    """
    if kv_kind == "e4m3fn":
        rows = quantise_e4m3fn(bf16_bits_to_f64(rows).astype(np.float32), kv_scale)
    elif kv_kind is not None:
        raise ValueError(f"unknown cache kind {kv_kind!r}")
    cache = latent_cache.copy()
    num_blocks, dx, bs, x = cache.shape
    s_count, t_count, width = rows.shape
    if width != dx * x:
        raise ValueError("rows must be [num_seqs, T, row width of the cache]")
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
            cache[b, :, p % bs, :] = rows[s, j].reshape(dx, x)
    return cache
