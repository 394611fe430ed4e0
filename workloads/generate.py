"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention arithmetic: it draws sequence lengths, scatters
each sequence's logical blocks over a physical pool through a table, fills the
pool with N(0,1) values in the pages' cache layouts, and (for the fp8 cache)
quantises them to OCP E4M3FN codes with one per-tensor scale.

Recipe (stated in full so both sides can be regenerated anywhere):
  * metadata from numpy.random.default_rng(seed), in this order:
      1. sequence lengths: "uniform" -> rng.integers(lo, hi + 1, S);
         "lognormal" -> rint(rng.lognormal(ln(median), sigma, S)) clipped to
         [1, cap]; "const"/"fixed" draw nothing; with prefix groups
         (group_size, prefix_tokens) every length gets prefix_tokens added;
      2. pool = rng.permutation(pool_blocks); sequence s takes the next
         ceil(L_s / block_size) entries, in sequence order;
      3. table entries past a sequence's last block hold ``pad_id``; with
         prefix groups, members after a group's first sequence take that
         sequence's first prefix_tokens / block_size entries instead of
         drawing their own.
  * values from torch.Generator(device).manual_seed(seed), in this order:
    query, K pool, V pool, each torch.randn in float32, then cast with
    round-to-nearest-even to bfloat16 when the dtype is bf16. For the fp8
    cache: s = max(|K|.max(), |V|.max()) / 448, codes =
    clamp(x / s, -448, 448) cast to float8_e4m3fn (round-to-nearest-even),
    k_scale = v_scale = s.
  * K pool layout [num_blocks, num_kv_heads, head_size/x, block_size, x] and
    V pool layout [num_blocks, num_kv_heads, head_size, block_size], with
    x = 16 bytes / element size (10100.com article, §2, for the layouts).
  * ALiBi slopes 2^(-8 (i+1) / H) for query head i (the long-context
    workload's slopes with H = 32); scale = 1/sqrt(head_size).
  * latent-cache (MLA) workloads (make_mla_case): the same metadata draw;
    values query [S, H, 576] then the latent pool [num_blocks, 72, bs, 8],
    each torch.randn in float32 cast to bf16; scale = 1/sqrt(128 + 64) (the
    query-key width of DeepSeek-V2 heads before absorption: 128 without
    position, 64 with).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from .configs import DecodeConfig

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}
FP8_NAN_CODE = 0x7F


def kv_elem(cfg: DecodeConfig) -> str:
    return cfg.q_dtype if cfg.kv_dtype == "auto" else cfg.kv_dtype


def default_x(cfg: DecodeConfig) -> int:
    return 16 // ELEM_BYTES[kv_elem(cfg)]


def alibi_slopes(num_heads: int) -> np.ndarray:
    return np.array([2.0 ** (-8.0 * (i + 1) / num_heads) for i in range(num_heads)],
                    dtype=np.float32)


def draw_seq_lens(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    kind = cfg.seq_lens[0]
    if kind == "fixed":
        lens = np.array(cfg.seq_lens[1], dtype=np.int64)
        if lens.shape != (cfg.num_seqs,):
            raise ValueError("fixed seq_lens must list one length per sequence")
        return lens
    if kind == "const":
        return np.full(cfg.num_seqs, cfg.seq_lens[1], dtype=np.int64)
    if kind == "uniform":
        lo, hi = cfg.seq_lens[1], cfg.seq_lens[2]
        return rng.integers(lo, hi + 1, cfg.num_seqs).astype(np.int64)
    if kind == "lognormal":
        median, sigma, cap = cfg.seq_lens[1:]
        raw = rng.lognormal(math.log(median), sigma, cfg.num_seqs)
        return np.clip(np.rint(raw), 1, cap).astype(np.int64)
    raise ValueError(f"unknown seq_len recipe {kind!r}")


@dataclass
class Metadata:
    seq_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray      # int32 [S, max_blocks]
    max_seq_len: int
    used_blocks: np.ndarray       # int64, physical ids referenced by valid tokens
    pad_id: int


def make_metadata(cfg: DecodeConfig, seed: int | None = None, *,
                  seq_lens=None, pad_id: int = 0, max_seq_len: int | None = None,
                  share_prefix_blocks: int = 0) -> Metadata:
    """Sequence lengths and a scattered block table.

    ``seq_lens`` overrides the recipe (no length draw then). ``max_seq_len``
    may exceed the longest sequence (table width follows it).
    ``share_prefix_blocks`` > 0 makes every sequence long enough reuse the
    first physical blocks of sequence 0 (read-only sharing).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    if seq_lens is None:
        lens = draw_seq_lens(cfg, rng)
    else:
        lens = np.asarray(seq_lens, dtype=np.int64)
        if lens.shape != (cfg.num_seqs,):
            raise ValueError("seq_lens must have num_seqs entries")
    group_size, prefix_tokens = cfg.prefix_groups if cfg.prefix_groups else (1, 0)
    if prefix_tokens % cfg.block_size:
        raise ValueError("a shared prefix must be whole blocks")
    if prefix_tokens and seq_lens is None:
        lens = lens + prefix_tokens
    longest = int(lens.max()) if lens.size else 0
    msl = longest if max_seq_len is None else int(max_seq_len)
    if msl < longest:
        raise ValueError("max_seq_len below the longest sequence")
    bs = cfg.block_size
    max_blocks = max(1, -(-msl // bs))
    need = [-(-int(n) // bs) for n in lens]
    perm = rng.permutation(cfg.pool_blocks).astype(np.int64)
    table = np.full((cfg.num_seqs, max_blocks), pad_id, dtype=np.int64)
    pos = 0
    prefix_blocks = prefix_tokens // bs
    for s in range(cfg.num_seqs):
        nb = need[s]
        shared = min(share_prefix_blocks, nb, need[0]) if s > 0 else 0
        if s % group_size and prefix_blocks:                 # a later member of a prompt group
            shared = min(prefix_blocks, nb)
            table[s, :shared] = table[s - s % group_size, :shared]
        elif shared:
            table[s, :shared] = table[0, :shared]
        own = nb - shared
        if pos + own > cfg.pool_blocks:
            raise ValueError(f"{cfg.name}: pool of {cfg.pool_blocks} blocks too small")
        table[s, shared:nb] = perm[pos:pos + own]
        pos += own
    used = np.unique(np.concatenate([table[s, :need[s]] for s in range(cfg.num_seqs)]
                                    + [np.zeros(0, np.int64)]))
    return Metadata(lens.astype(np.int32), table.astype(np.int32), msl, used, pad_id)


@dataclass
class Case:
    cfg: DecodeConfig
    meta: Metadata
    x: int
    query: torch.Tensor           # [S, H, D] f32 | bf16
    key_cache: torch.Tensor       # [NB, Hkv, D/x, bs, x] f32 | bf16 | uint8 (e4m3fn codes)
    value_cache: torch.Tensor     # [NB, Hkv, D, bs]
    block_tables: torch.Tensor    # int32 [S, max_blocks]
    seq_lens: torch.Tensor        # int32 [S]
    alibi_slopes: torch.Tensor | None
    scale: float
    k_scale: float
    v_scale: float
    extra: dict = field(default_factory=dict)

    @property
    def max_seq_len(self) -> int:
        return self.meta.max_seq_len

    @property
    def kv_cache_dtype(self) -> str:
        return self.cfg.kv_dtype


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _fill_pool(shape, dtype, gen, device, chunk_rows=4096):
    """N(0,1) pool of ``shape`` in ``dtype``, drawn in row chunks to bound the
    float32 temporary."""
    out = torch.empty(shape, dtype=dtype, device=device)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = _randn((r1 - r0,) + tuple(shape[1:]), gen, device).to(dtype)
    return out


def make_case(cfg: DecodeConfig, seed: int | None = None, device="cpu", *,
              seq_lens=None, max_seq_len=None, poison: bool = False,
              share_prefix_blocks: int = 0, x: int | None = None,
              k_scale: float | None = None, v_scale: float | None = None,
              pad_id: int | None = None) -> Case:
    """Build one workload instance on ``device``.

    poison=True writes NaN into every pool slot that no valid token uses: the
    tail slots of each sequence's last block, every unused block, and points
    every unused table entry at one NaN block.
    k_scale / v_scale override the fp8 amax-derived scales (codes unchanged).
    """
    seed = cfg.seed if seed is None else seed
    elem = kv_elem(cfg)
    x = default_x(cfg) if x is None else x
    d, hkv, bs, nb = cfg.head_size, cfg.num_kv_heads, cfg.block_size, cfg.pool_blocks
    if d % x:
        raise ValueError("x must divide head_size")
    meta = make_metadata(cfg, seed, seq_lens=seq_lens, max_seq_len=max_seq_len,
                         share_prefix_blocks=share_prefix_blocks,
                         pad_id=0 if pad_id is None else pad_id)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q_dtype = TORCH_DTYPE[cfg.q_dtype]
    query = _randn((cfg.num_seqs, cfg.num_heads, d), gen, device).to(q_dtype)
    k_shape = (nb, hkv, d // x, bs, x)
    v_shape = (nb, hkv, d, bs)
    ks = vs = 1.0
    if elem == "fp8_e4m3":
        k32 = _fill_pool(k_shape, torch.float32, gen, device)
        v32 = _fill_pool(v_shape, torch.float32, gen, device)
        amax = max(float(k32.abs().max()), float(v32.abs().max()))
        s = amax / 448.0
        key_cache = _quantise_e4m3(k32, s)
        del k32
        value_cache = _quantise_e4m3(v32, s)
        del v32
        ks = vs = s
    else:
        key_cache = _fill_pool(k_shape, TORCH_DTYPE[elem], gen, device)
        value_cache = _fill_pool(v_shape, TORCH_DTYPE[elem], gen, device)
    if k_scale is not None:
        ks = float(k_scale)
    if v_scale is not None:
        vs = float(v_scale)

    table = meta.block_tables.copy()
    if poison:
        _poison(cfg, meta, table, key_cache, value_cache, elem)
    slopes = None
    if cfg.alibi:
        slopes = torch.from_numpy(alibi_slopes(cfg.num_heads)).to(device)
    return Case(cfg=cfg, meta=meta, x=x, query=query, key_cache=key_cache,
                value_cache=value_cache,
                block_tables=torch.from_numpy(table).to(device),
                seq_lens=torch.from_numpy(meta.seq_lens).to(device),
                alibi_slopes=slopes, scale=1.0 / math.sqrt(d), k_scale=ks, v_scale=vs)


def _quantise_e4m3(vals: torch.Tensor, s: float) -> torch.Tensor:
    return (vals / s).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def _nan_fill(t: torch.Tensor, elem: str):
    if elem == "fp8_e4m3":
        t.fill_(FP8_NAN_CODE)
    else:
        t.fill_(float("nan"))


def _poison(cfg, meta, table, key_cache, value_cache, elem):
    bs = cfg.block_size
    used = np.zeros(cfg.pool_blocks, dtype=bool)
    used[meta.used_blocks] = True
    unused = np.flatnonzero(~used)
    if unused.size == 0:
        raise ValueError("poison needs at least one unused pool block")
    idx = torch.from_numpy(unused).to(key_cache.device)
    fill = FP8_NAN_CODE if elem == "fp8_e4m3" else float("nan")
    key_cache.index_fill_(0, idx, fill)
    value_cache.index_fill_(0, idx, fill)
    nan_block = int(unused[0])
    for s in range(cfg.num_seqs):
        n = int(meta.seq_lens[s])
        nblk = -(-n // bs)
        table[s, nblk:] = nan_block
        tail = n % bs
        if nblk and tail:
            last = int(table[s, nblk - 1])
            _nan_fill(key_cache[last, :, :, tail:, :], elem)
            _nan_fill(value_cache[last, :, :, tail:], elem)


# ---------------------------------------------------------------------------
# Host copies for the oracle side (pure relabelling of physical blocks).
# ---------------------------------------------------------------------------

def host_arrays(case: Case, seqs=None) -> dict:
    """numpy inputs for the oracle, restricted to sequences ``seqs``.

    Only the physical blocks those sequences reference are copied; they are
    renumbered 0..n-1 in ascending physical order and the table rows are
    rewritten to match. bf16 tensors are returned as uint16 bit patterns and
    fp8 caches as uint8 codes.
    """
    cfg = case.cfg
    seqs = list(range(cfg.num_seqs)) if seqs is None else list(seqs)
    lens = case.meta.seq_lens[seqs].astype(np.int64)
    table = case.block_tables.cpu().numpy()[seqs].astype(np.int64)
    bs = cfg.block_size
    nblk = [-(-int(n) // bs) for n in lens]
    ids = np.unique(np.concatenate([table[i, :nblk[i]] for i in range(len(seqs))]
                                   + [np.zeros(0, np.int64)]))
    if ids.size == 0:
        ids = np.zeros(1, np.int64)
    remap = {int(b): i for i, b in enumerate(ids.tolist())}
    new_table = np.zeros_like(table)
    for i in range(len(seqs)):
        for j in range(nblk[i]):
            new_table[i, j] = remap[int(table[i, j])]
    idx = torch.from_numpy(ids).to(case.key_cache.device)
    kc = case.key_cache.index_select(0, idx).cpu()
    vc = case.value_cache.index_select(0, idx).cpu()
    q = case.query.cpu()[seqs]
    return {
        "query": _to_np(q),
        "key_cache": _to_np(kc),
        "value_cache": _to_np(vc),
        "block_tables": new_table.astype(np.int32),
        "seq_lens": lens.astype(np.int32),
        "alibi_slopes": None if case.alibi_slopes is None else case.alibi_slopes.cpu().numpy(),
        "scale": case.scale,
        "q_kind": case.cfg.q_dtype,
        "kv_kind": {"f32": "f32", "bf16": "bf16", "fp8_e4m3": "e4m3fn"}[kv_elem(cfg)],
        "k_scale": case.k_scale if kv_elem(cfg) == "fp8_e4m3" else 1.0,
        "v_scale": case.v_scale if kv_elem(cfg) == "fp8_e4m3" else 1.0,
    }


def _to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


# ---------------------------------------------------------------------------
# Latent-cache (MLA) workloads.
# ---------------------------------------------------------------------------

MLA_LATENT, MLA_ROPE = 512, 64


@dataclass
class MlaCase:
    cfg: DecodeConfig
    meta: Metadata
    query: torch.Tensor           # bf16 [S, H, 576]
    latent_cache: torch.Tensor    # bf16 [NB, 72, bs, 8], or uint8 e4m3fn codes [NB, 36, bs, 16]
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    scale: float
    kv_scale: float = 1.0         # fp8 cache: value = code * kv_scale

    @property
    def max_seq_len(self) -> int:
        return self.meta.max_seq_len


def make_mla_case(cfg: DecodeConfig, seed: int | None = None, device="cpu", *, seq_lens=None,
                  max_seq_len=None, poison: bool = False, num_heads: int | None = None,
                  share_prefix_blocks: int = 0) -> MlaCase:
    """One MLA workload instance; poison=True writes NaN into every pool slot
    no valid token uses and points unused table entries at a NaN block.
    share_prefix_blocks > 0 maps the first blocks of every long enough
    sequence to sequence 0's physical blocks (read-only sharing). With
    cfg.kv_dtype "fp8_e4m3" the N(0,1) rows are stored as e4m3fn codes of
    value / s, s = amax / 448 over the pool (the fp8 workloads' recipe)."""
    seed = cfg.seed if seed is None else seed
    if num_heads is not None:
        cfg = cfg.with_(num_heads=num_heads)
    width = MLA_LATENT + MLA_ROPE
    meta = make_metadata(cfg, seed, seq_lens=seq_lens, max_seq_len=max_seq_len,
                         share_prefix_blocks=share_prefix_blocks)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    query = _randn((cfg.num_seqs, cfg.num_heads, width), gen, device).to(torch.bfloat16)
    fp8 = cfg.kv_dtype == "fp8_e4m3"
    kv_scale = 1.0
    if fp8:
        pool = _fill_pool((cfg.pool_blocks, width // 16, cfg.block_size, 16), torch.float32, gen, device)
        kv_scale = float(pool.abs().max()) / 448.0
        pool = _quantise_e4m3(pool, kv_scale)
    else:
        pool = _fill_pool((cfg.pool_blocks, width // 8, cfg.block_size, 8), torch.bfloat16, gen, device)
    nan = FP8_NAN_CODE if fp8 else float("nan")
    table = meta.block_tables.copy()
    if poison:
        used = np.zeros(cfg.pool_blocks, dtype=bool)
        used[meta.used_blocks] = True
        unused = np.flatnonzero(~used)
        if unused.size == 0:
            raise ValueError("poison needs at least one unused pool block")
        pool.index_fill_(0, torch.from_numpy(unused).to(pool.device), nan)
        bs = cfg.block_size
        for s in range(cfg.num_seqs):
            n = int(meta.seq_lens[s])
            nblk = -(-n // bs)
            table[s, nblk:] = int(unused[0])
            if nblk and n % bs:
                pool[int(table[s, nblk - 1]), :, n % bs:, :] = nan
    return MlaCase(cfg=cfg, meta=meta, query=query, latent_cache=pool,
                   block_tables=torch.from_numpy(table).to(device),
                   seq_lens=torch.from_numpy(meta.seq_lens).to(device),
                   scale=1.0 / math.sqrt(128 + 64), kv_scale=kv_scale)


def mla_host_arrays(case: MlaCase, seqs=None) -> dict:
    """numpy inputs for the MLA oracle, restricted to ``seqs``; the referenced
    physical blocks are copied and renumbered in ascending order (bf16 as
    uint16 bit patterns)."""
    cfg = case.cfg
    seqs = list(range(cfg.num_seqs)) if seqs is None else list(seqs)
    lens = case.meta.seq_lens[seqs].astype(np.int64)
    table = case.block_tables.cpu().numpy()[seqs].astype(np.int64)
    bs = cfg.block_size
    nblk = [-(-int(n) // bs) for n in lens]
    ids = np.unique(np.concatenate([table[i, :nblk[i]] for i in range(len(seqs))] + [np.zeros(0, np.int64)]))
    if ids.size == 0:
        ids = np.zeros(1, np.int64)
    remap = {int(b): i for i, b in enumerate(ids.tolist())}
    new_table = np.zeros_like(table)
    for i in range(len(seqs)):
        for j in range(nblk[i]):
            new_table[i, j] = remap[int(table[i, j])]
    pool = case.latent_cache.index_select(0, torch.from_numpy(ids).to(case.latent_cache.device)).cpu()
    return {
        "query": _to_np(case.query.cpu()[seqs]),
        "latent_cache": _to_np(pool),
        "block_tables": new_table.astype(np.int32),
        "seq_lens": lens.astype(np.int32),
        "scale": case.scale,
        "kv_kind": "e4m3fn" if case.cfg.kv_dtype == "fp8_e4m3" else "bf16",
        "kv_scale": case.kv_scale,
    }
