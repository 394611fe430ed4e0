"""The five decode workloads, as plain data.

Shapes follow the pages' workloads: head sizes 64/128 and 256-token partitions
(PR #47361 report, test and benchmark snippets), a pool of 128*1024 physical
blocks (same benchmark), block_size 16, and physical blocks scattered through a
per-sequence table (10100.com article, §1).

Readings where the workload text is silent:
  * lognormal lengths: sigma = 1.0 in natural-log units around ln(4096),
    rounded to the nearest integer, clipped to [1, 16384];
  * the long-context pool is 131072 blocks, like the other large configs;
  * one amax over all generated K and V values gives k_scale = v_scale =
    amax / 448 for the fp8 cache.
"""

from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    pool_blocks: int
    q_dtype: str          # "f32" or "bf16"; out has the same dtype
    kv_dtype: str         # "auto" (= q dtype) or "fp8_e4m3"
    seq_lens: tuple       # recipe: ("fixed", (..)), ("const", n), ("uniform", lo, hi),
                          #         ("lognormal", median, sigma, cap)
    alibi: bool
    seed: int
    # (group_size, prefix_tokens): consecutive sequences in groups of
    # group_size share the physical blocks of a prefix_tokens-token prompt
    # (a multiple of block_size); their lengths are prefix_tokens plus the
    # drawn length. None: no sharing.
    prefix_groups: tuple | None = None
    # "auto": the cache type's arithmetic; "fp8": fp8 arithmetic on an fp8
    # cache (MX-quantised q, e4m3 P).
    compute: str = "auto"

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


TINY = DecodeConfig("tiny", 2, 4, 4, 64, 16, 16, "f32", "auto",
                    ("fixed", (17, 40)), False, 0)
MHA = DecodeConfig("mha", 64, 32, 32, 128, 16, 32768, "bf16", "auto",
                   ("const", 4096), False, 1)
GQA = DecodeConfig("gqa", 128, 64, 8, 128, 16, 128 * 1024, "bf16", "auto",
                   ("uniform", 1, 8192), False, 2)
LONG = DecodeConfig("long", 8, 32, 8, 128, 16, 128 * 1024, "bf16", "auto",
                    ("const", 32768), True, 3)
FP8 = DecodeConfig("fp8", 256, 64, 8, 128, 16, 128 * 1024, "bf16", "fp8_e4m3",
                   ("lognormal", 4096, 1.0, 16384), False, 4)

# Shared-prompt decode (not one of the five reference workloads): parallel
# sampling with n = 8 over 16 prompts of 4096 tokens, each sample with its
# own U[1, 512] generated tokens; otherwise the GQA workload's shapes.
SHARED = DecodeConfig("shared", 128, 64, 8, 128, 16, 128 * 1024, "bf16", "auto",
                      ("uniform", 1, 512), False, 5, prefix_groups=(8, 4096))

# The GQA workload with 32-token blocks: same lengths (same seed), same pool
# capacity in tokens.
GQA32 = GQA.with_(name="gqa32", block_size=32, pool_blocks=64 * 1024)

# The fp8 workload with fp8 arithmetic (same inputs, same seed).
FP8C = FP8.with_(name="fp8c", compute="fp8")

CONFIGS = {c.name: c for c in (TINY, MHA, GQA, LONG, FP8)}
EXTRA_CONFIGS = {c.name: c for c in (SHARED, GQA32, FP8C)}

# Latent-cache (MLA) decode, not one of the five reference workloads: rows of
# [c_kv (512), k_rope (64)] in bf16, one latent head, 16-token blocks, lengths
# and pool as in the GQA workload. "mla" is one GPU's share of a 128-head
# model whose heads are split over 8 GPUs (16 query heads); "mla128" keeps all
# 128 heads on one GPU. head_size holds the row width.
MLA = DecodeConfig("mla", 256, 16, 1, 576, 16, 128 * 1024, "bf16", "auto",
                   ("uniform", 1, 8192), False, 6)
MLA128 = MLA.with_(name="mla128", num_heads=128, seed=7)
# The same with the latent rows stored as fp8 e4m3 codes and one scale.
MLA_FP8 = MLA.with_(name="mla_fp8", kv_dtype="fp8_e4m3", seed=8)
MLA128_FP8 = MLA128.with_(name="mla128_fp8", kv_dtype="fp8_e4m3", seed=9)
# 32-token cache blocks (the same 2.4 GB pool in half as many blocks).
MLA_BS32 = MLA.with_(name="mla_bs32", block_size=32, pool_blocks=64 * 1024)
MLA128_BS32 = MLA128.with_(name="mla128_bs32", block_size=32, pool_blocks=64 * 1024)
MLA_CONFIGS = {c.name: c for c in (MLA, MLA128, MLA_FP8, MLA128_FP8, MLA_BS32, MLA128_BS32)}
