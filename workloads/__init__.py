"""Seeded synthetic decode workloads (no attention arithmetic lives here)."""

from .configs import (  # noqa: F401
    CONFIGS, EXTRA_CONFIGS, FP8, FP8C, GQA, GQA32, LONG, MHA, MLA, MLA128, MLA128_BS32, MLA128_FP8, MLA_BS32, MLA_CONFIGS, MLA_FP8, SHARED, TINY, DecodeConfig,
)
from .generate import (  # noqa: F401
    Case,
    Metadata,
    alibi_slopes,
    default_x,
    draw_seq_lens,
    host_arrays,
    kv_elem,
    make_case,
    make_metadata,
    MlaCase,
    make_mla_case,
    mla_host_arrays,
)
