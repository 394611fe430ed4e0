"""Seeded synthetic decode workloads (no attention arithmetic lives here)."""

from .configs import CONFIGS, EXTRA_CONFIGS, FP8, FP8C, GQA, GQA32, LONG, MHA, SHARED, TINY, DecodeConfig  # noqa: F401
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
)
