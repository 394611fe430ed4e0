"""fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP library and imports nothing from it.

Sources (cited by page title and section):
  * "PR #47361 完整报告" (prhub.com.cn report on vLLM PR #47361, "Delete
    PagedAttention"), section "关键源码片段": the benchmark and test snippets
    give the call signature, the 256-token partitions and the workspace shapes.
  * The 10100.com article on why vLLM retired its CUDA PagedAttention kernels:
    §1 (block-table indexing), §2 (K/V cache layouts), §3 (two traversals vs a
    fused single traversal), §4 (fp8 e4m3 storage dequantised with a per-tensor
    scale).
  * "vLLM 0.25.0 解读：PagedAttention 退场，MRv2 接管", §1 (logical blocks mapped
    to non-contiguous physical blocks through a per-sequence table; shared
    blocks).

Parity status of each function is listed in ``decode_fp64.PINS``,
``kv_append.PINS``, ``decode_fp8_compute.PINS`` and ``mla_decode.PINS``.
"""

from .decode_fp64 import (  # noqa: F401
    E4M3FN_MAX,
    PINS,
    attention_weights,
    bf16_bits_to_f64,
    decode_cache_values,
    e4m3fn_table,
    gather_sequence,
    head_logits,
    merge_partitions,
    paged_decode,
    paged_decode_partitioned,
)
from .kv_append import PINS as APPEND_PINS  # noqa: F401,E402
from .kv_append import append_tokens, quantise_e4m3fn  # noqa: F401,E402
from .decode_fp8_compute import PINS as FP8_COMPUTE_PINS  # noqa: F401,E402
from .decode_fp8_compute import (  # noqa: F401,E402
    mx_dequantise,
    mx_quantise_e4m3,
    paged_decode_fp8_compute,
    round_to_e4m3fn,
)
from .mla_decode import PINS as MLA_PINS  # noqa: F401,E402
from .mla_decode import append_latent, gather_latent, mla_decode  # noqa: F401,E402
