"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call.

Fake device addresses (aligned integers) are safe here: every call below fails
validation, or is the num_seqs == 0 no-op, so nothing is dereferenced or launched.
"""

import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


@pytest.fixture(scope="module")
def pa():
    import __graft_entry__
    b = __graft_entry__._build_module()
    if not os.path.exists(b.LIB_PATH):
        b.build()
    import decode_attention_paged_07_amd as mod
    return mod


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("pa_paged_attention_decode", "pa_paged_attention_decode_split", "pa_decode_plan",
                     "pa_workspace_bytes", "pa_kv_layout", "pa_last_error", "pa_version",
                     "pa_timing_enable", "pa_timing_read", "pa_hbm_read_probe",
                     "pa_hbm_gather_probe", "pa_kv_cache_append", "pa_timing_read_append",
                     "pa_pool_create", "pa_pool_destroy", "pa_pool_num_free", "pa_pool_refcount",
                     "pa_pool_append", "pa_pool_fork", "pa_pool_release", "pa_copy_blocks",
                     "pa_mla_decode", "pa_mla_workspace_bytes", "pa_mla_cache_append"):
        assert required in names


def test_library_exports_every_declared_symbol(pa):
    out = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(ctypes.CDLL(pa.LIB_PATH), name)


def test_binding_names_match_c_entry_points(pa):
    for name in declared_functions():
        assert callable(getattr(pa, name)), name


FAKE = dict(out=0x10000, query=0x20000, key_cache=0x30000, value_cache=0x40000, num_seqs=2,
            num_heads=8, num_kv_heads=2, head_size=128, num_blocks=16, scale=0.1,
            block_tables=0x50000, max_blocks_per_seq=4, seq_lens=0x60000, block_size=16,
            max_seq_len=40, alibi_slopes=None, q_dtype=1, kv_cache_dtype=0, k_scale=None,
            v_scale=None, workspace=None, workspace_bytes=0, stream=None)
ORDER = list(FAKE)


def call(pa, **over):
    a = dict(FAKE)
    a.update(over)
    return pa.pa_paged_attention_decode(*[a[k] for k in ORDER])


@pytest.mark.parametrize("over,code", [
    (dict(out=None), -1), (dict(query=None), -1), (dict(key_cache=None), -1),
    (dict(value_cache=None), -1), (dict(block_tables=None), -1), (dict(seq_lens=None), -1),
    (dict(head_size=96), -2), (dict(head_size=256), -2), (dict(head_size=16), -2), (dict(block_size=8), -2),
    (dict(block_size=64), -2), (dict(block_size=32, max_seq_len=129), -2),
    (dict(num_heads=6, num_kv_heads=4), -2), (dict(num_heads=64, num_kv_heads=2), -2),
    (dict(num_kv_heads=0), -2), (dict(num_seqs=-1), -2), (dict(num_blocks=0), -2),
    (dict(max_blocks_per_seq=0), -2), (dict(max_seq_len=65), -2), (dict(max_seq_len=-1), -2),
    (dict(num_seqs=65536, query=1 << 40), -2),
    (dict(scale=float("inf")), -2), (dict(scale=float("nan")), -2),
    (dict(q_dtype=7), -3), (dict(kv_cache_dtype=5), -3), (dict(q_dtype=0, kv_cache_dtype=1), -3), (dict(q_dtype=0, kv_cache_dtype=2), -3),
    (dict(out=0x10008), -5), (dict(query=0x20004), -5), (dict(key_cache=0x30002), -5),
    (dict(block_tables=0x50002), -5), (dict(alibi_slopes=0x70001), -5),
    (dict(out=0x20000 + 64), -2),                                  # overlaps query
    (dict(), -4),                                                  # stream-K needs a workspace
    (dict(workspace=0x80000, workspace_bytes=16), -4),
    (dict(workspace=0x80008, workspace_bytes=64 << 20), -5),
])
def test_validation_rejects(pa, over, code):
    rc = call(pa, **over)
    assert rc == code, (rc, pa.pa_last_error())
    assert pa.pa_last_error() != ""


def test_zero_sequences_is_a_noop(pa):
    assert call(pa, num_seqs=0, out=None, query=None) == 0
    assert pa.pa_last_error() == ""


def test_split_size_must_be_partition_multiple(pa):
    a = dict(FAKE)
    rc = pa.pa_paged_attention_decode_split(*[a[k] for k in ORDER], 300)
    assert rc == -2
    with pytest.raises(ValueError):
        pa.pa_decode_plan(2, 8, 2, 128, 4096, 100)


def test_grid_dimension_limits(pa):
    # num_seqs and the number of splits each become a launch grid dimension
    assert pa.PA_MAX_SEQS == 65535
    assert pa.pa_decode_plan(65535, 8, 2, 128, 4096, 0)[1] == 0
    with pytest.raises(ValueError):
        pa.pa_decode_plan(65536, 8, 2, 128, 4096, 0)
    assert pa.pa_decode_plan(2, 8, 2, 128, 65535 * 256, 256)[1] == 65535
    with pytest.raises(ValueError):
        pa.pa_decode_plan(2, 8, 2, 128, 65535 * 256 + 1, 256)


def test_plan_partition_counts_follow_the_pages(pa):
    from tests import _golden
    for max_len, parts in _golden.partition_counts():
        st, ns, wb = pa.pa_decode_plan(3, 8, 2, 128, max_len, 256)
        assert (st, ns) == (256, parts)
        rows = 3 * 8 * parts
        if parts == 1:
            assert wb == 0
        else:
            def up(v):
                return (v + 255) // 256 * 256
            assert wb == up(rows * 128 * 4) + 2 * up(rows * 4)
        assert pa.pa_workspace_bytes(3, 8, 128, max_len) >= wb


def test_auto_plan_is_streamk_and_fits_workspace_bytes(pa):
    for s, h, hkv, L in [(128, 64, 8, 8192), (8, 32, 8, 32768), (256, 64, 8, 16384), (64, 32, 32, 4096),
                         (2, 4, 4, 40), (1, 16, 1, 1 << 20), (3, 48, 3, 100)]:
        st, ns, wb = pa.pa_decode_plan(s, h, hkv, 128, L)
        assert (st, ns) == (0, 0)                      # stream-K scheduler
        g = h // hkv
        # one slot per (sequence, kv head) plus one per stream-K wave: at most
        # 8 waves per compute unit on 256 compute units (MI355X; also the
        # count assumed where no device can be queried)
        slots = s * hkv + 8 * 256

        def up(v):
            return (v + 255) // 256 * 256
        assert wb == up(slots * g * 128 * 4) + 2 * up(slots * g * 4) + up(s * hkv * 8)
        assert wb <= pa.pa_workspace_bytes(s, h, 128, L)
        for split in (256, 1024):
            assert pa.pa_decode_plan(s, h, hkv, 128, L, split)[2] <= pa.pa_workspace_bytes(s, h, 128, L)


def test_kv_layout_matches_generator(pa):
    import workloads
    for name in ("tiny", "mha", "gqa", "long", "fp8"):
        cfg = workloads.CONFIGS[name]
        q = 0 if cfg.q_dtype == "f32" else 1
        kv = 1 if cfg.kv_dtype == "fp8_e4m3" else 0
        lay = pa.pa_kv_layout(cfg.num_kv_heads, cfg.head_size, 16, q, kv)
        assert lay["x"] == workloads.default_x(cfg)
        assert lay["k_head_stride"] == cfg.head_size * 16
        assert lay["k_block_stride"] == cfg.head_size * 16 * cfg.num_kv_heads
        k_shape, v_shape = pa.kv_cache_shapes(cfg.pool_blocks, cfg.num_kv_heads, cfg.head_size,
                                              torch.float32 if q == 0 else torch.bfloat16, cfg.kv_dtype)
        c = workloads.make_case(cfg.with_(pool_blocks=16, num_seqs=1, seq_lens=("fixed", (5,))))
        assert k_shape[1:] == tuple(c.key_cache.shape[1:])
        assert v_shape[1:] == tuple(c.value_cache.shape[1:])
        lay32 = pa.pa_kv_layout(cfg.num_kv_heads, cfg.head_size, 32, q, kv)
        assert lay32["k_head_stride"] == cfg.head_size * 32 and lay32["x"] == lay["x"]
        c32 = workloads.make_case(cfg.with_(pool_blocks=8, num_seqs=1, seq_lens=("fixed", (5,)), block_size=32))
        k32, v32 = pa.kv_cache_shapes(8, cfg.num_kv_heads, cfg.head_size,
                                      torch.float32 if q == 0 else torch.bfloat16, cfg.kv_dtype, 32)
        assert k32 == tuple(c32.key_cache.shape) and v32 == tuple(c32.value_cache.shape)


def test_tensor_call_refuses_cpu_tensors(pa):
    """No CPU fallback: host tensors are rejected before anything runs."""
    import workloads
    c = workloads.make_case(workloads.TINY)
    out = torch.empty_like(c.query)
    with pytest.raises(ValueError, match="GPU"):
        pa.paged_attention_decode(out, c.query, c.key_cache, c.value_cache, 4, c.scale,
                                  c.block_tables, c.seq_lens, 16, c.max_seq_len)


def test_tensor_call_rejects_bad_kv_dtype_name(pa):
    import workloads
    c = workloads.make_case(workloads.TINY)
    with pytest.raises(TypeError):
        pa.paged_attention_decode(torch.empty_like(c.query), c.query, c.key_cache, c.value_cache, 4,
                                  c.scale, c.block_tables, c.seq_lens, 16, c.max_seq_len,
                                  kv_cache_dtype="int8")


@pytest.mark.parametrize("args,code", [
    ((None, 1 << 20, 1024, 0x1000, None), -1), ((0x10000, 1 << 20, 1024, None, None), -1),
    ((0x10000, 0, 1024, 0x1000, None), -2), ((0x10000, 100, 1024, 0x1000, None), -2),
    ((0x10000, 1 << 20, 0, 0x1000, None), -2), ((0x10000, 1 << 20, (1 << 20) + 1, 0x1000, None), -2),
    ((0x10008, 1 << 20, 1024, 0x1000, None), -5), ((0x10000, 1 << 20, 1024, 0x1002, None), -5),
])
def test_read_probe_validation(pa, args, code):
    assert pa.pa_hbm_read_probe(*args) == code
    assert pa.pa_last_error() != ""


@pytest.mark.parametrize("over,code", [
    (dict(pool=None), -1), (dict(ids=None), -1), (dict(sink=None), -1), (dict(tile_bytes=3000), -2),
    (dict(pool_bytes=1000), -2), (dict(num_tiles=0), -2), (dict(depth=3), -2), (dict(workgroups=0), -2),
    (dict(pool=0x10008), -5), (dict(ids=0x20002), -5),
])
def test_gather_probe_validation(pa, over, code):
    a = dict(pool=0x10000, pool_bytes=1 << 20, tile_bytes=4096, ids=0x20000, num_tiles=16, depth=1,
             workgroups=64, sink=0x30000, stream=None)
    a.update(over)
    assert pa.pa_hbm_gather_probe(*a.values()) == code
    assert pa.pa_last_error() != ""


APPEND = dict(key_cache=0x10000, value_cache=0x20000, key=0x30000, value=0x40000, num_seqs=2,
              tokens_per_seq=1, num_kv_heads=2, head_size=128, num_blocks=16, block_tables=0x50000,
              max_blocks_per_seq=4, positions=0x60000, block_size=16, in_dtype=1, kv_cache_dtype=0,
              k_scale=None, v_scale=None, stream=None)


@pytest.mark.parametrize("over,code", [
    (dict(key_cache=None), -1), (dict(value=None), -1), (dict(positions=None), -1),
    (dict(block_tables=None), -1), (dict(head_size=96), -2), (dict(block_size=8), -2),
    (dict(block_size=64), -2), (dict(block_size=24), -2),
    (dict(tokens_per_seq=0), -2), (dict(num_kv_heads=0), -2), (dict(num_blocks=0), -2),
    (dict(max_blocks_per_seq=0), -2), (dict(num_seqs=-1), -2),
    (dict(num_seqs=1 << 20, tokens_per_seq=1 << 10, num_kv_heads=8), -2),
    (dict(in_dtype=5), -3), (dict(kv_cache_dtype=3), -3),
    (dict(key=0x30008), -5), (dict(value_cache=0x20004), -5), (dict(positions=0x60002), -5),
])
def test_append_validation_rejects(pa, over, code):
    a = dict(APPEND)
    a.update(over)
    assert pa.pa_kv_cache_append(*a.values()) == code, pa.pa_last_error()
    assert pa.pa_last_error() != ""


def test_append_zero_sequences_is_a_noop(pa):
    a = dict(APPEND, num_seqs=0, key=None, value=None)
    assert pa.pa_kv_cache_append(*a.values()) == 0


def test_tensor_append_refuses_cpu_tensors(pa):
    kc = torch.zeros((4, 2, 16, 16, 8), dtype=torch.bfloat16)
    vc = torch.zeros((4, 2, 128, 16), dtype=torch.bfloat16)
    k = torch.zeros((1, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        pa.kv_cache_append(kc, vc, k, k.clone(), torch.zeros((1, 4), dtype=torch.int32),
                           torch.zeros(1, dtype=torch.int32))


def test_timing_read_without_launches(pa):
    pa.pa_timing_enable(True)
    assert pa.pa_timing_read() == (0.0, 0, 0.0, 0)
    assert pa.pa_timing_read_append() == (0.0, 0)
    pa.pa_timing_enable(False)
