"""Paged decode attention for AMD MI355X (gfx950): Python binding.

A thin ctypes layer over ``libpa_decode.so`` (C ABI declared in
``include/pa_decode.h``). The ``pa_*`` functions mirror the C entry points one
to one (plain integers and device addresses); ``paged_attention_decode`` takes
torch tensors and only marshals their metadata, device addresses and the
current HIP stream. Every step of the computation runs in the library's
kernels; there is no fallback path. Importing this package fails with
ImportError when the library has not been built.

The call follows the ROCm decode call kept in the PR #47361 report
(prhub.com.cn, "关键源码片段"): out, query, key_cache, value_cache,
num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
alibi_slopes, kv_cache_dtype, k_scale, v_scale; its three partial-result
buffers are replaced by one workspace the binding keeps per device.
"""

from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

__all__ = [
    "PA_OK", "PA_ERR_NULL", "PA_ERR_SHAPE", "PA_ERR_DTYPE", "PA_ERR_WORKSPACE", "PA_ERR_ALIGN",
    "PA_ERR_HIP", "PA_DTYPE_F32", "PA_DTYPE_BF16", "PA_KV_AUTO", "PA_KV_FP8_E4M3", "PA_KV_FP8_E4M3_COMPUTE",
    "PA_BLOCK_SIZE", "PA_PARTITION_SIZE", "PA_MAX_GROUP", "PA_MAX_SEQS",
    "pa_paged_attention_decode", "pa_paged_attention_decode_split", "pa_paged_attention_decode_noalloc",
    "pa_decode_plan", "PA_NOALLOC_SCRATCH_BYTES",
    "pa_workspace_bytes", "pa_kv_layout", "pa_last_error", "pa_version", "pa_timing_enable",
    "pa_timing_read", "pa_timing_read_append", "pa_hbm_read_probe", "pa_hbm_gather_probe", "pa_kv_cache_append",
    "paged_attention_decode", "kv_cache_append", "PA_ERR_NOMEM", "pa_pool_create", "pa_pool_destroy",
    "pa_pool_num_free", "pa_pool_refcount", "pa_pool_append", "pa_pool_fork", "pa_pool_release",
    "pa_copy_blocks", "BlockPool", "copy_blocks", "pa_shared_workspace_bytes",
    "pa_paged_attention_decode_shared", "PrefixGroups", "prefix_groups", "find_prefix_groups",
    "paged_attention_decode_shared", "kv_cache_shapes", "LIB_PATH",
    "PagedAttentionError", "PA_MLA_LATENT_DIM", "PA_MLA_ROPE_DIM", "PA_MLA_MAX_HEADS",
    "pa_mla_workspace_bytes", "pa_mla_decode", "mla_decode", "mla_cache_shape", "pa_mla_cache_append",
    "mla_cache_append", "pa_mla_decode_fp8", "pa_mla_cache_append_fp8",
]

PA_OK = 0
PA_ERR_NULL = -1
PA_ERR_SHAPE = -2
PA_ERR_DTYPE = -3
PA_ERR_WORKSPACE = -4
PA_ERR_ALIGN = -5
PA_ERR_HIP = -6
PA_ERR_NOMEM = -7
PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
PA_KV_AUTO = 0
PA_KV_FP8_E4M3 = 1
PA_KV_FP8_E4M3_COMPUTE = 2
PA_BLOCK_SIZE = 16
PA_PARTITION_SIZE = 256
PA_MAX_GROUP = 16
PA_MAX_SEQS = 65535
PA_MLA_LATENT_DIM = 512
PA_MLA_ROPE_DIM = 64
PA_MLA_MAX_HEADS = 128
PA_NOALLOC_SCRATCH_BYTES = 32 << 20

# PA_DECODE_LIB names another build of the library to load instead of the
# in-tree one (e.g. a host-sanitizer build); it must exist like the default.
LIB_PATH = os.environ.get("PA_DECODE_LIB") or LIB_PATH
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
        "or python decode_attention_paged_07_amd/build.py). There is no non-HIP fallback.")

_lib = ctypes.CDLL(LIB_PATH)

_c_int, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class _LayoutDesc(ctypes.Structure):
    _fields_ = [("x", ctypes.c_int), ("elem_bytes", ctypes.c_int),
                ("k_block_stride", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
                ("v_block_stride", ctypes.c_int64), ("v_head_stride", ctypes.c_int64)]


_DECODE_ARGS = [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _c_int,
                _vp, _c_int, _c_int, _vp, _c_int, _c_int, _vp, _vp, _vp, _c_size, _vp]

_lib.pa_paged_attention_decode.argtypes = _DECODE_ARGS
_lib.pa_paged_attention_decode.restype = _c_int
_lib.pa_paged_attention_decode_split.argtypes = _DECODE_ARGS + [_c_int]
_lib.pa_paged_attention_decode_split.restype = _c_int
_lib.pa_paged_attention_decode_noalloc.argtypes = _DECODE_ARGS[:20] + [_vp]
_lib.pa_paged_attention_decode_noalloc.restype = _c_int
_lib.pa_decode_plan.argtypes = [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                ctypes.POINTER(_c_int), ctypes.POINTER(_c_int), ctypes.POINTER(_c_size)]
_lib.pa_decode_plan.restype = _c_int
_lib.pa_workspace_bytes.argtypes = [_c_int, _c_int, _c_int, _c_int, ctypes.POINTER(_c_size)]
_lib.pa_workspace_bytes.restype = _c_int
_lib.pa_kv_layout.argtypes = [_c_int, _c_int, _c_int, _c_int, _c_int, ctypes.POINTER(_LayoutDesc)]
_lib.pa_kv_layout.restype = _c_int
_lib.pa_last_error.argtypes = []
_lib.pa_last_error.restype = ctypes.c_char_p
_lib.pa_version.argtypes = []
_lib.pa_version.restype = _c_int
_lib.pa_timing_enable.argtypes = [_c_int]
_lib.pa_timing_enable.restype = _c_int
_lib.pa_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_c_int),
                                ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_c_int)]
_lib.pa_timing_read.restype = _c_int
_lib.pa_timing_read_append.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_c_int)]
_lib.pa_timing_read_append.restype = _c_int
_lib.pa_hbm_read_probe.argtypes = [_vp, _c_size, _c_int, _vp, _vp]
_lib.pa_hbm_read_probe.restype = _c_int
_lib.pa_hbm_gather_probe.argtypes = [_vp, _c_size, _c_int, _vp, _c_int, _c_int, _c_int, _vp, _vp]
_lib.pa_hbm_gather_probe.restype = _c_int
_lib.pa_kv_cache_append.argtypes = [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp,
                                    _c_int, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp]
_lib.pa_kv_cache_append.restype = _c_int


_i32p = ctypes.POINTER(ctypes.c_int32)
_lib.pa_pool_create.argtypes = [_c_int, _c_int, ctypes.POINTER(_vp)]
_lib.pa_pool_create.restype = _c_int
_lib.pa_pool_destroy.argtypes = [_vp]
_lib.pa_pool_destroy.restype = None
_lib.pa_pool_num_free.argtypes = [_vp, ctypes.POINTER(_c_int)]
_lib.pa_pool_num_free.restype = _c_int
_lib.pa_pool_refcount.argtypes = [_vp, ctypes.c_int32, ctypes.POINTER(_c_int)]
_lib.pa_pool_refcount.restype = _c_int
_lib.pa_pool_append.argtypes = [_vp, _i32p, _c_int, _c_int, _c_int, _i32p, _i32p, ctypes.POINTER(_c_int)]
_lib.pa_pool_append.restype = _c_int
_lib.pa_pool_fork.argtypes = [_vp, _i32p, _c_int, _i32p, _c_int]
_lib.pa_pool_fork.restype = _c_int
_lib.pa_pool_release.argtypes = [_vp, _i32p, _c_int]
_lib.pa_pool_release.restype = _c_int
_lib.pa_shared_workspace_bytes.argtypes = [_c_int] * 9 + [ctypes.POINTER(_c_size)]
_lib.pa_shared_workspace_bytes.restype = _c_int
_lib.pa_paged_attention_decode_shared.argtypes = _DECODE_ARGS[:20] + [_c_int, _vp, _vp, _c_int, _vp, _vp, _c_int,
                                                                      _c_int, _vp, _c_size, _vp]
_lib.pa_paged_attention_decode_shared.restype = _c_int
_lib.pa_copy_blocks.argtypes = [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_size, _vp]
_lib.pa_copy_blocks.restype = _c_int
_lib.pa_mla_workspace_bytes.argtypes = [_c_int, _c_int, ctypes.POINTER(_c_size)]
_lib.pa_mla_workspace_bytes.restype = _c_int
_lib.pa_mla_decode.argtypes = [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_float, _vp, _c_int, _vp, _c_int,
                               _c_int, _vp, _c_size, _vp]
_lib.pa_mla_decode.restype = _c_int
_lib.pa_mla_cache_append.argtypes = [_vp, _vp, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _c_int, _vp]
_lib.pa_mla_cache_append.restype = _c_int
_lib.pa_mla_decode_fp8.argtypes = [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_float, _vp, _c_int, _vp, _c_int,
                                   _c_int, _vp, _vp, _c_size, _vp]
_lib.pa_mla_decode_fp8.restype = _c_int
_lib.pa_mla_cache_append_fp8.argtypes = [_vp, _vp, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _c_int, _vp, _vp]
_lib.pa_mla_cache_append_fp8.restype = _c_int


class PagedAttentionError(RuntimeError):
    """A PA_ERR_HIP failure reported by the library."""


class PoolExhausted(MemoryError):
    """PA_ERR_NOMEM: the block pool has too few free blocks."""


def _raise_for(code: int, what: str):
    if code == PA_OK:
        return
    msg = f"{what}: {pa_last_error()} (code {code})"
    if code == PA_ERR_DTYPE:
        raise TypeError(msg)
    if code == PA_ERR_HIP:
        raise PagedAttentionError(msg)
    if code == PA_ERR_NOMEM:
        raise PoolExhausted(msg)
    raise ValueError(msg)


# ---------------------------------------------------------------------------
# One-to-one wrappers of the C entry points (integers and device addresses).
# ---------------------------------------------------------------------------

def pa_paged_attention_decode(out, query, key_cache, value_cache, num_seqs, num_heads,
                              num_kv_heads, head_size, num_blocks, scale, block_tables,
                              max_blocks_per_seq, seq_lens, block_size, max_seq_len,
                              alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale,
                              workspace, workspace_bytes, stream) -> int:
    return _lib.pa_paged_attention_decode(out, query, key_cache, value_cache, num_seqs, num_heads,
                                          num_kv_heads, head_size, num_blocks, scale, block_tables,
                                          max_blocks_per_seq, seq_lens, block_size, max_seq_len,
                                          alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale,
                                          workspace, workspace_bytes, stream)


def pa_paged_attention_decode_split(out, query, key_cache, value_cache, num_seqs, num_heads,
                                    num_kv_heads, head_size, num_blocks, scale, block_tables,
                                    max_blocks_per_seq, seq_lens, block_size, max_seq_len,
                                    alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale,
                                    workspace, workspace_bytes, stream, split_tokens) -> int:
    return _lib.pa_paged_attention_decode_split(out, query, key_cache, value_cache, num_seqs,
                                                num_heads, num_kv_heads, head_size, num_blocks,
                                                scale, block_tables, max_blocks_per_seq, seq_lens,
                                                block_size, max_seq_len, alibi_slopes, q_dtype,
                                                kv_cache_dtype, k_scale, v_scale, workspace,
                                                workspace_bytes, stream, split_tokens)


def pa_paged_attention_decode_noalloc(out, query, key_cache, value_cache, num_seqs, num_heads,
                                      num_kv_heads, head_size, num_blocks, scale, block_tables,
                                      max_blocks_per_seq, seq_lens, block_size, max_seq_len,
                                      alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale,
                                      stream) -> int:
    return _lib.pa_paged_attention_decode_noalloc(out, query, key_cache, value_cache, num_seqs,
                                                  num_heads, num_kv_heads, head_size, num_blocks,
                                                  scale, block_tables, max_blocks_per_seq, seq_lens,
                                                  block_size, max_seq_len, alibi_slopes, q_dtype,
                                                  kv_cache_dtype, k_scale, v_scale, stream)


def pa_decode_plan(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len,
                   requested_split_tokens=0):
    """-> (split_tokens, num_splits, workspace_bytes); raises on invalid sizes."""
    st, ns, wb = _c_int(), _c_int(), _c_size()
    rc = _lib.pa_decode_plan(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len,
                             requested_split_tokens, ctypes.byref(st), ctypes.byref(ns),
                             ctypes.byref(wb))
    _raise_for(rc, "pa_decode_plan")
    return st.value, ns.value, wb.value


def pa_workspace_bytes(num_seqs, num_heads, head_size, max_seq_len) -> int:
    out = _c_size()
    rc = _lib.pa_workspace_bytes(num_seqs, num_heads, head_size, max_seq_len, ctypes.byref(out))
    _raise_for(rc, "pa_workspace_bytes")
    return out.value


def pa_kv_layout(num_kv_heads, head_size, block_size, q_dtype, kv_cache_dtype) -> dict:
    d = _LayoutDesc()
    rc = _lib.pa_kv_layout(num_kv_heads, head_size, block_size, q_dtype, kv_cache_dtype,
                           ctypes.byref(d))
    _raise_for(rc, "pa_kv_layout")
    return {f: getattr(d, f) for f, _ in _LayoutDesc._fields_}


def pa_last_error() -> str:
    return _lib.pa_last_error().decode()


def pa_version() -> int:
    return _lib.pa_version()


def pa_timing_enable(on: bool) -> None:
    _raise_for(_lib.pa_timing_enable(1 if on else 0), "pa_timing_enable")


def pa_timing_read():
    """-> (partition_ms, partition_launches, reduce_ms, reduce_launches) since the last read."""
    pm, pn, rm, rn = ctypes.c_double(), _c_int(), ctypes.c_double(), _c_int()
    rc = _lib.pa_timing_read(ctypes.byref(pm), ctypes.byref(pn), ctypes.byref(rm), ctypes.byref(rn))
    _raise_for(rc, "pa_timing_read")
    return pm.value, pn.value, rm.value, rn.value


def pa_timing_read_append():
    """-> (append_ms, append_launches) since the last read."""
    ms, n = ctypes.c_double(), _c_int()
    _raise_for(_lib.pa_timing_read_append(ctypes.byref(ms), ctypes.byref(n)), "pa_timing_read_append")
    return ms.value, n.value


def pa_hbm_read_probe(buf, nbytes, workgroups, sink, stream) -> int:
    return _lib.pa_hbm_read_probe(buf, nbytes, workgroups, sink, stream)


def pa_hbm_gather_probe(pool, pool_bytes, tile_bytes, ids, num_tiles, depth, workgroups, sink,
                        stream) -> int:
    return _lib.pa_hbm_gather_probe(pool, pool_bytes, tile_bytes, ids, num_tiles, depth, workgroups,
                                    sink, stream)


def pa_kv_cache_append(key_cache, value_cache, key, value, num_seqs, tokens_per_seq, num_kv_heads,
                       head_size, num_blocks, block_tables, max_blocks_per_seq, positions, block_size,
                       in_dtype, kv_cache_dtype, k_scale, v_scale, stream) -> int:
    return _lib.pa_kv_cache_append(key_cache, value_cache, key, value, num_seqs, tokens_per_seq,
                                   num_kv_heads, head_size, num_blocks, block_tables,
                                   max_blocks_per_seq, positions, block_size, in_dtype,
                                   kv_cache_dtype, k_scale, v_scale, stream)


def pa_pool_create(num_blocks, block_size, pool_out) -> int:
    return _lib.pa_pool_create(num_blocks, block_size, pool_out)


def pa_pool_destroy(pool) -> None:
    _lib.pa_pool_destroy(pool)


def pa_pool_num_free(pool, num_free) -> int:
    return _lib.pa_pool_num_free(pool, num_free)


def pa_pool_refcount(pool, block, refcount) -> int:
    return _lib.pa_pool_refcount(pool, block, refcount)


def pa_pool_append(pool, table_row, max_blocks, seq_len, num_new, cow_src, cow_dst, num_cow) -> int:
    return _lib.pa_pool_append(pool, table_row, max_blocks, seq_len, num_new, cow_src, cow_dst, num_cow)


def pa_pool_fork(pool, src_row, seq_len, dst_row, max_blocks) -> int:
    return _lib.pa_pool_fork(pool, src_row, seq_len, dst_row, max_blocks)


def pa_pool_release(pool, table_row, seq_len) -> int:
    return _lib.pa_pool_release(pool, table_row, seq_len)


def pa_shared_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size, block_size, max_seq_len,
                              num_groups, max_group_size, max_prefix_blocks) -> int:
    out = _c_size()
    rc = _lib.pa_shared_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size, block_size, max_seq_len,
                                        num_groups, max_group_size, max_prefix_blocks, ctypes.byref(out))
    _raise_for(rc, "pa_shared_workspace_bytes")
    return out.value


def pa_paged_attention_decode_shared(out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads,
                                     head_size, num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens,
                                     block_size, max_seq_len, alibi_slopes, q_dtype, kv_cache_dtype, k_scale,
                                     v_scale, num_groups, group_start, group_seqs, num_members,
                                     group_prefix_blocks, seq_prefix_blocks, max_group_size,
                                     max_prefix_blocks, workspace, workspace_bytes, stream) -> int:
    return _lib.pa_paged_attention_decode_shared(
        out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale,
        block_tables, max_blocks_per_seq, seq_lens, block_size, max_seq_len, alibi_slopes, q_dtype,
        kv_cache_dtype, k_scale, v_scale, num_groups, group_start, group_seqs, num_members,
        group_prefix_blocks, seq_prefix_blocks, max_group_size, max_prefix_blocks, workspace,
        workspace_bytes, stream)


def pa_copy_blocks(key_cache, value_cache, src, dst, num_pairs, num_blocks, block_bytes, stream) -> int:
    return _lib.pa_copy_blocks(key_cache, value_cache, src, dst, num_pairs, num_blocks, block_bytes, stream)


class BlockPool:
    """Host block pool (include/pa_blocks.h): reference-counted physical
    blocks, on-demand growth, sharing by fork, copy-on-write of a shared
    partially filled block. Table rows are host int32 numpy arrays, updated in
    place; the caller mirrors them to the device table."""

    def __init__(self, num_blocks: int, block_size: int = PA_BLOCK_SIZE):
        h = _vp()
        _raise_for(_lib.pa_pool_create(num_blocks, block_size, ctypes.byref(h)), "pa_pool_create")
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if self._h:
            _lib.pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass

    @staticmethod
    def _row(row):
        import numpy as np
        if not (isinstance(row, np.ndarray) and row.dtype == np.int32 and row.ndim == 1
                and row.flags["C_CONTIGUOUS"]):
            raise TypeError("table rows must be contiguous 1-D int32 numpy arrays")
        return row.ctypes.data_as(_i32p)

    @property
    def num_free(self) -> int:
        n = _c_int()
        _raise_for(_lib.pa_pool_num_free(self._h, ctypes.byref(n)), "pa_pool_num_free")
        return n.value

    def refcount(self, block: int) -> int:
        n = _c_int()
        _raise_for(_lib.pa_pool_refcount(self._h, int(block), ctypes.byref(n)), "pa_pool_refcount")
        return n.value

    def append(self, row, seq_len: int, num_new: int):
        """Room for num_new tokens after seq_len; -> (src, dst) copy-on-write pair or None."""
        src, dst, n = ctypes.c_int32(), ctypes.c_int32(), _c_int()
        _raise_for(_lib.pa_pool_append(self._h, self._row(row), row.shape[0], int(seq_len), int(num_new),
                                       ctypes.byref(src), ctypes.byref(dst), ctypes.byref(n)), "pa_pool_append")
        return (src.value, dst.value) if n.value else None

    def fork(self, src_row, seq_len: int, dst_row) -> None:
        _raise_for(_lib.pa_pool_fork(self._h, self._row(src_row), int(seq_len), self._row(dst_row),
                                     dst_row.shape[0]), "pa_pool_fork")

    def release(self, row, seq_len: int) -> None:
        _raise_for(_lib.pa_pool_release(self._h, self._row(row), int(seq_len)), "pa_pool_release")


def copy_blocks(key_cache, value_cache, src, dst) -> None:
    """Copy physical blocks src[i] -> dst[i] in both caches (device int32
    tensors), on the current stream."""
    dev = key_cache.device
    _need(dev.type == "cuda", "caches must be on a GPU")
    for name, t in (("value_cache", value_cache), ("src", src), ("dst", dst)):
        _need(t.device == dev, f"{name} is not on the caches' device")
    _need(src.dtype == torch.int32 and dst.dtype == torch.int32 and src.shape == dst.shape and src.dim() == 1,
          "src and dst must be int32 vectors of one length")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous() and key_cache.shape[0] == value_cache.shape[0],
          "caches must be contiguous with one block count")
    block_bytes = key_cache[0].numel() * key_cache.element_size()
    _need(value_cache[0].numel() * value_cache.element_size() == block_bytes, "K and V blocks differ in size")
    rc = _lib.pa_copy_blocks(key_cache.data_ptr(), value_cache.data_ptr(), src.data_ptr(), dst.data_ptr(),
                             src.shape[0], key_cache.shape[0], block_bytes,
                             torch.cuda.current_stream(dev).cuda_stream)
    _raise_for(rc, "copy_blocks")


# ---------------------------------------------------------------------------
# Tensor-level call.
# ---------------------------------------------------------------------------

_Q_DTYPES = {torch.float32: PA_DTYPE_F32, torch.bfloat16: PA_DTYPE_BF16}
_KV_NAMES = {"auto": PA_KV_AUTO, "fp8": PA_KV_FP8_E4M3, "fp8_e4m3": PA_KV_FP8_E4M3}
_workspaces: dict = {}
_scalars: dict = {}


def kv_cache_shapes(num_blocks, num_kv_heads, head_size, q_dtype=torch.bfloat16,
                    kv_cache_dtype="auto", block_size=PA_BLOCK_SIZE):
    """Shapes of (key_cache, value_cache) in the library's layout."""
    lay = pa_kv_layout(num_kv_heads, head_size, block_size, _Q_DTYPES[q_dtype],
                       _KV_NAMES[kv_cache_dtype])
    x = lay["x"]
    return ((num_blocks, num_kv_heads, head_size // x, block_size, x),
            (num_blocks, num_kv_heads, head_size, block_size))


def _capturing() -> bool:
    """Whether the current stream is capturing a graph."""
    return torch.cuda.is_current_stream_capturing()


def _device_scalar(v, device):
    """A one-element float32 device tensor holding v. A Python float becomes a
    device tensor filled by a kernel (no host-to-device copy, so it can be
    captured); eager calls cache it per (device, value). Under graph capture it
    is made afresh and not cached: the fill runs only when the graph replays."""
    if isinstance(v, torch.Tensor):
        if v.dtype != torch.float32 or v.numel() != 1 or v.device != device:
            raise ValueError("k_scale/v_scale tensors must be one float32 element on the query's device")
        return v
    if _capturing():
        return torch.full((1,), float(v), dtype=torch.float32, device=device)
    key = (device, float(v))
    t = _scalars.get(key)
    if t is None:
        t = torch.full((1,), float(v), dtype=torch.float32, device=device)
        _scalars[key] = t
    return t


# Outgrown workspaces, each with an event recorded on its stream after its
# last use: kept until that event has completed (kernels queued before it may
# still write the buffer), then dropped.
_retired: list = []


def _workspace_for(device, nbytes):
    """A workspace of at least nbytes for a call on the current stream.

    Eager calls share one cached buffer per (device, stream), so calls on
    different streams never share one. A buffer outgrown by a larger call is
    replaced by one half as large again as it (or the request, if larger), so
    a slowly growing batch replaces it a logarithmic number of times; the old
    one stays alive until the work queued on its stream so far has finished.
    Under graph capture the call gets a buffer of its own from torch's
    allocator (the graph's memory pool, like any temporary of a captured op)
    that is never cached: the graph's replays use it alone, and later eager
    calls cannot replace it."""
    if nbytes == 0:
        return None
    if _capturing():
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if _retired:
        _retired[:] = [(b, e) for b, e in _retired if not e.query()]
    stream = torch.cuda.current_stream(device)
    key = (device, stream.cuda_stream)
    t = _workspaces.get(key)
    if t is None or t.numel() < nbytes:
        size = nbytes
        if t is not None:
            done = torch.cuda.Event()
            done.record(stream)
            _retired.append((t, done))
            size = max(nbytes, t.numel() + t.numel() // 2)
        t = torch.empty(size, dtype=torch.uint8, device=device)
        _workspaces[key] = t
    return t


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def paged_attention_decode(out, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
                           seq_lens, block_size, max_seq_len, alibi_slopes=None,
                           kv_cache_dtype="auto", k_scale=1.0, v_scale=1.0, *, workspace=None,
                           split_tokens=0, compute="auto") -> None:
    """Write softmax(scale*q.K^T + alibi).V for every (sequence, query head) into ``out``.

    out, query: [num_seqs, num_heads, head_size], float32 or bfloat16, contiguous, on one GPU.
    key_cache, value_cache: the library's layout (``kv_cache_shapes``); same dtype as query for
    kv_cache_dtype "auto", uint8 / float8_e4m3fn codes for "fp8" / "fp8_e4m3".
    block_tables int32 [num_seqs, max_blocks]; seq_lens int32 [num_seqs].
    alibi_slopes: float32 [num_heads] or None. k_scale / v_scale: float or one-element float32
    tensor (used for the fp8 cache only). compute: "auto" (bf16/f32 arithmetic) or "fp8"
    (fp8 cache only: MX-scaled fp8 q and e4m3 P on fp8 MFMA, PA_KV_FP8_E4M3_COMPUTE).
    Runs asynchronously on the current stream.
    """
    if kv_cache_dtype not in _KV_NAMES:
        raise TypeError(f"kv_cache_dtype {kv_cache_dtype!r} is not one of {sorted(_KV_NAMES)}")
    kvd = _KV_NAMES[kv_cache_dtype]
    if compute not in ("auto", "fp8"):
        raise TypeError(f"compute {compute!r} is not 'auto' or 'fp8'")
    if compute == "fp8":
        if kvd != PA_KV_FP8_E4M3:
            raise TypeError("compute='fp8' needs the fp8 cache")
        kvd = PA_KV_FP8_E4M3_COMPUTE
    if query.dtype not in _Q_DTYPES:
        raise TypeError(f"query dtype {query.dtype} is not float32 or bfloat16")
    qd = _Q_DTYPES[query.dtype]
    dev = query.device
    _need(dev.type == "cuda", "query must be on a GPU")
    for name, t in (("out", out), ("key_cache", key_cache), ("value_cache", value_cache),
                    ("block_tables", block_tables), ("seq_lens", seq_lens)):
        _need(t.device == dev, f"{name} is not on the query's device")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(query.is_contiguous(), "query must be contiguous")
    _need(out.dtype == query.dtype and out.shape == query.shape, "out must match query in shape and dtype")
    _need(query.dim() == 3, "query must be [num_seqs, num_heads, head_size]")
    num_seqs, num_heads, head_size = query.shape
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == num_seqs, "block_tables must be int32 [num_seqs, max_blocks]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.shape == (num_seqs,), "seq_lens must be int32 [num_seqs]")
    if kvd == PA_KV_AUTO:
        if key_cache.dtype != query.dtype or value_cache.dtype != query.dtype:
            raise TypeError("with kv_cache_dtype 'auto' the caches must have the query's dtype")
    elif key_cache.dtype not in (torch.uint8, torch.float8_e4m3fn) or value_cache.dtype != key_cache.dtype:
        raise TypeError("the fp8 cache must be uint8 or float8_e4m3fn codes")
    num_blocks = key_cache.shape[0]
    k_shape, v_shape = kv_cache_shapes(num_blocks, num_kv_heads, head_size, query.dtype,
                                       kv_cache_dtype, block_size)
    _need(tuple(key_cache.shape) == k_shape, f"key_cache shape {tuple(key_cache.shape)} != {k_shape}")
    _need(tuple(value_cache.shape) == v_shape, f"value_cache shape {tuple(value_cache.shape)} != {v_shape}")
    slopes_ptr = None
    if alibi_slopes is not None:
        _need(alibi_slopes.dtype == torch.float32 and alibi_slopes.shape == (num_heads,)
              and alibi_slopes.device == dev and alibi_slopes.is_contiguous(),
              "alibi_slopes must be contiguous float32 [num_heads] on the query's device")
        slopes_ptr = alibi_slopes.data_ptr()
    ks = _device_scalar(k_scale, dev) if kvd != PA_KV_AUTO else None
    vs = _device_scalar(v_scale, dev) if kvd != PA_KV_AUTO else None
    if workspace is None:
        _, _, need = pa_decode_plan(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len,
                                    split_tokens)
        workspace = _workspace_for(dev, need)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), num_seqs,
            num_heads, num_kv_heads, head_size, num_blocks, float(scale), block_tables.data_ptr(),
            block_tables.shape[1], seq_lens.data_ptr(), block_size, int(max_seq_len), slopes_ptr, qd,
            kvd, ks.data_ptr() if ks is not None else None, vs.data_ptr() if vs is not None else None,
            ws_ptr, ws_bytes, stream)
    if split_tokens:
        rc = _lib.pa_paged_attention_decode_split(*args, int(split_tokens))
    else:
        rc = _lib.pa_paged_attention_decode(*args)
    _raise_for(rc, "paged_attention_decode")


def pa_mla_workspace_bytes(num_seqs, num_heads) -> int:
    out = _c_size(0)
    _raise_for(_lib.pa_mla_workspace_bytes(num_seqs, num_heads, ctypes.byref(out)), "pa_mla_workspace_bytes")
    return out.value


def pa_mla_decode(out, query, latent_cache, num_seqs, num_heads, num_blocks, scale, block_tables,
                  max_blocks_per_seq, seq_lens, block_size, max_seq_len, workspace, workspace_bytes,
                  stream) -> int:
    return _lib.pa_mla_decode(out, query, latent_cache, num_seqs, num_heads, num_blocks, scale, block_tables,
                              max_blocks_per_seq, seq_lens, block_size, max_seq_len, workspace,
                              workspace_bytes, stream)


def pa_mla_cache_append(latent_cache, rows, num_seqs, tokens_per_seq, num_blocks, block_tables,
                        max_blocks_per_seq, positions, block_size, stream) -> int:
    return _lib.pa_mla_cache_append(latent_cache, rows, num_seqs, tokens_per_seq, num_blocks, block_tables,
                                    max_blocks_per_seq, positions, block_size, stream)


def pa_mla_decode_fp8(out, query, latent_cache, num_seqs, num_heads, num_blocks, scale, block_tables,
                      max_blocks_per_seq, seq_lens, block_size, max_seq_len, kv_scale, workspace,
                      workspace_bytes, stream) -> int:
    return _lib.pa_mla_decode_fp8(out, query, latent_cache, num_seqs, num_heads, num_blocks, scale, block_tables,
                                  max_blocks_per_seq, seq_lens, block_size, max_seq_len, kv_scale, workspace,
                                  workspace_bytes, stream)


def pa_mla_cache_append_fp8(latent_cache, rows, num_seqs, tokens_per_seq, num_blocks, block_tables,
                            max_blocks_per_seq, positions, block_size, kv_scale, stream) -> int:
    return _lib.pa_mla_cache_append_fp8(latent_cache, rows, num_seqs, tokens_per_seq, num_blocks, block_tables,
                                        max_blocks_per_seq, positions, block_size, kv_scale, stream)


def mla_cache_shape(num_blocks, block_size=16, fp8=False):
    """Shape of the latent cache: bf16 [num_blocks, 576/8, block_size, 8], or
    with fp8=True uint8 e4m3fn codes [num_blocks, 576/16, block_size, 16]."""
    x = 16 if fp8 else 8
    return (num_blocks, (PA_MLA_LATENT_DIM + PA_MLA_ROPE_DIM) // x, block_size, x)


_FP8_CODES = (torch.uint8, torch.float8_e4m3fn)


def mla_decode(out, query, latent_cache, scale, block_tables, seq_lens, max_seq_len, *,
               workspace=None, kv_scale=1.0) -> None:
    """Latent-cache (MLA) decode: out[s,h] = sum_t softmax_t(scale*q[s,h].row_t) * row_t[:512].

    query bf16 [num_seqs, num_heads, 576] (absorbed query and rope query), out bf16
    [num_seqs, num_heads, 512], latent_cache bf16 ``mla_cache_shape(num_blocks)``, or uint8 /
    float8_e4m3fn codes ``mla_cache_shape(num_blocks, fp8=True)`` whose values are code * kv_scale
    (float or one-element float32 device tensor); block_tables int32 [num_seqs, max_blocks];
    seq_lens int32 [num_seqs]. Runs on the current stream.
    """
    dev = query.device
    _need(dev.type == "cuda", "query must be on a GPU")
    for name, t in (("out", out), ("query", query), ("latent_cache", latent_cache),
                    ("block_tables", block_tables), ("seq_lens", seq_lens)):
        _need(t.device == dev, f"{name} is not on the query's device")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    width = PA_MLA_LATENT_DIM + PA_MLA_ROPE_DIM
    fp8 = latent_cache.dtype in _FP8_CODES
    if query.dtype != torch.bfloat16 or out.dtype != torch.bfloat16 or not (fp8 or latent_cache.dtype == torch.bfloat16):
        raise TypeError("query and out must be bfloat16, latent_cache bfloat16 or e4m3fn codes")
    _need(query.dim() == 3 and query.shape[2] == width, f"query must be [num_seqs, num_heads, {width}]")
    num_seqs, num_heads, _ = query.shape
    _need(tuple(out.shape) == (num_seqs, num_heads, PA_MLA_LATENT_DIM),
          f"out must be [num_seqs, num_heads, {PA_MLA_LATENT_DIM}]")
    _need(latent_cache.dim() == 4, "latent_cache must be [num_blocks, 576/x, block_size, x]")
    num_blocks, block_size = latent_cache.shape[0], latent_cache.shape[2]
    want = mla_cache_shape(num_blocks, block_size, fp8)
    _need(tuple(latent_cache.shape) == want, f"latent_cache shape {tuple(latent_cache.shape)} != {want}")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == num_seqs, "block_tables must be int32 [num_seqs, max_blocks]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.shape == (num_seqs,), "seq_lens must be int32 [num_seqs]")
    if workspace is None:
        workspace = _workspace_for(dev, pa_mla_workspace_bytes(num_seqs, num_heads))
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stream = torch.cuda.current_stream(dev).cuda_stream
    if fp8:
        ks = _device_scalar(kv_scale, dev)
        rc = _lib.pa_mla_decode_fp8(out.data_ptr(), query.data_ptr(), latent_cache.data_ptr(), num_seqs,
                                    num_heads, num_blocks, float(scale), block_tables.data_ptr(),
                                    block_tables.shape[1], seq_lens.data_ptr(), block_size, int(max_seq_len),
                                    ks.data_ptr(), ws_ptr, ws_bytes, stream)
    else:
        rc = _lib.pa_mla_decode(out.data_ptr(), query.data_ptr(), latent_cache.data_ptr(), num_seqs, num_heads,
                                num_blocks, float(scale), block_tables.data_ptr(), block_tables.shape[1],
                                seq_lens.data_ptr(), block_size, int(max_seq_len), ws_ptr, ws_bytes, stream)
    _raise_for(rc, "mla_decode")


def kv_cache_append(key_cache, value_cache, key, value, block_tables, positions,
                    kv_cache_dtype="auto", k_scale=1.0, v_scale=1.0, block_size=None) -> None:
    """Store new tokens' K/V rows in the paged cache (in place, current stream).

    key, value: [num_seqs, num_kv_heads, head_size] (one token per sequence) or
    [num_seqs, T, num_kv_heads, head_size], float32 or bfloat16, contiguous.
    Token j of sequence s is written at logical position positions[s] + j
    through block_tables (int32 [num_seqs, max_blocks]); positions int32
    [num_seqs], negative = skip. Caches in the library's layout
    (``kv_cache_shapes``): the input dtype for "auto", uint8 / float8_e4m3fn
    codes for "fp8" / "fp8_e4m3" (value / scale rounded to the nearest code).
    block_size: tokens per cache block (16 or 32); None takes it from the
    value cache's last dimension.
    """
    if kv_cache_dtype not in _KV_NAMES:
        raise TypeError(f"kv_cache_dtype {kv_cache_dtype!r} is not one of {sorted(_KV_NAMES)}")
    kvd = _KV_NAMES[kv_cache_dtype]
    if key.dtype not in _Q_DTYPES or value.dtype != key.dtype:
        raise TypeError("key/value must both be float32 or bfloat16")
    dev = key.device
    _need(dev.type == "cuda", "key must be on a GPU")
    for name, t in (("key_cache", key_cache), ("value_cache", value_cache), ("value", value),
                    ("block_tables", block_tables), ("positions", positions)):
        _need(t.device == dev, f"{name} is not on the key's device")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(key.is_contiguous(), "key must be contiguous")
    _need(key.shape == value.shape and key.dim() in (3, 4), "key/value must be [S, Hkv, D] or [S, T, Hkv, D]")
    num_seqs = key.shape[0]
    tokens = 1 if key.dim() == 3 else key.shape[1]
    num_kv_heads, head_size = key.shape[-2], key.shape[-1]
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == num_seqs, "block_tables must be int32 [num_seqs, max_blocks]")
    _need(positions.dtype == torch.int32 and positions.shape == (num_seqs,),
          "positions must be int32 [num_seqs]")
    if kvd == PA_KV_AUTO:
        if key_cache.dtype != key.dtype or value_cache.dtype != key.dtype:
            raise TypeError("with kv_cache_dtype 'auto' the caches must have the key's dtype")
    elif key_cache.dtype not in (torch.uint8, torch.float8_e4m3fn) or value_cache.dtype != key_cache.dtype:
        raise TypeError("the fp8 cache must be uint8 or float8_e4m3fn codes")
    num_blocks = key_cache.shape[0]
    if block_size is None:
        _need(value_cache.dim() == 4, "value_cache must be [num_blocks, num_kv_heads, head_size, block_size]")
        block_size = int(value_cache.shape[-1])
    # the layout depends only on the cache element type (fp8 codes for any input type)
    layout_dtype = key.dtype if kvd == PA_KV_AUTO else torch.bfloat16
    k_shape, v_shape = kv_cache_shapes(num_blocks, num_kv_heads, head_size, layout_dtype, kv_cache_dtype,
                                       block_size)
    _need(tuple(key_cache.shape) == k_shape, f"key_cache shape {tuple(key_cache.shape)} != {k_shape}")
    _need(tuple(value_cache.shape) == v_shape, f"value_cache shape {tuple(value_cache.shape)} != {v_shape}")
    ks = _device_scalar(k_scale, dev) if kvd == PA_KV_FP8_E4M3 else None
    vs = _device_scalar(v_scale, dev) if kvd == PA_KV_FP8_E4M3 else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = _lib.pa_kv_cache_append(
        key_cache.data_ptr(), value_cache.data_ptr(), key.data_ptr(), value.data_ptr(), num_seqs,
        tokens, num_kv_heads, head_size, num_blocks, block_tables.data_ptr(), block_tables.shape[1],
        positions.data_ptr(), int(block_size), _Q_DTYPES[key.dtype], kvd,
        ks.data_ptr() if ks is not None else None, vs.data_ptr() if vs is not None else None, stream)
    _raise_for(rc, "kv_cache_append")


def mla_cache_append(latent_cache, rows, block_tables, positions, kv_scale=1.0) -> None:
    """Store new tokens' latent rows [c_kv, k_rope] in the paged latent cache (in place, current stream).

    rows bf16 [num_seqs, 576] (one token per sequence) or [num_seqs, T, 576], contiguous; token j of
    sequence s is written at logical position positions[s] + j through block_tables (int32
    [num_seqs, max_blocks]); positions int32 [num_seqs], negative = skip. latent_cache bf16
    ``mla_cache_shape(num_blocks)``, or uint8 / float8_e4m3fn ``mla_cache_shape(num_blocks, fp8=True)``
    receiving the e4m3fn codes of row / kv_scale.
    """
    width = PA_MLA_LATENT_DIM + PA_MLA_ROPE_DIM
    dev = rows.device
    _need(dev.type == "cuda", "rows must be on a GPU")
    for name, t in (("latent_cache", latent_cache), ("rows", rows), ("block_tables", block_tables),
                    ("positions", positions)):
        _need(t.device == dev, f"{name} is not on the rows' device")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    fp8 = latent_cache.dtype in _FP8_CODES
    if rows.dtype != torch.bfloat16 or not (fp8 or latent_cache.dtype == torch.bfloat16):
        raise TypeError("rows must be bfloat16, latent_cache bfloat16 or e4m3fn codes")
    _need(rows.dim() in (2, 3) and rows.shape[-1] == width, f"rows must be [S, {width}] or [S, T, {width}]")
    num_seqs = rows.shape[0]
    tokens = 1 if rows.dim() == 2 else rows.shape[1]
    _need(latent_cache.dim() == 4, "latent_cache must be [num_blocks, 576/x, block_size, x]")
    num_blocks, block_size = latent_cache.shape[0], latent_cache.shape[2]
    want = mla_cache_shape(num_blocks, block_size, fp8)
    _need(tuple(latent_cache.shape) == want, f"latent_cache shape {tuple(latent_cache.shape)} != {want}")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == num_seqs, "block_tables must be int32 [num_seqs, max_blocks]")
    _need(positions.dtype == torch.int32 and positions.shape == (num_seqs,),
          "positions must be int32 [num_seqs]")
    stream = torch.cuda.current_stream(dev).cuda_stream
    if fp8:
        ks = _device_scalar(kv_scale, dev)
        rc = _lib.pa_mla_cache_append_fp8(latent_cache.data_ptr(), rows.data_ptr(), num_seqs, tokens, num_blocks,
                                          block_tables.data_ptr(), block_tables.shape[1], positions.data_ptr(),
                                          block_size, ks.data_ptr(), stream)
    else:
        rc = _lib.pa_mla_cache_append(latent_cache.data_ptr(), rows.data_ptr(), num_seqs, tokens, num_blocks,
                                      block_tables.data_ptr(), block_tables.shape[1], positions.data_ptr(),
                                      block_size, stream)
    _raise_for(rc, "mla_cache_append")


class PrefixGroups:
    """Device description of shared-prefix groups for paged_attention_decode_shared."""

    def __init__(self, groups, num_seqs, device):
        """groups: iterable of (member sequence ids, shared prefix blocks)."""
        groups = [(list(map(int, m)), int(p)) for m, p in groups if len(m) > 0]
        seen = set()
        start, seqs, pref = [0], [], []
        seq_pref = [0] * num_seqs
        for members, p in groups:
            if p < 0:
                raise ValueError("prefix blocks must be >= 0")
            for s in members:
                if not 0 <= s < num_seqs or s in seen:
                    raise ValueError(f"sequence {s} is out of range or in two groups")
                seen.add(s)
                seq_pref[s] = p
            seqs.extend(members)
            start.append(len(seqs))
            pref.append(p)
        i32 = dict(dtype=torch.int32, device=device)
        self.num_groups = len(groups)
        self.group_start = torch.tensor(start, **i32)
        self.group_seqs = torch.tensor(seqs if seqs else [0], **i32)
        self.num_members = len(seqs)
        self.group_prefix_blocks = torch.tensor(pref if pref else [0], **i32)
        self.seq_prefix_blocks = torch.tensor(seq_pref, **i32)
        self.max_group_size = max([len(m) for m, _ in groups], default=1)
        self.max_prefix_blocks = max(pref, default=0)


def prefix_groups(groups, num_seqs, device) -> PrefixGroups:
    return PrefixGroups(groups, num_seqs, device)


def find_prefix_groups(block_tables, seq_lens, block_size=PA_BLOCK_SIZE, min_prefix_blocks=1):
    """Groups of sequences whose leading full blocks are the same physical
    blocks, from host copies of the table and lengths: sequences are grouped
    by their first physical block, and a group's prefix is the longest run of
    leading table entries all members share, cut to each member's full
    blocks. Returns [(members, prefix_blocks)] for groups of two or more."""
    import numpy as np
    table = np.asarray(block_tables)
    lens = np.asarray(seq_lens)
    by_first = {}
    for s in range(table.shape[0]):
        if lens[s] >= block_size:
            by_first.setdefault(int(table[s, 0]), []).append(s)
    out = []
    for members in by_first.values():
        if len(members) < 2:
            continue
        full = min(int(lens[s]) // block_size for s in members)
        rows = table[members, :full]
        same = np.all(rows == rows[0], axis=0)
        p = int(np.argmin(same)) if not same.all() else full
        if p >= min_prefix_blocks:
            out.append((members, p))
    return out


def paged_attention_decode_shared(out, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
                                  seq_lens, block_size, max_seq_len, groups: PrefixGroups, alibi_slopes=None,
                                  kv_cache_dtype="auto", k_scale=1.0, v_scale=1.0, *, workspace=None,
                                  compute="auto") -> None:
    """paged_attention_decode for a batch with shared-prefix groups (PrefixGroups):
    each shared K/V block is read once per group. Same result as the plain call
    (compute as for paged_attention_decode)."""
    if kv_cache_dtype not in _KV_NAMES:
        raise TypeError(f"kv_cache_dtype {kv_cache_dtype!r} is not one of {sorted(_KV_NAMES)}")
    kvd = _KV_NAMES[kv_cache_dtype]
    if compute not in ("auto", "fp8"):
        raise TypeError(f"compute {compute!r} is not 'auto' or 'fp8'")
    if compute == "fp8":
        if kvd != PA_KV_FP8_E4M3:
            raise TypeError("compute='fp8' needs the fp8 cache")
        kvd = PA_KV_FP8_E4M3_COMPUTE
    if query.dtype not in _Q_DTYPES:
        raise TypeError(f"query dtype {query.dtype} is not float32 or bfloat16")
    dev = query.device
    _need(dev.type == "cuda", "query must be on a GPU")
    for name, t in (("out", out), ("key_cache", key_cache), ("value_cache", value_cache),
                    ("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("group_start", groups.group_start), ("group_seqs", groups.group_seqs),
                    ("group_prefix_blocks", groups.group_prefix_blocks),
                    ("seq_prefix_blocks", groups.seq_prefix_blocks)):
        _need(t.device == dev, f"{name} is not on the query's device")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(query.is_contiguous() and out.dtype == query.dtype and out.shape == query.shape,
          "out must match a contiguous query in shape and dtype")
    num_seqs, num_heads, head_size = query.shape
    _need(groups.seq_prefix_blocks.shape == (num_seqs,), "groups were built for another batch size")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == num_seqs,
          "block_tables must be int32 [num_seqs, max_blocks]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.shape == (num_seqs,), "seq_lens must be int32 [num_seqs]")
    num_blocks = key_cache.shape[0]
    k_shape, v_shape = kv_cache_shapes(num_blocks, num_kv_heads, head_size, query.dtype, kv_cache_dtype,
                                       block_size)
    _need(tuple(key_cache.shape) == k_shape and tuple(value_cache.shape) == v_shape,
          "caches are not in the library's layout")
    slopes_ptr = None
    if alibi_slopes is not None:
        _need(alibi_slopes.dtype == torch.float32 and alibi_slopes.shape == (num_heads,)
              and alibi_slopes.device == dev, "alibi_slopes must be float32 [num_heads] on the query's device")
        slopes_ptr = alibi_slopes.data_ptr()
    ks = _device_scalar(k_scale, dev) if kvd != PA_KV_AUTO else None
    vs = _device_scalar(v_scale, dev) if kvd != PA_KV_AUTO else None
    if workspace is None:
        need = pa_shared_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size, block_size, max_seq_len,
                                         groups.num_groups, groups.max_group_size, groups.max_prefix_blocks)
        workspace = _workspace_for(dev, need)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = _lib.pa_paged_attention_decode_shared(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), num_seqs, num_heads,
        num_kv_heads, head_size, num_blocks, float(scale), block_tables.data_ptr(), block_tables.shape[1],
        seq_lens.data_ptr(), block_size, int(max_seq_len), slopes_ptr, _Q_DTYPES[query.dtype], kvd,
        ks.data_ptr() if ks is not None else None, vs.data_ptr() if vs is not None else None,
        groups.num_groups, groups.group_start.data_ptr(), groups.group_seqs.data_ptr(), groups.num_members,
        groups.group_prefix_blocks.data_ptr(), groups.seq_prefix_blocks.data_ptr(), groups.max_group_size,
        groups.max_prefix_blocks, ws_ptr, ws_bytes, torch.cuda.current_stream(dev).cuda_stream)
    _raise_for(rc, "paged_attention_decode_shared")
