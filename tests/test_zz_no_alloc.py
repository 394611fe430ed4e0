"""The decode call that allocates nothing (pa_paged_attention_decode_noalloc),
through the C ABI: its output against pa_paged_attention_decode's (the same
kernels with a caller workspace) and against the fp64 oracle, on two calls in
a row, the second with a smaller input; and its host-side rejection of a call
whose workspace would not fit its scratch array."""

import ctypes

import pytest
import torch

import workloads
from tests import _run

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
KV = {"auto": 0, "fp8_e4m3": 1}
QD = {"f32": 0, "bf16": 1}


def _c_args(pa, case, out, scales):
    cfg = case.cfg
    s, h, d = case.query.shape
    ks, vs = scales
    return [out.data_ptr(), case.query.data_ptr(), case.key_cache.data_ptr(), case.value_cache.data_ptr(), s, h,
            cfg.num_kv_heads, d, case.key_cache.shape[0], ctypes.c_float(case.scale), case.block_tables.data_ptr(),
            case.block_tables.shape[1], case.seq_lens.data_ptr(), cfg.block_size, case.max_seq_len,
            case.alibi_slopes.data_ptr() if case.alibi_slopes is not None else None, QD[cfg.q_dtype],
            KV[cfg.kv_dtype], ks.data_ptr() if ks is not None else None, vs.data_ptr() if vs is not None else None]


def _noalloc_and_workspace_call(pa, case):
    cfg = case.cfg
    scales = (None, None)
    if cfg.kv_dtype != "auto":
        scales = tuple(torch.tensor([v], dtype=torch.float32, device=DEV) for v in (case.k_scale, case.v_scale))
    stream = torch.cuda.current_stream(DEV).cuda_stream
    out_na = torch.full_like(case.query, float("nan"))
    out_ws = torch.full_like(case.query, float("nan"))
    print(f"[case] noalloc S={case.query.shape[0]} kv={cfg.kv_dtype} lens={case.meta.seq_lens.tolist()}",
          flush=True)
    rc = pa.pa_paged_attention_decode_noalloc(*_c_args(pa, case, out_na, scales), stream)
    assert rc == pa.PA_OK, pa.pa_last_error()
    _, _, need = pa.pa_decode_plan(case.query.shape[0], case.query.shape[1], cfg.num_kv_heads,
                                   case.query.shape[2], case.max_seq_len, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    rc = pa.pa_paged_attention_decode(*_c_args(pa, case, out_ws, scales), ws.data_ptr(), need, stream)
    assert rc == pa.PA_OK, pa.pa_last_error()
    torch.cuda.synchronize()
    return out_na, out_ws


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    import decode_attention_paged_07_amd as pa
    big = workloads.GQA.with_(num_seqs=12, pool_blocks=1024, seq_lens=("uniform", 1, 1500))
    small = workloads.FP8.with_(num_seqs=3, pool_blocks=128, seq_lens=("fixed", (40, 600, 5)))
    for cfg in (big, small):
        case = workloads.make_case(cfg, device=DEV, poison=True)
        out_na, out_ws = _noalloc_and_workspace_call(pa, case)
        # The same kernels and plan on the same inputs: bitwise equal outputs.
        assert torch.equal(out_na, out_ws)
        _run.compare(out_na, _run.run_oracle(case), cfg.q_dtype, what=f"noalloc {cfg.name}")


def test_noalloc_rejects_a_call_beyond_its_scratch():
    """Host validation only (fake, aligned device addresses; nothing is
    launched): 4096 sequences x 8 kv heads of 8 query heads at head size 128
    need about 138 MB of stream-K workspace, beyond the 32 MiB scratch."""
    import decode_attention_paged_07_amd as pa
    s, h, hkv, d = 4096, 64, 8, 128
    big = 1 << 32
    rc = pa.pa_paged_attention_decode_noalloc(big, 2 * big, 3 * big, 4 * big, s, h, hkv, d, 1024,
                                              ctypes.c_float(0.1), 5 * big, 64, 6 * big, 16, 1024, None, 1, 0,
                                              None, None, None)
    assert rc == pa.PA_ERR_WORKSPACE
    assert "no-alloc scratch" in pa.pa_last_error()
    # The same call with an ordinary workspace argument would be accepted by
    # the plan: the need is the stream-K plan's.
    _, _, need = pa.pa_decode_plan(s, h, hkv, d, 1024, 0)
    assert need > pa.PA_NOALLOC_SCRATCH_BYTES
    # Invalid arguments are reported as for the decode call.
    rc = pa.pa_paged_attention_decode_noalloc(big, 2 * big, 3 * big, 4 * big, 2, 8, 3, d, 16,
                                              ctypes.c_float(0.1), 5 * big, 4, 6 * big, 16, 40, None, 1, 0,
                                              None, None, None)
    assert rc == pa.PA_ERR_SHAPE
