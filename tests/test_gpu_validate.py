"""PA_VALIDATE_DEVICE=1: the decode calls copy seq_lens and the table entries
each sequence uses to the host and reject out-of-range values with
PA_ERR_SHAPE before launching anything (the output keeps its sentinel). Valid
inputs give the same result as without the check, bit for bit. Entries past
a sequence's blocks are not checked (they are never read)."""

import ctypes

import numpy as np
import pytest
import torch

import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
SENTINEL = 7.0


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("PA_VALIDATE_DEVICE", "1")
    return monkeypatch


def small(kv="auto", lens=(17, 300, 1, 640)):
    cfg = (workloads.GQA if kv == "auto" else workloads.FP8).with_(
        num_seqs=len(lens), pool_blocks=200, seq_lens=("fixed", tuple(lens)))
    return workloads.make_case(cfg, device=DEV, max_seq_len=704)


def sentinel_out(case):
    return torch.full_like(case.query, SENTINEL)


@pytest.mark.parametrize("kv", ["auto", "fp8_e4m3"])
@pytest.mark.parametrize("split", [0, 256])
def test_valid_inputs_give_the_same_output(validate, kv, split):
    case = small(kv)
    print(f"[case] validate valid kv={kv} split={split}", flush=True)
    a = _run.run_hip(case, split_tokens=split)
    validate.delenv("PA_VALIDATE_DEVICE")
    b = _run.run_hip(case, split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _expect_rejected(case, match, **kw):
    out = sentinel_out(case)
    with pytest.raises(ValueError, match=match):
        _run.run_hip(case, out=out, **kw)
    torch.cuda.synchronize()
    assert (out.float() == SENTINEL).all(), "a rejected call must launch nothing"


@pytest.mark.parametrize("bad", [705, -3])
def test_length_outside_range_is_rejected(validate, bad):
    case = small()
    case.seq_lens[1] = bad
    print(f"[case] validate seq_len {bad}", flush=True)
    _expect_rejected(case, r"seq_lens\[1\] = " + str(bad))


@pytest.mark.parametrize("bad", [200, 10 ** 6, -1])
def test_used_table_entry_outside_pool_is_rejected(validate, bad):
    case = small()
    case.block_tables[3, 39] = bad            # the last block of the 640-token sequence
    print(f"[case] validate table entry {bad}", flush=True)
    _expect_rejected(case, r"block_tables\[3\]\[39\] = " + str(bad))
    _expect_rejected(case, r"block_tables\[3\]\[39\]", split_tokens=256)


def test_unused_table_entries_are_not_checked(validate):
    case = small()
    case.block_tables[2, 1:] = -5             # sequence 2 has one token: only entry 0 is read
    case.block_tables[0, 2:] = 10 ** 6        # sequence 0 has 17 tokens: entries 0 and 1
    print("[case] validate unused entries", flush=True)
    out = _run.run_hip(case)
    torch.cuda.synchronize()
    _run.compare(out, _run.run_oracle(case), "bf16", what="unused entries out of range")


def test_noalloc_call_is_checked(validate):
    import decode_attention_paged_07_amd as pa
    case = small()
    case.block_tables[1, 5] = 999
    out = sentinel_out(case)
    cfg = case.cfg
    s, h, d = case.query.shape
    print("[case] validate noalloc", flush=True)
    rc = pa.pa_paged_attention_decode_noalloc(
        out.data_ptr(), case.query.data_ptr(), case.key_cache.data_ptr(), case.value_cache.data_ptr(), s, h,
        cfg.num_kv_heads, d, case.key_cache.shape[0], ctypes.c_float(case.scale), case.block_tables.data_ptr(),
        case.block_tables.shape[1], case.seq_lens.data_ptr(), cfg.block_size, case.max_seq_len, None, 1, 0, None,
        None, torch.cuda.current_stream(DEV).cuda_stream)
    torch.cuda.synchronize()
    assert rc == pa.PA_ERR_SHAPE and "block_tables[1][5] = 999" in pa.pa_last_error()
    assert (out.float() == SENTINEL).all()


def test_shared_prefix_call_is_checked(validate):
    import decode_attention_paged_07_amd as pa
    cfg = workloads.SHARED.with_(num_seqs=8, pool_blocks=400, prefix_groups=(4, 512))
    case = workloads.make_case(cfg, device=DEV)
    groups = pa.find_prefix_groups(case.meta.block_tables, case.meta.seq_lens, cfg.block_size)
    g = pa.prefix_groups(groups, cfg.num_seqs, DEV)
    case.seq_lens[5] = case.max_seq_len + 1
    out = sentinel_out(case)
    print("[case] validate shared", flush=True)
    with pytest.raises(ValueError, match=r"seq_lens\[5\]"):
        pa.paged_attention_decode_shared(out, case.query, case.key_cache, case.value_cache, cfg.num_kv_heads,
                                         case.scale, case.block_tables, case.seq_lens, cfg.block_size,
                                         case.max_seq_len, g)
    torch.cuda.synchronize()
    assert (out.float() == SENTINEL).all()


@pytest.mark.parametrize("kv", ["auto", "fp8_e4m3"])
@pytest.mark.parametrize("heads", [16, 128])
def test_latent_cache_calls_are_checked(validate, kv, heads):
    import decode_attention_paged_07_amd as pa
    lens = [40, 300, 7]
    base = workloads.MLA if kv == "auto" else workloads.MLA_FP8
    cfg = base.with_(num_seqs=3, num_heads=heads, pool_blocks=60)
    case = workloads.make_mla_case(cfg, seed=3, device=DEV, seq_lens=lens)
    out = torch.empty(3, heads, 512, dtype=torch.bfloat16, device=DEV)
    print(f"[case] validate mla kv={kv} H={heads}", flush=True)
    pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens,
                  case.max_seq_len, kv_scale=case.kv_scale)            # valid: runs
    torch.cuda.synchronize()
    case.block_tables[1, 18] = 60               # the 300-token sequence's last block (entry 18)
    out.fill_(SENTINEL)
    with pytest.raises(ValueError, match=r"block_tables\[1\]\[18\] = 60"):
        pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens,
                      case.max_seq_len, kv_scale=case.kv_scale)
    torch.cuda.synchronize()
    assert (out.float() == SENTINEL).all()


def test_capture_skips_the_check_and_replays(validate):
    """Under graph capture the check (which synchronises) is skipped; the
    captured call replays like an eager one."""
    case = small()
    out = _run.run_hip(case)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run.run_hip(case, out=out)
    for rep in range(2):
        out.fill_(SENTINEL)
        graph.replay()
        torch.cuda.synchronize()
        eager = _run.run_hip(case)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
