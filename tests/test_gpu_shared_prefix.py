"""GPU parity of the shared-prefix decode (through the C ABI) against the fp64
oracle, which needs no notion of groups: shared physical blocks are just equal
table entries. Tolerances as for the plain decode."""

import numpy as np
import pytest
import torch

import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def run_shared(case, groups=None):
    import decode_attention_paged_07_amd as pa
    if groups is None:
        groups = pa.find_prefix_groups(case.meta.block_tables, case.meta.seq_lens, case.cfg.block_size)
    g = pa.prefix_groups(groups, case.cfg.num_seqs, DEV)
    out = torch.empty_like(case.query)
    pa.paged_attention_decode_shared(out, case.query, case.key_cache, case.value_cache, case.cfg.num_kv_heads,
                                     case.scale, case.block_tables, case.seq_lens, case.cfg.block_size,
                                     case.max_seq_len, g, alibi_slopes=case.alibi_slopes,
                                     kv_cache_dtype=case.cfg.kv_dtype, k_scale=case.k_scale,
                                     v_scale=case.v_scale)
    return out, groups


def check(case, what, groups=None, seqs=None):
    print(f"[case] {what}: bs={case.cfg.block_size} S={case.cfg.num_seqs} H={case.cfg.num_heads} "
          f"Hkv={case.cfg.num_kv_heads} "
          f"D={case.cfg.head_size} kv={case.cfg.kv_dtype} groups={case.cfg.prefix_groups}", flush=True)
    out, groups = run_shared(case, groups)
    torch.cuda.synchronize()
    assert groups, "the case has no shared prefix"
    ref = _run.run_oracle(case, seqs)
    return out, _run.compare(out, ref, case.cfg.q_dtype, seqs=seqs, what=what)


SMALL = {
    "gqa8-group8": workloads.GQA.with_(num_seqs=16, pool_blocks=1024, seq_lens=("uniform", 1, 600),
                                       prefix_groups=(8, 320)),
    "gqa8-group11": workloads.GQA.with_(num_seqs=22, pool_blocks=1024, seq_lens=("uniform", 1, 300),
                                        prefix_groups=(11, 160)),
    "mha-group20": workloads.MHA.with_(num_seqs=20, num_heads=8, num_kv_heads=8, pool_blocks=512,
                                       seq_lens=("uniform", 1, 200), prefix_groups=(20, 256)),
    "alibi-g4-group6": workloads.LONG.with_(num_seqs=12, pool_blocks=1024, seq_lens=("uniform", 1, 900),
                                            prefix_groups=(6, 1024)),
    "fp8-group8": workloads.FP8.with_(num_seqs=16, pool_blocks=1024, seq_lens=("uniform", 1, 500),
                                      prefix_groups=(8, 480)),
    "f32-d128-group5": workloads.TINY.with_(num_seqs=10, num_heads=16, num_kv_heads=2, head_size=128,
                                            pool_blocks=512, seq_lens=("uniform", 1, 200),
                                            prefix_groups=(5, 96)),
    "f32-d64-group4": workloads.TINY.with_(num_seqs=8, num_heads=8, num_kv_heads=4, pool_blocks=256,
                                           seq_lens=("uniform", 1, 100), prefix_groups=(4, 64)),
    "gqa8-d32-group8": workloads.GQA.with_(num_seqs=16, pool_blocks=1024, seq_lens=("uniform", 1, 600),
                                           prefix_groups=(8, 320), head_size=32),
    "fp8-d32-group8": workloads.FP8.with_(num_seqs=16, pool_blocks=1024, seq_lens=("uniform", 1, 500),
                                          prefix_groups=(8, 480), head_size=32),
    "f32-d32-group4": workloads.TINY.with_(num_seqs=8, num_heads=8, num_kv_heads=4, pool_blocks=256,
                                           seq_lens=("uniform", 1, 100), prefix_groups=(4, 64), head_size=32),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_shared_prefix_matches_oracle(name):
    check(workloads.make_case(SMALL[name], device=DEV), name)


def test_members_out_of_order_and_ungrouped_neighbours():
    """Groups given with shuffled member order; some sequences in no group,
    one of length zero, one whose whole length is the prefix."""
    cfg = workloads.GQA.with_(num_seqs=12, pool_blocks=1024, seq_lens=("uniform", 1, 400), prefix_groups=(4, 256))
    lens = None
    case = workloads.make_case(cfg, device=DEV, seq_lens=lens)
    import decode_attention_paged_07_amd as pa
    groups = pa.find_prefix_groups(case.meta.block_tables, case.meta.seq_lens)
    assert len(groups) == 3
    groups = [(list(reversed(m)), p) for m, p in groups[:2]]          # group 3 left out: plain path
    # sequence 1 ends exactly at the prefix; sequence 10 (ungrouped) is empty
    sl = case.meta.seq_lens.copy()
    sl[1] = 256
    sl[10] = 0
    case.meta.seq_lens = sl
    case.seq_lens = torch.from_numpy(sl).to(DEV)
    check(case, "out of order + ungrouped", groups=groups)


def test_shared_equals_plain_decode():
    import decode_attention_paged_07_amd as pa
    case = workloads.make_case(SMALL["gqa8-group8"], device=DEV)
    out_s, _ = run_shared(case)
    out_p = _run.run_hip(case)
    torch.cuda.synchronize()
    assert (out_s.float() - out_p.float()).abs().max().item() < 2e-2


def test_full_size_shared_workload_sampled():
    cfg = workloads.SHARED
    case = workloads.make_case(cfg, device=DEV)
    rng = np.random.default_rng(0)
    seqs = sorted(set(rng.choice(cfg.num_seqs, 6, replace=False).tolist()) | {0, 7, 127})
    out, (mabs, mrel) = check(case, "shared full size", seqs=seqs)
    print(f"[full] shared: sampled seqs {seqs} max_abs={mabs:.2e} max_rel={mrel:.2e}", flush=True)
    assert torch.isfinite(out.float()).all()


def test_no_groups_is_the_plain_decode():
    """With no groups the shared call runs only its per-sequence part and the
    merge; it must still equal the oracle (and the plain call)."""
    import decode_attention_paged_07_amd as pa
    case = workloads.make_case(SMALL["gqa8-group8"], device=DEV)
    g = pa.prefix_groups([], case.cfg.num_seqs, DEV)
    out = torch.empty_like(case.query)
    print("[case] shared call without groups", flush=True)
    pa.paged_attention_decode_shared(out, case.query, case.key_cache, case.value_cache, case.cfg.num_kv_heads,
                                     case.scale, case.block_tables, case.seq_lens, case.cfg.block_size,
                                     case.max_seq_len, g)
    torch.cuda.synchronize()
    _run.compare(out, _run.run_oracle(case), case.cfg.q_dtype, what="no groups")
