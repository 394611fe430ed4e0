"""GPU parity of the fp8-arithmetic decode (PA_KV_FP8_E4M3_COMPUTE, through
the C ABI) against its fp64 oracle, which applies the same quantisation rules:
MX-quantised q, per-block e4m3 P relative to 2^ceil(block max). Both sides
round a computed 2^(z - c) to e4m3, the kernel from a float32 z, so where that
value sits within float32 error of a rounding midpoint they may pick
neighbouring codes; tests/_fp8tol.py bounds what such picks can move, and the
comparison allows exactly that on top of the bf16 output tolerance."""

import numpy as np
import pytest
import torch

import workloads
from tests import _fp8tol, _golden, _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def check(case, split_tokens=0, seqs=None, what=""):
    cfg = case.cfg
    print(f"[case] {what}: bs={cfg.block_size} S={cfg.num_seqs} H={cfg.num_heads} Hkv={cfg.num_kv_heads} "
          f"D={cfg.head_size} alibi={cfg.alibi} split={split_tokens}", flush=True)
    out = _run.run_hip(case, split_tokens=split_tokens, compute="fp8")
    torch.cuda.synchronize()
    ref = _run.run_oracle_fp8(case, seqs)
    extra = _fp8tol.row_bounds(workloads.host_arrays(case, seqs))
    mabs, mrel = _run.compare(out, ref, "bf16", seqs=seqs, what=what, extra=extra)
    g = out.float().cpu().numpy()[list(seqs) if seqs is not None else slice(None)]
    strict = np.abs(g - ref) <= 1e-2 + 1e-2 * np.abs(ref)
    print(f"[ok] {what}: max_abs={mabs:.2e} max_rel={mrel:.2e}; elements needing the rounding "
          f"allowance: {int((~strict).sum())} of {strict.size}; largest allowance {extra.max():.2e}", flush=True)
    return out, ref


SMALL = workloads.FP8.with_(num_seqs=10, pool_blocks=1024, seq_lens=("lognormal", 300, 1.0, 1800))


@pytest.mark.parametrize("d", [128, 64, 32])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("split", [0, 256])
def test_small_fp8_compute(d, bs, split):
    cfg = SMALL.with_(head_size=d, block_size=bs, pool_blocks=1024 * 16 // bs)
    check(workloads.make_case(cfg, device=DEV), split_tokens=split, what=f"fp8c-d{d}-bs{bs}")


@pytest.mark.parametrize("group", [1, 4, 8, 16])
def test_group_sizes_fp8_compute(group):
    cfg = SMALL.with_(num_seqs=4, num_kv_heads=2, num_heads=2 * group, pool_blocks=256,
                      seq_lens=("uniform", 1, 900))
    check(workloads.make_case(cfg, device=DEV), what=f"fp8c-group{group}")


def test_alibi_fp8_compute():
    cfg = SMALL.with_(alibi=True, num_heads=32, num_kv_heads=8)
    check(workloads.make_case(cfg, device=DEV), split_tokens=512, what="fp8c-alibi")


@pytest.mark.parametrize("bs", [16, 32])
def test_edge_lengths_with_nan_poison_fp8_compute(bs):
    lens = (1, 7, 8, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 2)
    cfg = SMALL.with_(num_seqs=len(lens), num_heads=16, num_kv_heads=4, pool_blocks=8192 // bs,
                      seq_lens=("fixed", lens), block_size=bs)
    for split in (0, 256):
        case = workloads.make_case(cfg, device=DEV, poison=True, max_seq_len=900)
        out, _ = check(case, split_tokens=split, what=f"fp8c-edge-bs{bs}-{split}")
        assert torch.isfinite(out.float()).all()


def test_golden_example_on_gpu():
    """The hand-derived example of tests/golden/fp8_compute_example.txt."""
    import decode_attention_paged_07_amd as pa
    ex = _golden.fp8_compute_example()
    q = torch.from_numpy(ex["query"].view(np.int16)).view(torch.bfloat16).to(DEV)
    kc = torch.from_numpy(ex["key_cache"]).to(DEV)
    vc = torch.from_numpy(ex["value_cache"]).to(DEV)
    out = torch.empty_like(q)
    print("[case] fp8-compute golden example", flush=True)
    pa.paged_attention_decode(out, q, kc, vc, 1, ex["scale"], torch.from_numpy(ex["block_tables"]).to(DEV),
                              torch.from_numpy(ex["seq_lens"]).to(DEV), 16, 16, kv_cache_dtype="fp8",
                              compute="fp8")
    torch.cuda.synchronize()
    _run.compare(out, ex["expect"], "bf16", what="fp8-compute golden")


def test_full_size_fp8_compute_sampled():
    """The fp8 workload (256 sequences, lognormal lengths up to 16384) in the
    automatic launch plan; sampled sequences against the fp8-arithmetic oracle
    (the oracle runs at well under a sequence per second, so the batch is
    sampled) and against exact attention of the unquantised queries, within
    the derived bound tests/_fp8tol.exact_attention_bound (q and P
    quantisation) plus the kernel-to-oracle allowance and the bf16 output
    tolerance. The fp8 arithmetic is not held to the 1e-2 tolerance of the
    bf16-arithmetic paths against exact attention: its P carries three
    mantissa bits."""
    cfg = workloads.FP8
    case = workloads.make_case(cfg, device=DEV)
    lens = case.meta.seq_lens
    rng = np.random.default_rng(cfg.seed)
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens))} |
                  set(int(i) for i in rng.choice(len(lens), 3, replace=False)))
    out, ref = check(case, seqs=seqs, what="fp8c-full")
    h = workloads.host_arrays(case, seqs)
    extra = _fp8tol.row_bounds(h)
    exact, bound = _fp8tol.exact_attention_bound(h)
    g = out.float().cpu().numpy()[seqs]
    dev = np.abs(g - exact)
    allowed = 1e-2 + 1e-2 * np.abs(ref) + extra + bound
    print(f"[full] fp8 compute vs exact attention on seqs {seqs}: max_abs={dev.max():.3e} "
          f"mean_abs={dev.mean():.3e}; largest derived bound {bound.max():.3e}; largest fraction of the "
          f"allowance used {(dev / allowed).max():.3f}", flush=True)
    assert (dev <= allowed).all()
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("bs", [16, 32])
def test_shared_prefix_fp8_compute(bs):
    """The shared-prefix call with fp8 arithmetic: prefix blocks read once per
    group, each block's P quantised by the same rule, so the same oracle."""
    import decode_attention_paged_07_amd as pa
    cfg = SMALL.with_(num_seqs=16, pool_blocks=16384 // bs, seq_lens=("uniform", 1, 500), prefix_groups=(8, 480),
                      block_size=bs)
    case = workloads.make_case(cfg, device=DEV)
    groups = pa.find_prefix_groups(case.meta.block_tables, case.meta.seq_lens, bs)
    assert groups
    g = pa.prefix_groups(groups, cfg.num_seqs, DEV)
    out = torch.empty_like(case.query)
    print(f"[case] shared fp8 compute bs={bs}", flush=True)
    pa.paged_attention_decode_shared(out, case.query, case.key_cache, case.value_cache, cfg.num_kv_heads,
                                     case.scale, case.block_tables, case.seq_lens, bs, case.max_seq_len, g,
                                     kv_cache_dtype="fp8", k_scale=case.k_scale, v_scale=case.v_scale,
                                     compute="fp8")
    torch.cuda.synchronize()
    ref = _run.run_oracle_fp8(case)
    extra = _fp8tol.row_bounds(workloads.host_arrays(case))
    mabs, _ = _run.compare(out, ref, "bf16", what=f"shared fp8 compute bs{bs}", extra=extra)
    print(f"[ok] shared fp8 compute bs{bs}: max_abs={mabs:.2e}", flush=True)

