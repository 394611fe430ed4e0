"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance (element-wise, |gpu - oracle| <= atol + rtol*|oracle|): 1e-5 / 1e-5
for fp32 inputs and outputs, 1e-2 / 1e-2 for bf16 and fp8-dequantised inputs
with bf16 outputs (fp32 accumulation throughout).
"""

import math

import numpy as np
import pytest
import torch

import workloads
from tests import _golden, _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def check(case, seqs=None, split_tokens=0, what=""):
    print(f"[case] {what} cfg={case.cfg.name} S={case.cfg.num_seqs} H={case.cfg.num_heads} "
          f"Hkv={case.cfg.num_kv_heads} D={case.cfg.head_size} kv={case.cfg.kv_dtype} "
          f"split={split_tokens}", flush=True)
    out = _run.run_hip(case, split_tokens=split_tokens)
    torch.cuda.synchronize()
    ref = _run.run_oracle(case, seqs)
    return out, _run.compare(out, ref, case.cfg.q_dtype, seqs=seqs, what=what or case.cfg.name)


# ---------------------------------------------------------------------------
# Hand-derived example and the tiny fp32 workload.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("alibi", [False, True])
def test_worked_example(alibi):
    import decode_attention_paged_07_amd as pa
    ex = _golden.worked_example(alibi)
    t = {k: torch.from_numpy(v).to(DEV) for k, v in ex.items()
         if isinstance(v, np.ndarray) and k != "expect"}
    out = torch.empty_like(t["query"])
    pa.paged_attention_decode(out, t["query"], t["key_cache"], t["value_cache"], 1, ex["scale"],
                              t["block_tables"], t["seq_lens"], 16, 3,
                              alibi_slopes=t.get("alibi_slopes"))
    torch.cuda.synchronize()
    _run.compare(out, ex["expect"], "f32", what="worked example")


def test_tiny_config():
    check(workloads.make_case(workloads.TINY, device=DEV), what="tiny")


# ---------------------------------------------------------------------------
# Reduced-size versions of each workload: several splits, ragged tails.
# ---------------------------------------------------------------------------

SMALL = {
    "mha": workloads.MHA.with_(num_seqs=6, pool_blocks=512, seq_lens=("uniform", 1, 1100)),
    "gqa": workloads.GQA.with_(num_seqs=10, pool_blocks=1024, seq_lens=("uniform", 1, 1500)),
    "long": workloads.LONG.with_(num_seqs=2, pool_blocks=512, seq_lens=("const", 3000)),
    "fp8": workloads.FP8.with_(num_seqs=10, pool_blocks=1024, seq_lens=("lognormal", 300, 1.0, 1800)),
    "tiny128": workloads.TINY.with_(head_size=128, num_seqs=5, num_heads=8, num_kv_heads=2,
                                    pool_blocks=128, seq_lens=("uniform", 1, 700)),
}


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("split", [0, 256, 512])
def test_small_workloads(name, split):
    case = workloads.make_case(SMALL[name], device=DEV)
    check(case, split_tokens=split, what=f"{name}-small")


@pytest.mark.parametrize("name", ["gqa", "fp8", "mha"])
def test_head_size_64(name):
    cfg = SMALL[name].with_(head_size=64)
    check(workloads.make_case(cfg, device=DEV), what=f"{name}-d64")


@pytest.mark.parametrize("name", ["gqa", "fp8", "mha", "long", "tiny128"])
@pytest.mark.parametrize("split", [0, 256])
def test_head_size_32(name, split):
    """Head size 32: one K chunk step for bf16, two for f32, and half-chunk
    K loads for the fp8 cache (a token has only two 16-byte chunks)."""
    cfg = SMALL[name].with_(head_size=32)
    check(workloads.make_case(cfg, device=DEV), split_tokens=split, what=f"{name}-d32")


@pytest.mark.parametrize("group", [1, 2, 3, 4, 7, 8, 16])
@pytest.mark.parametrize("kv", ["auto", "fp8_e4m3"])
def test_group_sizes(group, kv):
    cfg = workloads.GQA.with_(num_seqs=4, num_kv_heads=2, num_heads=2 * group, pool_blocks=256,
                              seq_lens=("uniform", 1, 900), kv_dtype=kv)
    check(workloads.make_case(cfg, device=DEV), what=f"group{group}-{kv}")


# ---------------------------------------------------------------------------
# Edge cases.
# ---------------------------------------------------------------------------

EDGE_LENS = (1, 15, 16, 17, 255, 256, 257, 511, 512, 513, 40, 2)


@pytest.mark.parametrize("kv,q", [("auto", "bf16"), ("fp8_e4m3", "bf16"), ("auto", "f32")])
def test_edge_lengths_with_nan_poison(kv, q):
    """Tail slots, unused blocks and unused table entries hold NaN; never read."""
    cfg = workloads.GQA.with_(num_seqs=len(EDGE_LENS), num_heads=16, num_kv_heads=4,
                              pool_blocks=160, seq_lens=("fixed", EDGE_LENS), kv_dtype=kv, q_dtype=q)
    for split in (0, 256):
        case = workloads.make_case(cfg, device=DEV, poison=True, max_seq_len=900)
        out, _ = check(case, split_tokens=split, what=f"edge-poison-{kv}-{q}-{split}")
        assert torch.isfinite(out.float()).all()


def test_zero_length_sequences():
    cfg = workloads.GQA.with_(num_seqs=4, num_heads=16, num_kv_heads=4, pool_blocks=64,
                              seq_lens=("fixed", (0, 20, 0, 300)))
    case = workloads.make_case(cfg, device=DEV)
    out = torch.full_like(case.query, float("nan"))
    _run.run_hip(case, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out[0].float().cpu(), torch.zeros(16, 128))
    assert torch.equal(out[2].float().cpu(), torch.zeros(16, 128))
    ref = _run.run_oracle(case, [1, 3])
    _run.compare(out, ref, "bf16", seqs=[1, 3], what="zero-length neighbours")


@pytest.mark.parametrize("num_seqs", [129, 1100])
def test_many_sequences(num_seqs):
    # More than 128 sequences take the stream-K start-up scan in batches of
    # 16 x 64 sequences; 1100 spans two batches, the second one partial, and
    # about a fifth of the sequences are empty, some at chunk boundaries.
    rng = np.random.default_rng(num_seqs)
    lens = rng.integers(1, 41, num_seqs)
    lens[rng.random(num_seqs) < 0.2] = 0
    lens[[i for i in (63, 64, 127, 128, 511, 512) if i < num_seqs]] = 0
    cfg = workloads.GQA.with_(num_seqs=num_seqs, num_heads=8, num_kv_heads=2, pool_blocks=4096,
                              seq_lens=("fixed", tuple(int(x) for x in lens)))
    print(f"[case] {num_seqs} sequences, {int((lens == 0).sum())} empty", flush=True)
    case = workloads.make_case(cfg, device=DEV, poison=True)
    out = _run.run_hip(case)
    torch.cuda.synchronize()
    ref = _run.run_oracle(case)
    _run.compare(out, ref, "bf16", what=f"{num_seqs} sequences")


def test_max_seq_len_above_longest():
    cfg = workloads.GQA.with_(num_seqs=5, pool_blocks=256, seq_lens=("uniform", 1, 400))
    case = workloads.make_case(cfg, device=DEV, max_seq_len=3000)
    check(case, what="max_seq_len>max(L)")


def test_shared_prefix_blocks():
    cfg = workloads.GQA.with_(num_seqs=6, pool_blocks=512, seq_lens=("fixed", (600, 300, 520, 40, 1, 700)))
    case = workloads.make_case(cfg, device=DEV, share_prefix_blocks=20)
    check(case, what="shared-prefix")


def test_fp8_distinct_scales():
    """k_scale != v_scale, both keeping decoded values of unit scale (the
    tolerance is stated for N(0,1)-sized inputs: the bf16 rounding of the
    softmax weights gives an error proportional to |V|)."""
    cfg = SMALL["fp8"]
    s = workloads.make_case(cfg, device=DEV).k_scale
    case = workloads.make_case(cfg, device=DEV, k_scale=0.5 * s, v_scale=2.0 * s)
    assert case.k_scale != case.v_scale
    check(case, what="fp8 k_scale!=v_scale")


def test_alibi_with_gqa_and_fp8():
    cfg = SMALL["fp8"].with_(alibi=True)
    check(workloads.make_case(cfg, device=DEV), what="fp8+alibi")


def test_scale_edge_values():
    cfg = SMALL["gqa"]
    case = workloads.make_case(cfg, device=DEV)
    for scale in (0.0, 1.0):
        case.scale = scale
        check(case, what=f"scale={scale}")


def test_deterministic_bitwise():
    case = workloads.make_case(SMALL["gqa"], device=DEV)
    a = _run.run_hip(case).clone()
    b = _run.run_hip(case).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_split_sizes_agree():
    case = workloads.make_case(SMALL["long"], device=DEV)
    outs = []
    for split in (256, 512, 1024, 2048, 4096):
        out, _ = check(case, split_tokens=split, what=f"long split {split}")
        outs.append(out.float())
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() < 2e-2


def _split_partials(ws, s, h, ns, d):
    """(tmp_out [S,H,P,D], max_logits [S,H,P], exp_sums [S,H,P]) from a split
    plan's workspace, carved as pa_decode_plan documents: fp32 arrays, each at
    a 256-byte-aligned offset."""
    rows = s * h * ns

    def up(v):
        return (v + 255) // 256 * 256
    f = ws.cpu().view(torch.float32).numpy()
    tmp = f[:rows * d].reshape(s, h, ns, d)
    o1 = up(rows * d * 4) // 4
    ml = f[o1: o1 + rows].reshape(s, h, ns)
    o2 = (up(rows * d * 4) + up(rows * 4)) // 4
    es = f[o2: o2 + rows].reshape(s, h, ns)
    return tmp, ml, es


def _check_partials(case, ws, ns, what):
    """The GPU's per-partition (tmp_out, max_logits, exp_sums) against the
    oracle's partitioned form, for every partition a sequence uses."""
    import oracle
    s, h, d = case.query.shape
    tmp, ml, es = _split_partials(ws, s, h, ns, d)
    hst = workloads.host_arrays(case)
    _, o_tmp, o_ml, o_es = oracle.paged_decode_partitioned(
        hst["query"], hst["key_cache"], hst["value_cache"], hst["block_tables"], hst["seq_lens"],
        hst["scale"], q_kind=hst["q_kind"], kv_kind=hst["kv_kind"], alibi_slopes=hst["alibi_slopes"],
        k_scale=hst["k_scale"], v_scale=hst["v_scale"])
    for si, n in enumerate(case.meta.seq_lens.tolist()):
        used = math.ceil(n / 256)
        if used <= 1:
            continue                                   # one partition: written to out directly
        np.testing.assert_allclose(ml[si, :, :used], o_ml[si, :, :used], rtol=1e-4, atol=1e-3,
                                   err_msg=f"{what} max_logits seq {si}")
        np.testing.assert_allclose(es[si, :, :used], o_es[si, :, :used], rtol=1e-2, atol=1e-2,
                                   err_msg=f"{what} exp_sums seq {si}")
        np.testing.assert_allclose(tmp[si, :, :used], o_tmp[si, :, :used], rtol=1e-2, atol=1e-2,
                                   err_msg=f"{what} tmp_out seq {si}")


def test_workspace_partials_match_oracle_partitions():
    """With 256-token splits the workspace holds the pages' per-partition
    (tmp_out, max_logits, exp_sums); compare them with the oracle's."""
    import decode_attention_paged_07_amd as pa
    cfg = SMALL["long"].with_(seq_lens=("fixed", (1000, 513)))
    case = workloads.make_case(cfg, device=DEV)
    s, h, d = case.query.shape
    st, ns, wb = pa.pa_decode_plan(s, h, cfg.num_kv_heads, d, case.max_seq_len, 256)
    assert st == 256 and ns == math.ceil(case.max_seq_len / 256)
    ws = torch.full((wb,), 0, dtype=torch.uint8, device=DEV)
    _run.run_hip(case, split_tokens=256, workspace=ws)
    torch.cuda.synchronize()
    _check_partials(case, ws, ns, "long-small")


def test_alibi_partition_golden_on_gpu():
    """tests/golden/alibi_partitions.txt on the GPU: with 256-token splits the
    workspace's max_logits are the hand-derived -5.5 and 0 (the ALiBi term is
    zero on the newest token), the exp-sums and partial outputs their closed
    forms; both plans give the closed-form output."""
    import decode_attention_paged_07_amd as pa
    ex = _golden.alibi_partitions()
    t = {k: torch.from_numpy(v).to(DEV) for k, v in ex.items()
         if isinstance(v, np.ndarray) and k in ("query", "key_cache", "value_cache", "block_tables", "seq_lens",
                                                  "alibi_slopes")}
    n = int(ex["seq_lens"][0])
    st, ns, wb = pa.pa_decode_plan(1, 1, 1, 64, n, 256)
    assert (st, ns) == (256, 2)
    ws = torch.full((wb,), 0, dtype=torch.uint8, device=DEV)
    for split in (256, 0):
        print(f"[case] alibi partition golden split={split}", flush=True)
        out = torch.full_like(t["query"], float("nan"))
        pa.paged_attention_decode(out, t["query"], t["key_cache"], t["value_cache"], 1, ex["scale"],
                                  t["block_tables"], t["seq_lens"], 16, n, alibi_slopes=t["alibi_slopes"],
                                  split_tokens=split, workspace=ws if split else None)
        torch.cuda.synchronize()
        _run.compare(out, ex["expect"], "f32", what=f"alibi partition golden split={split}")
        if split:
            tmp, ml, es = _split_partials(ws, 1, 1, 2, 64)
            np.testing.assert_allclose(ml[0, 0], ex["m"], rtol=0, atol=1e-5)
            np.testing.assert_allclose(es[0, 0], ex["s"], rtol=1e-5, atol=0)
            np.testing.assert_allclose(tmp[0, 0], ex["tmp"], rtol=1e-5, atol=1e-6)


C_KV = {"auto": 0, "fp8_e4m3": 1}
C_Q = {"f32": 0, "bf16": 1}


@pytest.mark.parametrize("name,kw", [
    ("gqa", {}), ("fp8", {}), ("tiny128", {}), ("long", {"alibi": True}), ("mha", {"head_size": 64}),
])
def test_plain_c_entry_point(name, kw):
    """pa_paged_attention_decode, the headline C entry, called directly through
    ctypes with a workspace sized by pa_decode_plan."""
    import ctypes
    import decode_attention_paged_07_amd as pa
    cfg = SMALL[name].with_(**kw)
    case = workloads.make_case(cfg, device=DEV, poison=True)
    s, h, d = case.query.shape
    ks = vs = None
    if cfg.kv_dtype != "auto":
        ks = torch.tensor([case.k_scale], dtype=torch.float32, device=DEV)
        vs = torch.tensor([case.v_scale], dtype=torch.float32, device=DEV)
    _, _, need = pa.pa_decode_plan(s, h, cfg.num_kv_heads, d, case.max_seq_len, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.full_like(case.query, float("nan"))
    print(f"[case] plain C entry {name} {kw}", flush=True)
    rc = pa.pa_paged_attention_decode(
        out.data_ptr(), case.query.data_ptr(), case.key_cache.data_ptr(), case.value_cache.data_ptr(), s, h,
        cfg.num_kv_heads, d, case.key_cache.shape[0], ctypes.c_float(case.scale), case.block_tables.data_ptr(),
        case.block_tables.shape[1], case.seq_lens.data_ptr(), cfg.block_size, case.max_seq_len,
        case.alibi_slopes.data_ptr() if case.alibi_slopes is not None else None, C_Q[cfg.q_dtype],
        C_KV[cfg.kv_dtype], ks.data_ptr() if ks is not None else None, vs.data_ptr() if vs is not None else None,
        ws.data_ptr(), need, torch.cuda.current_stream(DEV).cuda_stream)
    assert rc == pa.PA_OK, pa.pa_last_error()
    torch.cuda.synchronize()
    _run.compare(out, _run.run_oracle(case), cfg.q_dtype, what=f"plain C entry {name}")


# ---------------------------------------------------------------------------
# Full-size workloads: every sequence against the oracle, in the launch
# configuration the benchmark times (the default stream-K plan) and in the
# pages' 256-token partition plan.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["gqa", "fp8", "mha", "long"])
def test_full_size_every_sequence(name):
    cfg = workloads.CONFIGS[name]
    case = workloads.make_case(cfg, device=DEV)
    print(f"[case] {name} full size: {cfg.num_seqs} sequences, {int(case.meta.seq_lens.sum())} tokens",
          flush=True)
    ref = _run.run_oracle(case)
    for split in (0, 256):
        out = torch.full_like(case.query, float("nan"))
        _run.run_hip(case, split_tokens=split, out=out)
        torch.cuda.synchronize()
        mabs, mrel = _run.compare(out, ref, cfg.q_dtype, what=f"{name}-full split={split}")
        print(f"[full] {name} split={split}: all {cfg.num_seqs} sequences, max_abs={mabs:.2e} "
              f"max_rel={mrel:.2e}", flush=True)
        assert torch.isfinite(out.float()).all()
    del case, out
    _free()


def test_full_size_long_partition_partials():
    """The long-context workload (8 x 32768 tokens, ALiBi) in the pages'
    256-token partition plan: 128 partitions per sequence, every partition's
    (tmp_out, max_logits, exp_sums) against the oracle's partitioned form."""
    import decode_attention_paged_07_amd as pa
    cfg = workloads.CONFIGS["long"]
    case = workloads.make_case(cfg, device=DEV)
    s, h, d = case.query.shape
    st, ns, wb = pa.pa_decode_plan(s, h, cfg.num_kv_heads, d, case.max_seq_len, 256)
    assert (st, ns) == (256, 128)
    ws = torch.zeros(wb, dtype=torch.uint8, device=DEV)
    print("[case] long full size, 256-token partials", flush=True)
    _run.run_hip(case, split_tokens=256, workspace=ws)
    torch.cuda.synchronize()
    _check_partials(case, ws, ns, "long-full")
    del case, ws
    _free()
