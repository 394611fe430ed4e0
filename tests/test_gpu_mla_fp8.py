"""GPU parity of the fp8 (e4m3fn) latent cache: decode (pa_mla_decode_fp8)
against the fp64 MLA oracle on the codes' values times the scale, and the fp8
latent append (pa_mla_cache_append_fp8) against the oracle's codes bit for bit.

The decode converts the codes to bf16 exactly and then runs the bf16
arithmetic, so the tolerance is the bf16 one: |gpu - oracle| <= 1e-2 +
1e-2 * |oracle| element-wise.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _run

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
WIDTH = 576


def host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def run_mla(case, out=None, kv_scale=None):
    import decode_attention_paged_07_amd as pa
    if out is None:
        out = torch.empty(case.cfg.num_seqs, case.cfg.num_heads, 512, dtype=torch.bfloat16, device=DEV)
    pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens,
                  case.max_seq_len, kv_scale=case.kv_scale if kv_scale is None else kv_scale)
    return out


def oracle_mla(case, seqs=None):
    h = workloads.mla_host_arrays(case, seqs)
    assert h["kv_kind"] == "e4m3fn"
    return oracle.mla_decode(h["query"], h["latent_cache"], h["block_tables"], h["seq_lens"], h["scale"], 512,
                             q_kind="bf16", kv_kind="e4m3fn", kv_scale=h["kv_scale"])


def check(case, seqs=None, what=""):
    print(f"[case] mla fp8 {what} S={case.cfg.num_seqs} H={case.cfg.num_heads} "
          f"lens={case.meta.seq_lens[:8].tolist()} kv_scale={case.kv_scale:.4g}", flush=True)
    out = run_mla(case)
    torch.cuda.synchronize()
    return out, _run.compare(out, oracle_mla(case, seqs), "bf16", seqs=seqs, what=what)


def small(lens, heads=16, seed=11, poison=True, pool=None):
    lens = list(lens)
    need = sum(-(-n // 16) for n in lens)
    cfg = workloads.MLA_FP8.with_(num_seqs=len(lens), num_heads=heads, pool_blocks=pool or need + 8)
    return workloads.make_mla_case(cfg, seed=seed, device=DEV, seq_lens=lens, poison=poison)


def test_cache_holds_codes_in_the_x16_layout():
    import decode_attention_paged_07_amd as pa
    case = small([5])
    assert case.latent_cache.dtype == torch.uint8
    assert tuple(case.latent_cache.shape) == pa.mla_cache_shape(case.cfg.pool_blocks, fp8=True)


@pytest.mark.parametrize("lens", [[1], [16], [17, 40, 3], [255, 256, 257], [1000, 31, 512]])
def test_ragged_lengths_poisoned_tails(lens):
    check(small(lens), what=f"lens {lens}")


@pytest.mark.parametrize("heads", [1, 8, 17, 40, 64, 65, 100, 128])
def test_head_counts(heads):
    # from 65 heads the fp8 cache runs the 16-heads-per-wave kernel with two
    # workgroups per share
    check(small([70, 300, 5, 129], heads=heads, seed=heads), what=f"H={heads}")


def requantise(case, s):
    """Re-store the case's row values (codes times its scale, about N(0,1))
    as the e4m3fn codes of value / s and make s the scale: the values keep
    their size while the codes and the scale change (s below amax/448 clips
    them at 448 s, above it rounds them more coarsely). NaN codes stay NaN."""
    vals = case.latent_cache.view(torch.float8_e4m3fn).to(torch.float32) * case.kv_scale
    case.latent_cache.copy_((vals / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8))
    case.kv_scale = s


@pytest.mark.parametrize("kv_scale", [1.0 / 64, 1.0 / 8, 0.5])
def test_scale_values(kv_scale):
    case = small([33, 700, 2], seed=4)
    requantise(case, kv_scale)
    check(case, what=f"kv_scale {kv_scale}")


def test_scale_as_device_tensor_matches_float():
    case = small([300, 45], seed=6)
    a = run_mla(case)
    b = run_mla(case, kv_scale=torch.tensor([case.kv_scale], dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_zero_length_sequences_give_zero_rows():
    out, _ = check(small([0, 5, 0, 33]), what="zero lengths")
    assert not out[0].any() and not out[2].any()


def test_long_sequences_cut_into_many_segments():
    check(small([8192, 3000]), what="segments")


def test_long_sequences_many_heads():
    check(small([6000, 2500, 17], heads=128, seed=5), what="segments H=128")


def test_many_short_sequences():
    lens = np.random.default_rng(8).integers(1, 65, 300).tolist()
    check(small(lens, seed=8, poison=False), what="300 short")


@pytest.mark.parametrize("seed", range(6))
def test_random_configurations(seed):
    rng = np.random.default_rng(2000 + seed)
    heads = int(rng.integers(1, 129))
    n = int(rng.integers(1, 41))
    lens = rng.integers(0, 3001, n)
    lens[rng.random(n) < 0.1] = 0
    check(small(lens.tolist(), heads=heads, seed=seed), what=f"random {seed}: H={heads}")


@pytest.mark.parametrize("name", ["mla_fp8", "mla128_fp8"])
def test_full_size_workload(name):
    """The full-size fp8 latent-cache workloads in the benchmark's launch
    configuration: every sequence (16 heads) or every 8th (128 heads)."""
    cfg = workloads.MLA_CONFIGS[name]
    case = workloads.make_mla_case(cfg, device=DEV)
    seqs = None if cfg.num_heads <= 16 else list(range(0, cfg.num_seqs, 8))
    out, (max_abs, max_rel) = check(case, seqs=seqs, what=f"{name} full size")
    print(f"[{name}] max_abs={max_abs:.3e} max_rel={max_rel:.3e}", flush=True)
    assert torch.isfinite(out.float()).all()
    del case
    torch.cuda.empty_cache()


def test_captured_call_replays_like_eager():
    cfg = workloads.MLA_FP8.with_(num_seqs=5, pool_blocks=500)
    case = workloads.make_mla_case(cfg, seed=21, device=DEV, seq_lens=[1, 300, 1200, 17, 2500])
    ks = torch.tensor([case.kv_scale], dtype=torch.float32, device=DEV)
    out = run_mla(case, kv_scale=ks)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_mla(case, out, kv_scale=ks)
    torch.cuda.synchronize()
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    for rep, f in enumerate((1.25, 0.8, 1.0)):          # the last replay at the cache's own scale
        case.query.copy_(torch.randn(case.query.shape, generator=g, device=DEV).to(torch.bfloat16))
        ks.fill_(case.kv_scale * f)
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = run_mla(case, kv_scale=ks)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
    case.kv_scale = float(ks.item())
    _run.compare(got, oracle_mla(case), "bf16", what="graph mla fp8")


# --- fp8 append ---------------------------------------------------------------

def make_append(S, T, pool, seed, positions=None):
    import decode_attention_paged_07_amd as pa
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    rng = np.random.default_rng(seed)
    cache = torch.randint(0, 256, pa.mla_cache_shape(pool, fp8=True), generator=g, device=DEV,
                          dtype=torch.int32).to(torch.uint8)
    max_blocks = pool // S
    table = rng.permutation(pool)[:S * max_blocks].reshape(S, max_blocks).astype(np.int32)
    if positions is None:
        positions = rng.integers(-1, max_blocks * 16 - T + 1, S).astype(np.int32)
    rows = (torch.randn((S, T, WIDTH), generator=g, device=DEV) * 3).to(torch.bfloat16)
    return dict(cache=cache, table=torch.from_numpy(table).to(DEV),
                positions=torch.from_numpy(np.asarray(positions, np.int32)).to(DEV), rows=rows)


def check_append(c, kv_scale, what):
    import decode_attention_paged_07_amd as pa
    print(f"[case] mla fp8 append {what}: rows={tuple(c['rows'].shape)} scale={kv_scale}", flush=True)
    before = host(c["cache"])
    pa.mla_cache_append(c["cache"], c["rows"], c["table"], c["positions"], kv_scale=kv_scale)
    torch.cuda.synchronize()
    ref = oracle.append_latent(before, host(c["rows"]), host(c["table"]), host(c["positions"]),
                               kv_kind="e4m3fn", kv_scale=float(np.float32(kv_scale)))
    bad = np.argwhere(host(c["cache"]) != ref)
    assert bad.size == 0, f"{what}: latent cache differs in {len(bad)} bytes, first {bad[:4].tolist()}"


@pytest.mark.parametrize("T", [1, 3, 16, 19])
@pytest.mark.parametrize("kv_scale", [1.0, 0.0117, 5.0])
def test_append_matches_oracle(T, kv_scale):
    check_append(make_append(S=6, T=T, pool=48, seed=T * 7 + 3), kv_scale, f"T={T}")


def test_append_every_bf16_pattern():
    """All 65536 bf16 bit patterns (NaN, +-0, subnormals, huge values) as row
    elements: every code equals the oracle's."""
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    S, T = 16, 8                                       # 16 * 8 * 576 >= 65536
    c = make_append(S=S, T=T, pool=64, seed=2, positions=[16 * (s % 4) for s in range(S)])
    flat = torch.cat([bits, bits[: S * T * WIDTH - 65536]])
    c["rows"] = flat.reshape(S, T, WIDTH).to(DEV).contiguous()
    check_append(c, 0.3, "every bf16 pattern")


def test_append_edge_positions_and_bad_entries():
    c = make_append(S=8, T=2, pool=64, seed=3, positions=[0, 15, 16, 31, 8 * 16 - 2, -1, 8 * 16 - 1, -100])
    t = c["table"].cpu()
    t[1, 1] = 10 ** 6
    t[3, 2] = -3
    c["table"] = t.to(DEV)
    check_append(c, 0.05, "edge positions, bad entries")


def test_append_then_decode_reads_the_new_rows():
    import decode_attention_paged_07_amd as pa
    lens = [1, 15, 16, 17, 300, 704]
    need = sum(-(-n // 16) for n in lens) + len(lens)
    cfg = workloads.MLA_FP8.with_(num_seqs=len(lens), num_heads=16, pool_blocks=need + 8)
    case = workloads.make_mla_case(cfg, seed=44, device=DEV, seq_lens=lens, max_seq_len=720)
    meta = case.meta
    used = set(meta.used_blocks.tolist())
    free = (b for b in range(cfg.pool_blocks) if b not in used)
    table = case.block_tables.cpu().numpy()
    for s, n in enumerate(lens):
        if n % 16 == 0:
            table[s, n // 16] = next(free)
    case.block_tables = torch.from_numpy(table).to(DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    rows = torch.randn((len(lens), WIDTH), generator=g, device=DEV).to(torch.bfloat16)
    pos = case.seq_lens.clone()
    before = host(case.latent_cache)
    print("[case] mla fp8 append then decode", flush=True)
    pa.mla_cache_append(case.latent_cache, rows, case.block_tables, pos, kv_scale=case.kv_scale)
    case.seq_lens += 1
    out = torch.empty(len(lens), 16, 512, dtype=torch.bfloat16, device=DEV)
    pa.mla_decode(out, case.query, case.latent_cache, case.scale, case.block_tables, case.seq_lens, 720,
                  kv_scale=case.kv_scale)
    torch.cuda.synchronize()
    ks = float(np.float32(case.kv_scale))
    grown = oracle.append_latent(before, host(rows)[:, None], host(case.block_tables), host(pos),
                                 kv_kind="e4m3fn", kv_scale=ks)
    ref = oracle.mla_decode(host(case.query), grown, host(case.block_tables), host(case.seq_lens), case.scale,
                            512, q_kind="bf16", kv_kind="e4m3fn", kv_scale=ks)
    _run.compare(out, ref, "bf16", what="mla fp8 append then decode")
