"""Benchmark of one paged decode-attention step on one MI355X.

A step is one call of the library's decode entry point (partition kernel plus,
when a sequence spans several splits, the reduce kernel) over one batch with
all inputs resident in HBM. Prints one JSON line.

Default workload: the bf16 GQA decode batch (128 sequences, 64 query / 8 kv
heads, head_size 128, block_size 16, lengths uniform in [1, 8192], 128K-block
pool), the configuration the bandwidth target is stated for.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "paged decode attn: seqs/s + effective KV-read HBM GB/s (% of MI355X peak)"
KERNEL_SRC = os.path.join(ROOT, "decode_attention_paged_07_amd", "csrc", "pa_kernels.hip")
WORKLOAD_TEXT = {
    "tiny": "tiny fp32 paged decode: 2 seqs {17,40}, 4/4 heads, D=64, bs=16, 16-block pool",
    "mha": "bf16 MHA decode: 64 seqs x 4096, 32/32 heads, D=128, bs=16, 32768-block pool",
    "gqa": "bf16 GQA decode: 128 seqs, lens U[1,8192] (seed 2), 64/8 heads, D=128, bs=16, "
           "131072-block pool",
    "long": "long-context split-KV + ALiBi: 8 seqs x 32768, 32/8 heads, D=128, bs=16, "
            "131072-block pool",
    "fp8": "fp8 e4m3 KV cache: 256 seqs, lognormal lens (median 4096, sigma 1, cap 16384, seed 4), "
           "64/8 heads, D=128, bs=16, bf16 q, 131072-block pool",
}


def kernel_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def kv_bytes(case) -> int:
    cfg = case.cfg
    e = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[cfg.q_dtype if cfg.kv_dtype == "auto" else cfg.kv_dtype]
    tokens = int(case.meta.seq_lens.astype("int64").sum())
    return tokens * cfg.num_kv_heads * cfg.head_size * 2 * e


def traffic_from_profiles(config: str):
    """HBM bytes per partition launch from committed rocprofv3 counter runs,
    only while the kernel source is unchanged since they were taken."""
    path = os.path.join(ROOT, "profiles", f"pa_partition_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(case, budget_s: float):
    """Time the fp64 oracle on the host over the first sequences of the batch
    until about budget_s seconds of work, and check the GPU output on them."""
    import numpy as np
    import threadpoolctl

    import oracle
    import workloads
    from tests import _run

    cores = min(len(os.sched_getaffinity(0)), 16)
    done, wall, cpu = [], 0.0, 0.0
    per_seq_est = None
    n = case.cfg.num_seqs
    with threadpoolctl.threadpool_limits(limits=cores):
        i = 0
        while i < n:
            # batches of sequences, sized from the measured per-sequence cost
            step = 1 if per_seq_est is None else max(1, min(n - i, int((budget_s - wall) / per_seq_est)))
            seqs = list(range(i, min(n, i + step)))
            h = workloads.host_arrays(case, seqs)           # host copy, not timed
            t0, c0 = time.perf_counter(), time.process_time()
            ref = oracle.paged_decode(h["query"], h["key_cache"], h["value_cache"], h["block_tables"],
                                      h["seq_lens"], h["scale"], q_kind=h["q_kind"],
                                      kv_kind=h["kv_kind"], alibi_slopes=h["alibi_slopes"],
                                      k_scale=h["k_scale"], v_scale=h["v_scale"])
            wall += time.perf_counter() - t0
            cpu += time.process_time() - c0
            done.append((seqs, ref))
            i += len(seqs)
            per_seq_est = wall / i
            if wall >= budget_s:
                break
    nseq = sum(len(s) for s, _ in done)
    tokens = int(case.meta.seq_lens[:nseq].astype("int64").sum())
    return {
        "value": nseq / wall, "unit": "seqs/s", "cores": cores, "kind": "oracle",
        "sample": f"first {nseq} of {n} sequences ({tokens} tokens), fp64 numpy oracle, "
                  f"host copy untimed, {wall:.1f} s wall",
        "cpu_util": round(cpu / wall, 2) if wall > 0 else None,
    }, done


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="gqa", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--split", type=int, default=0, help="split tokens (0 = library's choice)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path has no multi-GPU mode in this build).", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": args.steps}))
        return

    import decode_attention_paged_07_amd as pa
    import workloads
    from tests import _run

    cfg = workloads.CONFIGS[args.config]
    print(f"[bench] building {args.config} inputs", file=sys.stderr, flush=True)
    case = workloads.make_case(cfg, device=dev)
    out = torch.empty_like(case.query)
    split_tokens, num_splits, _ = pa.pa_decode_plan(cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads,
                                                    cfg.head_size, case.max_seq_len, args.split)

    def step():
        _run.run_hip(case, split_tokens=args.split, out=out)

    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # Timed region: exactly `steps` calls, synchronised on both sides.
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps, {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)

    # The same loop again with the library's per-kernel HIP events (recorded on
    # the stream the kernels run on) for the dominant kernel's launch time.
    pa.pa_timing_read()                       # drop anything recorded earlier
    pa.pa_timing_enable(True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    pa.pa_timing_enable(False)
    part_ms, part_n, red_ms, red_n = pa.pa_timing_read()
    ms_with_events = e0.elapsed_time(e1) / args.steps

    nbytes = kv_bytes(case)
    seqs_per_s = cfg.num_seqs / (ms_per_step / 1e3)
    gbps = nbytes / (ms_per_step / 1e3) / 1e9
    part_avg = part_ms / max(part_n, 1)
    achieved = nbytes / (part_avg / 1e3) / 1e9
    dtype = {"f32": "f32", "bf16": "bf16"}[cfg.q_dtype]
    if cfg.kv_dtype == "fp8_e4m3":
        dtype = "bf16 (fp8 e4m3 KV dequantised to bf16)"
    rec = {
        "metric": METRIC,
        "value": round(seqs_per_s, 1),
        "unit": "seqs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) values, seeded lengths and block tables)",
        "config": {
            "workload": WORKLOAD_TEXT[args.config],
            "num_seqs": cfg.num_seqs, "num_heads": cfg.num_heads, "num_kv_heads": cfg.num_kv_heads,
            "head_size": cfg.head_size, "block_size": cfg.block_size, "pool_blocks": cfg.pool_blocks,
            "tokens": int(case.meta.seq_lens.astype("int64").sum()), "max_seq_len": case.max_seq_len,
            "kv_bytes": nbytes,
            "scheduler": "stream-K" if split_tokens == 0 else f"split grid, {split_tokens}-token splits",
            "num_splits": num_splits,
        },
        "effective_kv_gbps": round(gbps, 1),
        "frac_of_peak_hbm": round(gbps / PEAK_HBM_GBPS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_streamk_kernel" if split_tokens == 0 else "pa_split_kernel",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic_from_profiles(args.config),
            "avg_launch_ms": round(part_avg, 5),
            "algorithmic_bytes_per_launch": nbytes,
        },
        "reduce_avg_ms": round(red_ms / red_n, 5) if red_n else 0.0,
        "ms_per_step_with_kernel_events": round(ms_with_events, 5),
        "kernel_sha": kernel_sha(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        step()
        torch.cuda.synchronize()
        base, done = cpu_baseline(case, args.cpu_seconds)
        worst = (0.0, 0.0)
        for seqs, ref in done:
            worst = tuple(max(a, b) for a, b in zip(worst, _run.compare(out, ref, cfg.q_dtype, seqs=seqs)))
        base["gpu_speedup"] = round(seqs_per_s / base["value"], 1)
        rec["cpu_baseline"] = base
        rec["parity_on_sample"] = {"max_abs": float(f"{worst[0]:.3e}"), "max_rel": float(f"{worst[1]:.3e}")}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
