#!/usr/bin/env python3
"""Benchmark of the sparse softmax-L1Norm hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
the metadata call (host work split) plus the main call (gather, MFMA QK,
mask, exp(s - lse), head mean, zero-filled row write), inputs already in
HBM. Default workload: DeepSeek-V3.2-shaped BSND (B=1, S1=S2=4096, N1=128,
N2=1, D=512, topk=2048, right-down causal, bf16).

Prints ONE JSON line. ``value`` is QK TFLOP/s = 2*N1*D*(valid pairs) / the
average step time; the effective HBM GB/s of the same step is given too.
``roofline`` reports the dominant kernel (the only kernel) against the
MI355X dense bf16/fp16 MFMA peak or the HBM peak, whichever bounds the
workload; its duration is measured with HIP events on the stream the kernel
is launched on. ``cpu_baseline`` times the CPU oracle (the test checker, as
it stands) on a bounded sample of the same workload's rows.

softmax_lse: timing runs use a stand-in of the right shape and magnitude
(log n + D*scale^2/2 per row), not the oracle's exact values; the work done
does not depend on the values.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}   # MI355X dense, published
PEAK_HBM_GBPS = 8000.0                                  # MI355X HBM3E, published
KERNELS = {0: "smla_l1norm_kernel", 1: "smla_wide_kernel"}  # metadata field 24
HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "sparse_mla_attention_02_amd", "csrc", "smla_kernels.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic(p, op="l1norm"):
    """(QK flops, unique HBM bytes) of one call on Problem p: the main call
    (softmax_lse in, the zero-filled output row out) or the lse call (the
    softmax_lse out, no output row)."""
    pairs = p.valid_pairs()
    flops = 2.0 * p.heads_q * p.head_dim * pairs
    nbytes = (p.q.numel() * p.q.element_size() + p.k.numel() * p.k.element_size()
              + p.rows * p.groups * 4                       # softmax_lse (in or out)
              + (p.sparse_indices.size * 4 if p.sparse_indices is not None else 0)
              + (p.topk_length.size * 4 if p.topk_length is not None else 0)
              + (p.cu_seqlens_q.size * 8 if p.cu_seqlens_q is not None else 0)
              + (p.cmp_residual_k.size * 4 if p.cmp_residual_k is not None else 0)
              + (p.rows * p.out_width * 4 if op == "l1norm" else 0))  # output row
    return flops, float(nbytes), pairs


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    profiles/<kernel>_<workload>_hbm_traffic.md (FETCH_SIZE + WRITE_SIZE,
    each scaled by the same counter's reading for a copy of known size), or
    None when there is none or the kernel source has changed since."""
    path = os.path.join(HERE, "profiles", f"{kernel}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            line = line.strip().strip("`")
            if ":" in line and line.split(":", 1)[0] in (
                    "kernel_source_sha256", "fetch_bytes_per_launch", "write_bytes_per_launch"):
                k, v = line.split(":", 1)
                fields[k] = v.strip()
    with open(KERNEL_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != sha:
        return None
    try:
        return int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(p, target_s, op="l1norm"):
    """Time the CPU oracle (oracle_l1norm given lse, or oracle_lse) on evenly
    spaced rows of the workload."""
    import oracle
    R = p.rows
    n = p.row_entries.reshape(R).astype(np.int64)
    # calibrate on a few rows per thread, then size the sample for ~target_s
    threads = oracle.num_threads()
    cal = np.linspace(0, R - 1, min(R, 4 * threads)).astype(np.int64)
    def run(rows):
        if op == "lse":
            oracle.lse(p, rows=rows)
        else:
            oracle.l1norm(p, rows=rows)

    run(cal[:threads])       # warm the thread pool
    t0 = time.perf_counter()
    run(cal)
    t_cal = time.perf_counter() - t0
    per_pair = t_cal / max(int(n[cal].sum()), 1)
    want_pairs = target_s / max(per_pair, 1e-12)
    count = int(np.clip(want_pairs / max(n.mean(), 1.0), 8, R))
    rows = np.linspace(0, R - 1, count).astype(np.int64)
    log(f"cpu baseline: oracle on {count} rows (~{count * n.mean() * per_pair:.1f} s)")
    t0 = time.perf_counter()
    run(rows)
    t = time.perf_counter() - t0
    pairs = int(n[rows].sum())
    flops = 2.0 * p.heads_q * p.head_dim * pairs
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{count} evenly spaced rows of {R} ({pairs} valid pairs), "
                      + ("oracle_lse" if op == "lse" else "oracle_l1norm given lse")
                      + f", {t:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--prewarm-seconds", type=float, default=0.5,
                    help="untimed steps run for this long before the warmup steps: an idle "
                         "GPU takes on the order of 100 ms of load to reach its working clock")
    ap.add_argument("--workload", default="dsv32")
    ap.add_argument("--op", choices=("l1norm", "lse"), default="l1norm",
                    help="l1norm: the Softmax-L1Norm call (the hot path); lse: the GPU "
                         "softmax_lse producer on the same workload")
    ap.add_argument("--kwide", action="store_true",
                    help="the main call with the K-wide output (entry t at column t)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (the "
                         "known-size reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.prewarm_seconds < 0:
        ap.error("--steps must be >= 1, --warmup and --prewarm-seconds >= 0")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    rank = int(os.environ.get("RANK", "0"))
    if args.gpus != 1 or world != 1:
        if rank == 0:
            print("bench.py measures one GPU only: this path has no multi-GPU mode "
                  "(query rows shard across GPUs with no exchange); run with --gpus 1",
                  file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import sparse_mla_attention_02_amd as smla
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": n}), flush=True)
        return

    log(f"generating workload {args.workload}")
    p = workloads.generate(args.workload)
    p.kwide = args.kwide and args.op == "l1norm"
    flops, nbytes, pairs = algorithmic(p, args.op)
    lse = workloads.lse_standin(p)
    p.softmax_lse = lse

    def t(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, k = p.q.to(dev), p.k.to(dev)
    lse_d = t(lse)
    idx, tlen = t(p.sparse_indices), t(p.topk_length)
    cu_q, cu_k, res = t(p.cu_seqlens_q), t(p.cu_seqlens_k), t(p.cmp_residual_k)
    cu_q_h = None if p.cu_seqlens_q is None else torch.from_numpy(p.cu_seqlens_q)
    cu_k_h = None if p.cu_seqlens_k is None else torch.from_numpy(p.cu_seqlens_k)
    if args.op == "lse":
        out = torch.empty(p.lse_shape(), dtype=torch.float32, device=dev)
    else:
        out = torch.empty(p.out_shape(), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(before=None, after=None):
        md = smla.smla_l1norm_metadata(
            p.heads_q, p.heads_k, p.head_dim, cu_seqlens_q=cu_q_h, cu_seqlens_k=cu_k_h,
            batch_size=p.batch, max_seqlen_q=p.max_seqlen_q, max_seqlen_k=p.max_seqlen_k,
            topk=p.topk, layout_q=p.layout, layout_k=p.layout, mask_mode=p.mask_mode,
            cmp_ratio=p.cmp_ratio, device=0)
        kw = dict(sparse_indices=idx, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                  cmp_residual_k=res, topk_length=tlen, metadata=md,
                  softmax_scale=p.softmax_scale, max_seqlen_k=p.max_seqlen_k,
                  cmp_ratio=p.cmp_ratio, mask_mode=p.mask_mode, layout_q=p.layout,
                  layout_k=p.layout, out=out)
        if before is not None:
            before.record(stream)
        if args.op == "lse":
            smla.smla_softmax_lse(q, k, **kw)
        else:
            smla.smla_softmax_l1norm(q, k, lse_d, kwide=p.kwide, **kw)
        if after is not None:
            after.record(stream)
        return md

    t_pre = time.perf_counter()
    n_pre = 0
    while time.perf_counter() - t_pre < args.prewarm_seconds:
        for _ in range(10):
            step()
        n_pre += 10
        torch.cuda.synchronize()
    log(f"prewarm {n_pre} steps; warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, each kernel bracketed by events on its stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        md = step(ev[i][0], ev[i][1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    ms_step = wall * 1e3 / args.steps
    kms = float(np.mean(kernel_ms))

    tflops = flops / (ms_step * 1e-3) / 1e12
    gbps = nbytes / (ms_step * 1e-3) / 1e9
    k_tflops = flops / (kms * 1e-3) / 1e12
    k_gbps = nbytes / (kms * 1e-3) / 1e9
    intensity = flops / nbytes
    ridge = PEAK_MFMA_TFLOPS[p.dtype] * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if intensity >= ridge:
        roof = {"bound": "mfma", "achieved": round(k_tflops, 2),
                "peak": PEAK_MFMA_TFLOPS[p.dtype], "unit": "TFLOP/s",
                "frac": round(k_tflops / PEAK_MFMA_TFLOPS[p.dtype], 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(k_gbps, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(k_gbps / PEAK_HBM_GBPS, 4)}
    kernel = "smla_lse_kernel" if args.op == "lse" else KERNELS.get(int(md[24]), "unknown")
    # (the committed counter summaries cover the S2-wide main call and the lse call)
    roof["traffic"] = None if p.kwide else measured_traffic(kernel, p.name)
    roof["kernel"] = kernel
    roof["kernel_ms"] = round(kms, 4)
    roof["algorithmic_flops"] = flops
    roof["algorithmic_bytes"] = nbytes

    metric = "QK TFLOP/s + HBM GB/s, sparse softmax-L1Norm N1=128 topk=2048 D=512"
    if args.op == "lse":
        metric = "QK TFLOP/s, GPU softmax_lse over the same selected keys"
    elif p.kwide:
        metric = "QK TFLOP/s, sparse softmax-L1Norm with the K-wide output"
    line = {
        "metric": metric,
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "prewarm_steps": n_pre, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p.dtype, "data": "synthetic",
        "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
        "config": {"workload": p.name, "layout": p.layout, "batch": p.batch,
                   "seqlen_q": p.seqlen_q, "seqlen_k": p.seqlen_k, "heads_q": p.heads_q,
                   "heads_k": p.heads_k, "head_dim": p.head_dim, "topk": p.topk,
                   "mask_mode": p.mask_mode, "cmp_ratio": p.cmp_ratio,
                   "valid_pairs": pairs, "op": args.op, "kwide": p.kwide,
                   "workgroups": int(md[4]) if args.op == "l1norm" else None,
                   "lse": "stand-in" if args.op == "l1norm" else "computed"},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds, args.op)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
