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

softmax_lse: computed on the GPU by the library's own lse call
(smla_softmax_lse) before the timed region, so the timed main call runs on
real inputs and its output is a proper distribution per row.

The line checks itself: after timing, the timed output is compared with the
CPU oracle (fed the same lse) on the rows the CPU baseline evaluates, every
row's sum is checked against 1, and the GPU lse against the oracle's lse on
a row sample; ``parity`` reports the result and a mismatch makes the run
exit with status 1. ``kernel_ms`` is the median of the per-launch HIP event
times; ``clock_mhz`` is the GPU's graphics clock from amdsmi's metrics table
(the mean over the XCDs of each snapshot), over the snapshots the driver
published while the untimed prewarm and warmup steps and the timed steps ran
(it refreshes them about once per second; null where amdsmi cannot read
them or none fell in that window).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

import numpy as np

PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}   # MI355X dense, published
PEAK_HBM_GBPS = 8000.0                                  # MI355X HBM3E, published
KERNELS = {0: "smla_l1norm_kernel", 1: "smla_wide_kernel", 2: "smla_narrow_kernel"}  # field 24
HERE = os.path.dirname(os.path.abspath(__file__))


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
    None when there is none or the kernel's source files have changed since."""
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
    from sparse_mla_attention_02_amd import _build
    if fields.get("kernel_source_sha256") != _build.kernel_source_sha256(kernel):
        return None
    try:
        return int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(p, target_s, op="l1norm", timed=True):
    """Time the CPU oracle (oracle_l1norm given lse, or oracle_lse) on evenly
    spaced rows of the workload. Returns (baseline dict or None, rows, the
    oracle's outputs on those rows); with ``timed`` False only a small sample
    is evaluated, for the parity check."""
    import oracle
    R = p.rows
    n = p.row_entries.reshape(R).astype(np.int64)
    threads = oracle.num_threads()

    def run(rows):
        if op == "lse":
            return oracle.lse(p, rows=rows)[0]
        return oracle.l1norm(p, rows=rows)

    if not timed:
        rows = np.unique(np.linspace(0, R - 1, min(R, 2 * threads)).astype(np.int64))
        return None, rows, run(rows)
    # calibrate on a few rows per thread, then size the sample for ~target_s
    cal = np.linspace(0, R - 1, min(R, 4 * threads)).astype(np.int64)
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
    out = run(rows)
    t = time.perf_counter() - t0
    pairs = int(n[rows].sum())
    flops = 2.0 * p.heads_q * p.head_dim * pairs
    base = {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{count} evenly spaced rows of {R} ({pairs} valid pairs), "
                      + ("oracle_lse" if op == "lse" else "oracle_l1norm given lse")
                      + f", {t:.1f} s wall"}
    return base, rows, out


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class ClockSampler:
    """Reads the GPU's graphics clocks (MHz) from amdsmi's metrics table in a
    thread while the steps run. The driver refreshes the table about once per
    second, so only snapshots that changed since the previous read count, and
    only those published at least `settle_s` after the sampler started (the
    clock needs load to rise). Every failure leaves the figures null: the
    clock is reported, never required."""

    def __init__(self, torch, dev_index=0, period_s=0.02, settle_s=0.25):
        self.snapshots = []  # mean clock over the XCDs, per fresh snapshot
        self.error = None
        self.period = period_s
        self.settle = settle_s
        self._stop = threading.Event()
        self._thread = None
        self._smi = None
        self._h = None
        self._last = None
        self._t0 = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            props = torch.cuda.get_device_properties(dev_index)
            want = (int(getattr(props, "pci_domain_id", 0)), int(props.pci_bus_id),
                    int(getattr(props, "pci_device_id", 0)))
            handles = amdsmi.amdsmi_get_processor_handles()
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)      # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self._h = h
            if self._h is None and len(handles) == 1:
                self._h = handles[0]
            if self._h is None:
                raise RuntimeError("no amdsmi handle matches the device's PCI address")
            self._smi = amdsmi
            self._read()
        except Exception as e:  # noqa: BLE001 (reporting only)
            self.error = f"{type(e).__name__}: {e}"
            self._smi = None

    def _read(self):
        """(snapshot key, mean graphics clock over the XCDs) of the current
        metrics table."""
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        clks = [float(c) for c in (m.get("current_gfxclks") or [])
                if isinstance(c, (int, float)) and 0 < c < 0xffff]
        if not clks:
            clks = [float(m["current_gfxclk"])]
        key = (m.get("system_clock_counter"), tuple(clks))
        return key, float(np.mean(clks))

    def _loop(self):
        while not self._stop.is_set():
            try:
                key, mhz = self._read()
            except Exception as e:  # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"
                return
            if self._last is not None and key != self._last and \
                    time.perf_counter() - self._t0 >= self.settle:
                self.snapshots.append(mhz)
            self._last = key
            self._stop.wait(self.period)

    def __enter__(self):
        if self._smi is not None:
            self._t0 = time.perf_counter()
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self):
        src = "amdsmi gpu metrics, current_gfxclks averaged over the XCDs"
        window = "prewarm, warmup and timed steps"
        if not self.snapshots:
            return {"median": None, "min": None, "max": None, "snapshots": 0, "source": src,
                    "window": window,
                    "error": self.error or "no metrics snapshot published in the window"}
        a = np.array(self.snapshots)
        return {"median": round(float(np.median(a)), 1), "min": round(float(a.min()), 1),
                "max": round(float(a.max()), 1), "snapshots": int(a.size), "source": src,
                "window": window}


TOL = 2e-5          # per element, and per lse value
ROWSUM_TOL = 1e-4   # per row with a used entry


def parity_check(p, op, out_rows, lse_rows, rows, expect, lse_sample):
    """The timed output against the oracle. ``out_rows``: (R, W) output (main
    call) or (R, G) lse (lse call) as numpy; ``expect``: the oracle on
    ``rows``; ``lse_sample``: (rows, oracle lse) for the main call's lse."""
    res = {"rows_checked": int(len(rows))}
    err = np.abs(out_rows[rows].astype(np.float64) - expect.astype(np.float64))
    if op == "lse":
        dead = np.isneginf(expect)
        ok_inf = bool(np.array_equal(np.isneginf(out_rows[rows]), dead))
        e = err[~dead]
        res["max_abs_err"] = float(e.max()) if e.size else 0.0
        res["ok"] = ok_inf and res["max_abs_err"] <= TOL
        return res
    res["max_abs_err"] = float(err.max()) if err.size else 0.0
    live = p.row_entries.reshape(p.rows) > 0
    sums = out_rows.astype(np.float64).sum(axis=1)
    res["max_rowsum_dev"] = float(np.abs(sums[live] - 1.0).max()) if live.any() else 0.0
    res["empty_rows_zero"] = bool(not out_rows[~live].any())
    lrows, lwant = lse_sample
    got = lse_rows[lrows]
    dead = np.isneginf(lwant)
    lerr = np.abs(got[~dead].astype(np.float64) - lwant[~dead].astype(np.float64))
    res["lse_rows_checked"] = int(len(lrows))
    res["lse_max_abs_err"] = float(lerr.max()) if lerr.size else 0.0
    res["ok"] = bool(res["max_abs_err"] <= TOL and res["max_rowsum_dev"] <= ROWSUM_TOL
                     and res["empty_rows_zero"] and res["lse_max_abs_err"] <= TOL
                     and np.array_equal(np.isneginf(got), dead))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--prewarm-seconds", type=float, default=1.5,
                    help="untimed steps run for this long before the warmup steps: an idle "
                         "GPU takes on the order of 100 ms of load to reach its working "
                         "clock, and the clock figures come from metrics the driver "
                         "refreshes about once per second")
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

    def t(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, k = p.q.to(dev), p.k.to(dev)
    idx, tlen = t(p.sparse_indices), t(p.topk_length)
    cu_q, cu_k, res = t(p.cu_seqlens_q), t(p.cu_seqlens_k), t(p.cmp_residual_k)
    cu_q_h = None if p.cu_seqlens_q is None else torch.from_numpy(p.cu_seqlens_q)
    cu_k_h = None if p.cu_seqlens_k is None else torch.from_numpy(p.cu_seqlens_k)
    if args.op == "lse":
        out = torch.empty(p.lse_shape(), dtype=torch.float32, device=dev)
    else:
        out = torch.empty(p.out_shape(), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def metadata():
        return smla.smla_l1norm_metadata(
            p.heads_q, p.heads_k, p.head_dim, cu_seqlens_q=cu_q_h, cu_seqlens_k=cu_k_h,
            batch_size=p.batch, max_seqlen_q=p.max_seqlen_q, max_seqlen_k=p.max_seqlen_k,
            topk=p.topk, layout_q=p.layout, layout_k=p.layout, mask_mode=p.mask_mode,
            cmp_ratio=p.cmp_ratio, device=0)

    def call_args(md, o):
        return dict(sparse_indices=idx, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                    cmp_residual_k=res, topk_length=tlen, metadata=md,
                    softmax_scale=p.softmax_scale, max_seqlen_k=p.max_seqlen_k,
                    cmp_ratio=p.cmp_ratio, mask_mode=p.mask_mode, layout_q=p.layout,
                    layout_k=p.layout, out=o)

    # the main call's softmax_lse input, computed untimed by the GPU lse call
    lse_d = None
    if args.op == "l1norm":
        lse_d = torch.empty(p.lse_shape(), dtype=torch.float32, device=dev)
        smla.smla_softmax_lse(q, k, **call_args(metadata(), lse_d))
        torch.cuda.synchronize()
        p.softmax_lse = lse_d.cpu().numpy()

    def step(before=None, after=None):
        md = metadata()
        kw = call_args(md, out)
        if before is not None:
            before.record(stream)
        if args.op == "lse":
            smla.smla_softmax_lse(q, k, **kw)
        else:
            smla.smla_softmax_l1norm(q, k, lse_d, kwide=p.kwide, **kw)
        if after is not None:
            after.record(stream)
        return md

    # the graphics clock, read while the untimed and the timed steps run
    clock = ClockSampler(torch, 0)
    clock.__enter__()
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
    try:
        t0 = time.perf_counter()
        for i in range(args.steps):
            md = step(ev[i][0], ev[i][1])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        clock.__exit__(None, None, None)
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    ms_step = wall * 1e3 / args.steps
    kms = float(np.median(kernel_ms))

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
    if args.op == "lse":
        # up to 64 heads: the small-head pipelined kernel; 65..128 heads with at
        # most 2048 indices (or dense): the one for 65..128 heads
        if p.groups <= 64:
            kernel = "smla_lse_narrow_kernel"
        elif p.sparse_indices is None or p.topk <= 2048:
            kernel = "smla_lse_wide_kernel"
        else:
            kernel = "smla_lse_kernel"
    else:
        kernel = KERNELS.get(int(md[24]), "unknown")
    # (the committed counter summaries cover the S2-wide main call and the lse call)
    roof["traffic"] = None if p.kwide else measured_traffic(kernel, p.name)
    roof["kernel"] = kernel
    roof["kernel_ms"] = round(kms, 4)
    roof["kernel_ms_mean"] = round(float(np.mean(kernel_ms)), 4)
    roof["kernel_ms_min"] = round(float(np.min(kernel_ms)), 4)
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
                   "lse": "computed (smla_softmax_lse, untimed)" if args.op == "l1norm"
                          else "output"},
        "roofline": roof,
        "clock_mhz": clock.summary(),
        "cpu_baseline": None,
        "parity": None,
    }
    # the timed output (every step wrote the same values) against the oracle
    out_rows = out.reshape(p.rows, -1).cpu().numpy()
    base, rows, expect = cpu_baseline(p, args.cpu_seconds, args.op,
                                      timed=not args.no_cpu_baseline)
    line["cpu_baseline"] = base
    lse_sample = None
    lse_rows = None
    if args.op == "l1norm":
        import oracle
        lrows = np.unique(np.linspace(0, p.rows - 1, min(p.rows, 64)).astype(np.int64))
        lse_sample = (lrows, oracle.lse(p, rows=lrows)[0])
        lse_rows = p.softmax_lse.reshape(p.rows, p.groups)
    line["parity"] = parity_check(p, args.op, out_rows, lse_rows, rows, expect, lse_sample)
    print(json.dumps(line), flush=True)
    if not line["parity"]["ok"]:
        log(f"PARITY FAILED: {line['parity']}")
        sys.exit(1)


if __name__ == "__main__":
    main()
