#!/usr/bin/env python3
"""Benchmark one decode step of attention over a KV cache on one MI355X.

A step is one kvattn_decode call over one batch of the workload: one kernel
launch (every split-KV workgroup, with the log-sum-exp merge done by the last
workgroup of each sequence and KV head), the whole batch, one layer.  Inputs are
seeded synthetic tensors already resident in HBM.  Several identical copies of
the K/V caches are rotated between steps so that each step streams its K/V from
HBM rather than from the 256 MB last-level (Infinity) cache.

Prints ONE JSON line:
  value           effective HBM GB/s = algorithmic bytes / wall time per step, for the
                  default workload: the largest of the five (paged_100k, 819 MB a step)
  roofline        the decode kernel timed with HIP events on the library's stream,
                  against MI355X's 8 TB/s HBM3E peak
  other_workloads the other workloads of the 70 %-of-peak target (decode_7b,
                  spec_verify, sink_window), timed the same way in the same run, and
                  decode_7b / spec_verify with the KV append fused in
                  (kvattn_append_decode, "+append": one launch writes the new rows
                  and attends; bytes add the new rows read and written)
  ceiling_gbs     a plain streaming read of 256 MiB and 1 GiB (the library's
                  yardstick kernel): the read bandwidth this device reaches in practice
  cpu_baseline    the oracle (test infrastructure) timed on the host cores over a
                  bounded sample of the same workload, with the host CPU model
"""
import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from kv_cache_attention_amd import accounting, workloads  # noqa: E402
from kv_cache_attention_amd import binding as kb  # noqa: E402

METRIC = "decode-attention effective HBM GB/s (% of MI355X peak) and µs/step, 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # dense matrix-core peaks, MI355X
MALL_BYTES = 256 << 20
COPY_BYTES = 1 << 30   # plain copy of known size, the yardstick for the traffic counters
PROFILES = os.path.join(ROOT, "profiles")
KERNELS = ["valu", "mfma", "prefill_mfma"]
# the other workloads of the 70 %-of-peak target (the default line is the largest)
OTHERS = ("decode_7b", "spec_verify", "sink_window")
# the same steps with the KV append fused in (one launch: write the new rows, attend)
APPEND_OTHERS = ("decode_7b+append", "spec_verify+append")
DEVICE_WARMUP_MS = 100  # plain streaming reads before the warmup steps (clock ramp)


def kernel_source_hash() -> str:
    """Hash of the HIP sources and of the build script (its compiler flags): HBM traffic
    measured for other sources or flags is not reported."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "kv_cache_attention_amd")
    csrc = os.path.join(pkg, "csrc")
    files = [(name, os.path.join(csrc, name)) for name in sorted(os.listdir(csrc))
             if name.endswith((".hip", ".hpp", ".cpp"))]
    files.append(("build.py", os.path.join(pkg, "build.py")))
    for name, path in files:
        with open(path, "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, layout: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel sources (else None)."""
    import json as _json
    path = os.path.join(PROFILES, f"traffic_{workload}_{layout}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = _json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="paged_100k", choices=list(workloads.CONFIGS))
    ap.add_argument("--layout", default="head_major", choices=["token_major", "head_major"])
    ap.add_argument("--split-len", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="K/V copies rotated (0 = auto)")
    ap.add_argument("--others", default=",".join(OTHERS + APPEND_OTHERS),
                    help="further workloads timed in the same run ('' = none)")
    ap.add_argument("--other-steps", type=int, default=100)
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = auto)")
    return ap.parse_args()


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, d, out, n_rows, step_bytes):
    """Time the oracle on the host over a sample of output rows (median of three runs)
    and check those rows."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(1234)
    total = case.batch * case.q_len * case.num_q_heads
    idx = np.sort(rng.choice(total, size=min(n_rows, total), replace=False))
    rows = np.stack([idx // (case.q_len * case.num_q_heads),
                     (idx // case.num_q_heads) % case.q_len,
                     idx % case.num_q_heads], axis=1).astype(np.int32)
    q, kc, vc = d["q"].cpu(), d["k_cache"].cpu(), d["v_cache"].cpu()
    bt = d["block_table"].cpu() if d["block_table"] is not None else None
    sl = d["seq_lens"].cpu()
    tm = d["tree_mask"].cpu() if d.get("tree_mask") is not None else None
    threads = oracle.threads()
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        ref = oracle.decode_rows(case, q, kc, vc, bt, sl, rows, k_scale=d["k_scale"],
                                 v_scale=d["v_scale"], tree_mask=tm)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[1]
    # the sample's share of the step's algorithmic bytes, so the rate is in the metric's unit
    byts = step_bytes * len(rows) / total
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    err = float(np.abs(got - ref).max())
    return {"value": round(byts / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{len(rows)} of {total} output rows of the same workload "
                      f"(float64 naive softmax, OpenMP over rows; median of 3 runs)",
            "host_cpu": host_cpu(), "nproc": os.cpu_count(),
            "parity_max_abs_on_sample": err}


class Workload:
    """One workload resident on the device, with rotated K/V copies and a handle bound
    to its own stream."""

    def __init__(self, case, layout, split_len=0, copies=0, dev=None, append=False):
        self.case = case
        d = workloads.make_inputs(case, device="cuda")
        self.d = d
        sl_host = d["seq_lens"].cpu().tolist()
        self.step_bytes = accounting.step_bytes(case, sl_host)
        # append fused into the step (kvattn_append_decode): the q_len new K and V rows
        # per sequence and KV head are read from k_new / v_new and written to the cache
        self.append = append
        if append:
            g = torch.Generator().manual_seed(case.seed + 1000)
            shape = (case.batch, case.q_len, case.num_kv_heads, case.head_dim)
            dt = kb.TORCH_DTYPE[case.kv_dtype or case.dtype]
            assert dt != torch.uint8, "fused-append workloads use 16-bit or 32-bit caches"
            self.k_new = torch.randn(shape, generator=g).to(dt).to(d["q"].device)
            self.v_new = torch.randn(shape, generator=g).to(dt).to(d["q"].device)
            self.step_bytes += 2 * 2 * self.k_new.numel() * self.k_new.element_size()
        self.step_flops = accounting.step_flops(case, sl_host)
        # multiply-adds the rows really do (row by row; the union count above is an upper
        # bound): decides whether the step is bound by the matrix cores or by HBM
        self.row_flops = (4 * case.head_dim * accounting.attended_pairs(case, sl_host)
                          if case.mask_mode != "tree" else self.step_flops)
        self.mfma_bound = (case.dtype in MFMA_PEAK_TFLOPS and self.row_flops / self.step_bytes >
                           MFMA_PEAK_TFLOPS[case.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9))
        self.seq_lens_sum = int(sum(sl_host))
        kv_attended = self.step_bytes - 2 * case.batch * case.q_len * case.num_q_heads * \
            case.head_dim * accounting.ELEM_BYTES[case.dtype]
        self.copies = copies or min(64, max(2, -(-4 * MALL_BYTES // max(kv_attended, 1))))
        kcs, vcs = [d["k_cache"]], [d["v_cache"]]
        for _ in range(self.copies - 1):
            kcs.append(d["k_cache"].clone())
            vcs.append(d["v_cache"].clone())
        if layout == "head_major":
            kcs = [k.permute(0, 2, 1, 3).contiguous() for k in kcs]
            vcs = [v.permute(0, 2, 1, 3).contiguous() for v in vcs]
        self.kcs, self.vcs = kcs, vcs
        self.h = kb.KVAttn.for_case(case, layout=layout)
        if split_len:
            self.h.set_split_len(split_len)
        if getattr(case, "kv_dtype", None) == "fp8":
            self.h.set_kv_scales(d["k_scale"], d["v_scale"])
        self.plan = self.h.plan(case.q_len, case.mask_mode, case.n_sink, case.window)
        self.stream = torch.cuda.Stream(dev)   # default priority
        self.out = torch.empty_like(d["q"])
        kb.kvattn_set_stream(self.h.h, self.stream.cuda_stream)
        self.mask = kb.MASK[case.mask_mode]

    def step(self, c, out=None):
        case, d = self.case, self.d
        out = self.out if out is None else out
        if self.append:
            kb.kvattn_append_decode(self.h.h, d["q"], self.k_new, self.v_new, self.kcs[c],
                                    self.vcs[c], d["block_table"], d["seq_lens"], case.q_len,
                                    self.mask, case.n_sink, case.window, out)
        elif case.mask_mode == "tree":
            kb.kvattn_decode_tree(self.h.h, d["q"], self.kcs[c], self.vcs[c], d["block_table"],
                                  d["seq_lens"], case.q_len, d["tree_mask"], out)
        else:
            kb.kvattn_decode(self.h.h, d["q"], self.kcs[c], self.vcs[c], d["block_table"],
                             d["seq_lens"], case.q_len, self.mask, case.n_sink, case.window, out)

    def settle(self, ms=DEVICE_WARMUP_MS):
        """Keep the device busy for `ms` with plain streaming reads of the K/V copies before
        the warmup steps: after the seconds of host-side input drawing the device has
        dropped its clocks, and the first launches would be timed while they ramp up."""
        sink = torch.zeros(4, dtype=torch.int32, device=self.d["q"].device)
        t0 = time.perf_counter()
        n = 0
        while (time.perf_counter() - t0) * 1e3 < ms:
            c = n % self.copies
            kb.kvattn_stream_read(self.kcs[c], sink, self.stream.cuda_stream)
            kb.kvattn_stream_read(self.vcs[c], sink, self.stream.cuda_stream)
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()

    def time(self, steps, warmup):
        """The timed region: `steps` back-to-back steps, bracketed by a host sync and wall
        clock and by HIP events recorded on the handle's stream (average launch duration
        = event time / steps).  Then the same steps again, each bracketed by its own
        pair of events (launch-by-launch spread)."""
        self.settle()
        for w in range(warmup):
            self.step(w % self.copies)
        torch.cuda.synchronize()
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        r0.record(self.stream)
        for s in range(steps):
            self.step(s % self.copies)
        r1.record(self.stream)
        t_enq = time.perf_counter() - t0
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        region_ms = r0.elapsed_time(r1)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for s in range(steps):
            evs[s][0].record(self.stream)
            self.step(s % self.copies)
            evs[s][1].record(self.stream)
        torch.cuda.synchronize()
        ev_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        return {"ms_per_step": wall * 1e3 / steps, "enqueue_us": t_enq * 1e6 / steps,
                "launch_ms": region_ms / steps,
                "ev_mean_ms": sum(ev_ms) / len(ev_ms), "ev_med_ms": ev_ms[len(ev_ms) // 2]}

    def output_for_copy0(self):
        out = torch.empty_like(self.d["q"])
        self.step(0, out)
        torch.cuda.synchronize()
        return out

    def close(self):
        self.h.close()


def ceiling(dev, sizes=(256 << 20, 1 << 30), reps=30):
    """Achievable read bandwidth: the library's plain streaming read, `reps` back-to-back
    launches between HIP events, over buffers rotated so every read comes from HBM (at
    least 1 GiB in rotation)."""
    stream = torch.cuda.Stream(dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    res = {}
    for size in sizes:
        n = max(2, -(-(1 << 30) // size) + 1)
        bufs = [torch.ones(size // 4, dtype=torch.float32, device=dev) for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(3):
            kb.kvattn_stream_read(bufs[i % n], sink, stream.cuda_stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            kb.kvattn_stream_read(bufs[i % n], sink, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[f"{size >> 20}MiB"] = round(size / (ms * 1e-3) / 1e9, 1)
        del bufs
    torch.cuda.empty_cache()
    return res


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this library's "
              f"decode path is single-GPU, see the sharding notes.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kb.load()  # fail loudly if the HIP library is missing
    case = workloads.CONFIGS[a.config]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = Workload(case, a.layout, a.split_len, a.copies, dev)
    n_split, split_len, kernel = w.plan
    t = w.time(a.steps, a.warmup)
    ms_per_step, launch_ms = t["ms_per_step"], t["launch_ms"]
    step_bytes, row_flops = w.step_bytes, w.row_flops

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = step_bytes / (launch_ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "host_enqueue_us_per_step": round(t["enqueue_us"], 2),
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "device_warmup": f"{DEVICE_WARMUP_MS} ms of plain streaming reads of the K/V copies "
                         "before the warmup steps (the clocks ramp up after host-side setup)",
        "vs_baseline": None,
        "dtype": case.dtype if not getattr(case, "kv_dtype", None) else
                 f"{case.dtype} (K/V {case.kv_dtype} e4m3)",
        "data": "synthetic (seeded N(0,1) x scale, host CPU generators)",
        "config": {
            "workload": case.name, "batch": case.batch, "num_q_heads": case.num_q_heads,
            "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
            "q_len": case.q_len, "cache": case.cache_mode, "capacity": case.capacity,
            "mask": case.mask_mode, "n_sink": case.n_sink, "window": case.window,
            "seq_lens_sum": w.seq_lens_sum, "layout": a.layout,
            "n_split": n_split, "split_len": split_len,
            "kernel": KERNELS[kernel], "kv_copies_rotated": w.copies,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "row_flops_per_step": row_flops,
            "traffic": measured_traffic(case.name, a.layout),
            "bytes_per_step": step_bytes,
            "flops_per_step": w.step_flops,
            "launch_us": round(launch_ms * 1e3, 2),
            "bracketed_us_mean": round(t["ev_mean_ms"] * 1e3, 2),
            "bracketed_us_median": round(t["ev_med_ms"] * 1e3, 2),
            "timed": "the decode kernel (split-KV + fused merge), one launch per step: "
                     "HIP events on the library's stream around the timed region's "
                     f"{a.steps} back-to-back launches (launch_us = region / steps); "
                     "bracketed_us_* = the same steps each between its own event pair",
        },
    }
    if w.mfma_bound:  # the matrix cores bound this step: flops per launch against their peak
        tf = row_flops / (launch_ms * 1e-3) / 1e12
        rec["roofline"].update({"bound": "mfma", "achieved": round(tf, 2),
                                "peak": MFMA_PEAK_TFLOPS[case.dtype], "unit": "TFLOP/s",
                                "frac": round(tf / MFMA_PEAK_TFLOPS[case.dtype], 4),
                                "hbm_gbs": round(achieved, 2)})
    rec["config"]["kernel_source_hash"] = kernel_source_hash()
    out0 = None if a.no_cpu_baseline else w.output_for_copy0()
    w.close()
    del w
    torch.cuda.empty_cache()

    # the other workloads of the 70 %-of-peak target, timed the same way in the same run
    others = {}
    for name in [n for n in a.others.split(",") if n and n != case.name]:
        base, _, suffix = name.partition("+")  # "<workload>+append": kvattn_append_decode
        o = Workload(workloads.CONFIGS[base], a.layout, 0, 0, dev, append=suffix == "append")
        ot = o.time(a.other_steps, a.warmup)
        ach = o.step_bytes / (ot["launch_ms"] * 1e-3) / 1e9
        others[name] = {"us_per_step": round(ot["ms_per_step"] * 1e3, 2),
                        "launch_us": round(ot["launch_ms"] * 1e3, 2),
                        "bracketed_us_mean": round(ot["ev_mean_ms"] * 1e3, 2),
                        "bytes_per_step": o.step_bytes, "achieved_gbs": round(ach, 1),
                        "bound": "hbm", "frac": round(ach / HBM_PEAK_GBS, 4),
                        "kernel": KERNELS[o.plan[2]]}
        if o.mfma_bound:  # the matrix cores bound this step: row flops against their peak
            tf = o.row_flops / (ot["launch_ms"] * 1e-3) / 1e12
            others[name].update({"bound": "mfma", "row_flops_per_step": o.row_flops,
                                 "achieved_tflops": round(tf, 1),
                                 "frac": round(tf / MFMA_PEAK_TFLOPS[o.case.dtype], 4)})
        o.close()
        del o
        torch.cuda.empty_cache()
    if others:
        rec["other_workloads"] = others

    # yardstick for the memory counters: one plain device copy of known size
    # (outside the timed region; a profiler run scales FETCH/WRITE_SIZE by it)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    if not a.no_ceiling:
        rec["ceiling_gbs"] = ceiling(dev)
        rec["ceiling_gbs"]["kernel"] = "plain streaming read (kvattn_stream_read), event-timed"
    if out0 is not None:
        rows = a.cpu_rows or default_cpu_rows(case)
        d = workloads.make_inputs(case)   # the same values, on the host
        rec["cpu_baseline"] = cpu_baseline(case, d, out0, rows, step_bytes)
    print(json.dumps(rec), flush=True)


def default_cpu_rows(case):
    # a bounded sample: about 1-30 s of oracle work on the host cores
    per_row = {"tiny": 4, "decode_7b": 512, "spec_verify": 320, "sink_window": 128,
               "paged_100k": 64}
    return per_row.get(case.name.replace("_fp8", ""), 64)


if __name__ == "__main__":
    main()
