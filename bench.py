#!/usr/bin/env python3
"""Benchmark one decode step of attention over a KV cache on one MI355X.

A step is one kvattn_decode call over one batch of the workload: one kernel
launch (every split-KV workgroup, with the log-sum-exp merge done by the last
workgroup of each sequence and KV head), the whole batch, one layer.  Inputs are
seeded synthetic tensors already resident in HBM.  Several identical copies of
the K/V caches are rotated between steps so that each step streams its K/V from
HBM rather than from the 256 MB last-level (Infinity) cache.

Prints ONE JSON line:
  value        effective HBM GB/s = algorithmic bytes / wall time per step
  roofline     the decode kernel(s) timed with HIP events on the library's stream,
               against MI355X's 8 TB/s HBM3E peak
  cpu_baseline the oracle (test infrastructure) timed on the host cores over a
               bounded sample of the same workload
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


def kernel_source_hash() -> str:
    """Hash of the HIP sources: HBM traffic measured for other sources is not reported."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(csrc, name), "rb") as f:
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
    ap.add_argument("--config", default="decode_7b", choices=list(workloads.CONFIGS))
    ap.add_argument("--layout", default="head_major", choices=["token_major", "head_major"])
    ap.add_argument("--split-len", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="K/V copies rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = auto)")
    return ap.parse_args()


def cpu_baseline(case, d, out, n_rows, step_bytes):
    """Time the oracle on the host over a sample of output rows and check those rows."""
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
    threads = oracle.threads()
    t0 = time.perf_counter()
    tm = d["tree_mask"].cpu() if d.get("tree_mask") is not None else None
    ref = oracle.decode_rows(case, q, kc, vc, bt, sl, rows, k_scale=d["k_scale"],
                             v_scale=d["v_scale"], tree_mask=tm)
    dt = time.perf_counter() - t0
    # the sample's share of the step's algorithmic bytes, so the rate is in the metric's unit
    byts = step_bytes * len(rows) / total
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    err = float(np.abs(got - ref).max())
    return {"value": round(byts / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{len(rows)} of {total} output rows of the same workload "
                      f"(float64 naive softmax, OpenMP over rows)",
            "parity_max_abs_on_sample": err}


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
    d = workloads.make_inputs(case, device="cuda")
    sl_host = d["seq_lens"].cpu().tolist()
    step_bytes = accounting.step_bytes(case, sl_host)
    step_flops = accounting.step_flops(case, sl_host)
    # multiply-adds the rows really do (row by row; the union count above is an upper
    # bound): decides whether the step is bound by the matrix cores or by HBM
    row_flops = (4 * case.head_dim * accounting.attended_pairs(case, sl_host)
                 if case.mask_mode != "tree" else step_flops)
    mfma_bound = (case.dtype in MFMA_PEAK_TFLOPS and row_flops / step_bytes >
                  MFMA_PEAK_TFLOPS[case.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9))
    kv_attended = step_bytes - 2 * case.batch * case.q_len * case.num_q_heads * case.head_dim * \
        accounting.ELEM_BYTES[case.dtype]

    copies = a.copies or min(64, max(2, -(-4 * MALL_BYTES // max(kv_attended, 1))))
    kcs, vcs = [d["k_cache"]], [d["v_cache"]]
    for _ in range(copies - 1):
        kcs.append(d["k_cache"].clone())
        vcs.append(d["v_cache"].clone())
    if a.layout == "head_major":
        kcs = [k.permute(0, 2, 1, 3).contiguous() for k in kcs]
        vcs = [v.permute(0, 2, 1, 3).contiguous() for v in vcs]

    h = kb.KVAttn.for_case(case, layout=a.layout)
    if a.split_len:
        h.set_split_len(a.split_len)
    if getattr(case, "kv_dtype", None) == "fp8":
        h.set_kv_scales(d["k_scale"], d["v_scale"])
    n_split, split_len, kernel = h.plan(case.q_len, case.mask_mode, case.n_sink, case.window)
    stream = torch.cuda.Stream(dev)   # default priority
    out = torch.empty_like(d["q"])
    kb.kvattn_set_stream(h.h, stream.cuda_stream)
    mask = kb.MASK[case.mask_mode]

    def step(c):
        if case.mask_mode == "tree":
            kb.kvattn_decode_tree(h.h, d["q"], kcs[c], vcs[c], d["block_table"], d["seq_lens"],
                                  case.q_len, d["tree_mask"], out)
        else:
            kb.kvattn_decode(h.h, d["q"], kcs[c], vcs[c], d["block_table"], d["seq_lens"],
                             case.q_len, mask, case.n_sink, case.window, out)

    for w in range(a.warmup):
        step(w % copies)
    torch.cuda.synchronize()

    # timed region: K steps, synchronised on both sides
    t0 = time.perf_counter()
    for s in range(a.steps):
        step(s % copies)
    t_enq = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / a.steps

    # the same steps again, each bracketed by HIP events on the library's stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    for s in range(a.steps):
        evs[s][0].record(stream)
        step(s % copies)
        evs[s][1].record(stream)
    torch.cuda.synchronize()
    ev_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    ev_mean = sum(ev_ms) / len(ev_ms)
    ev_med = ev_ms[len(ev_ms) // 2]

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = step_bytes / (ev_mean * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "host_enqueue_us_per_step": round(t_enq * 1e6 / a.steps, 2),
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype if not getattr(case, "kv_dtype", None) else
                 f"{case.dtype} (K/V {case.kv_dtype} e4m3)",
        "data": "synthetic (seeded N(0,1) x scale, device generator)",
        "config": {
            "workload": case.name, "batch": case.batch, "num_q_heads": case.num_q_heads,
            "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
            "q_len": case.q_len, "cache": case.cache_mode, "capacity": case.capacity,
            "mask": case.mask_mode, "n_sink": case.n_sink, "window": case.window,
            "seq_lens_sum": int(sum(sl_host)), "layout": a.layout,
            "n_split": n_split, "split_len": split_len,
            "kernel": ["valu", "mfma", "prefill_mfma"][kernel], "kv_copies_rotated": copies,
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
            "flops_per_step": step_flops,
            "event_us_mean": round(ev_mean * 1e3, 2),
            "event_us_median": round(ev_med * 1e3, 2),
            "timed": "the decode kernel (split-KV + fused merge), one launch per step, "
                     "HIP events on the library's stream",
        },
    }
    if mfma_bound:  # the matrix cores bound this step: flops per launch against their peak
        tf = row_flops / (ev_mean * 1e-3) / 1e12
        rec["roofline"].update({"bound": "mfma", "achieved": round(tf, 2),
                                "peak": MFMA_PEAK_TFLOPS[case.dtype], "unit": "TFLOP/s",
                                "frac": round(tf / MFMA_PEAK_TFLOPS[case.dtype], 4),
                                "hbm_gbs": round(achieved, 2)})
    # yardstick for the memory counters: one plain device copy of known size
    # (outside the timed region; a profiler run scales FETCH/WRITE_SIZE by it)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    rec["config"]["kernel_source_hash"] = kernel_source_hash()
    if not a.no_cpu_baseline:
        rows = a.cpu_rows or default_cpu_rows(case)
        rec["cpu_baseline"] = cpu_baseline(case, d, out_for_copy0(h, d, kcs, vcs, case, mask),
                                           rows, step_bytes)
    print(json.dumps(rec), flush=True)


def default_cpu_rows(case):
    # about 10-30 s of single-threaded-equivalent oracle work on a few host cores
    per_row = {"tiny": 4, "decode_7b": 512, "spec_verify": 320, "sink_window": 128,
               "paged_100k": 64}
    return per_row.get(case.name.replace("_fp8", ""), 64)


def out_for_copy0(h, d, kcs, vcs, case, mask):
    out = torch.empty_like(d["q"])
    if case.mask_mode == "tree":
        kb.kvattn_decode_tree(h.h, d["q"], kcs[0], vcs[0], d["block_table"], d["seq_lens"],
                              case.q_len, d["tree_mask"], out)
    else:
        kb.kvattn_decode(h.h, d["q"], kcs[0], vcs[0], d["block_table"], d["seq_lens"],
                         case.q_len, mask, case.n_sink, case.window, out)
    torch.cuda.synchronize()
    return out


if __name__ == "__main__":
    main()
