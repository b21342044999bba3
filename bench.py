"""Benchmark of the MLA decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one mla_decode call over the paged bf16 workload the headline metric
is quoted on: batch 64, 128 query heads, every sequence 4096 tokens, 64-token
pages scattered through a 4096-page pool by a random block table, q and KV
N(0,1) in bf16, softmax scale 192^-0.5.  The call runs the whole path on the
GPU: work split, query tile load, block-table translation, KV streaming, QK^T,
online softmax, PV, epilogue and the split-KV merge, in one kernel launch.
Inputs are seeded, generated on the host and resident in HBM before timing.

Prints one JSON line: whole-step algorithmic HBM throughput (GB/s) as
`value`, µs/step, tokens/s, a `roofline` object for the decode kernel (timed
with HIP events on its stream) and a `cpu_baseline` object (the float64 CPU
oracle on a bounded sample of the same workload).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode µs/step + achieved HBM GB/s (% of peak) at B=64,H=128,s_k=4096"
HBM_PEAK_GBS = 8000.0
CALIB_BYTES = 256 << 20  # plain copy used to scale the HBM traffic counters
WORKLOAD = "paged_bf16_4096"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_paged_bf16_4096_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "mqa_latent_kv_amd", "csrc", f) for f in ("decode.hip",)]


def algorithmic_bytes(inp) -> int:
    """Bytes the decode must move at least once: the KV rows of every attended
    token, the queries, the outputs (bf16 O + fp32 LSE) and the block-table
    entries and sequence lengths it reads."""
    B, H = inp["batch"], inp["heads"]
    seq = inp["seqlens"].astype(np.int64)
    row = 576 * 2 if inp["kv_format"] == "bf16" else 512 + 128 + 16
    qb = 576 * (2 if inp["q_format"] == "bf16" else 1)
    pages = int(np.sum((seq + 63) // 64))
    return int(seq.sum()) * row + B * H * qb + B * H * (512 * 2 + 4) + pages * 4 + B * 4


def algorithmic_flops(inp) -> int:
    return int(inp["seqlens"].astype(np.int64).sum()) * 2 * inp["heads"] * (576 + 512)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; else None."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_hash") != kernel_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def cpu_baseline(inp, budget_s: float = 12.0):
    """The float64 oracle (as it stands) on whole sequences of the workload,
    until the time budget is spent; throughput in the metric's unit."""
    from threadpoolctl import threadpool_info

    from oracle import mla_oracle as mo

    done = 0
    t0 = time.perf_counter()
    while done < inp["batch"] and time.perf_counter() - t0 < budget_s:
        mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], batches=[done])
        done += 1
    dt = time.perf_counter() - t0
    per_seq = algorithmic_bytes(inp) / inp["batch"]
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("internal_api") in ("openblas", "mkl", "blis")] or [1])
    return {
        "value": round(per_seq * done / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {inp['batch']} sequences (all 128 heads x 4096 tokens each), {dt:.1f} s, "
                  f"{done * 4096 / dt:.0f} KV tokens/s; host has {os.cpu_count()} logical CPUs",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="for rocprofv3 counter runs: run the steps untimed, then a plain device copy of "
                         f"{CALIB_BYTES >> 20} MiB (read {CALIB_BYTES >> 20} MiB, write as much) per step as the "
                         "calibration of the FETCH_SIZE / WRITE_SIZE counters; prints no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (the decode path is measured on "
              "one GPU's share; multi-GPU sharding is not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import mqa_latent_kv_amd as mla
    from mqa_latent_kv_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.workload_inputs(WORKLOAD)
    d = mla.to_device(inp, dev)
    B, H = inp["batch"], inp["heads"]
    params = mla.decode_params(batch=B, heads=H, num_pages=inp["kv"].shape[0],
                               max_pages_per_seq=inp["block_table"].shape[1])
    stream = torch.cuda.current_stream(dev)
    ws = mla.decode_workspace(params, dev, stream)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)

    def step():
        mla.mla_decode(d["q"], d["kv"], d["block_table"], d["seqlens"], out=out, lse=lse, workspace=ws,
                       stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.profile_run:
        for _ in range(args.steps):
            step()
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.int32, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"profile run: {args.steps} decode steps, {args.steps} copies of {CALIB_BYTES} bytes", flush=True)
        return

    # timed region: K back-to-back steps; an event pair around every launch
    # gives the kernel's own duration on its stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_all0, t_all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record(stream)
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_all0.elapsed_time(t_all1)
    kern_ms = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    ms_per_step = total_ms / args.steps

    # cold-cache figure (secondary): a 512 MB write between steps evicts the
    # 256 MB Infinity Cache and the L2s; only the decode launch is timed
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(min(args.steps, 20)):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush

    nbytes = algorithmic_bytes(inp)
    flops = algorithmic_flops(inp)
    kern_avg_s = float(kern_ms.mean()) / 1e3
    achieved = nbytes / kern_avg_s / 1e9
    traffic = measured_traffic()
    value = nbytes / (ms_per_step / 1e3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(B / (ms_per_step / 1e3), 1),
        "kv_tokens_per_s": round(float(inp["seqlens"].sum()) / (ms_per_step / 1e3), 1),
        "cold_us_per_step_median": round(float(np.median(cold)) * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q and KV, random permuted block table)",
        "config": {
            "workload": "paged bf16 MLA decode: batch 64, 128 heads, seq_len 4096 each, 64-token pages, "
                        "4096-page pool, d_qk 576, d_v 512",
            "batch": B,
            "heads": H,
            "seq_len": 4096,
            "page_size": 64,
            "algorithmic_bytes": nbytes,
            "algorithmic_flops": flops,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "mla_decode_bf16_kernel<2,false>",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_us_avg": round(kern_avg_s * 1e6, 2),
            "mfma_tflops": round(flops / kern_avg_s / 1e12, 1),
        },
        "wall_s_timed_region": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
