"""Benchmark of the MLA decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--profile-run] [--graph]

A step is one pass of the hot path over one batch of synthetic input, with
every input resident in HBM before timing:

  paged_bf16_4096 (default, the headline): one mla_decode call over the paged
      bf16 cache, batch 64, 128 query heads, every sequence 4096 tokens,
      64-token pages scattered through a 4096-page pool by a random block
      table, q and KV N(0,1) in bf16, softmax scale 192^-0.5.
  paged_bf16: the same pool with seeded lengths uniform in [1024, 4096].
  fp8_cache: batch 32, 64 heads, lengths uniform in [8192, 32768], e4m3 cache
      (512 codes + 64 bf16 rope per row) with per-row per-tile fp32 scales.
  topk_sparse: batch 32, 128 heads, 2048 sorted top-k positions per sequence
      over 65536-token contexts (trailing -1 padding), e4m3 cache.
  query_decode: mla_query (RMSNorm, Q_B, W_UK, FP8) for 64 tokens x 8 heads,
      then mla_decode of those FP8 queries over a bf16 cache of 8192 tokens
      per sequence.
  insert_decode: mla_kv_insert of the 64 new tokens' latent rows (RMSNorm,
      per-tensor e4m3) at each sequence's last position, then mla_decode over
      that all-FP8 cache: batch 64, 128 heads, 4096 tokens each, 4096-page pool.
  mtp_bf16: two new query tokens per sequence (causal), batch 64, 128 heads,
      4096 tokens each, over the headline's bf16 pool: 256 query rows read
      every KV row once.

The decode call runs the work split, block-table translation (or the top-k
translation), KV streaming, QK^T, softmax, PV, epilogue and the split-KV merge on
the GPU.  Each step calls the entry points from Python; with --graph the
step's calls are recorded once into a HIP graph and every timed step replays
it (measured slower on this ROCm: the replay adds more per-kernel time than the
calls cost the host, and the host stays ahead of the GPU either way).  Either
way the timed steps must reproduce the first step's output bit for bit.  Prints one JSON line: algorithmic HBM throughput (GB/s) as
`value`, µs/step, tokens/s, a `roofline` object (the step's kernels timed with
HIP events on their stream) and a `cpu_baseline` object (the float64 CPU
oracle on a bounded sample of the same workload).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode µs/step + achieved HBM GB/s (% of peak) at B=64,H=128,s_k=4096"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CALIB_BYTES = 256 << 20  # plain copy used to scale the HBM traffic counters
DECODE_SOURCES = ("decode_common.h", "decode.hip", "decode_ws.hip")
QUERY_WORKLOADS = ("query_decode", "query_narrow_decode", "insert_decode")  # also run query.hip kernels
COLD_FLUSH_BYTES = 512 << 20  # read between cold steps: twice the 256 MB Infinity Cache

WORKLOADS = {
    "paged_bf16_4096": "paged bf16 MLA decode: batch 64, 128 heads, seq_len 4096 each, 64-token pages, "
                       "4096-page pool, d_qk 576, d_v 512",
    "paged_bf16": "paged bf16 MLA decode: batch 64, 128 heads, seq_len uniform 1024..4096, 64-token pages, "
                  "4096-page pool",
    "fp8_cache": "FP8 (e4m3 + fp32 tile scales) MLA decode: batch 32, 64 heads, seq_len uniform 8192..32768, "
                 "16384-page pool",
    "topk_sparse": "top-k sparse MLA decode: batch 32, 128 heads, 2048 positions (<=256 padded) of 65536, "
                   "e4m3 cache, 32768-page pool",
    "query_decode": "MLA query front end (64 tokens, 8 heads: RMSNorm, Q_B 1536x1536, W_UK, FP8) then decode "
                    "of the FP8 queries over bf16 pages, 8192 tokens each",
    "insert_decode": "KV-cache insert (64 tokens: RMSNorm of the 512-wide latent row, per-tensor e4m3 of the 576 "
                     "columns) then decode over the all-FP8 cache: batch 64, 128 heads, seq_len 4096 each, "
                     "4096-page pool",
    "mtp_bf16": "paged bf16 MLA decode of 2 new query tokens per sequence (causal): batch 64, 128 heads, "
                "seq_len 4096 each, 4096-page pool",
    "query_narrow_decode": "MLA query front end in its narrow-batch form (4 tokens, 128 heads: RMSNorm, Q_B "
                           "24576x1536, W_UK, FP8) then decode of the FP8 queries over bf16 pages, 8192 tokens each",
}


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")


def causal_limits(inp) -> np.ndarray:
    """[B, T] positions visible to each query token: seqlen - T + 1 + t."""
    T = inp.get("tokens_per_seq", 1)
    seq = inp["seqlens"].astype(np.int64)[:, None]
    return np.maximum(seq - T + 1 + np.arange(T)[None, :], 0)


def kv_tokens(inp) -> int:
    """KV rows the decode must read: every position once for all query tokens
    (dense), or the valid entries of every top-k list."""
    if inp.get("topk_idx") is not None:
        B, T = inp["batch"], inp.get("tokens_per_seq", 1)
        t = inp["topk_idx"].reshape(B, T, -1)
        return int(np.sum((t >= 0) & (t < causal_limits(inp)[:, :, None])))
    return int(inp["seqlens"].astype(np.int64).sum())


def attended_pairs(inp) -> int:
    """(query token, KV row) pairs the scores are computed for."""
    if inp.get("topk_idx") is not None:
        return kv_tokens(inp)
    return int(causal_limits(inp).sum())


def decode_bytes(inp) -> int:
    """Bytes the decode must move at least once: the KV rows it attends
    (bf16 1152 B; FP8 512 codes + 128 B rope + 16 B scales; per-tensor FP8
    576 codes), the queries, the
    outputs (bf16 O + fp32 LSE), the block-table entries it reads, the
    sequence lengths and the top-k lists."""
    B, H = inp["batch"], inp["heads"] * inp.get("tokens_per_seq", 1)  # query rows per sequence
    row = {"bf16": 576 * 2, "fp8": 512 + 128 + 16, "fp8_tensor": 576}[inp["kv_format"]]
    qb = 576 * (2 if inp["q_format"] == "bf16" else 1)
    if inp.get("topk_idx") is not None:
        tables = inp["topk_idx"].size * 4 + kv_tokens(inp) * 4  # lists + one block-table entry per valid entry
    else:
        seq = inp["seqlens"].astype(np.int64)
        tables = int(np.sum((seq + 63) // 64)) * 4
    return kv_tokens(inp) * row + B * H * qb + B * H * (512 * 2 + 4) + tables + B * 4


def decode_flops(inp) -> int:
    return attended_pairs(inp) * 2 * inp["heads"] * (576 + 512)


def query_bytes(qin) -> int:
    """qkv rows read, the three weights, the FP8 output."""
    B, H = qin["batch"], qin["heads"]
    return B * 1536 * 2 + 1536 * 2 + H * 192 * 1536 * 2 + H * 128 * 512 * 2 + B * H * 576


def insert_bytes(tokens: int) -> int:
    """Latent + rope bf16 read per token, its slot, the 576 codes written,
    w_kva and the scale."""
    return tokens * (576 * 2 + 8 + 576) + 512 * 2 + 4


def insert_flops(tokens: int) -> int:
    return tokens * 512 * 4  # square-accumulate, normalise, weight


def query_flops(qin) -> int:
    B, H = qin["batch"], qin["heads"]
    return 2 * B * 1536 * H * 192 + 2 * B * H * 128 * 512


def kernel_sources(workload: str):
    names = DECODE_SOURCES + (("query.hip",) if workload in QUERY_WORKLOADS else ())
    return [os.path.join(ROOT, "mqa_latent_kv_amd", "csrc", f) for f in names]


def kernel_hash(workload: str) -> str:
    """Hash of the sources of the workload's kernels with // comments dropped
    and whitespace runs collapsed, so a comment edit does not disown counters
    taken on the same code."""
    h = hashlib.sha256()
    for p in kernel_sources(workload):
        text = re.sub(r"//[^\n]*", "", open(p, encoding="utf-8").read())
        h.update(re.sub(r"\s+", " ", text).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per step from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    try:
        d = json.load(open(traffic_file(workload)))
    except (OSError, ValueError):
        return None
    if d.get("kernel_hash") != kernel_hash(workload):
        return None
    return d.get("traffic_bytes_per_step")


SETTLE_S = 1.5  # seconds of untimed steps that bring the GPU clock to its steady state
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)


def step_event_times(stream, run, steps: int, before=None):
    """Milliseconds of each of `steps` calls of run(), from HIP events
    recorded on `stream` before and after it (before(), when given, runs
    ahead of each step's first event, untimed).  The events are created with
    hipEventDisableSystemFence: a default event's system-scope release
    writes back the caches when it is recorded, and that writeback would be
    timed as part of the step."""
    import ctypes

    hip = ctypes.CDLL("libamdhip64.so")
    evs = []
    for _ in range(2 * steps):
        e = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        evs.append(e)
    sp = ctypes.c_void_p(stream.cuda_stream)
    for i in range(steps):
        if before is not None:
            before()
        hip.hipEventRecord(evs[2 * i], sp)
        run()
        hip.hipEventRecord(evs[2 * i + 1], sp)
    if hip.hipEventSynchronize(evs[-1]) != 0:
        raise RuntimeError("hipEventSynchronize failed")
    out = []
    for i in range(steps):
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), evs[2 * i], evs[2 * i + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        out.append(ms.value)
    for e in evs:
        hip.hipEventDestroy(e)
    return out


def cpu_threads() -> int:
    from threadpoolctl import threadpool_info

    return int(max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("internal_api") in ("openblas", "mkl", "blis")] or [1]))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, nbytes: int, budget_s: float = 12.0, qin=None, ins=None):
    """The float64 oracle (as it stands) on whole sequences of the workload
    until the time budget is spent, scaled to the metric's unit."""
    from oracle import mla_oracle as mo

    t0 = time.perf_counter()
    if qin is not None:
        mo.mla_query(qin["qkv"], qin["w_qa"], qin["w_qb"], qin["w_uk"], qin["q_scale_inv"], eps=qin["eps"])
    if ins is not None:
        mo.kv_insert(ins["qkv"], ins["w_kva"], inp["kv"], ins["slots"], float(inp["kv_scales"][0]), ins["eps"])
    done = 0
    while done < inp["batch"] and time.perf_counter() - t0 < budget_s:
        mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], inp.get("topk_idx"),
                      inp.get("kv_scales"), q_format=inp["q_format"], kv_format=inp["kv_format"],
                      q_descale=inp["q_descale"], batches=[done])
        done += 1
    dt = time.perf_counter() - t0
    frac = done / inp["batch"]
    return {
        "value": round(nbytes * frac / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": cpu_threads(),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"{done} of {inp['batch']} sequences{' plus the whole query front end' if qin else ''}"
                  f"{' plus the whole insert' if ins else ''}, "
                  f"{dt:.1f} s; host has {os.cpu_count()} logical CPUs",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="paged_bf16_4096", choices=list(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay a HIP graph of the step instead of calling the entry points every step")
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
    name = args.workload
    inp = synth.workload_inputs(name)
    qin = None
    if name in ("query_decode", "query_narrow_decode"):
        qin = synth.make_query_inputs(5 if name == "query_decode" else 8, batch=inp["batch"], heads=inp["heads"])
    d = mla.to_device(inp, dev)
    B, H = inp["batch"], inp["heads"]
    ins = None
    if name == "insert_decode":
        # the new token of sequence b is its last position
        bt, last = inp["block_table"], inp["seqlens"].astype(np.int64) - 1
        ins = synth.make_insert_inputs(6, tokens=B, num_pages=1)
        slots = bt[np.arange(B), last // 64].astype(np.int64) * 64 + last % 64
        di = mla.insert_to_device(ins, dev)
        di["slots"] = torch.from_numpy(slots).to(dev)
    T = inp.get("tokens_per_seq", 1)
    topk = 0 if inp.get("topk_idx") is None else inp["topk_idx"].shape[-1]
    params = mla.decode_params(batch=B, heads=H, num_pages=inp["kv"].shape[0],
                               max_pages_per_seq=inp["block_table"].shape[1], topk=topk,
                               q_fp8=inp["q_format"] != "bf16", kv_format=inp["kv_format"],
                               q_descale=inp["q_descale"], tokens_per_seq=T)
    stream = torch.cuda.current_stream(dev)
    ws = mla.decode_workspace(params, dev, stream)
    rows = (B, H) if T == 1 else (B, T, H)
    out = torch.empty(rows + (512,), dtype=torch.bfloat16, device=dev)
    lse = torch.empty(rows, dtype=torch.float32, device=dev)
    q = d["q"]
    if qin is not None:
        dq = mla.query_to_device(qin, dev)
        q = torch.empty((B, H, 576), dtype=torch.uint8, device=dev)
        qws = torch.empty(max(mla.mla_query_workspace_size(mla.QueryParams(B, H, 1536, qin["eps"])), 1),
                          dtype=torch.uint8, device=dev)

    # the cold figure's sweep buffer, written once here (float32 ones)
    flush = torch.ones(COLD_FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    # every call goes to the current stream (the capture stream while a graph
    # of the step is recorded)
    def step():
        if ins is not None:
            mla.mla_kv_insert(di["qkv"], di["w_kva"], di["slots"], d["kv_scales"], d["kv"], eps=ins["eps"])
        if qin is not None:
            mla.mla_query(dq["qkv"], dq["w_qa"], dq["w_qb"], dq["w_uk"], dq["q_scale_inv"], out=q, eps=qin["eps"],
                          workspace=qws)
        mla.mla_decode(q, d["kv"], d["block_table"], d["seqlens"], d["topk_idx"], d["kv_scales"], out=out, lse=lse,
                       q_descale=inp["q_descale"], workspace=ws)

    # the GPU clock ramps up over the first ~100 ms of sustained work: run
    # steps for SETTLE_S seconds before the warm-up steps, so the timed steps
    # see the steady clock (untimed; the same calls as a step)
    t_settle = time.perf_counter()
    settle_steps = 0
    while not args.profile_run and time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(20):
            step()
        settle_steps += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    first_out = (out.clone(), lse.clone())
    run = step
    if args.graph:
        # the step's kernels recorded once into a HIP graph and replayed: the
        # same launches with the same arguments, without the Python and
        # launch overhead of every call (no memset nodes: the library clears
        # nothing with hipMemsetAsync)
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
    if args.profile_run:
        for _ in range(args.steps):
            run()
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.int32, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"profile run: {name}, {args.steps} steps, {args.steps} copies of {CALIB_BYTES} bytes", flush=True)
        return

    # timed region: K back-to-back steps between one event pair
    t_all0, t_all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record(stream)
    for _ in range(args.steps):
        run()
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # the kernels of each step, timed by a HIP event pair around it on the
    # stream the library launches on (K more steps, right after): events
    # without the system-scope fence, whose cache writeback would otherwise
    # be timed with the kernels
    kern_ms = np.array(step_event_times(stream, run, args.steps))
    # the timed steps must reproduce the warm-up's output bit for bit (the kernels are deterministic)
    if not (torch.equal(out.view(torch.int16), first_out[0].view(torch.int16))
            and torch.equal(lse.view(torch.int32), first_out[1].view(torch.int32))):
        print("bench.py: the timed steps did not reproduce the warm-up step's output", file=sys.stderr)
        sys.exit(1)
    total_ms = t_all0.elapsed_time(t_all1)
    ms_per_step = total_ms / args.steps

    # cold-cache figure: before each step a read-only sweep of a buffer
    # written once at setup evicts the KV from the Infinity Cache and the L2s
    # without leaving dirty lines to be written back during the step; the
    # step alone is timed, with the same fence-free events
    sweep_acc = torch.zeros((), dtype=torch.float32, device=dev)
    cold = np.array(step_event_times(stream, run, min(args.steps, 30),
                                     before=lambda: torch.sum(flush, 0, out=sweep_acc)))
    # context: a plain device copy of 1 GiB (read 1 GiB, write 1 GiB), the
    # bandwidth a streaming kernel reaches on this GPU
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * (1 << 30) / (c0.elapsed_time(c1) / 1e3) / 1e9
    # and a read-only stream: the library GEMV of torch.mv over the same 1 GiB
    # as a [2^19, 1024] bf16 matrix (writes 1 MB), the fastest read-only
    # primitive at hand here, which bounds what a kernel that only reads HBM
    # reaches (torch's reductions stay near 3.8 TB/s)
    rd = src.view(torch.bfloat16).view(-1, 1024)
    xv = torch.ones(1024, dtype=torch.bfloat16, device=dev)
    yv = torch.empty(rd.shape[0], dtype=torch.bfloat16, device=dev)
    torch.mv(rd, xv, out=yv)
    c0.record(stream)
    for _ in range(5):
        torch.mv(rd, xv, out=yv)
    c1.record(stream)
    torch.cuda.synchronize()
    read_gbs = 5 * (1 << 30) / (c0.elapsed_time(c1) / 1e3) / 1e9
    del flush, sweep_acc, src, dst, rd, xv, yv

    nbytes = decode_bytes(inp) + (query_bytes(qin) if qin else 0) + (insert_bytes(B) if ins else 0)
    flops = decode_flops(inp) + (query_flops(qin) if qin else 0) + (insert_flops(B) if ins else 0)
    kern_avg_s = float(kern_ms.mean()) / 1e3
    achieved = nbytes / kern_avg_s / 1e9
    tflops = flops / kern_avg_s / 1e12
    value = nbytes / (ms_per_step / 1e3) / 1e9
    kernels = {"topk_sparse": "mla_decode_ws_kernel<1,false,false,true> + mla_merge_kernel<true>",
               "fp8_cache": "mla_decode_ws_kernel<1,false,false,false> + mla_merge_wide_kernel<true>",
               "query_decode": "mla_qbn_kernel + mla_qlm_kernel + mla_decode_kernel<4,true,0,false> + "
                               "mla_merge_wide_kernel<false>",
               "query_narrow_decode": "mla_qb_gemv_kernel + mla_ql_gemv_kernel + "
                                      "mla_decode_ws_kernel<0,true,false,false> + mla_merge_wide_kernel<true>",
               "insert_decode": "mla_kv_insert_kernel + mla_decode_ws_kernel<2,false,false,false> + "
                                "mla_merge_kernel<true>",
               "mtp_bf16": "mla_decode_ws_kernel<0,false,true,false> + mla_merge_kernel<true>"}
    kernel = kernels.get(name, "mla_decode_ws_kernel<0,false,false,false> + mla_merge_kernel<true>")
    # above the ridge (2.5 PFLOP/s over 8 TB/s = 312.5 flop/B) the step is bound by the bf16 MFMA rate:
    # top-k (345 flop/B) and the per-tensor FP8 cache at 128 heads (432 flop/B)
    mfma_bound = flops / nbytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    roofline = {
        "bound": "mfma" if mfma_bound else "hbm",
        "kernel": kernel + " (one call, timed together: HIP events without the system fence around each call)",
        "achieved": round(tflops if mfma_bound else achieved, 1),
        "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
        "unit": "TFLOP/s" if mfma_bound else "GB/s",
        "frac": round((tflops / MFMA_BF16_PEAK_TFLOPS) if mfma_bound else (achieved / HBM_PEAK_GBS), 4),
        "traffic": measured_traffic(name),
        "kernel_us_avg": round(kern_avg_s * 1e6, 2),
        "hbm_gbs": round(achieved, 1),
        "mfma_tflops": round(tflops, 1),
        "copy_ceiling_gbs": round(copy_gbs, 1),
        "read_ceiling_gbs": round(read_gbs, 1),
    }
    seq = inp["seqlens"]
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
        "tokens_per_s": round(B * T / (ms_per_step / 1e3), 1),
        "kv_tokens_per_s": round(kv_tokens(inp) / (ms_per_step / 1e3), 1),
        "cold_us_per_step_median": round(float(np.median(cold)) * 1e3, 2),
        "cold_frac_of_hbm_peak": round(nbytes / (float(np.median(cold)) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "cold_method": f"{len(cold)} steps, each after a read-only sweep of a {COLD_FLUSH_BYTES >> 20} MiB buffer "
                       "written once at setup; the step alone timed with fence-free HIP events",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp["kv_format"] == "bf16" else "bf16 (e4m3 cache codes)",
        "data": "synthetic (seeded; q and KV from N(0,1), random permuted block table)",
        "config": {
            "workload": WORKLOADS[name],
            "batch": B,
            "heads": H,
            "seq_len": int(seq.max()) if int(seq.min()) == int(seq.max()) else [int(seq.min()), int(seq.max())],
            "page_size": 64,
            "topk": topk,
            "algorithmic_bytes": int(nbytes),
            "algorithmic_flops": int(flops),
        },
        "roofline": roofline,
        "wall_s_timed_region": round(wall, 4),
        "settle": {"seconds": SETTLE_S, "steps": settle_steps},
    }
    if ins is not None:
        ins["slots"] = slots
    if T > 1:
        res["config"]["tokens_per_seq"] = T
    res["config"]["launch"] = "HIP graph of the step's kernels, one replay per step" if args.graph else \
        "one call per entry point per step"
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(inp, nbytes, qin=qin, ins=ins)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
