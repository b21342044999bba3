"""Independent calls in flight at once on separate streams (run on an
MI355X).  Each stream owns its workspace and outputs; the inputs are shared
and only read.  Every call must reproduce, bit for bit, the same call made
alone with nothing else running: the library keeps no per-call state outside
the workspace it is given (the allocation-free decode's static scratch is
used by one stream only, which is the documented condition for it).  All
streams are created at the default priority."""
import numpy as np
import pytest
import torch

import mqa_latent_kv_amd as mla
from mqa_latent_kv_amd import synth

pytestmark = pytest.mark.gpu

# decode problems covering the kernels a call can take: the wave-specialised
# kernel with split sequences (merged), top-k lists over the per-tile FP8
# cache, several query tokens per sequence, and the split-reduction kernel
# at 8 heads
DECODES = [
    ("dense_split_h128", dict(seed=501, batch=3, heads=128, seqlens=[1, 200, 6000])),
    ("topk_fp8_h64", dict(seed=502, batch=3, heads=64, seqlens=[3000, 900, 50], kv_format="fp8", topk=700)),
    ("mtp_h64", dict(seed=503, batch=2, heads=64, seqlens=[33, 2500], tokens_per_seq=3)),
    ("h8_ragged", dict(seed=504, batch=5, heads=8, seqlen_range=(1, 3000))),
]


def _say(msg):
    print(msg, flush=True)


class _Decode:
    def __init__(self, name, kw, dev, noalloc=False):
        self.name, self.noalloc = name, noalloc
        inp = synth.make_decode_inputs(**kw)
        self.inp, self.d = inp, mla.to_device(inp, dev)
        B, H, T = inp["batch"], inp["heads"], inp["tokens_per_seq"]
        rows = (B, H) if T == 1 else (B, T, H)
        self.out = torch.empty(rows + (512,), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(rows, dtype=torch.float32, device=dev)
        topk = 0 if inp["topk_idx"] is None else inp["topk_idx"].shape[-1]
        params = mla.decode_params(batch=B, heads=H, num_pages=inp["kv"].shape[0],
                                   max_pages_per_seq=inp["block_table"].shape[1], topk=topk,
                                   q_fp8=inp["q_format"] != "bf16", kv_format=inp["kv_format"],
                                   q_descale=inp["q_descale"], tokens_per_seq=T)
        self.ws = None if noalloc else mla.decode_workspace(params, dev)

    def __call__(self, stream):
        d = self.d
        args = (d["q"], d["kv"], d["block_table"], d["seqlens"], d["topk_idx"], d["kv_scales"])
        if self.noalloc:
            mla.mla_decode_noalloc(*args, out=self.out, lse=self.lse, q_descale=self.inp["q_descale"], stream=stream)
        else:
            mla.mla_decode(*args, out=self.out, lse=self.lse, q_descale=self.inp["q_descale"], workspace=self.ws,
                           stream=stream)

    def poison(self):
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))

    def result(self):
        return [self.out.clone(), self.lse.clone()]


class _Query:
    name = "query_h16"

    def __init__(self, dev):
        qin = synth.make_query_inputs(505, batch=40, heads=16, width=2112)
        self.qin, self.dq = qin, mla.query_to_device(qin, dev)
        self.ws = torch.empty(mla.mla_query_workspace_size(mla.QueryParams(40, 16, 2112, qin["eps"])),
                              dtype=torch.uint8, device=dev)
        self.out = torch.empty((40, 16, 576), dtype=torch.uint8, device=dev)

    def __call__(self, stream):
        dq = self.dq
        mla.mla_query(dq["qkv"], dq["w_qa"], dq["w_qb"], dq["w_uk"], dq["q_scale_inv"], out=self.out,
                      eps=self.qin["eps"], workspace=self.ws, stream=stream)

    def poison(self):
        self.out.fill_(0xFF)

    def result(self):
        return [self.out.clone()]


class _Insert:
    name = "insert_300"

    def __init__(self, dev):
        ins = synth.make_insert_inputs(506, tokens=300, num_pages=12)
        self.ins, self.di = ins, mla.insert_to_device(ins, dev)
        self.cache0 = self.di["cache"].clone()

    def __call__(self, stream):
        di = self.di
        mla.mla_kv_insert(di["qkv"], di["w_kva"], di["slots"], di["k_scale_inv"], di["cache"], eps=self.ins["eps"],
                          stream=stream)

    def poison(self):
        self.di["cache"].copy_(self.cache0)

    def result(self):
        return [self.di["cache"].clone()]


def _same(a, b):
    """bit-for-bit equality of two tensors (NaN payloads included)"""
    x = a.contiguous().view(torch.uint8).cpu().numpy()
    y = b.contiguous().view(torch.uint8).cpu().numpy()
    return np.array_equal(x, y)


def test_concurrent_streams_match_calls_alone():
    dev = torch.device("cuda:0")
    jobs = [_Decode(n, kw, dev) for n, kw in DECODES]
    jobs.append(_Decode("noalloc_dense_h128", dict(seed=507, batch=6, heads=128, seqlen_range=(100, 4000)), dev,
                        noalloc=True))
    jobs += [_Query(dev), _Insert(dev)]
    cur = torch.cuda.current_stream(dev)

    # each call alone: launched, then waited for, before the next one
    want = {}
    for j in jobs:
        _say(f"[streams] alone: {j.name}")
        j.poison()
        j(cur)
        torch.cuda.synchronize()
        want[j.name] = j.result()

    # all of them at once, three rounds launched round-robin over the streams
    streams = [torch.cuda.Stream(device=dev) for _ in jobs]
    for j in jobs:
        j.poison()
    for s in streams:
        s.wait_stream(cur)
    _say(f"[streams] {len(jobs)} streams, 3 rounds")
    for _ in range(3):
        for j, s in zip(jobs, streams):
            with torch.cuda.stream(s):
                j(s)
    for s in streams:
        cur.wait_stream(s)
    torch.cuda.synchronize()
    for j in jobs:
        got = j.result()
        for k, (g, w) in enumerate(zip(got, want[j.name])):
            assert _same(g, w), f"{j.name}: output {k} differs from the call made alone"
    _say("[streams] every output equals its call made alone")
