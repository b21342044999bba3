"""mla_decode_noalloc: the decode entry point that allocates nothing and takes
its scratch from the library's static per-GPU array.  On the GPU its outputs
must equal mla_decode's (same kernels, same plan) bit for bit, on calls in a
row whose later ones are smaller, and inside a replayed HIP graph; a problem
whose scratch would exceed the array is refused before anything launches."""
import ctypes
import os

import pytest
import torch

import mqa_latent_kv_amd as mla
from mqa_latent_kv_amd import synth


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mla.LIB_PATH):
        from mqa_latent_kv_amd import build

        build.build()
    return mla.lib()


def test_noalloc_exported_and_validated_on_host(L):
    assert hasattr(L, "mla_decode_noalloc")
    assert mla.mla_status_string(mla.MLA_ERR_SCRATCH_LIMIT) not in ("ok", "unknown status")
    fake = ctypes.c_void_p(0x1000)
    p = mla.decode_params(batch=2, heads=128, num_pages=8, max_pages_per_seq=4)
    args = [fake] * 4 + [None, None, fake, fake, None]
    assert L.mla_decode_noalloc(None, *args) == -1
    # a missing output and a misaligned query are caught before any device call
    assert L.mla_decode_noalloc(ctypes.byref(p), *args[:6], None, fake, None) == -1
    assert L.mla_decode_noalloc(ctypes.byref(p), ctypes.c_void_p(0x1008), *args[1:]) == -1
    if not torch.cuda.is_available():
        assert L.mla_decode_noalloc(ctypes.byref(p), *args) == -5


def _inputs(kind):
    if kind == "dense_bf16_128":  # wave-specialised kernel, sequences split over several ranges
        return synth.make_decode_inputs(401, batch=12, heads=128, seqlen_range=(1, 5000))
    if kind == "mtp_bf16_64":
        return synth.make_decode_inputs(402, batch=4, heads=32, seqlens=[2, 700, 3000, 65], tokens_per_seq=2)
    if kind == "topk_fp8_16":
        return synth.make_decode_inputs(403, batch=3, heads=16, seqlens=[900, 40, 2000], kv_format="fp8", topk=300)
    return synth.make_decode_inputs(404, batch=2, heads=8, seqlens=[5, 130], kv_format="fp8_tensor",
                                    q_format="fp8", q_descale=4.0)


def _both(inp, dev):
    d = mla.to_device(inp, dev)
    kw = dict(q_descale=inp["q_descale"])
    want = mla.mla_decode(d["q"], d["kv"], d["block_table"], d["seqlens"], d["topk_idx"], d["kv_scales"], **kw)
    got = mla.mla_decode_noalloc(d["q"], d["kv"], d["block_table"], d["seqlens"], d["topk_idx"], d["kv_scales"], **kw)
    torch.cuda.synchronize()
    return want, got


def _same(want, got, what):
    (wo, wl), (go, gl) = want, got
    assert torch.equal(go.view(torch.int16), wo.view(torch.int16)), f"{what}: out differs"
    assert torch.equal(gl.view(torch.int32), wl.view(torch.int32)), f"{what}: lse differs"


@pytest.mark.gpu
def test_noalloc_matches_workspace_decode_on_shrinking_calls():
    dev = torch.device("cuda:0")
    # largest first: each later call is smaller and finds the previous call's
    # bytes in the shared scratch
    for kind in ("dense_bf16_128", "mtp_bf16_64", "topk_fp8_16", "fp8_tensor_8"):
        _say(f"[noalloc] {kind}")
        inp = _inputs(kind)
        _same(*_both(inp, dev), kind)
    # the second of two calls in a row on the same sizes, smaller again
    small = synth.make_decode_inputs(405, batch=2, heads=128, seqlens=[3000, 17])
    _say("[noalloc] dense_bf16_128 small")
    _same(*_both(small, dev), "small")


@pytest.mark.gpu
def test_noalloc_refuses_problems_beyond_its_scratch():
    dev = torch.device("cuda:0")
    B, H = 8192, 128
    p = mla.decode_params(batch=B, heads=H, num_pages=1, max_pages_per_seq=1)
    assert mla.mla_decode_workspace_size(p) > mla.DECODE_SCRATCH_BYTES
    # real, correctly sized tensors (every sequence empty), so the refusal is
    # the only thing under test
    q = torch.zeros((B, H, 576), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((1, 64, 576), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, 1), dtype=torch.int32, device=dev)
    sl = torch.zeros((B,), dtype=torch.int32, device=dev)
    out = torch.full((B, H, 512), 7.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H), 7.0, dtype=torch.float32, device=dev)
    code = mla.lib().mla_decode_noalloc(ctypes.byref(p), *(ctypes.c_void_p(t.data_ptr()) for t in (q, kv, bt, sl)),
                                        None, None, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    torch.cuda.synchronize()
    assert code == mla.MLA_ERR_SCRATCH_LIMIT
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all()), "a refused call wrote its outputs"


@pytest.mark.gpu
def test_noalloc_graph_replays_match_eager():
    dev = torch.device("cuda:0")
    inp = synth.make_decode_inputs(406, batch=3, heads=128, seqlens=[1, 200, 6000])
    d = mla.to_device(inp, dev)
    out = torch.empty((3, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((3, 128), dtype=torch.float32, device=dev)

    def step():
        mla.mla_decode_noalloc(d["q"], d["kv"], d["block_table"], d["seqlens"], out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    want_o, want_l = out.clone(), lse.clone()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    _say("[noalloc] capture")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    # between replays: poison the outputs and run another no-alloc decode,
    # which leaves its own bytes in the shared scratch
    other = mla.to_device(synth.make_decode_inputs(407, batch=2, heads=32, seqlens=[500, 90]), dev)
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        mla.mla_decode_noalloc(other["q"], other["kv"], other["block_table"], other["seqlens"])
        torch.cuda.synchronize()
        _say(f"[noalloc] replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want_o.view(torch.int16)), f"replay {r}: out differs"
        assert torch.equal(lse.view(torch.int32), want_l.view(torch.int32)), f"replay {r}: lse differs"
