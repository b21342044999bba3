"""The entry points recorded into a HIP graph and replayed (run on an MI355X):
every replay, with the program's own eager work and synchronisations between
replays, must reproduce the eager calls' outputs bit for bit (the kernels are
deterministic and clear nothing with memset nodes)."""
import numpy as np
import pytest
import torch

import mqa_latent_kv_amd as mla
from mqa_latent_kv_amd import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("kind", ["dense_split", "topk", "mtp", "insert_query_decode"])
def test_graph_replays_match_eager(kind):
    dev = torch.device("cuda:0")
    if kind == "dense_split":
        inp = synth.make_decode_inputs(301, batch=3, heads=128, seqlens=[1, 200, 6000])
    elif kind == "topk":
        inp = synth.make_decode_inputs(302, batch=3, heads=64, seqlens=[3000, 900, 50], kv_format="fp8", topk=700)
    elif kind == "mtp":
        inp = synth.make_decode_inputs(303, batch=2, heads=64, seqlens=[33, 2500], tokens_per_seq=3)
    else:
        inp = synth.make_decode_inputs(304, batch=4, heads=16, seqlens=[100, 700, 1, 64], kv_format="fp8_tensor",
                                       q_format="fp8", q_descale=8.0)
    d = mla.to_device(inp, dev)
    B, H, T = inp["batch"], inp["heads"], inp["tokens_per_seq"]
    rows = (B, H) if T == 1 else (B, T, H)
    out = torch.empty(rows + (512,), dtype=torch.bfloat16, device=dev)
    lse = torch.empty(rows, dtype=torch.float32, device=dev)
    topk = 0 if inp["topk_idx"] is None else inp["topk_idx"].shape[-1]
    params = mla.decode_params(batch=B, heads=H, num_pages=inp["kv"].shape[0],
                               max_pages_per_seq=inp["block_table"].shape[1], topk=topk,
                               q_fp8=inp["q_format"] != "bf16", kv_format=inp["kv_format"],
                               q_descale=inp["q_descale"], tokens_per_seq=T)
    ws = mla.decode_workspace(params, dev)
    q = d["q"]
    extra = []
    if kind == "insert_query_decode":
        qin = synth.make_query_inputs(305, batch=B, heads=H, width=2112)
        dq = mla.query_to_device(qin, dev)
        ins = synth.make_insert_inputs(306, tokens=B, num_pages=inp["kv"].shape[0])
        di = mla.insert_to_device(ins, dev)
        qws = torch.empty(mla.mla_query_workspace_size(mla.QueryParams(B, H, 2112, qin["eps"])), dtype=torch.uint8,
                          device=dev)
        q = torch.empty((B, H, 576), dtype=torch.uint8, device=dev)

        def front():
            mla.mla_kv_insert(dq["qkv"], di["w_kva"], di["slots"], d["kv_scales"], d["kv"], eps=ins["eps"])
            mla.mla_query(dq["qkv"], dq["w_qa"], dq["w_qb"], dq["w_uk"], dq["q_scale_inv"], out=q, eps=qin["eps"],
                          workspace=qws)
        extra.append(front)

    def step():
        for f in extra:
            f()
        mla.mla_decode(q, d["kv"], d["block_table"], d["seqlens"], d["topk_idx"], d["kv_scales"], out=out, lse=lse,
                       q_descale=inp["q_descale"], workspace=ws)

    _say(f"[graph] {kind}: eager")
    step()
    torch.cuda.synchronize()
    want_o, want_l = out.clone(), lse.clone()
    kv_after = d["kv"].clone()

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    _say(f"[graph] {kind}: capture")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    # eager work between replays: poison the outputs, run an unrelated eager
    # decode with its own workspace, synchronise
    other = synth.make_decode_inputs(307, batch=2, heads=32, seqlens=[500, 90])
    do = mla.to_device(other, dev)
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        mla.mla_decode(do["q"], do["kv"], do["block_table"], do["seqlens"])
        torch.cuda.synchronize()
        _say(f"[graph] {kind}: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want_o.view(torch.int16)), f"replay {r}: out differs"
        assert torch.equal(lse.view(torch.int32), want_l.view(torch.int32)), f"replay {r}: lse differs"
        assert torch.equal(d["kv"], kv_after)
