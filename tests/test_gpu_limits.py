"""Parity at the limits the C ABI accepts (run on an MI355X): the largest
batch, the most query tokens per sequence, long top-k lists, a context of
131072 tokens, and a large insert.  Checked against the float64 oracle on
sampled sequences (decode) or in full (insert), with the same bars as the
other parity tests."""
import numpy as np
import pytest
import torch

import mqa_latent_kv_amd as mla
from mqa_latent_kv_amd import synth
from oracle import mla_oracle as mo

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 1e-3


def _say(msg):
    print(msg, flush=True)


def _check(inp, out, lse, batches):
    ref = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], inp["topk_idx"], inp["kv_scales"],
                        q_format=inp["q_format"], kv_format=inp["kv_format"], q_descale=inp["q_descale"],
                        batches=batches)
    o = out.float().cpu().numpy().astype(np.float64)[batches]
    l = lse.cpu().numpy().astype(np.float64)[batches]
    ro, rl = ref["O"][batches], ref["LSE"][batches]
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(l), empty)
    err_o = np.max(np.abs(o - ro))
    err_l = np.max(np.abs(l[~empty] - rl[~empty])) if np.any(~empty) else 0.0
    _say(f"   max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= O_TOL and err_l <= LSE_TOL


def _run(inp):
    d = mla.to_device(inp)
    out, lse = mla.mla_decode(d["q"], d["kv"], d["block_table"], d["seqlens"], d["topk_idx"], d["kv_scales"],
                              q_descale=inp["q_descale"])
    torch.cuda.synchronize()
    return out, lse


def test_largest_batch():
    """MLA_MAX_BATCH sequences of 0 to 100 tokens, 64 heads."""
    inp = synth.make_decode_inputs(201, batch=8192, heads=64, seqlen_range=(0, 100), pages_per_seq=2)
    _say("[limits] B=8192 H=64 seqlen 0..100")
    out, lse = _run(inp)
    sample = [0, 1, 2, 4095, 8190, 8191] + list(np.random.default_rng(3).choice(8192, 10, replace=False))
    _check(inp, out, lse, sorted(set(sample)))


def test_most_tokens_per_sequence_at_128_heads():
    """T = 16 query tokens of 128 heads: 2048 rows over one sequence's KV."""
    inp = synth.make_decode_inputs(202, batch=2, heads=128, seqlens=[15, 300], tokens_per_seq=16)
    _say("[limits] T=16 H=128")
    out, lse = _run(inp)
    _check(inp, out, lse, [0, 1])


def test_long_topk_lists():
    inp = synth.make_decode_inputs(203, batch=2, heads=64, seqlens=[20000, 9000], kv_format="fp8", topk=8192,
                                   topk_pad_max=1000)
    _say("[limits] top-k 8192 of 20000")
    out, lse = _run(inp)
    _check(inp, out, lse, [0, 1])


def test_context_of_131072_tokens():
    inp = synth.make_decode_inputs(204, batch=1, heads=128, seqlens=[131072])
    _say("[limits] s_k=131072 H=128")
    out, lse = _run(inp)
    _check(inp, out, lse, [0])


def test_large_insert():
    """20000 tokens (1000 skipped) into a 1024-page per-tensor cache."""
    inp = synth.make_insert_inputs(205, tokens=20000, num_pages=1024, skipped=1000)
    _say("[limits] insert T=20000")
    d = mla.insert_to_device(inp)
    mla.mla_kv_insert(d["qkv"], d["w_kva"], d["slots"], d["k_scale_inv"], d["cache"], eps=inp["eps"])
    torch.cuda.synchronize()
    got = d["cache"].cpu().numpy()
    want = mo.kv_insert(inp["qkv"], inp["w_kva"], inp["cache"], inp["slots"], inp["k_scale_inv"], inp["eps"])["cache"]
    rank = lambda c: np.where(c & 0x80, -(c.astype(np.int32) & 0x7F), c.astype(np.int32) & 0x7F)
    step = np.abs(rank(got) - rank(want))
    _say(f"   identical {np.mean(got == want) * 100:.4f}%, max step {step.max()}")
    assert step.max() <= 1 and np.mean(step[:, :, 512:] == 0) == 1.0
    assert np.mean(got == want) >= 0.999


@pytest.mark.parametrize("batch,heads", [(8192, 8), (8, 128)])
def test_query_largest_batch_per_form(batch, heads):
    """The query front end at the largest batch of its wide (MFMA) form and
    of its narrow (wave FMA) form, checked on sampled tokens: every token's
    output depends on its own q_a row only, so the oracle runs on those rows.
    Bars as in the query parity tests: every code equal to the oracle's or
    one e4m3 step away, at least 99.9 % identical."""
    qin = synth.make_query_inputs(205 + heads, batch=batch, heads=heads)
    _say(f"[limits] query B={batch} H={heads}")
    d = mla.query_to_device(qin)
    out = mla.mla_query(d["qkv"], d["w_qa"], d["w_qb"], d["w_uk"], d["q_scale_inv"], eps=qin["eps"])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    sample = sorted(set([0, batch - 1] + list(np.random.default_rng(9).choice(batch, min(batch, 6), replace=False))))
    want = mo.mla_query(qin["qkv"][sample], qin["w_qa"], qin["w_qb"], qin["w_uk"], qin["q_scale_inv"],
                        eps=qin["eps"])["out"]
    g = got[sample]
    assert not np.any(g == 0xFF) and not np.any(g == 0x7F), "NaN code for finite input"
    rank = lambda c: np.where(np.asarray(c, np.int32) & 0x80, -(np.asarray(c, np.int32) & 0x7F),
                              np.asarray(c, np.int32) & 0x7F)
    step = np.abs(rank(g) - rank(want))
    same = np.mean(step == 0)
    _say(f"   codes identical {same * 100:.3f}%, max step {step.max()}")
    assert step.max() <= 1 and same >= 0.999
