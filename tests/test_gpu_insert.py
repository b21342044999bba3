"""GPU parity of mla_kv_insert (RMSNorm of the latent KV row -> bf16 ->
per-tensor e4m3 at slot -> page/offset) against the float64 oracle, and of the
insert -> decode chain over the per-tensor FP8 cache (run on an MI355X).

Bars: the placement is bit-exact (every byte outside the written rows keeps
its value, skipped tokens write nothing); the rope codes are bit-exact (both
sides encode the exact product of the same bf16 value and fp32 scale); the
latent codes equal the oracle's or are its neighbour in value order, at least
99.9% identical (the fp32 RMSNorm can land on the other side of a bf16
rounding boundary than the float64 one); no NaN code for finite input.
"""
import numpy as np
import pytest
import torch

import mqa_latent_kv_amd as mla
from mqa_latent_kv_amd import synth
from oracle import codecs
from oracle import mla_oracle as mo
from oracle.codecs import f64_to_e4m3

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def code_rank(c):
    """Position of an e4m3fn code in value order (sign-magnitude; both zeros 0)."""
    c = np.asarray(c, dtype=np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def run_insert(inp, qkv=None, slots=None, stride_pad=0):
    d = mla.insert_to_device(inp)
    q = d["qkv"] if qkv is None else qkv
    if stride_pad:
        wide = torch.zeros((q.shape[0], q.shape[1] + stride_pad), dtype=q.dtype, device=q.device)
        wide[:, : q.shape[1]] = q
        q = wide
    s = d["slots"] if slots is None else slots
    mla.mla_kv_insert(q, d["w_kva"], s, d["k_scale_inv"], d["cache"], eps=inp["eps"])
    torch.cuda.synchronize()
    return d["cache"].cpu().numpy()


def check_insert(inp, got):
    ref = mo.kv_insert(inp["qkv"], inp["w_kva"], inp["cache"], inp["slots"], inp["k_scale_inv"], inp["eps"])
    want = ref["cache"]
    assert got.shape == want.shape
    P = want.shape[0]
    live = [(int(s) // 64, int(s) % 64) for s in inp["slots"] if 0 <= s < P * 64]
    written = np.zeros(want.shape[:2], dtype=bool)
    for pg, off in live:
        written[pg, off] = True
    np.testing.assert_array_equal(got[~written], inp["cache"][~written])  # untouched rows: bit-exact
    g, w = got[written], want[written]
    np.testing.assert_array_equal(g[:, 512:], w[:, 512:])  # rope codes: bit-exact
    assert not np.any(g == 0xFF) and not np.any(g == 0x7F), "NaN code for finite input"
    step = np.abs(code_rank(g[:, :512]) - code_rank(w[:, :512]))
    same = np.mean(step == 0) if step.size else 1.0
    _say(f"   rows written {len(live)}, latent codes identical {same * 100:.3f}%, max step {step.max(initial=0)}")
    assert step.max(initial=0) <= 1
    assert same >= 0.999
    return ref


CASES = {
    "t300_p20_skips": dict(seed=61, tokens=300, num_pages=20, skipped=37),
    "one_token": dict(seed=62, tokens=1, num_pages=1),
    "t64_ksi_pow2": dict(seed=63, tokens=64, num_pages=4, k_scale_inv=32.0),
    "t1000_ragged_waves": dict(seed=64, tokens=1001, num_pages=40, skipped=100),
    "eps_large": dict(seed=65, tokens=50, num_pages=2, eps=0.5),
    "ksi_small": dict(seed=66, tokens=70, num_pages=3, k_scale_inv=0.01),
}


def _sweep_case(i):
    """Configuration i of the seeded sweep: token count, pool size (from a
    tight fit to a pool many times larger), skipped tokens, scale and eps at
    random."""
    rng = np.random.default_rng(7000 + i)
    tokens = int(rng.integers(1, 601))
    num_pages = -(-tokens // 64) + int(rng.integers(0, 30))
    return dict(tokens=tokens, num_pages=num_pages, skipped=int(rng.integers(0, tokens // 4 + 1)),
                k_scale_inv=float(rng.choice([0.01, 1.0, 3.0, 32.0, 37.0])), eps=float(rng.choice([1e-6, 1e-3, 0.5])))


@pytest.mark.parametrize("i", range(16))
def test_insert_random_configurations(i):
    """A seeded sweep of the insert's sizes, skips, scales and eps."""
    kw = _sweep_case(i)
    inp = synth.make_insert_inputs(8000 + i, **kw)
    _say(f"[insert sweep] i={i} {kw}")
    check_insert(inp, run_insert(inp))


@pytest.mark.parametrize("name", list(CASES))
def test_insert_matches_oracle(name):
    kw = dict(CASES[name])
    inp = synth.make_insert_inputs(kw.pop("seed"), **kw)
    _say(f"[insert] case={name} T={inp['tokens']} pages={inp['cache'].shape[0]}")
    check_insert(inp, run_insert(inp))


def test_insert_row_stride_and_edge_slots():
    """Rows padded past 2112 columns; the first and last slot of the pool; a
    slot one past the end (skipped, never written); every token skipped."""
    inp = synth.make_insert_inputs(67, tokens=6, num_pages=3)
    P = 3
    inp["slots"] = np.array([0, P * 64 - 1, P * 64, -1, 65, 130], dtype=np.int64)
    _say("[insert] stride 2176, edge slots")
    got = run_insert(inp, stride_pad=64)
    check_insert(inp, got)
    inp["slots"] = np.full(6, -1, dtype=np.int64)
    _say("[insert] all skipped")
    got = run_insert(inp)
    np.testing.assert_array_equal(got, inp["cache"])


def test_insert_saturates_and_zero_rows():
    """A huge k_scale_inv saturates to 0x7E / 0xFE; an all-zero latent row
    (eps > 0) gives zero codes."""
    inp = synth.make_insert_inputs(68, tokens=8, num_pages=1, k_scale_inv=1.0e5)
    inp["qkv"][3, 1536:2112] = 0
    _say("[insert] saturation, zero row")
    got = run_insert(inp)
    ref = check_insert(inp, got)
    assert np.mean(np.isin(ref["codes"], (0x7E, 0xFE))) > 0.5
    assert np.all(ref["codes"][3] == 0)


def test_insert_then_decode_chain():
    """New tokens written by mla_kv_insert at the last position of each
    sequence, then mla_decode over the per-tensor cache, against the oracle's
    insert and decode of the same inputs."""
    dec = synth.make_decode_inputs(69, batch=4, heads=64, seqlens=[1, 700, 1500, 64], kv_format="fp8_tensor")
    ins = synth.make_insert_inputs(70, tokens=4, num_pages=1)
    slots = np.array([mo.physical_rows(dec["block_table"][b], np.array([int(dec["seqlens"][b]) - 1]))[0]
                      for b in range(4)], dtype=np.int64)
    ksi = float(dec["kv_scales"][0])
    ins.update(cache=dec["kv"], slots=slots, k_scale_inv=ksi)
    _say("[insert -> decode] B=4 H=64")
    d = mla.to_device(dec)
    di = mla.insert_to_device(ins)
    mla.mla_kv_insert(di["qkv"], di["w_kva"], di["slots"], d["kv_scales"], d["kv"], eps=ins["eps"])
    out, lse = mla.mla_decode(d["q"], d["kv"], d["block_table"], d["seqlens"], None, d["kv_scales"])
    torch.cuda.synchronize()
    ref_cache = check_insert(ins, d["kv"].cpu().numpy())["cache"]
    ref = mo.mla_decode(dec["q"], ref_cache, dec["block_table"], dec["seqlens"], None, dec["kv_scales"],
                        kv_format="fp8_tensor")
    err_o = np.max(np.abs(out.float().cpu().numpy() - ref["O"]))
    err_l = np.max(np.abs(lse.cpu().numpy() - ref["LSE"]))
    _say(f"   max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= 2e-2 and err_l <= 1e-3


def test_insert_full_size_in_benchmark_configuration():
    """The 64-token insert into the 4096-page per-tensor cache of the
    benchmarked insert + decode step (slots at each sequence's last position),
    every written row and the rest of the pool checked."""
    dec = synth.workload_inputs("insert_decode")
    ins = synth.make_insert_inputs(6, tokens=dec["batch"], num_pages=1)
    last = dec["seqlens"].astype(np.int64) - 1
    slots = np.array([mo.physical_rows(dec["block_table"][b], last[b : b + 1])[0] for b in range(dec["batch"])],
                     dtype=np.int64)
    ins.update(cache=dec["kv"], slots=slots, k_scale_inv=float(dec["kv_scales"][0]))
    _say(f"[insert full-size] T={ins['tokens']} pages={dec['kv'].shape[0]}")
    check_insert(ins, run_insert(ins))


@pytest.mark.parametrize("ksi", [0.3, 1.0 / 3.0, 0.125, 448.0 / 3.0, 1e-3, 7.0, 3.0517578125e-05 * 1.7])
def test_insert_encodes_every_bf16_value(ksi):
    """The device FP8 encoder on every finite bf16 value: 1024 tokens whose 64
    rope values run through all 65536 bf16 bit patterns (non-finite ones
    replaced by 0), with latent inputs of 1 and eps = 0 so that the RMSNorm
    factor is exactly 1 and the latent values are the w_kva weights
    themselves.  Every code must equal the e4m3 code of the exact product
    value * k_scale_inv, bit for bit; scales 0.3 and 1/3 put fp32 products on
    e4m3 midpoints, where the exact product decides."""
    T = 1024
    bits = np.arange(T * 64, dtype=np.uint32).astype(np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] = 0
    rng = np.random.default_rng(7)
    wbits = rng.integers(0, 1 << 16, 512).astype(np.uint16)
    wbits[(wbits & 0x7F80) == 0x7F80] = 0x3F80
    qkv = np.zeros((T, 2112), dtype=np.uint16)
    qkv[:, 1536:2048] = 0x3F80  # 1.0
    qkv[:, 2048:] = bits.reshape(T, 64)
    inp = {"qkv": qkv, "w_kva": wbits, "cache": np.zeros((16, 64, 576), dtype=np.uint8),
           "slots": np.arange(T, dtype=np.int64), "k_scale_inv": float(ksi), "eps": 0.0, "tokens": T}
    _say(f"[insert encoder sweep] k_scale_inv={ksi!r}")
    got = run_insert(inp).reshape(T, 576)
    q = float(np.float32(ksi))
    want_rope = f64_to_e4m3(codecs.bf16_bits_to_f64(bits) * q).reshape(T, 64)
    want_lat = f64_to_e4m3(codecs.bf16_bits_to_f64(wbits) * q)
    np.testing.assert_array_equal(got[:, 512:], want_rope)
    np.testing.assert_array_equal(got[:, :512], np.broadcast_to(want_lat, (T, 512)))
