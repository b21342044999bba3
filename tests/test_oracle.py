"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against an independent fact: a library routine
with a different implementation (torch casts, torch SDPA, torch RMSNorm), a
brute-force search or pure-Python loop on tiny inputs, a closed form, or an
invariant of the mathematics.  They are chosen so that a dropped term, a wrong
sign or index, or a transposed operand in the oracle fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs
from oracle import mla_oracle as mo
from mqa_latent_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = 192.0**-0.5

# ------------------------------------------------------------------ codecs: bf16


def test_bf16_golden_values():
    d = json.load(open(os.path.join(GOLDEN, "bf16_values.json")))
    for code, val in d["decode"].items():
        assert codecs.bf16_bits_to_f64(np.array([int(code, 16)]))[0] == val
    for val, code in d["round"]:
        assert int(codecs.f64_to_bf16_bits(np.array([val]))[0]) == int(code, 16), (val, code)


def test_bf16_round_matches_torch_on_f32_inputs():
    g = torch.Generator().manual_seed(11)
    x = torch.randn(200000, generator=g, dtype=torch.float32) * torch.exp2(torch.randint(-140, 128, (200000,), generator=g).float())
    # exact ties and subnormal-range values
    ties = torch.tensor([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 2.0**-133 * 1.5, 2.0**-134, 3.0 * 2**-135], dtype=torch.float32)
    x = torch.cat([x, ties])
    x = x[torch.isfinite(x)]
    ours = codecs.f64_to_bf16_bits(x.double().numpy())
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_round_brute_force_nearest_even_from_f64():
    """Direct f64 -> bf16 rounding vs brute force over all finite bf16 values
    (no intermediate f32 rounding, which torch's double cast would do)."""
    allbits = np.arange(0x7F80, dtype=np.uint16)  # non-negative finite values, ascending
    vals = codecs.bf16_bits_to_f64(allbits)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-130, 120, 20000))
    # midpoints between neighbours, and midpoints nudged by one f64 ulp
    mids = (vals[1000:1010] + vals[1001:1011]) / 2
    x = np.concatenate([x, mids, np.nextafter(mids, np.inf), np.nextafter(mids, 0), -mids])
    ax = np.abs(x)
    i = np.clip(np.searchsorted(vals, ax), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    pick_hi = (ax - lo > hi - ax) | ((ax - lo == hi - ax) & (allbits[i] % 2 == 0))
    expect = np.where(pick_hi, allbits[i], allbits[i - 1]) | (np.signbit(x).astype(np.uint16) << 15)
    assert np.array_equal(codecs.f64_to_bf16_bits(x), expect)


def test_bf16_specials():
    b = codecs.f64_to_bf16_bits(np.array([np.inf, -np.inf, np.nan, -0.0, 0.0, 1e39, -1e39]))
    assert b.tolist() == [0x7F80, 0xFF80, 0x7FC0, 0x8000, 0x0000, 0x7F80, 0xFF80]


# ------------------------------------------------------------------ codecs: e4m3fn


def test_e4m3_golden_values():
    d = json.load(open(os.path.join(GOLDEN, "e4m3fn_values.json")))
    for code, val in d["codes"].items():
        v = codecs.e4m3_to_f64(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert v == val and math.copysign(1, v) == math.copysign(1, val)
    for code in d["nan_codes"]:
        assert np.isnan(codecs.E4M3_TABLE[int(code, 16)])
    assert np.isnan(codecs.E4M3_TABLE).sum() == 2


def test_e4m3_decode_table_matches_torch():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = codecs.E4M3_TABLE
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_encode_matches_torch_within_range():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(300000, generator=g, dtype=torch.float32) * torch.exp2(torch.randint(-12, 9, (300000,), generator=g).float())
    x = x.clamp(-448, 448)
    # all midpoints between neighbouring codes (ties to even)
    pos = torch.tensor(codecs.E4M3_TABLE[:0x7F], dtype=torch.float64)
    mids = ((pos[1:] + pos[:-1]) / 2).float()
    x = torch.cat([x, mids, -mids, torch.tensor([448.0, -448.0, 0.0, -0.0])])
    ours = codecs.f64_to_e4m3(x.double().numpy())
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_brute_force_nearest_even():
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = codecs.E4M3_TABLE[:0x7F]
    rng = np.random.default_rng(9)
    x = rng.uniform(-448, 448, 50000) * np.exp2(rng.integers(-14, 1, 50000))
    ax = np.abs(x)
    d = np.abs(ax[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equidistant candidates pick the even code
    pick = np.where(cand.sum(axis=1) > 1, np.argmax(cand & (codes[None, :] % 2 == 0), axis=1), np.argmin(d, axis=1))
    expect = codes[pick] | (np.signbit(x).astype(np.uint8) << 7)
    assert np.array_equal(codecs.f64_to_e4m3(x), expect)


def test_e4m3_saturation_nan_and_no_0xff():
    x = np.array([448.0, 460.0, 464.0, 465.0, 1e6, np.inf, -1e6, -np.inf, np.nan])
    c = codecs.f64_to_e4m3(x)
    assert c.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F]
    rng = np.random.default_rng(0)
    y = rng.standard_normal(100000) * 1000
    assert not np.any(codecs.f64_to_e4m3(y) == 0xFF)


# ------------------------------------------------------------------ decode helpers


def _tiny_decode_inputs(seed, B, H, seqlens, kv_format="bf16", topk=0, extra_pages=3):
    pages = max(1, -(-max(seqlens) // 64))
    return synth.make_decode_inputs(
        seed, batch=B, heads=H, seqlens=seqlens, pages_per_seq=pages,
        num_pages=B * pages + extra_pages, kv_format=kv_format, topk=topk, topk_pad_max=min(8, topk) if topk else 0,
    )


def _dense_kq(inp, b):
    """Gather K rows (f64) of sequence b with a pure-Python loop over positions."""
    rows = []
    for j in range(int(inp["seqlens"][b])):
        page = int(inp["block_table"][b][j // 64])
        rows.append(page * 64 + j % 64)
    k = mo.dequant_rows(inp["kv"], np.array(rows, dtype=np.int64), inp["kv_format"], inp["kv_scales"])
    q = codecs.bf16_bits_to_f64(inp["q"][b])
    return k, q


def test_physical_rows_matches_python_loop():
    rng = np.random.default_rng(1)
    bt = rng.permutation(1000)[:37].astype(np.int32)
    pos = rng.integers(0, 37 * 64, 500)
    expect = [int(bt[p // 64]) * 64 + int(p % 64) for p in pos]
    assert mo.physical_rows(bt, pos).tolist() == expect


@pytest.mark.parametrize("H,seqlens", [(16, [128]), (4, [1]), (3, [63, 64]), (4, [65, 200]), (2, [200])])
def test_decode_matches_torch_sdpa(H, seqlens):
    inp = _tiny_decode_inputs(100 + H, len(seqlens), H, seqlens)
    res = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"])
    for b in range(len(seqlens)):
        k, q = _dense_kq(inp, b)
        kt = torch.from_numpy(k)[None, None].expand(1, H, -1, -1)  # shared K for every head
        qt = torch.from_numpy(q)[None, :, None, :]
        vt = torch.from_numpy(k[:, :512])[None, None].expand(1, H, -1, -1)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SCALE)[0, :, 0].numpy()
        np.testing.assert_allclose(res["O"][b], o, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seqlens", [[7], [64, 130], [300]])
def test_lse_matches_sdpa_with_sentinel_key(seqlens):
    """LSE from an independent library path: append a key whose score is
    exactly 0 (zero vector) and whose value is a one-hot extra column; SDPA then
    returns w = 1 / (1 + sum_t exp(S_t)) in that column, so
    LSE = log(1 / w - 1)."""
    H = 3
    inp = _tiny_decode_inputs(7, len(seqlens), H, seqlens)
    res = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"])
    for b in range(len(seqlens)):
        k, q = _dense_kq(inp, b)
        n = k.shape[0]
        k2 = np.vstack([k, np.zeros((1, 576))])
        v2 = np.zeros((n + 1, 513))
        v2[:n, :512] = k[:, :512]
        v2[n, 512] = 1.0
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :],
            torch.from_numpy(k2)[None, None].expand(1, H, -1, -1),
            torch.from_numpy(v2)[None, None].expand(1, H, -1, -1),
            scale=SCALE,
        )[0, :, 0].numpy()
        lse = np.log(1.0 / o[:, 512] - 1.0)
        np.testing.assert_allclose(res["LSE"][b], lse, rtol=0, atol=1e-9)


def test_attend_brute_force_python():
    rng = np.random.default_rng(4)
    H, n = 2, 5
    q = rng.standard_normal((H, 576))
    k = rng.standard_normal((n, 576))
    o, lse, p = mo.attend(q, k, SCALE)
    for h in range(H):
        s = [sum(q[h, d] * k[t, d] for d in range(576)) * SCALE for t in range(n)]
        z = sum(math.exp(x) for x in s)
        assert abs(lse[h] - math.log(z)) < 1e-12
        for c in (0, 17, 511):
            ref = sum(math.exp(s[t]) / z * k[t, c] for t in range(n))
            assert abs(o[h, c] - ref) < 1e-12


def test_softmax_rows_sum_to_one_and_lse_identity():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((8, 576))
    k = rng.standard_normal((333, 576))
    o, lse, p = mo.attend(q, k, SCALE)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12
    s = q @ k.T * SCALE
    # exp(S - LSE) = P, and O = sum_t exp(S_t - LSE) V_t
    np.testing.assert_allclose(np.exp(s - lse[:, None]), p, rtol=1e-12, atol=0)
    np.testing.assert_allclose(o, np.exp(s - lse[:, None]) @ k[:, :512], rtol=0, atol=1e-12)


@pytest.mark.parametrize("split", [1, 64, 100, 299])
def test_split_combine_identity(split):
    rng = np.random.default_rng(split)
    q = rng.standard_normal((5, 576))
    k = rng.standard_normal((300, 576))
    o, lse, _ = mo.attend(q, k, SCALE)
    o1, l1, _ = mo.attend(q, k[:split], SCALE)
    o2, l2, _ = mo.attend(q, k[split:], SCALE)
    oc, lc = mo.combine([(o1, l1), (o2, l2)])
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lc, lse, rtol=0, atol=1e-12)
    # an empty part changes nothing
    oe, le, _ = mo.attend(q, k[:0], SCALE)
    oc2, lc2 = mo.combine([(oc, lc), (oe, le)])
    np.testing.assert_allclose(oc2, o, rtol=0, atol=1e-12)


def test_empty_attended_set():
    inp = _tiny_decode_inputs(2, 2, 4, [0, 5])
    res = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"])
    assert np.all(res["O"][0] == 0) and np.all(np.isneginf(res["LSE"][0]))
    assert np.all(np.isfinite(res["LSE"][1]))


@pytest.mark.parametrize("kv_format", ["bf16", "fp8"])
def test_dense_equals_sparse_with_full_index_list(kv_format):
    seqlens = [150, 64]
    inp = _tiny_decode_inputs(21, 2, 4, seqlens, kv_format=kv_format)
    dense = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], kv_scales=inp["kv_scales"], kv_format=kv_format)
    topk = np.full((2, 160), -1, dtype=np.int32)
    for b, n in enumerate(seqlens):
        topk[b, :n] = np.arange(n)
    sparse = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], topk_idx=topk, kv_scales=inp["kv_scales"], kv_format=kv_format)
    assert np.array_equal(dense["O"], sparse["O"]) and np.array_equal(dense["LSE"], sparse["LSE"])
    # padding and out-of-range entries contribute nothing
    topk2 = topk.copy()
    topk2[0, 150:] = [10**6, -5, 150, 151, 9999, -1, -1, -1, -1, -1]
    sparse2 = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], topk_idx=topk2, kv_scales=inp["kv_scales"], kv_format=kv_format)
    assert np.array_equal(dense["O"], sparse2["O"])


def test_sparse_subset_equals_attend_on_gathered_rows():
    inp = _tiny_decode_inputs(5, 1, 4, [500], topk=64)
    res = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], topk_idx=inp["topk_idx"])
    k_all, q = _dense_kq(inp, 0)
    sel = [int(j) for j in inp["topk_idx"][0] if j >= 0]
    o, lse, _ = mo.attend(q, k_all[sel], SCALE)
    np.testing.assert_allclose(res["O"][0], o, rtol=0, atol=1e-13)


def test_page_permutation_invariance():
    inp = _tiny_decode_inputs(31, 2, 4, [200, 77], extra_pages=5)
    res = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"])
    P = inp["kv"].shape[0]
    perm = np.random.default_rng(3).permutation(P)
    inv = np.argsort(perm)
    kv2 = inp["kv"][perm]  # new page i holds old page perm[i]
    bt2 = inv[inp["block_table"]].astype(np.int32)
    res2 = mo.mla_decode(inp["q"], kv2, bt2, inp["seqlens"])
    assert np.array_equal(res["O"], res2["O"]) and np.array_equal(res["LSE"], res2["LSE"])


def test_closed_forms():
    rng = np.random.default_rng(12)
    n = 97
    k = rng.standard_normal((n, 576))
    # q = 0: uniform attention
    o, lse, _ = mo.attend(np.zeros((2, 576)), k, SCALE)
    np.testing.assert_allclose(lse, np.log(n), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0], k[:, :512].mean(axis=0), rtol=0, atol=1e-14)
    # all rows equal: O is that row, LSE = s + log n
    q = rng.standard_normal((3, 576))
    krep = np.repeat(k[:1], n, axis=0)
    o, lse, _ = mo.attend(q, krep, SCALE)
    np.testing.assert_allclose(o, np.repeat(k[:1, :512], 3, axis=0), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, (q @ k[0]) * SCALE + np.log(n), rtol=0, atol=1e-12)
    # duplicating every row adds log 2 to LSE and leaves O unchanged
    o1, l1, _ = mo.attend(q, k, SCALE)
    o2, l2, _ = mo.attend(q, np.vstack([k, k]), SCALE)
    np.testing.assert_allclose(l2 - l1, np.log(2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    # one token: LSE is its score, O its V row
    o, lse, _ = mo.attend(q, k[5:6], SCALE)
    np.testing.assert_allclose(lse, (q @ k[5]) * SCALE, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, np.repeat(k[5:6, :512], 3, axis=0), rtol=0, atol=0)


def test_rope_columns_count_in_score_but_not_in_v():
    """Score = nope dot + rope dot; V = the 512 nope columns only."""
    n = 2
    k = np.zeros((n, 576))
    k[0, 512] = 1.0  # rope column only
    k[1, 0] = 1.0  # nope column only
    k[0, 3] = 7.0  # a V value of row 0
    q = np.zeros((1, 576))
    q[0, 512] = math.log(3.0) / SCALE  # row 0 scores log 3 via rope; row 1 scores 0
    o, lse, p = mo.attend(q, k, SCALE)
    np.testing.assert_allclose(p[0], [0.75, 0.25], atol=1e-15)
    assert abs(o[0, 3] - 0.75 * 7.0) < 1e-14 and o.shape == (1, 512)
    assert abs(lse[0] - math.log(4.0)) < 1e-14


def test_one_hot_query_selects_row():
    inp = _tiny_decode_inputs(44, 1, 4, [256])
    k, _ = _dense_kq(inp, 0)
    jstar = [3, 100, 200, 255]
    q = np.stack([5.0 * k[j] for j in jstar])
    o, _, _ = mo.attend(codecs.bf16_round(q), k, SCALE)
    for h, j in enumerate(jstar):
        np.testing.assert_allclose(o[h], k[j, :512], rtol=0, atol=1e-20)


def test_fp8_dequant_matches_torch_float8_path():
    inp = _tiny_decode_inputs(9, 1, 2, [100], kv_format="fp8")
    rows = np.arange(0, 128, 3)
    ours = mo.dequant_rows(inp["kv"], rows, "fp8", inp["kv_scales"])
    rec = torch.from_numpy(inp["kv"].reshape(-1, 640)[rows])
    codes = rec[:, :512].contiguous().view(torch.float8_e4m3fn).double()
    sc = torch.from_numpy(inp["kv_scales"].reshape(-1, 4)[rows]).double()
    ref_nope = (codes.view(-1, 4, 128) * sc[:, :, None]).view(-1, 512)
    ref_rope = rec[:, 512:].contiguous().view(torch.bfloat16).double()
    np.testing.assert_array_equal(ours[:, :512], ref_nope.numpy())
    np.testing.assert_array_equal(ours[:, 512:], ref_rope.numpy())


def test_fp8_q_descale():
    inp = synth.make_decode_inputs(3, batch=1, heads=2, seqlens=[70], q_format="fp8", q_descale=8.0)
    r8 = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], q_format="fp8", q_descale=8.0)
    qf = codecs.e4m3_to_f64(inp["q"][0]) * 8.0
    k, _ = _dense_kq(inp, 0)
    o, lse, _ = mo.attend(qf, k, SCALE)
    np.testing.assert_allclose(r8["O"][0], o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(r8["LSE"][0], lse, rtol=0, atol=1e-14)


# ------------------------------------------------------------------ query front end


def _q_inputs(B=5, H=3, seed=17):
    return synth.make_query_inputs(seed, batch=B, heads=H)


def test_rms_norm_matches_torch():
    inp = _q_inputs()
    res = mo.mla_query(inp["qkv"], inp["w_qa"], inp["w_qb"], inp["w_uk"], inp["q_scale_inv"], inp["eps"])
    x = torch.from_numpy(codecs.bf16_bits_to_f64(inp["qkv"][:, :1536]))
    w = torch.from_numpy(codecs.bf16_bits_to_f64(inp["w_qa"]))
    ref = torch.nn.functional.rms_norm(x, (1536,), w, eps=inp["eps"]).numpy()
    np.testing.assert_allclose(res["xn_pre"], ref, rtol=1e-12, atol=0)
    assert np.array_equal(res["xn"], codecs.bf16_round(res["xn_pre"]))


def test_query_projections_match_torch_and_python():
    inp = _q_inputs()
    H = 3
    res = mo.mla_query(inp["qkv"], inp["w_qa"], inp["w_qb"], inp["w_uk"], inp["q_scale_inv"], inp["eps"])
    wqb = torch.from_numpy(codecs.bf16_bits_to_f64(inp["w_qb"]))
    ref = (torch.from_numpy(res["xn"]) @ wqb.T).view(5, H, 192).numpy()
    np.testing.assert_allclose(res["qb_pre"], ref, rtol=1e-12, atol=1e-15)
    # Q_B row h*192 + r belongs to head h, position r
    b, h, r = 2, 1, 150
    s = sum(res["xn"][b, k] * codecs.bf16_bits_to_f64(inp["w_qb"][h * 192 + r, k]) for k in range(1536))
    assert abs(res["qb_pre"][b, h, r] - s) < 1e-13
    # W_UK contraction: the 128 axis of W_uk[h] against the nope part of Q_B
    wuk = codecs.bf16_bits_to_f64(inp["w_uk"])
    c = 300
    s = sum(res["qb"][b, h, p] * wuk[h, p, c] for p in range(128))
    assert abs(res["ql_pre"][b, h, c] - s) < 1e-13


def test_absorption_identity():
    """ql . kv_latent == qn . (W_uk kv_latent): absorbing W_UK into the query
    equals up-projecting the cached latent into the 128-wide nope key space."""
    inp = _q_inputs()
    res = mo.mla_query(inp["qkv"], inp["w_qa"], inp["w_qb"], inp["w_uk"], inp["q_scale_inv"], inp["eps"])
    wuk = codecs.bf16_bits_to_f64(inp["w_uk"])
    lat = np.random.default_rng(1).standard_normal((7, 512))
    for h in range(3):
        lhs = res["ql_pre"][:, h, :] @ lat.T
        k_nope = lat @ wuk[h].T  # [7, 128]: up-projected keys
        rhs = res["qb"][:, h, :128] @ k_nope.T
        np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-13)


def test_query_output_layout_and_encoding():
    inp = _q_inputs(B=4, H=2)
    res = mo.mla_query(inp["qkv"], inp["w_qa"], inp["w_qb"], inp["w_uk"], inp["q_scale_inv"], inp["eps"])
    out = res["out"]
    assert out.shape == (4, 2, 576) and out.dtype == np.uint8
    np.testing.assert_array_equal(out[..., :512], codecs.f64_to_e4m3(res["ql"] * 0.125))
    np.testing.assert_array_equal(out[..., 512:], codecs.f64_to_e4m3(res["qb"][..., 128:] * 0.125))
    assert not np.any(out == 0xFF)


def test_query_identity_weights_closed_form():
    """With W_qb selecting input columns and W_uk an identity block, the output
    is the e4m3 encoding of the bf16 RMSNorm values placed at known columns."""
    B, H = 3, 1
    inp = _q_inputs(B=B, H=H, seed=2)
    wqb = np.zeros((192, 1536))
    for r in range(192):
        wqb[r, 7 * r] = 1.0
    wuk = np.zeros((1, 128, 512))
    for p in range(128):
        wuk[0, p, 511 - p] = 1.0
    res = mo.mla_query(inp["qkv"], inp["w_qa"], codecs.f64_to_bf16_bits(wqb), codecs.f64_to_bf16_bits(wuk), 0.125, 1e-6)
    x = codecs.bf16_bits_to_f64(inp["qkv"][:, :1536])
    w = codecs.bf16_bits_to_f64(inp["w_qa"])
    xn = codecs.bf16_round(x / np.sqrt((x * x).mean(axis=1, keepdims=True) + 1e-6) * w)
    for p in range(128):
        np.testing.assert_array_equal(res["out"][:, 0, 511 - p], codecs.f64_to_e4m3(xn[:, 7 * p] * 0.125))
    for r in range(128, 192):
        np.testing.assert_array_equal(res["out"][:, 0, 512 + r - 128], codecs.f64_to_e4m3(xn[:, 7 * r] * 0.125))
    assert np.all(codecs.e4m3_to_f64(res["out"][:, 0, :384]) == 0)


# ------------------------------------------------------------------ KV-cache insert, per-tensor FP8 cache


def _bf16_bits(values):
    return torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _insert_rows(latent, rope, T=None):
    """qkv bf16 bits [T, 2112]: q_a zeros, then the given latent and rope rows."""
    latent = np.atleast_2d(np.asarray(latent, dtype=np.float64))
    rope = np.atleast_2d(np.asarray(rope, dtype=np.float64))
    T = latent.shape[0]
    x = np.zeros((T, 2112))
    x[:, 1536:2048] = latent
    x[:, 2048:2112] = rope
    return _bf16_bits(x)


def test_insert_slot_placement_by_hand():
    """Slots map to (page, offset) = (slot // 64, slot % 64); -1 writes nothing
    and every other byte of the cache keeps its prior value."""
    inp = synth.make_insert_inputs(31, tokens=5, num_pages=3)
    slots = np.array([130, -1, 0, 191, 64], dtype=np.int64)
    where = {0: (2, 2), 2: (0, 0), 3: (2, 63), 4: (1, 0)}  # written out by hand
    # a slot past the pool (3 pages: 192 rows) writes nothing either
    past = mo.kv_insert(inp["qkv"][:1], inp["w_kva"], inp["cache"], [192], inp["k_scale_inv"], inp["eps"])
    np.testing.assert_array_equal(past["cache"], inp["cache"])
    res = mo.kv_insert(inp["qkv"], inp["w_kva"], inp["cache"], slots, inp["k_scale_inv"], inp["eps"])
    out = res["cache"]
    touched = np.zeros(out.shape[:2], dtype=bool)
    for t, (pg, off) in where.items():
        np.testing.assert_array_equal(out[pg, off], res["codes"][t])
        touched[pg, off] = True
    np.testing.assert_array_equal(out[~touched], inp["cache"][~touched])
    assert not np.array_equal(res["codes"][1], out[0, 1])  # the skipped token's row landed nowhere


def test_insert_constant_rows_closed_form():
    """A constant latent row c has RMS |c|, so with w = 1 and eps = 0 every
    normalised value is sign(c); the rope columns are encoded unnormalised.
    The e4m3fn codes follow from the format's definition: 1.0 = 0x38, 4.0 =
    0x48, 3.0 = 0x44, 0.5 = 0x30, sign bit 0x80."""
    lat = np.array([[0.75] * 512, [-3.0] * 512, [2.0**-9] * 512])
    rope = np.array([[1.5] * 64, [-1.5] * 64, [0.125] * 64])
    qkv = _insert_rows(lat, rope)
    ones = _bf16_bits(np.ones(512))
    cache = np.zeros((1, 64, 576), dtype=np.uint8)
    slots = np.array([0, 1, 2])
    r1 = mo.kv_insert(qkv, ones, cache, slots, 1.0, 0.0)["cache"][0]
    assert np.all(r1[0, :512] == 0x38) and np.all(r1[1, :512] == 0xB8) and np.all(r1[2, :512] == 0x38)
    assert np.all(r1[0, 512:] == 0x3C) and np.all(r1[1, 512:] == 0xBC) and np.all(r1[2, 512:] == 0x20)
    r4 = mo.kv_insert(qkv, ones, cache, slots, 4.0, 0.0)["cache"][0]
    assert np.all(r4[0, :512] == 0x48) and np.all(r4[1, :512] == 0xC8)
    # rope 1.5 * 4 = 6.0 = 1.5 * 2^2: exponent field 9, mantissa 100
    assert np.all(r4[0, 512:] == 0x4C) and np.all(r4[2, 512:] == 0x30)
    half = _bf16_bits(np.full(512, 0.5))
    rh = mo.kv_insert(qkv, half, cache, slots, 1.0, 0.0)["cache"][0]
    assert np.all(rh[0, :512] == 0x30) and np.all(rh[1, :512] == 0xB0)
    # rope 1.5 * 2 = 3.0
    assert np.all(mo.kv_insert(qkv, ones, cache, slots, 2.0, 0.0)["cache"][0][0, 512:] == 0x44)


def test_insert_rms_invariants():
    """With w = 1 and eps = 0 the normalised rows have mean square 1 and are
    unchanged by scaling the input by a power of two; a huge eps reduces the
    norm to x * w / sqrt(eps); an all-zero row gives zero codes."""
    inp = synth.make_insert_inputs(32, tokens=6, num_pages=1)
    ones = _bf16_bits(np.ones(512))
    cache = np.zeros((1, 64, 576), dtype=np.uint8)
    slots = np.arange(6)
    r = mo.kv_insert(inp["qkv"], ones, cache, slots, 1.0, 0.0)
    np.testing.assert_allclose((r["normed_pre"] ** 2).mean(axis=1), 1.0, rtol=1e-13)
    x = codecs.bf16_bits_to_f64(inp["qkv"])
    r8 = mo.kv_insert(codecs.f64_to_bf16_bits(x * 8.0), ones, cache, slots, 1.0, 0.0)
    np.testing.assert_array_equal(r8["codes"][:, :512], r["codes"][:, :512])
    big = mo.kv_insert(inp["qkv"], inp["w_kva"], cache, slots, 1.0, 1e12)
    w = codecs.bf16_bits_to_f64(inp["w_kva"])
    np.testing.assert_allclose(big["normed_pre"], x[:, 1536:2048] * w / 1e6, rtol=1e-9)
    z = mo.kv_insert(_insert_rows(np.zeros((1, 512)), np.zeros((1, 64))), inp["w_kva"], cache, [0], 37.0, 1e-6)
    assert np.all(z["cache"][0, 0] == 0)


def test_insert_matches_torch_rmsnorm_and_float8_cast():
    """The normalised latent row against torch's RMSNorm (float64), and the
    codes against torch's float8_e4m3fn cast, with a power-of-two k_scale_inv so
    that the product is exact in float32."""
    inp = synth.make_insert_inputs(33, tokens=9, num_pages=2, skipped=2)
    res = mo.kv_insert(inp["qkv"], inp["w_kva"], inp["cache"], inp["slots"], 16.0, inp["eps"])
    x = torch.from_numpy(inp["qkv"].view(np.int16)).view(torch.bfloat16).double()
    w = torch.from_numpy(inp["w_kva"].view(np.int16)).view(torch.bfloat16).double()
    ref = torch.nn.functional.rms_norm(x[:, 1536:2048], (512,), w, eps=inp["eps"])
    np.testing.assert_allclose(res["normed_pre"], ref.numpy(), rtol=1e-12, atol=1e-15)
    normed = torch.from_numpy(res["normed"]).float()
    lat = (normed * 16.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    rope = (x[:, 2048:2112].float() * 16.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(res["codes"][:, :512], lat)
    np.testing.assert_array_equal(res["codes"][:, 512:], rope)


def test_per_tensor_dequant_matches_torch_float8():
    inp = synth.make_decode_inputs(34, batch=1, heads=2, seqlens=[90], kv_format="fp8_tensor")
    ksi = float(inp["kv_scales"][0])
    rows = np.arange(0, 128, 5)
    ours = mo.dequant_rows(inp["kv"], rows, "fp8_tensor", inp["kv_scales"])
    codes = torch.from_numpy(inp["kv"].reshape(-1, 576)[rows]).view(torch.float8_e4m3fn).double()
    np.testing.assert_array_equal(ours, (codes / ksi).numpy())


def test_per_tensor_decode_equals_bf16_decode_of_its_values():
    """With a power-of-two k_scale_inv every dequantised value is exact in bf16,
    so decode over the per-tensor FP8 cache equals decode over a bf16 cache that
    holds those values (decoded here by torch), dense and top-k."""
    inp = synth.make_decode_inputs(35, batch=2, heads=4, seqlens=[130, 77], kv_format="fp8_tensor", topk=0)
    ksi = np.array([0.25], dtype=np.float32)
    vals = torch.from_numpy(inp["kv"]).view(torch.float8_e4m3fn).float() / 0.25
    kv16 = vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(vals.to(torch.bfloat16).float().numpy(), vals.numpy())
    topk = np.array([[5, 129, -1, 64, 7], [76, 0, 3, 200, -1]], dtype=np.int32)
    for tk in (None, topk):
        a = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], tk, ksi, kv_format="fp8_tensor")
        b = mo.mla_decode(inp["q"], kv16, inp["block_table"], inp["seqlens"], tk)
        np.testing.assert_array_equal(a["O"], b["O"])
        np.testing.assert_array_equal(a["LSE"], b["LSE"])


def test_insert_then_dequant_within_e4m3_bound():
    """Rows written by the insert and read back through the per-tensor format
    are the bf16 normalised (and rope) values within e4m3's rounding bound:
    relative 2^-4 for normal codes, absolute 2^-10 / k_scale_inv below 2^-6."""
    inp = synth.make_insert_inputs(36, tokens=12, num_pages=1, skipped=3)
    res = mo.kv_insert(inp["qkv"], inp["w_kva"], inp["cache"], inp["slots"], inp["k_scale_inv"], inp["eps"])
    ksi = inp["k_scale_inv"]
    live = inp["slots"] >= 0
    back = mo.dequant_rows(res["cache"], inp["slots"][live], "fp8_tensor", np.array([ksi], np.float32))
    want = res["fp8_in"][live] / ksi
    err = np.abs(back - want)
    bound = np.maximum(np.abs(want) * 2.0**-4, 2.0**-10 / ksi)
    assert np.all(err <= bound)


# ------------------------------------------------------------------ several query tokens per sequence (causal)


def test_multi_token_causal_mask_by_hand_against_sdpa():
    """seqlen 5, T = 3: token 0 sees positions 0..2, token 1 sees 0..3, token 2
    sees 0..4 (the mask below is written out by hand), checked against torch's
    SDPA in float64 with that boolean mask."""
    inp = synth.make_decode_inputs(37, batch=1, heads=2, seqlens=[5], num_pages=1, tokens_per_seq=3)
    res = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"])
    assert res["O"].shape == (1, 3, 2, 512) and res["LSE"].shape == (1, 3, 2)
    visible = np.array([[1, 1, 1, 0, 0], [1, 1, 1, 1, 0], [1, 1, 1, 1, 1]], dtype=bool)
    k, _ = _dense_kq(inp, 0)
    q = torch.from_numpy(codecs.bf16_bits_to_f64(inp["q"][0]))  # [T, H, 576]
    kt = torch.from_numpy(k)
    for h in range(2):
        o = torch.nn.functional.scaled_dot_product_attention(
            q[:, h][None], kt[None], kt[:, :512][None], attn_mask=torch.from_numpy(visible)[None], scale=SCALE)[0]
        np.testing.assert_allclose(res["O"][0, :, h], o.numpy(), rtol=1e-12, atol=1e-14)
        s = (q[:, h] @ kt.T).numpy() * SCALE
        lse = [np.log(np.exp(s[t, visible[t]]).sum()) for t in range(3)]
        np.testing.assert_allclose(res["LSE"][0, :, h], lse, rtol=1e-13)


def test_multi_token_reduces_to_single_token_at_each_position():
    """Token t of a T-token decode equals a one-token decode of the same
    sequence cut to its causal length, dense and sparse (the one-token path is
    pinned against SDPA above)."""
    T = 4
    for topk in (0, 40):
        inp = synth.make_decode_inputs(38 + topk, batch=3, heads=4, seqlens=[70, 3, 129], tokens_per_seq=T,
                                       topk=topk, topk_pad_max=5)
        res = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], inp["topk_idx"])
        for t in range(T):
            cut = np.maximum(inp["seqlens"] - T + 1 + t, 0).astype(np.int32)
            one = mo.mla_decode(inp["q"][:, t], inp["kv"], inp["block_table"], cut,
                                None if topk == 0 else inp["topk_idx"][:, t])
            np.testing.assert_array_equal(res["O"][:, t], one["O"])
            np.testing.assert_array_equal(res["LSE"][:, t], one["LSE"])


def test_multi_token_nothing_visible_and_sparse_cut():
    """seqlen 2 with T = 4: tokens 0 and 1 see nothing (O = 0, LSE = -inf),
    token 2 sees position 0 only, token 3 positions 0 and 1.  A sparse list
    entry at or past the token's own position is masked."""
    inp = synth.make_decode_inputs(39, batch=1, heads=2, seqlens=[2], num_pages=1, tokens_per_seq=4)
    res = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"])
    assert np.all(res["O"][0, :2] == 0) and np.all(np.isneginf(res["LSE"][0, :2]))
    k, _ = _dense_kq(inp, 0)
    np.testing.assert_allclose(res["O"][0, 2], np.broadcast_to(k[0, :512], (2, 512)), rtol=0, atol=1e-15)
    # sparse: seqlen 10, T = 2; lists [9, 8, 1] for both tokens -> token 0 drops 9
    inp = synth.make_decode_inputs(40, batch=1, heads=2, seqlens=[10], num_pages=1, tokens_per_seq=2)
    lists = np.array([[[9, 8, 1], [9, 8, 1]]], dtype=np.int32)
    res = mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], lists)
    k, _ = _dense_kq(inp, 0)
    qf = codecs.bf16_bits_to_f64(inp["q"][0])
    o0, l0, _ = mo.attend(qf[0], k[[8, 1]], SCALE)
    o1, l1, _ = mo.attend(qf[1], k[[9, 8, 1]], SCALE)
    np.testing.assert_array_equal(res["O"][0, 0], o0)
    np.testing.assert_array_equal(res["O"][0, 1], o1)
