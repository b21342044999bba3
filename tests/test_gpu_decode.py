"""GPU parity of mla_decode against the float64 oracle (run on an MI355X).

Every case draws seeded inputs from mqa_latent_kv_amd.synth, runs the HIP path
through the C ABI and compares element by element with oracle.mla_decode on
the same bits.  Bars: bf16 O max-abs <= 2e-2 and fp32 LSE max-abs <= 1e-3;
gathers (block-table lookups, sequence boundaries) are checked bit-exactly
through one-hot queries.
"""
import numpy as np
import pytest
import torch

import mqa_latent_kv_amd as mla
from mqa_latent_kv_amd import synth
from oracle import codecs
from oracle import mla_oracle as mo

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 1e-3


def _say(msg):
    print(msg, flush=True)


def run_gpu(inp, **kw):
    d = mla.to_device(inp)
    out, lse = mla.mla_decode(d["q"], d["kv"], d["block_table"], d["seqlens"], d["topk_idx"], d["kv_scales"],
                              q_descale=inp["q_descale"], **kw)
    torch.cuda.synchronize()
    return out, lse


def run_oracle(inp, batches=None):
    return mo.mla_decode(inp["q"], inp["kv"], inp["block_table"], inp["seqlens"], inp["topk_idx"], inp["kv_scales"],
                         q_format=inp["q_format"], kv_format=inp["kv_format"], q_descale=inp["q_descale"],
                         batches=batches)


def abs_weighted_v(inp):
    """sum_t p_t |V_t| per (b, h, c): the size of the terms that O sums, which
    bounds the effect of rounding P to bf16 (dense inputs only)."""
    out = np.zeros((inp["batch"], inp["heads"], 512))
    for b in range(inp["batch"]):
        pos = mo.valid_positions(inp["seqlens"][b])
        kf = mo.dequant_rows(inp["kv"], mo.physical_rows(inp["block_table"][b], pos), inp["kv_format"], inp["kv_scales"])
        _, _, p = mo.attend(mo.query_rows(inp["q"], b, inp["q_format"], inp["q_descale"]), kf, 192.0**-0.5)
        out[b] = p @ np.abs(kf[:, :512])
    return out


def compare(inp, out, lse, batches=None, rtol=0.0, scale=None):
    """Element-wise bars: |dO| <= O_TOL + rtol*scale and |dLSE| <= LSE_TOL.
    rtol is 0 for the N(0,1) workloads; inputs with large |V| add the bf16
    rounding of P and of O (unit roundoff 2^-8 each, bf16 keeping 8
    significant bits) times scale = sum p|V| >= |O|."""
    ref = run_oracle(inp, batches)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    sel = slice(None) if batches is None else list(batches)
    ro, rl = ref["O"][sel], ref["LSE"][sel]
    go, gl = o[sel], l[sel]
    assert np.all(np.isfinite(go)), "non-finite output"
    err_o = np.max(np.abs(go - ro))
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), "LSE -inf pattern differs"
    err_l = np.max(np.abs(gl[~empty] - rl[~empty])) if np.any(~empty) else 0.0
    exc = np.abs(go - ro) - rtol * (scale[sel] if scale is not None else 0.0)
    excess = np.max(exc)
    if excess > O_TOL:
        i = np.unravel_index(np.argmax(exc), exc.shape)
        sc_i = "none" if scale is None else f"{scale[sel][i]:.6g}"
        _say(f"   worst at {i}: gpu={go[i]:.6g} ref={ro[i]:.6g} scale={sc_i} "
             f"lse gpu={gl[i[:-1]]:.6g} ref={rl[i[:-1]]:.6g}")
    _say(f"   max|dO|={err_o:.3e} (max|O|={np.max(np.abs(ro)):.3e}, max excess over rtol term={excess:.3e})"
         f"  max|dLSE|={err_l:.3e}")
    assert err_l <= LSE_TOL
    assert excess <= O_TOL
    return ref


CASES = {
    # name: make_decode_inputs kwargs
    "tiny_dense_b1_h16_s128": dict(seed=1, batch=1, heads=16, seqlens=[128], num_pages=2, pages_per_seq=2),
    "h128_ragged": dict(seed=11, batch=3, heads=128, seqlens=[1, 200, 2100], pages_per_seq=34, num_pages=120),
    "h64_ragged": dict(seed=12, batch=5, heads=64, seqlen_range=(1, 700)),
    "h32_ragged": dict(seed=13, batch=4, heads=32, seqlen_range=(30, 900)),
    "h16_ragged": dict(seed=14, batch=4, heads=16, seqlen_range=(30, 900)),
    "h8_ragged": dict(seed=15, batch=6, heads=8, seqlen_range=(1, 1300)),
    "h8_fp8q": dict(seed=16, batch=6, heads=8, seqlen_range=(100, 1300), q_format="fp8", q_descale=8.0),
    "h128_fp8q": dict(seed=17, batch=2, heads=128, seqlen_range=(500, 1500), q_format="fp8", q_descale=8.0),
    "many_short_seqs": dict(seed=18, batch=300, heads=64, seqlen_range=(1, 100)),
    "one_long_seq": dict(seed=19, batch=1, heads=128, seqlens=[20000]),
    "with_empty_seqs": dict(seed=20, batch=5, heads=64, seqlens=[0, 77, 0, 300, 0], pages_per_seq=5),
    "exact_pages": dict(seed=21, batch=3, heads=128, seqlens=[64, 128, 4096]),
    # 128 heads: ranges of many short sequences, empty sequences
    "h128_many_short": dict(seed=23, batch=300, heads=128, seqlen_range=(1, 100)),
    "h128_with_empty_seqs": dict(seed=24, batch=5, heads=128, seqlens=[0, 33, 0, 1000, 0], pages_per_seq=16),
    # FP8 cache: e4m3 codes with one fp32 scale per row and 128-column tile
    "fp8_h128_ragged": dict(seed=71, batch=3, heads=128, seqlens=[1, 300, 2100], kv_format="fp8"),
    "fp8_h64_ragged": dict(seed=72, batch=5, heads=64, seqlen_range=(1, 1500), kv_format="fp8"),
    "fp8_h32_ragged": dict(seed=73, batch=4, heads=32, seqlen_range=(30, 900), kv_format="fp8"),
    "fp8_h8_fp8q": dict(seed=74, batch=6, heads=8, seqlen_range=(100, 1300), kv_format="fp8", q_format="fp8",
                        q_descale=8.0),
    "fp8_with_empty_seqs": dict(seed=75, batch=4, heads=64, seqlens=[0, 500, 0, 65], pages_per_seq=8,
                                kv_format="fp8"),
    # top-k: sorted distinct positions, trailing -1 padding
    "topk_fp8_h128": dict(seed=81, batch=3, heads=128, seqlens=[3000, 5000, 100], kv_format="fp8", topk=512,
                          topk_pad_max=100),
    "topk_fp8_h64": dict(seed=82, batch=4, heads=64, seqlen_range=(200, 4000), kv_format="fp8", topk=1000),
    "topk_fp8_h16": dict(seed=83, batch=3, heads=16, seqlen_range=(50, 3000), kv_format="fp8", topk=300),
    "topk_bf16_h64": dict(seed=84, batch=3, heads=64, seqlen_range=(500, 3000), topk=700),
    "topk_bf16_h128": dict(seed=85, batch=2, heads=128, seqlens=[4000, 33], topk=256, topk_pad_max=40),
    # per-tensor FP8 cache (the layout mla_kv_insert writes): 576 e4m3 codes per row, one k_scale_inv
    "fp8t_h128_ragged": dict(seed=101, batch=3, heads=128, seqlens=[1, 300, 2100], kv_format="fp8_tensor"),
    "fp8t_h64_ragged": dict(seed=102, batch=5, heads=64, seqlen_range=(1, 1500), kv_format="fp8_tensor"),
    "fp8t_h16_fp8q": dict(seed=103, batch=4, heads=16, seqlen_range=(30, 900), kv_format="fp8_tensor",
                          q_format="fp8", q_descale=8.0),
    "fp8t_h8": dict(seed=104, batch=6, heads=8, seqlen_range=(1, 1300), kv_format="fp8_tensor"),
    "fp8t_with_empty_seqs": dict(seed=105, batch=4, heads=32, seqlens=[0, 500, 0, 65], pages_per_seq=8,
                                 kv_format="fp8_tensor"),
    "topk_fp8t_h128": dict(seed=106, batch=3, heads=128, seqlens=[3000, 5000, 100], kv_format="fp8_tensor",
                           topk=512, topk_pad_max=100),
    "topk_fp8t_h64": dict(seed=107, batch=4, heads=64, seqlen_range=(200, 4000), kv_format="fp8_tensor", topk=1000),
    # T new query tokens per sequence, causal: token t sees positions below seqlen - T + 1 + t.
    # Lengths put the hidden tail inside one slot, across two slots (seqlen % 32 < T - 1) and
    # before any position (seqlen < T).
    "mtp_t2_h64": dict(seed=111, batch=5, heads=64, seqlens=[1, 33, 64, 700, 2049], tokens_per_seq=2),
    "mtp_t3_h128": dict(seed=112, batch=3, heads=128, seqlens=[2, 129, 1500], tokens_per_seq=3),
    "mtp_t4_h8": dict(seed=113, batch=6, heads=8, seqlens=[3, 4, 32, 34, 97, 1300], tokens_per_seq=4),
    "mtp_t16_h8": dict(seed=114, batch=3, heads=8, seqlens=[10, 47, 600], tokens_per_seq=16),
    "mtp_t2_h16_fp8q": dict(seed=115, batch=4, heads=16, seqlen_range=(30, 900), tokens_per_seq=2, q_format="fp8",
                            q_descale=8.0),
    "mtp_t2_h64_fp8": dict(seed=116, batch=4, heads=64, seqlens=[1, 65, 500, 1025], tokens_per_seq=2,
                           kv_format="fp8"),
    "mtp_t3_h32_fp8t": dict(seed=117, batch=4, heads=32, seqlens=[2, 35, 300, 999], tokens_per_seq=3,
                            kv_format="fp8_tensor"),
    "mtp_long_split_t2_h128": dict(seed=118, batch=1, heads=128, seqlens=[20000], tokens_per_seq=2),
    # the hidden tail reaches back into the first of two or more slots (lengths 33, 40 with T = 16;
    # 33 with T = 3), or into a slot before the last (65 with T = 3), at 128 and 384 query rows
    "mtp_t16_h8_first_slot_masked": dict(seed=122, batch=4, heads=8, seqlens=[33, 40, 47, 64], tokens_per_seq=16),
    "mtp_t3_h128_first_slot_masked": dict(seed=123, batch=3, heads=128, seqlens=[33, 34, 65], tokens_per_seq=3),
    # the same on the per-tensor FP8 register-fill path (masked first slot of a multi-slot segment)
    "mtp_t16_h8_first_slot_masked_fp8t": dict(seed=124, batch=4, heads=8, seqlens=[33, 40, 47, 64],
                                              tokens_per_seq=16, kv_format="fp8_tensor"),
    "mtp_t3_h128_first_slot_masked_fp8t": dict(seed=125, batch=3, heads=128, seqlens=[33, 34, 65],
                                               tokens_per_seq=3, kv_format="fp8_tensor"),
    # segments of three or more slots with seqlen % 32 < T - 1: the hidden tail starts in the
    # slot before the last, a masked slot that is neither the first nor the last (64 and 128 rows)
    "mtp_t3_h64_fp8t_masked_mid_slot": dict(seed=126, batch=4, heads=64, seqlens=[97, 129, 226, 1025],
                                            tokens_per_seq=3, kv_format="fp8_tensor"),
    "mtp_t4_h32_fp8t_masked_mid_slot": dict(seed=127, batch=3, heads=32, seqlens=[66, 130, 1026],
                                            tokens_per_seq=4, kv_format="fp8_tensor"),
    # one sequence cut into one-page pieces (51 and 91 of them), combined by the many-piece merge,
    # whose last piece holds only the final 2 (1) positions: rows of the first T - 2 (T - 1) tokens
    # see none of it, a piece with LSE -inf for those rows; then the many-piece merge at 384 query
    # rows over the per-tensor cache, two sequences in three-page pieces
    "wide_merge_t4_h64_hidden_last_piece": dict(seed=131, batch=1, heads=64, seqlens=[64 * 50 + 2],
                                                tokens_per_seq=4),
    "wide_merge_t2_h64_hidden_last_piece": dict(seed=132, batch=1, heads=64, seqlens=[64 * 90 + 1],
                                                tokens_per_seq=2),
    "wide_merge_t3_h128_fp8t_hidden_last_piece": dict(seed=133, batch=2, heads=128, seqlens=[64 * 70 + 2, 64 * 3],
                                                      tokens_per_seq=3, kv_format="fp8_tensor"),
    "mtp_topk_t2_h64_fp8": dict(seed=119, batch=3, heads=64, seqlens=[3000, 800, 40], tokens_per_seq=2,
                                kv_format="fp8", topk=512, topk_pad_max=60),
    "mtp_topk_t3_h128_bf16": dict(seed=120, batch=2, heads=128, seqlens=[2000, 300], tokens_per_seq=3, topk=256,
                                  topk_pad_max=30),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name):
    kw = dict(CASES[name])
    inp = synth.make_decode_inputs(kw.pop("seed"), **kw)
    _say(f"[decode parity] case={name} B={inp['batch']} H={inp['heads']} seqlens[:8]={inp['seqlens'][:8].tolist()}")
    out, lse = run_gpu(inp)
    compare(inp, out, lse)


def test_multi_token_causal_boundary():
    """Every query row points at the first position its token must not see
    (q = 8 k at that position; the last token, which sees everything, points
    at its own position): a row that leaked it would put nearly all its weight
    there, far outside the tolerance."""
    T = 3
    inp = synth.make_decode_inputs(121, batch=4, heads=64, seqlens=[3, 40, 64, 1111], tokens_per_seq=T)
    kv = inp["kv"].reshape(-1, 576)
    q = np.empty_like(inp["q"])
    for b in range(4):
        for t in range(T):
            lim = mo.causal_limit(inp["seqlens"][b], T, t)
            pos = min(lim, int(inp["seqlens"][b]) - 1)
            row = mo.physical_rows(inp["block_table"][b], np.array([pos]))[0]
            q[b, t] = codecs.f64_to_bf16_bits(8.0 * codecs.bf16_bits_to_f64(kv[row]))[None]
    inp["q"] = q
    _say("[decode causal boundary] T=3 H=64")
    out, lse = run_gpu(inp)
    compare(inp, out, lse)


@pytest.mark.parametrize("heads", [128, 64, 8])
def test_running_max_jumps(heads):
    """KV rows scaled up along each sequence make every slot's max exceed the
    running reference by far more than the lazy-rescale threshold, so the
    set-aside-and-restart path runs on most slots (and across split pieces)."""
    inp = synth.make_decode_inputs(61 + heads, batch=3, heads=heads, seqlens=[700, 1500, 129], pages_per_seq=24)
    kv = codecs.bf16_bits_to_f64(inp["kv"]).reshape(-1, 576)
    bt = inp["block_table"]
    for b in range(3):
        n = int(inp["seqlens"][b])
        rows = mo.physical_rows(bt[b], np.arange(n))
        kv[rows] *= (1.0 + np.arange(n) / 16.0)[:, None]
    inp["kv"] = codecs.f64_to_bf16_bits(kv).reshape(inp["kv"].shape)
    _say(f"[decode growing scores] H={heads}")
    out, lse = run_gpu(inp)
    compare(inp, out, lse, rtol=2.0**-7, scale=abs_weighted_v(inp))


@pytest.mark.parametrize("kv_format", ["bf16", "fp8_tensor"])
@pytest.mark.parametrize("half", [0, 1])
def test_running_max_jumps_in_one_token_half(half, kv_format):
    """As above, but only the positions in one half of every 32-token slot
    (p % 32 < 16, or >= 16) grow: with 128 heads each token half of a slot
    has its own softmax wave after a segment's first slot, so only one wave
    sees the jumps and the restart must still use the maximum over both
    halves.  Run on the bf16 copy path and on the per-tensor FP8 register
    fill (there the grown values are re-encoded as e4m3 codes)."""
    inp = synth.make_decode_inputs(131 + half, batch=3, heads=128, seqlens=[700, 1500, 129], pages_per_seq=24,
                                   kv_format=kv_format)
    if kv_format == "bf16":
        kv = codecs.bf16_bits_to_f64(inp["kv"]).reshape(-1, 576)
    else:
        kv = codecs.e4m3_to_f64(inp["kv"]).reshape(-1, 576)
    bt = inp["block_table"]
    for b in range(3):
        n = int(inp["seqlens"][b])
        pos = np.arange(n)
        rows = mo.physical_rows(bt[b], pos)
        grow = ((pos % 32) >= 16) == bool(half)
        kv[rows] *= np.where(grow, 1.0 + pos / 16.0, 1.0)[:, None]
    if kv_format == "bf16":
        inp["kv"] = codecs.f64_to_bf16_bits(kv).reshape(inp["kv"].shape)
    else:
        inp["kv"] = codecs.f64_to_e4m3(kv).reshape(inp["kv"].shape)
    _say(f"[decode growing scores, token half {half}] H=128 kv={kv_format}")
    out, lse = run_gpu(inp)
    compare(inp, out, lse, rtol=2.0**-7, scale=abs_weighted_v(inp))


@pytest.mark.parametrize("heads,e", [(128, 40), (128, -40), (64, 40), (8, 40)])
def test_split_partials_far_from_unit_scale(heads, e):
    """V scaled by 2^e (latent columns times 2^e, the queries' latent columns
    times 2^-e: every score, and so every p, stays the same bit for bit) on
    sequences that split over several ranges.  O scales by 2^e exactly, so
    the bar is the usual one times 2^e.  At 64 and more rows the pieces store
    fp16 partials with a power-of-two factor per row and 128 columns: without
    the factor 2^40 would overflow fp16 and 2^-40 would fall below its
    subnormals."""
    inp = synth.make_decode_inputs(151 + heads + e, batch=3, heads=heads, seqlens=[20000, 3000, 129])
    kv = codecs.bf16_bits_to_f64(inp["kv"]).reshape(-1, 576)
    kv[:, :512] *= 2.0**e
    inp["kv"] = codecs.f64_to_bf16_bits(kv).reshape(inp["kv"].shape)
    q = codecs.bf16_bits_to_f64(inp["q"])
    q[..., :512] *= 2.0**-e
    inp["q"] = codecs.f64_to_bf16_bits(q)
    _say(f"[decode split partials, V x 2^{e}] H={heads}")
    out, lse = run_gpu(inp)
    ref = run_oracle(inp)
    go = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(go)), "non-finite output"
    err_o = np.max(np.abs(go - ref["O"])) * 2.0**-e
    err_l = np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref["LSE"]))
    _say(f"   max|dO|/2^e={err_o:.3e} (max|O|/2^e={np.max(np.abs(ref['O'])) * 2.0**-e:.3e})  max|dLSE|={err_l:.3e}")
    assert err_o <= O_TOL and err_l <= LSE_TOL


def test_topk_masking_rules():
    """Entries that are -1, negative, or at/after seqlen contribute nothing; a
    sequence whose entries are all masked gets O = 0 and LSE = -inf."""
    inp = synth.make_decode_inputs(91, batch=3, heads=64, seqlens=[700, 1200, 900], kv_format="fp8", topk=400)
    t = inp["topk_idx"]
    t[0, ::7] = -1
    t[0, 1::11] = 700 + np.arange(len(t[0, 1::11]), dtype=np.int32)  # at and past seqlen
    t[1, ::5] = -3
    t[2, :] = -1  # nothing to attend
    _say("[decode top-k masking]")
    out, lse = run_gpu(inp)
    compare(inp, out, lse)
    assert torch.all(out[2].float() == 0) and torch.all(torch.isneginf(lse[2]))


def test_outputs_fully_written_and_deterministic():
    inp = synth.make_decode_inputs(31, batch=7, heads=128, seqlen_range=(1, 3000))
    d = mla.to_device(inp)
    _say("[decode] NaN-poisoned outputs, two runs")
    outs = []
    for _ in range(2):
        out = torch.full((7, 128, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((7, 128), float("nan"), dtype=torch.float32, device="cuda")
        mla.mla_decode(d["q"], d["kv"], d["block_table"], d["seqlens"], out=out, lse=lse)
        torch.cuda.synchronize()
        assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
        outs.append((out.clone(), lse.clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))


def _pow2_scales(inp, seed):
    """Replace the FP8 scales by powers of two in {1/2, 1, 2}: code * scale is
    then exact in bf16, so a one-hot softmax must return the row bit for bit."""
    rng = np.random.default_rng(seed)
    inp["kv_scales"] = (2.0 ** rng.integers(-1, 2, inp["kv_scales"].shape)).astype(np.float32)


@pytest.mark.parametrize("heads,kv_format,topk", [(128, "fp8", 0), (64, "fp8", 0), (8, "fp8", 0),
                                                  (128, "fp8", 600), (64, "bf16", 600),
                                                  (128, "fp8_tensor", 0), (8, "fp8_tensor", 0),
                                                  (64, "fp8_tensor", 600)])
def test_one_hot_gather_fp8_and_topk_bit_exact(heads, kv_format, topk):
    """As the bf16 one-hot test, for the FP8 caches (power-of-two scales) and
    for top-k gathers: j* is one of the listed entries, and the expected row
    is the oracle's dequantised V[row(j*)], exact in bf16."""
    B = 3
    inp = synth.make_decode_inputs(141 + heads + topk, batch=B, heads=heads, seqlen_range=(700, 2500),
                                   kv_format=kv_format, topk=topk, topk_pad_max=50)
    if kv_format == "fp8":
        _pow2_scales(inp, heads)
    if kv_format == "fp8_tensor":
        inp["kv_scales"] = np.array([2.0], dtype=np.float32)  # code / 2 is exact in bf16
    rng = np.random.default_rng(heads + topk)
    q = np.empty_like(inp["q"])
    want = np.empty((B, heads, 512), dtype=np.uint16)
    for b in range(B):
        n = int(inp["seqlens"][b])
        if topk:
            cand = inp["topk_idx"][b]
            cand = cand[(cand >= 0) & (cand < n)]
            js = rng.choice(cand, heads)
            js[0] = cand[-1]
        else:
            js = rng.integers(0, n, heads)
            js[0] = n - 1
        rows = mo.physical_rows(inp["block_table"][b], js)
        kf = mo.dequant_rows(inp["kv"], rows, inp["kv_format"], inp["kv_scales"])
        # gain 32 (exact in bf16): every other token then trails by so many
        # logits that its weight is 0 in fp32, also where V[row(j*)] has exact
        # zeros (e4m3 codes 0x00 / 0x80), which a smaller gain would leave at
        # ~1e-30 instead of 0
        q[b] = codecs.f64_to_bf16_bits(32.0 * kf)
        want[b] = codecs.f64_to_bf16_bits(kf[:, :512])
        assert np.array_equal(codecs.bf16_bits_to_f64(want[b]), kf[:, :512])  # exact in bf16
    inp["q"] = q
    _say(f"[decode one-hot] H={heads} kv={kv_format} topk={topk}")
    out, lse = run_gpu(inp)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    # e4m3 code 0x80 is -0: the sum p * V gives +0 for it, and the two zeros
    # count as equal
    g, wv = _plus_zero(got), _plus_zero(want)
    bad = np.argwhere(g != wv)
    for i in bad[:8]:
        i = tuple(i)
        gv = float(codecs.bf16_bits_to_f64(np.array([g[i]], dtype=np.uint16))[0])
        wf = float(codecs.bf16_bits_to_f64(np.array([wv[i]], dtype=np.uint16))[0])
        _say(f"   mismatch at {i}: gpu={gv:.6g} ({int(g[i]):#06x}) want={wf:.6g} ({int(wv[i]):#06x})")
    np.testing.assert_array_equal(g, wv)


def _plus_zero(bits):
    return np.where((bits & 0x7FFF) == 0, 0, bits).astype(np.uint16)


@pytest.mark.parametrize("heads", [128, 64, 8])
def test_one_hot_gather_is_bit_exact(heads):
    """q[b,h] = 5 * k[row(j*)] makes position j* win by a logit gap of ~170, so
    p(j*) = 1 exactly in fp32 and O must equal V[row(j*)] bit for bit: a wrong
    block-table lookup, tail mask or slot offset shows up as a wrong row."""
    B = 4
    inp = synth.make_decode_inputs(41 + heads, batch=B, heads=heads, seqlen_range=(300, 2500))
    rng = np.random.default_rng(heads)
    kvf = inp["kv"].reshape(-1, 576)
    jstar = np.zeros((B, heads), dtype=np.int64)
    q = np.empty_like(inp["q"])
    for b in range(B):
        n = int(inp["seqlens"][b])
        js = rng.integers(0, n, heads)
        js[0] = n - 1  # the last valid token (tail of the last page)
        js[1 % heads] = 0
        jstar[b] = js
        rows = mo.physical_rows(inp["block_table"][b], js)
        q[b] = codecs.f64_to_bf16_bits(5.0 * codecs.bf16_bits_to_f64(kvf[rows]))
    inp["q"] = q
    _say(f"[decode one-hot] H={heads}")
    out, lse = run_gpu(inp)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    for b in range(B):
        rows = mo.physical_rows(inp["block_table"][b], jstar[b])
        np.testing.assert_array_equal(got[b], kvf[rows][:, :512])


def test_page_permutation_invariance_bitwise():
    inp = synth.make_decode_inputs(51, batch=3, heads=64, seqlen_range=(100, 1500), num_pages=80, pages_per_seq=24)
    _say("[decode] page permutation")
    out1, lse1 = run_gpu(inp)
    P = inp["kv"].shape[0]
    perm = np.random.default_rng(2).permutation(P)
    inv = np.argsort(perm)
    inp2 = dict(inp)
    inp2["kv"] = np.ascontiguousarray(inp["kv"][perm])
    inp2["block_table"] = inv[inp["block_table"]].astype(np.int32)
    out2, lse2 = run_gpu(inp2)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))


def _sweep_case(i):
    """Configuration i of the seeded sweep: cache format, heads, query tokens
    per sequence, top-k length, query format, batch and lengths drawn at
    random (empty sequences and page-multiple lengths included), at sizes the
    oracle finishes in about a second."""
    rng = np.random.default_rng(1000 + i)
    kv = str(rng.choice(["bf16", "fp8", "fp8_tensor"]))
    heads = int(rng.choice([8, 16, 32, 64, 128], p=[0.15, 0.15, 0.15, 0.25, 0.3]))
    topk = 0 if rng.random() < 0.6 else int(rng.choice([64, 200, 777, 1024]))
    T = 1 if rng.random() < 0.6 else int(rng.integers(2, 5))
    qf = "fp8" if rng.random() < 0.3 else "bf16"
    big = heads * T >= 256
    batch = int(rng.integers(1, 4 if big else 7))
    seqlens = rng.integers(0, (1500 if big else 3000) + 1, batch)
    if rng.random() < 0.3:
        seqlens[rng.integers(0, batch)] = 0
    if rng.random() < 0.3:
        seqlens[rng.integers(0, batch)] = 64 * int(rng.integers(1, 24))
    pps = max(1, -(-int(seqlens.max()) // 64)) + int(rng.integers(0, 3))
    kw = dict(batch=batch, heads=heads, seqlens=seqlens.tolist(), pages_per_seq=pps,
              num_pages=batch * pps + int(rng.integers(0, 17)), kv_format=kv, q_format=qf, topk=topk,
              tokens_per_seq=T)
    if qf == "fp8":
        kw["q_descale"] = 8.0
    return kw


def _sweep_case_long(i):
    """Configuration i of the second sweep: fewer, longer sequences (up to
    6000 tokens) with up to 512 query rows (T up to 4 at 128 heads), so that
    sequences split over many ranges and slabs."""
    rng = np.random.default_rng(5000 + i)
    kv = str(rng.choice(["bf16", "fp8", "fp8_tensor"]))
    heads = int(rng.choice([64, 128]))
    T = int(rng.choice([1, 1, 2, 4]))
    topk = 0 if rng.random() < 0.7 else int(rng.choice([1024, 2048]))
    qf = "fp8" if rng.random() < 0.3 else "bf16"
    batch = int(rng.integers(1, 3))
    seqlens = rng.integers(2000, 6001, batch)
    pps = -(-int(seqlens.max()) // 64)
    kw = dict(batch=batch, heads=heads, seqlens=seqlens.tolist(), pages_per_seq=pps,
              num_pages=batch * pps + int(rng.integers(0, 9)), kv_format=kv, q_format=qf, topk=topk, tokens_per_seq=T)
    if qf == "fp8":
        kw["q_descale"] = 8.0
    return kw


@pytest.mark.parametrize("i", range(32))
def test_decode_random_long_configurations(i):
    """The second seeded sweep (long sequences, many rows), against the oracle."""
    kw = _sweep_case_long(i)
    inp = synth.make_decode_inputs(6000 + i, **kw)
    _say(f"[decode sweep long] i={i} kv={kw['kv_format']} q={kw['q_format']} H={kw['heads']} T={kw['tokens_per_seq']} "
         f"topk={kw['topk']} seqlens={kw['seqlens']}")
    out, lse = run_gpu(inp)
    compare(inp, out, lse)


@pytest.mark.parametrize("i", range(40))
def test_decode_random_configurations(i):
    """A seeded sweep over the decode's configuration space, each against the
    oracle element by element (the fixed cases above pin the named corners;
    this covers their combinations: FP8 queries on per-tile caches, top-k
    lists with several query tokens, empty sequences beside long ones)."""
    kw = _sweep_case(i)
    inp = synth.make_decode_inputs(2000 + i, **kw)
    _say(f"[decode sweep] i={i} kv={kw['kv_format']} q={kw['q_format']} H={kw['heads']} T={kw['tokens_per_seq']} "
         f"topk={kw['topk']} seqlens={kw['seqlens']}")
    out, lse = run_gpu(inp)
    compare(inp, out, lse)


@pytest.mark.parametrize("name", ["paged_bf16_4096", "paged_bf16", "query_decode", "query_narrow_decode", "fp8_cache", "topk_sparse",
                                  "insert_decode", "mtp_bf16"])
def test_full_size_workloads_sampled(name):
    """The full-size decode workloads, in the launch configuration the
    benchmark times, checked on a sample of sequences the oracle computes."""
    inp = synth.workload_inputs(name)
    _say(f"[decode full-size] {name} B={inp['batch']} H={inp['heads']}")
    out, lse = run_gpu(inp)
    B = inp["batch"]
    sample = sorted(set([0, B - 1] + list(np.random.default_rng(7).choice(B, 4, replace=False))))
    compare(inp, out, lse, batches=sample)
