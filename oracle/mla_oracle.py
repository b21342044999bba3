"""Plain CPU float64 oracle for absorbed MLA decode and the MLA query front end.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the GPU library (``mqa_latent_kv_amd``) and imports nothing from it;
inputs arrive as raw bit arrays produced by the seeded generators.

What is computed (sources are the three pages this library is built from):

* Decode.  Multi-query attention where every query head reads the same latent
  KV row ("STAGE_D2" design note, "DSV4 is MQA" shapes: Q per head, one shared
  K/V).  A row holds 576 values: 512 latent ("nope") columns followed by 64
  rope columns; the score of head h against row t is the sum of the nope dot
  product and the rope dot product (FlashMLA issue "dual gemm": the rope part
  is treated as an extra 64-wide block of the same QK^T).  Softmax is per head
  row ("Strategy A: Head-Packed M Dimension": each row of the packed tile is
  one head's attention).  V is the 512 latent columns of the same row.
  The oracle computes the plain definition

      S = (Q @ K^T) * scale,   LSE = log(sum_t exp(S_t)),
      P = exp(S - LSE),        O = P @ V

  in float64, one batch entry at a time, with no blocking or online softmax.

* Paged storage.  Logical position j of sequence b lives in physical row
  ``block_table[b, j // 64] * 64 + j % 64`` of a pool of 64-row pages (the
  page/offset split of a slot, vLLM ``MlaQuery.insert``: page = slot // page
  size, offset = slot % page size).

* Sparse (top-k) decode attends only to listed positions; padding (-1) and
  positions outside [0, seqlen) are masked (FlashMLA issue: invalid slots are
  masked when P is formed).

* Several new query tokens per sequence (T > 1: multi-token prediction or
  speculative decode).  The STAGE_D2 note packs the T*H query rows of a
  sequence into one tile over the same KV rows.  The pages do not state the
  mask; the reading taken is causal: the KV cache already holds the T new
  tokens, and query token t (0-based) sees positions [0, seqlen - T + 1 + t),
  itself included and its successors excluded.  Sparse lists are per query
  token and are cut at the same limit.

* FP8 cache: 512 e4m3fn codes with one fp32 scale per 128-column tile, the 64
  rope values kept in bf16; value = code * scale (the issue's per-buffer
  "dequant" K tiles).

* Per-tensor FP8 cache (the layout ``MlaQuery.insert`` writes): all 576
  columns of a row, rope included, are e4m3fn codes of value * k_scale_inv
  with one fp32 k_scale_inv for the whole cache; value = code / k_scale_inv.

* KV-cache insert (vLLM ``MlaQuery`` API page, ``insert``): for each new
  token with slot >= 0, RMSNorm the 512 latent columns qkv[1536:2048] with
  ``w_kva`` (mean over those 512 columns), round to bf16, then write the e4m3
  codes of (normed * k_scale_inv) and of (qkv[2048:2112] * k_scale_inv) to row
  offset = slot % 64 of page = slot // 64.  Slots < 0 write nothing.

* Query front end (vLLM ``MlaQuery`` API page, ``kernel``): RMSNorm of the
  1536-wide q_a part of ``qkv`` with ``w_qa``; Q_B projection to 192 rows per
  head (128 nope + 64 rope); absorption of the nope part through W_UK[h]
  (128 -> 512); FP8 encoding of the 512 absorbed values and the 64 rope values
  after multiplying by ``q_scale_inv``.  The page rounds to bf16 after RMSNorm,
  after Q_B and after W_UK; the oracle reproduces those three roundings and the
  final FP8 encoding, and does everything else in float64.

Readings of points the pages leave open are listed in the design notes; the
ones that change arithmetic are: LSE is the natural log; the softmax scale
multiplies the full 576-wide dot; no causal mask at one query token; an empty
attended set gives O = 0 and LSE = -inf; no RoPE rotation is applied anywhere;
the RMSNorm factor is 1/sqrt(mean(x^2) + eps) applied as (x * rr) * w.
"""
from __future__ import annotations

import numpy as np

from .codecs import (
    bf16_bits_to_f64,
    bf16_round,
    e4m3_to_f64,
    f64_to_bf16_bits,
    f64_to_e4m3,
)

PAGE = 64
D_QK = 576
D_NOPE = 512
D_ROPE = 64
D_V = 512
FP8_ROW_BYTES = 640  # 512 e4m3 codes + 64 bf16 rope values
FP8T_ROW_BYTES = 576  # per-tensor FP8 cache: 576 e4m3 codes
FP8_TILE = 128  # columns per fp32 scale
Q_A = 1536  # width of the q_a part of qkv
QB_ROWS = 192  # Q_B rows per head: 128 nope + 64 rope
QB_NOPE = 128
KV_LATENT = 1536  # first qkv column of the latent KV row
KV_ROPE = 2048  # first qkv column of the rope key
QKV_WIDTH = 2112  # q_a 1536 | latent 512 | rope 64

# ----------------------------------------------------------------------------- decode


def attend(qf: np.ndarray, kf: np.ndarray, scale: float):
    """Attention of ``H`` query rows over ``n`` shared KV rows, by definition.

    qf: [H, 576] f64, kf: [n, 576] f64.  Returns (O [H, 512], LSE [H], P [H, n]).
    An empty ``kf`` gives O = 0, LSE = -inf.
    """
    H = qf.shape[0]
    n = kf.shape[0]
    if n == 0:
        return np.zeros((H, D_V)), np.full(H, -np.inf), np.zeros((H, 0))
    s = (qf @ kf.T) * scale  # [H, n]
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    p = np.exp(s - lse[:, None])
    o = p @ kf[:, :D_V]
    return o, lse, p


def combine(parts):
    """Merge attention results over disjoint KV subsets (the split-KV combine):
    LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
    ``parts`` is a list of (O_s [..., 512], LSE_s [...]).  Subsets with
    LSE_s = -inf (empty) contribute nothing; all empty gives O = 0, LSE = -inf."""
    lses = np.stack([p[1] for p in parts])  # [S, ...]
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    msafe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - msafe), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, msafe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    o = np.zeros(parts[0][0].shape)
    for (o_s, _), w_s in zip(parts, w):
        o = o + (w_s / np.where(finite, tot, 1.0))[..., None] * o_s
    return o, lse


def valid_positions(seqlen: int, topk_row=None) -> np.ndarray:
    """Logical positions attended by one sequence: all of [0, seqlen) when dense,
    else the listed indices in list order, dropping -1 and anything outside
    [0, seqlen)."""
    if topk_row is None:
        return np.arange(int(seqlen), dtype=np.int64)
    idx = np.asarray(topk_row, dtype=np.int64).reshape(-1)
    return idx[(idx >= 0) & (idx < int(seqlen))]


def physical_rows(block_table_row, positions: np.ndarray) -> np.ndarray:
    """Pool row of each logical position through the block table (int64, exact)."""
    bt = np.asarray(block_table_row, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    return bt[positions // PAGE] * PAGE + positions % PAGE


def dequant_rows(kv, rows: np.ndarray, kv_format: str, kv_scales=None) -> np.ndarray:
    """Latent rows [n, 576] in f64.

    bf16 cache: ``kv`` is uint16 [pages, 64, 576].
    FP8 cache: ``kv`` is uint8 [pages, 64, 640] (512 e4m3 codes, then the 64 rope
    values as little-endian bf16) and ``kv_scales`` float32 [pages, 64, 4]; column
    d < 512 is code * scale[d // 128].
    Per-tensor FP8 cache (``fp8_tensor``): ``kv`` is uint8 [pages, 64, 576], all
    e4m3 codes, and ``kv_scales`` the one fp32 k_scale_inv; value = code / k_scale_inv."""
    if kv_format == "bf16":
        flat = np.asarray(kv).reshape(-1, D_QK)
        return bf16_bits_to_f64(flat[rows])
    if kv_format == "fp8":
        flat = np.asarray(kv).reshape(-1, FP8_ROW_BYTES)[rows]
        sc = np.asarray(kv_scales, dtype=np.float32).reshape(-1, D_NOPE // FP8_TILE)[rows]
        k = np.empty((len(rows), D_QK))
        k[:, :D_NOPE] = e4m3_to_f64(flat[:, :D_NOPE]) * np.repeat(sc.astype(np.float64), FP8_TILE, axis=1)
        rope = np.ascontiguousarray(flat[:, D_NOPE:]).view("<u2")
        k[:, D_NOPE:] = bf16_bits_to_f64(rope)
        return k
    if kv_format == "fp8_tensor":
        flat = np.asarray(kv).reshape(-1, FP8T_ROW_BYTES)[rows]
        ksi = float(np.asarray(kv_scales, dtype=np.float32).reshape(-1)[0])
        return e4m3_to_f64(flat) / ksi
    raise ValueError(f"unknown kv_format {kv_format!r}")


def query_rows(q, b: int, q_format: str, q_descale: float) -> np.ndarray:
    """Query rows of batch entry b as f64 [H, 576].  bf16 queries are exact;
    FP8 queries are code value * q_descale (descale = 1 / q_scale_inv)."""
    qb = np.asarray(q)[b].reshape(-1, D_QK)
    if q_format == "bf16":
        return bf16_bits_to_f64(qb)
    if q_format == "fp8":
        return e4m3_to_f64(qb) * float(q_descale)
    raise ValueError(f"unknown q_format {q_format!r}")


def causal_limit(seqlen: int, T: int, t: int) -> int:
    """Positions visible to query token t of T new tokens: [0, seqlen - T + 1 + t)
    (none when that is empty)."""
    return max(int(seqlen) - int(T) + 1 + int(t), 0)


def mla_decode(
    q,
    kv,
    block_table,
    seqlens,
    topk_idx=None,
    kv_scales=None,
    *,
    q_format: str = "bf16",
    kv_format: str = "bf16",
    q_descale: float = 1.0,
    softmax_scale: float = 192.0**-0.5,
    batches=None,
):
    """Absorbed MLA decode of T new query tokens per sequence.

    q: [B, H, 576] (one token) or [B, T, H, 576] (uint16 bf16 bits or uint8 e4m3
       codes).  kv / kv_scales: see ``dequant_rows``.  block_table: int32
       [B, max_pages].  seqlens: int32 [B], the cache length including the T
       new tokens.  topk_idx: None (dense) or int32 [B, topk] / [B, T, topk]
       logical positions with -1 padding, one list per query token.
    Query token t sees positions below ``causal_limit(seqlen, T, t)``.
    ``batches`` restricts the work to a subset of batch entries (for sampled
    checks of large configurations); other rows of the result stay NaN.

    Returns a dict with f64 ``O`` [B, H, 512] and ``LSE`` [B, H] (natural log)
    when T = 1, [B, T, H, 512] and [B, T, H] when T > 1, plus the stored forms
    ``out_bf16`` (uint16 bits, RNE) and ``lse_f32``.
    """
    q = np.asarray(q)
    if q.ndim == 3:
        q = q[:, None]
    B, T, H = q.shape[0], q.shape[1], q.shape[2]
    seqlens = np.asarray(seqlens).reshape(-1)
    if topk_idx is not None:
        topk_idx = np.asarray(topk_idx).reshape(B, T, -1)
    O = np.full((B, T, H, D_V), np.nan)
    LSE = np.full((B, T, H), np.nan)
    for b in range(B) if batches is None else batches:
        for t in range(T):
            lim = causal_limit(seqlens[b], T, t)
            pos = valid_positions(lim, None if topk_idx is None else topk_idx[b, t])
            rows = physical_rows(np.asarray(block_table)[b], pos)
            kf = dequant_rows(kv, rows, kv_format, kv_scales)
            qf = query_rows(q[:, t], b, q_format, q_descale)
            O[b, t], LSE[b, t], _ = attend(qf, kf, softmax_scale)
    if T == 1:
        O, LSE = O[:, 0], LSE[:, 0]
    # stored forms, of the computed rows only when a subset was asked for
    if batches is None:
        out_bf16 = f64_to_bf16_bits(O)
    else:
        idx = sorted(set(int(b) for b in batches))
        out_bf16 = np.zeros(O.shape, dtype=np.uint16)
        out_bf16[idx] = f64_to_bf16_bits(O[idx])
    return {
        "O": O,
        "LSE": LSE,
        "out_bf16": out_bf16,
        "lse_f32": LSE.astype(np.float32),
    }


# ----------------------------------------------------------------------------- query


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float):
    """RMSNorm over the last axis (width n): rr = 1 / sqrt(sum(x^2) / n + eps),
    applied as (x * rr) * w, before the bf16 rounding.  The q_a rows have
    n = 1536, the latent KV rows n = 512."""
    ss = (x * x).sum(axis=-1, keepdims=True)
    rr = 1.0 / np.sqrt(ss / x.shape[-1] + eps)
    return (x * rr) * w


def mla_query(qkv, w_qa, w_qb, w_uk, q_scale_inv: float, eps: float = 1e-6, heads: int | None = None):
    """The MLA query front end for a batch of tokens.

    qkv: uint16 bf16 bits [B, >=1536] (only columns 0..1535, q_a, are read).
    w_qa: uint16 [1536].  w_qb: uint16 [H*192, 1536], row h*192 + r (r < 128
    nope, 128 <= r < 192 rope).  w_uk: uint16 [H, 128, 512].
    Returns a dict: ``out`` uint8 e4m3fn codes [B, H, 576] (cols 0..511 the
    absorbed latent query, 512..575 the rope query), plus the f64 values before
    each rounding (``xn_pre``, ``qb_pre``, ``ql_pre``), the rounded ones
    (``xn``, ``qb``, ``ql``) and the pre-encoding FP8 inputs (``fp8_in``).
    """
    qkv = np.asarray(qkv)
    B = qkv.shape[0]
    x = bf16_bits_to_f64(qkv[:, :Q_A])
    w = bf16_bits_to_f64(w_qa)
    wqb = bf16_bits_to_f64(w_qb)  # [H*192, 1536]
    wuk = bf16_bits_to_f64(w_uk)  # [H, 128, 512]
    H = wuk.shape[0] if heads is None else heads
    xn_pre = rms_norm(x, w, eps)
    xn = bf16_round(xn_pre)
    qb_pre = (xn @ wqb.T).reshape(B, H, QB_ROWS)
    qb = bf16_round(qb_pre)
    qn, qr = qb[..., :QB_NOPE], qb[..., QB_NOPE:]
    ql_pre = np.empty((B, H, D_NOPE))
    for h in range(H):
        ql_pre[:, h, :] = qn[:, h, :] @ wuk[h]
    ql = bf16_round(ql_pre)
    qsi = float(np.float32(q_scale_inv))
    fp8_in = np.concatenate([ql * qsi, qr * qsi], axis=-1)
    out = f64_to_e4m3(fp8_in)
    return {
        "out": out,
        "xn_pre": xn_pre,
        "xn": xn,
        "qb_pre": qb_pre,
        "qb": qb,
        "ql_pre": ql_pre,
        "ql": ql,
        "fp8_in": fp8_in,
    }


# ----------------------------------------------------------------------------- KV-cache insert


def slot_page_offset(slot: int, page_size: int = PAGE):
    """Page and row offset of a cache slot (integer division, exact)."""
    return int(slot) // page_size, int(slot) % page_size


def kv_insert(qkv, w_kva, cache, slots, k_scale_inv: float, eps: float = 1e-6):
    """The KV-cache insert of the new tokens' latent rows.

    qkv: uint16 bf16 bits [T, >=2112] (columns 1536..2047 the latent KV row,
    2048..2111 the rope key).  w_kva: uint16 [512].  cache: uint8 e4m3 codes
    [pages, 64, 576] (not modified; a written copy is returned).  slots: int
    [T], slot < 0 skips the token.  k_scale_inv: the fp32 per-tensor factor.

    Returns a dict: ``cache`` (the written copy), ``normed_pre`` [T, 512] f64
    (before the bf16 rounding), ``normed`` (after it) and ``fp8_in`` [T, 576]
    (the values that are encoded).  Duplicate non-negative slots: the later
    token's row wins (the GPU leaves that case unspecified).  A slot at or
    past pages * 64 names no row and, like a negative one, writes nothing.
    """
    qkv = np.asarray(qkv)
    x = bf16_bits_to_f64(qkv[:, KV_LATENT:KV_ROPE])
    rope = bf16_bits_to_f64(qkv[:, KV_ROPE:QKV_WIDTH])
    w = bf16_bits_to_f64(w_kva)
    normed_pre = rms_norm(x, w, eps)
    normed = bf16_round(normed_pre)
    ksi = float(np.float32(k_scale_inv))
    fp8_in = np.concatenate([normed * ksi, rope * ksi], axis=-1)
    codes = f64_to_e4m3(fp8_in)
    out = np.array(cache, dtype=np.uint8, copy=True)
    page_size = out.shape[1]
    for t, slot in enumerate(np.asarray(slots).reshape(-1)):
        if slot < 0 or slot >= out.shape[0] * page_size:
            continue
        page, offset = slot_page_offset(slot, page_size)
        out[page, offset, :] = codes[t]
    return {"cache": out, "normed_pre": normed_pre, "normed": normed, "fp8_in": fp8_in, "codes": codes}
