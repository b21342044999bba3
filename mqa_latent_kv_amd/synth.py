"""Seeded synthetic inputs for MLA decode and the MLA query front end.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the GPU path's tests/benchmark and the CPU oracle are
fed from it.  Everything is drawn on the host with a CPU ``torch.Generator``
seeded explicitly, in a fixed order, and returned as numpy arrays of raw bits:

  * bf16 tensors as ``uint16`` (float32 normal samples rounded to bf16 by
    torch's round-to-nearest-even cast),
  * FP8 codes as ``uint8`` (float32 N(0,1) samples cast to e4m3fn by torch;
    |x| < 448 always holds for these samples, so no saturation is involved),
  * fp32 scales as ``float32``, int32 tables as ``int32``.

Draw order for a decode input: q, seqlens, KV pool (nope codes / bf16 rows,
then rope, then scales; or, for the per-tensor FP8 cache, all 576 codes of each
row, then the one k_scale_inv), block table, top-k lists.  For a KV-cache
insert: qkv rows, w_kva, the cache's prior contents, the slots, then which
tokens are skipped (slot -1).  The per-workload recipes
(shapes, distributions, page pools) are in ``WORKLOADS``.
"""
from __future__ import annotations

import numpy as np
import torch

PAGE = 64
D_QK = 576
D_NOPE = 512
D_ROPE = 64
FP8_ROW_BYTES = 640
QKV_WIDTH = 2112  # q_a 1536 | latent KV 512 | rope key 64
_CHUNK = 1 << 24  # elements per host draw, bounds peak memory for large pools


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def bf16_normal(g: torch.Generator, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """bf16 bits of N(mean, std^2) samples, drawn in float32 then rounded (RNE)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        x = torch.randn(m, generator=g, dtype=torch.float32)
        if std != 1.0 or mean != 0.0:
            x = x * std + mean
        out[s : s + m] = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return out.reshape(shape)


def fp8_normal(g: torch.Generator, shape) -> np.ndarray:
    """e4m3fn codes of float32 N(0,1) samples (torch's RNE cast)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        x = torch.randn(m, generator=g, dtype=torch.float32)
        out[s : s + m] = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out.reshape(shape)


def log_uniform_scales(g: torch.Generator, shape, lo_exp: float = -2.0, hi_exp: float = 0.0) -> np.ndarray:
    """fp32 scales 10**U(lo_exp, hi_exp)."""
    u = torch.rand(tuple(shape), generator=g, dtype=torch.float64)
    return (10.0 ** (lo_exp + (hi_exp - lo_exp) * u)).to(torch.float32).numpy()


def fp8_records(codes: np.ndarray, rope_bits: np.ndarray) -> np.ndarray:
    """Pack [P, 64, 512] e4m3 codes and [P, 64, 64] bf16 rope bits into the FP8
    cache rows [P, 64, 640] (codes, then rope as little-endian bf16)."""
    P = codes.shape[0]
    rec = np.empty((P, PAGE, FP8_ROW_BYTES), dtype=np.uint8)
    rec[..., :D_NOPE] = codes
    rec[..., D_NOPE:] = np.ascontiguousarray(rope_bits).astype("<u2").view(np.uint8).reshape(P, PAGE, 2 * D_ROPE)
    return rec


def make_decode_inputs(
    seed: int,
    *,
    batch: int,
    heads: int,
    seqlens=None,
    seqlen_range=None,
    num_pages: int | None = None,
    pages_per_seq: int | None = None,
    kv_format: str = "bf16",
    q_format: str = "bf16",
    topk: int = 0,
    topk_pad_max: int = 256,
    q_descale: float = 1.0,
    tokens_per_seq: int = 1,
) -> dict:
    """Seeded inputs for one decode call.

    seqlens: explicit list, or ``seqlen_range=(lo, hi)`` integer-uniform inclusive.
    pages_per_seq: block-table width (default: pages of the longest sequence).
    num_pages: pool size (default: batch * pages_per_seq); the block table is the
    first batch*pages_per_seq entries of a random permutation of the pool.
    topk > 0: per sequence (and query token), ``topk`` distinct positions drawn
    uniformly from [0, seqlen), sorted, then the last U{0..topk_pad_max} slots
    set to -1.
    tokens_per_seq = T > 1: q is [B, T, H, 576] and the top-k lists [B, T, topk].
    """
    g = _gen(seed)
    B, H, T = batch, heads, tokens_per_seq
    qshape = (B, H, D_QK) if T == 1 else (B, T, H, D_QK)
    if q_format == "bf16":
        q = bf16_normal(g, qshape)
    elif q_format == "fp8":
        q = fp8_normal(g, qshape)
    else:
        raise ValueError(q_format)
    if seqlens is None:
        lo, hi = seqlen_range
        seqlens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).numpy()
    seqlens = np.asarray(seqlens, dtype=np.int32).reshape(B)
    if pages_per_seq is None:
        pages_per_seq = max(1, int(-(-int(seqlens.max()) // PAGE)))
    if num_pages is None:
        num_pages = B * pages_per_seq
    assert num_pages >= B * pages_per_seq
    if kv_format == "bf16":
        kv = bf16_normal(g, (num_pages, PAGE, D_QK))
        kv_scales = None
    elif kv_format == "fp8":
        codes = fp8_normal(g, (num_pages, PAGE, D_NOPE))
        rope = bf16_normal(g, (num_pages, PAGE, D_ROPE))
        kv = fp8_records(codes, rope)
        del codes, rope
        kv_scales = log_uniform_scales(g, (num_pages, PAGE, D_NOPE // 128))
    elif kv_format == "fp8_tensor":
        kv = fp8_normal(g, (num_pages, PAGE, D_QK))
        kv_scales = log_uniform_scales(g, (1,), 0.0, 0.5)  # k_scale_inv in [1, 3.16]
    else:
        raise ValueError(kv_format)
    perm = torch.randperm(num_pages, generator=g).numpy().astype(np.int32)
    block_table = np.ascontiguousarray(perm[: B * pages_per_seq].reshape(B, pages_per_seq))
    topk_idx = None
    if topk:
        topk_idx = np.full((B * T, topk), -1, dtype=np.int32)
        for bt in range(B * T):
            n = int(seqlens[bt // T])
            k = min(topk, n)
            sel = torch.randperm(n, generator=g)[:k].sort().values.numpy().astype(np.int32)
            pad = int(torch.randint(0, topk_pad_max + 1, (1,), generator=g).item())
            topk_idx[bt, :k] = sel
            if pad:
                topk_idx[bt, topk - pad :] = -1
        topk_idx = topk_idx.reshape((B, topk) if T == 1 else (B, T, topk))
    return {
        "q": q,
        "kv": kv,
        "kv_scales": kv_scales,
        "block_table": block_table,
        "seqlens": seqlens,
        "topk_idx": topk_idx,
        "q_format": q_format,
        "kv_format": kv_format,
        "q_descale": float(q_descale),
        "softmax_scale": 192.0**-0.5,
        "heads": H,
        "batch": B,
        "tokens_per_seq": T,
    }


def make_query_inputs(seed: int, *, batch: int, heads: int, width: int = 1536, q_scale_inv: float = 0.125, eps: float = 1e-6) -> dict:
    """Seeded inputs for the query front end: qkv bf16 [B, width] N(0,1);
    w_qa bf16 N(1, 0.1^2) [1536]; W_qb bf16 N(0, 0.02^2) [H*192, 1536];
    W_uk bf16 N(0, 0.02^2) [H, 128, 512]."""
    g = _gen(seed)
    return {
        "qkv": bf16_normal(g, (batch, width)),
        "w_qa": bf16_normal(g, (1536,), mean=1.0, std=0.1),
        "w_qb": bf16_normal(g, (heads * 192, 1536), std=0.02),
        "w_uk": bf16_normal(g, (heads, 128, 512), std=0.02),
        "q_scale_inv": float(q_scale_inv),
        "eps": float(eps),
        "heads": heads,
        "batch": batch,
    }


def make_insert_inputs(seed: int, *, tokens: int, num_pages: int, skipped: int = 0, k_scale_inv: float = 37.0,
                       eps: float = 1e-6) -> dict:
    """Seeded inputs for the KV-cache insert: qkv bf16 [T, 2112] N(0,1); w_kva
    bf16 N(1, 0.1^2) [512]; the per-tensor FP8 cache's prior contents, e4m3
    codes of N(0,1) samples [num_pages, 64, 576]; int64 slots, T distinct slots
    of the pool in random order, then ``skipped`` randomly chosen tokens set to
    -1."""
    g = _gen(seed)
    qkv = bf16_normal(g, (tokens, QKV_WIDTH))
    w_kva = bf16_normal(g, (D_NOPE,), mean=1.0, std=0.1)
    cache = fp8_normal(g, (num_pages, PAGE, D_QK))
    assert tokens <= num_pages * PAGE
    slots = torch.randperm(num_pages * PAGE, generator=g)[:tokens].numpy().astype(np.int64)
    if skipped:
        slots[torch.randperm(tokens, generator=g)[:skipped].numpy()] = -1
    return {
        "qkv": qkv,
        "w_kva": w_kva,
        "cache": cache,
        "slots": slots,
        "k_scale_inv": float(k_scale_inv),
        "eps": float(eps),
        "tokens": tokens,
    }


# Workloads: shapes and distributions of the decode configurations this library
# is measured and tested on.  Seed k for workload k.
WORKLOADS = {
    "tiny_dense": dict(seed=1, batch=1, heads=16, seqlens=[128], num_pages=2, pages_per_seq=2),
    "paged_bf16": dict(seed=2, batch=64, heads=128, seqlen_range=(1024, 4096), num_pages=4096, pages_per_seq=64),
    "paged_bf16_4096": dict(seed=2, batch=64, heads=128, seqlens=[4096] * 64, num_pages=4096, pages_per_seq=64),
    "fp8_cache": dict(seed=3, batch=32, heads=64, seqlen_range=(8192, 32768), num_pages=16384, pages_per_seq=512, kv_format="fp8"),
    "topk_sparse": dict(seed=4, batch=32, heads=128, seqlens=[65536] * 32, num_pages=32768, pages_per_seq=1024, kv_format="fp8", topk=2048, topk_pad_max=256),
    "insert_decode": dict(seed=6, batch=64, heads=128, seqlens=[4096] * 64, num_pages=4096, pages_per_seq=64, kv_format="fp8_tensor"),
    "mtp_bf16": dict(seed=7, batch=64, heads=128, seqlens=[4096] * 64, num_pages=4096, pages_per_seq=64, tokens_per_seq=2),
    "query_decode": dict(seed=5, batch=64, heads=8, seqlens=[8192] * 64, num_pages=8192, pages_per_seq=128, q_format="fp8", q_descale=8.0),
    # the narrow-batch form of the query front end: 4 tokens, all 128 heads
    "query_narrow_decode": dict(seed=8, batch=4, heads=128, seqlens=[8192] * 4, num_pages=512, pages_per_seq=128, q_format="fp8", q_descale=8.0),
}


def workload_inputs(name: str, seed: int | None = None, **overrides) -> dict:
    spec = dict(WORKLOADS[name])
    s = spec.pop("seed")
    spec.update(overrides)
    return make_decode_inputs(s if seed is None else seed, **spec)
