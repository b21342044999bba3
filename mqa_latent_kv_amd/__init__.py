"""MI355X-native absorbed MLA decode: thin Python binding of libmla.so.

The binding only marshals arguments (tensor checks, pointers, the current HIP
stream) into the C ABI declared in include/mla.h; every step of the
computation runs in the library's gfx950 kernels.  PyTorch provides device
memory and streams.  The functions raise if libmla.so is missing or a call
returns an error status; there is no fallback path.

Entry points (same names as the C ABI):
    mla_decode(q, kv_cache, block_table, seqlens, topk_idx=None, kv_scales=None,
               out=None, lse=None, ...)
    mla_query(qkv, w_qa, w_qb, w_uk, q_scale_inv, out=None, ...)
    mla_kv_insert(qkv, w_kva, slots, k_scale_inv, kv_cache, ...)
    mla_decode_noalloc(q, kv_cache, block_table, seqlens, ...)  (library-owned scratch)
    mla_decode_workspace_size(params), mla_decode_workspace_init(params, ws),
    mla_query_workspace_size(params)
    mla_status_string(code), mla_version()
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_DTYPE_BF16 = 1
MLA_DTYPE_FP8_E4M3 = 2
MLA_DTYPE_FP8_E4M3_TENSOR = 3
MLA_ERR_SCRATCH_LIMIT = -6
DECODE_SCRATCH_BYTES = 64 << 20
D_QK = 576
D_V = 512
PAGE_SIZE = 64
FP8_ROW_BYTES = 640
FP8T_ROW_BYTES = 576
QKV_WIDTH = 2112
KV_DTYPES = {"bf16": MLA_DTYPE_BF16, "fp8": MLA_DTYPE_FP8_E4M3, "fp8_tensor": MLA_DTYPE_FP8_E4M3_TENSOR}


class MlaError(RuntimeError):
    pass


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_descale", ctypes.c_float),
        ("tokens_per_seq", ctypes.c_int32),
    ]


class InsertParams(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("qkv_stride", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


class QueryParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("qkv_stride", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmla.so (built in-tree by mqa_latent_kv_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MlaError(f"{LIB_PATH} is missing: build it with `python -m mqa_latent_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.mla_version.restype = i32
        L.mla_version.argtypes = []
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_status_string.argtypes = [i32]
        L.mla_decode_workspace_size.restype = i32
        L.mla_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeParams), ctypes.POINTER(sz)]
        L.mla_decode_workspace_init.restype = i32
        L.mla_decode_workspace_init.argtypes = [ctypes.POINTER(DecodeParams), vp, sz, vp]
        L.mla_decode.restype = i32
        L.mla_decode.argtypes = [ctypes.POINTER(DecodeParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.mla_decode_noalloc.restype = i32
        L.mla_decode_noalloc.argtypes = [ctypes.POINTER(DecodeParams), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.mla_query_workspace_size.restype = i32
        L.mla_query_workspace_size.argtypes = [ctypes.POINTER(QueryParams), ctypes.POINTER(sz)]
        L.mla_query.restype = i32
        L.mla_query.argtypes = [ctypes.POINTER(QueryParams), vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.mla_kv_insert.restype = i32
        L.mla_kv_insert.argtypes = [ctypes.POINTER(InsertParams), vp, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def mla_version() -> int:
    return int(lib().mla_version())


def mla_status_string(code: int) -> str:
    return lib().mla_status_string(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise MlaError(f"{what} failed: {mla_status_string(code)} ({code})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, device):
    import torch

    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _expect(t, name, dtypes, shape=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def decode_params(*, batch, heads, num_pages, max_pages_per_seq, topk=0, q_fp8=False, kv_format="bf16",
                  softmax_scale=192.0**-0.5, q_descale=1.0, tokens_per_seq=1) -> DecodeParams:
    """kv_format: "bf16", "fp8" (per-tile scales) or "fp8_tensor" (one per-tensor scale)."""
    return DecodeParams(
        batch, heads, num_pages, max_pages_per_seq, topk,
        MLA_DTYPE_FP8_E4M3 if q_fp8 else MLA_DTYPE_BF16,
        KV_DTYPES[kv_format],
        float(softmax_scale), float(q_descale), int(tokens_per_seq),
    )


def mla_decode_workspace_size(params: DecodeParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mla_decode_workspace_size(ctypes.byref(params), ctypes.byref(n)), "mla_decode_workspace_size")
    return int(n.value)


def mla_decode_workspace_init(params: DecodeParams, workspace, stream=None) -> None:
    _check(lib().mla_decode_workspace_init(ctypes.byref(params), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                           _stream_handle(stream, workspace.device)), "mla_decode_workspace_init")


def decode_workspace(params: DecodeParams, device="cuda", stream=None):
    """Allocate and prepare a decode workspace (reusable across calls that fit)."""
    import torch

    ws = torch.empty(max(mla_decode_workspace_size(params), 1), dtype=torch.uint8, device=device)
    mla_decode_workspace_init(params, ws, stream)
    return ws


def _decode_call(q, kv_cache, block_table, seqlens, topk_idx, kv_scales, out, lse, softmax_scale, q_descale):
    """Check the tensors of a decode call; returns (params, out, lse)."""
    import torch

    _expect(q, "q", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn))
    if q.dim() == 3:
        B, H, dq = q.shape
        T = 1
        oshape, lshape = (B, H, D_V), (B, H)
    elif q.dim() == 4:
        B, T, H, dq = q.shape
        oshape, lshape = (B, T, H, D_V), (B, T, H)
    else:
        raise ValueError("q must be [B, H, 576] or [B, T, H, 576]")
    if dq != D_QK:
        raise ValueError("q must have 576 columns")
    q_fp8 = q.dtype != torch.bfloat16
    if kv_cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        _expect(kv_cache, "kv_cache", (torch.uint8, torch.float8_e4m3fn))
        if tuple(kv_cache.shape[1:]) == (PAGE_SIZE, FP8_ROW_BYTES):
            kv_format = "fp8"
            _expect(kv_scales, "kv_scales", (torch.float32,), (kv_cache.shape[0], PAGE_SIZE, 4))
        elif tuple(kv_cache.shape[1:]) == (PAGE_SIZE, FP8T_ROW_BYTES):
            kv_format = "fp8_tensor"
            _expect(kv_scales, "kv_scales", (torch.float32,), (1,))
        else:
            raise ValueError("FP8 kv_cache must be [P, 64, 640] (tile scales) or [P, 64, 576] (per-tensor scale)")
    else:
        kv_format = "bf16"
        _expect(kv_cache, "kv_cache", (torch.bfloat16,))
        if tuple(kv_cache.shape[1:]) != (PAGE_SIZE, D_QK):
            raise ValueError("bf16 kv_cache must be [P, 64, 576]")
        if kv_scales is not None:
            raise ValueError("kv_scales is only for an FP8 cache")
    P = kv_cache.shape[0]
    _expect(block_table, "block_table", (torch.int32,))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    _expect(seqlens, "seqlens", (torch.int32,), (B,))
    topk = 0
    if topk_idx is not None:
        _expect(topk_idx, "topk_idx", (torch.int32,))
        if topk_idx.numel() % (B * T) != 0:
            raise ValueError("topk_idx must be [B, topk] or [B, T, topk]")
        topk = topk_idx.numel() // (B * T)
    dev = q.device
    if out is None:
        out = torch.empty(oshape, dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty(lshape, dtype=torch.float32, device=dev)
    _expect(out, "out", (torch.bfloat16,), oshape)
    _expect(lse, "lse", (torch.float32,), lshape)
    params = decode_params(batch=B, heads=H, num_pages=P, max_pages_per_seq=block_table.shape[1], topk=topk,
                           q_fp8=q_fp8, kv_format=kv_format, softmax_scale=softmax_scale, q_descale=q_descale,
                           tokens_per_seq=T)
    return params, out, lse


def mla_decode(q, kv_cache, block_table, seqlens, topk_idx=None, kv_scales=None, out=None, lse=None, *,
               softmax_scale=192.0**-0.5, q_descale=1.0, workspace=None, stream=None):
    """Absorbed MLA decode (see include/mla.h).

    q: [B, H, 576] (one query token per sequence) or [B, T, H, 576] (T new
    tokens, causal), torch.bfloat16, or uint8 / float8_e4m3fn codes.
    kv_cache: bf16 [P, 64, 576]; or uint8 [P, 64, 640] FP8 rows (then kv_scales
    float32 [P, 64, 4]); or uint8 [P, 64, 576] per-tensor FP8 rows (then
    kv_scales the float32 [1] k_scale_inv).  block_table int32 [B, max_pages], seqlens int32 [B],
    topk_idx int32 [B, topk] ([B, T, topk] for T tokens) or None.  Returns (out bf16 [B, H, 512], lse
    fp32 [B, H]), or [B, T, H, 512] and [B, T, H] for a 4-D q.
    """
    import torch

    params, out, lse = _decode_call(q, kv_cache, block_table, seqlens, topk_idx, kv_scales, out, lse,
                                    softmax_scale, q_descale)
    dev = q.device
    if workspace is None:
        workspace = decode_workspace(params, dev, stream)
    _expect(workspace, "workspace", (torch.uint8,))
    code = lib().mla_decode(
        ctypes.byref(params), _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seqlens), _ptr(topk_idx),
        _ptr(kv_scales), _ptr(out), _ptr(lse), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
        _stream_handle(stream, dev),
    )
    _check(code, "mla_decode")
    return out, lse


def mla_decode_noalloc(q, kv_cache, block_table, seqlens, topk_idx=None, kv_scales=None, out=None, lse=None, *,
                       softmax_scale=192.0**-0.5, q_descale=1.0, stream=None):
    """mla_decode with the library-owned scratch (DECODE_SCRATCH_BYTES per GPU)
    instead of a workspace: the C entry point allocates nothing.  Pass `out`
    and `lse` to keep this wrapper from allocating them.  Calls that overlap
    on one GPU race on the shared scratch; order them on one stream."""
    params, out, lse = _decode_call(q, kv_cache, block_table, seqlens, topk_idx, kv_scales, out, lse,
                                    softmax_scale, q_descale)
    code = lib().mla_decode_noalloc(
        ctypes.byref(params), _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seqlens), _ptr(topk_idx),
        _ptr(kv_scales), _ptr(out), _ptr(lse), _stream_handle(stream, q.device),
    )
    _check(code, "mla_decode_noalloc")
    return out, lse


def mla_query_workspace_size(params: QueryParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mla_query_workspace_size(ctypes.byref(params), ctypes.byref(n)), "mla_query_workspace_size")
    return int(n.value)


def mla_query(qkv, w_qa, w_qb, w_uk, q_scale_inv, out=None, *, eps=1e-6, workspace=None, stream=None):
    """MLA query front end (see include/mla.h).  qkv bf16 [B, >=1536];
    w_qa bf16 [1536]; w_qb bf16 [H*192, 1536]; w_uk bf16 [H, 128, 512];
    q_scale_inv float32 [1] on the device.  Returns uint8 e4m3 codes [B, H, 576]."""
    import torch

    _expect(qkv, "qkv", (torch.bfloat16,))
    B, width = qkv.shape
    _expect(w_uk, "w_uk", (torch.bfloat16,))
    H = w_uk.shape[0]
    _expect(w_uk, "w_uk", (torch.bfloat16,), (H, 128, D_V))
    _expect(w_qa, "w_qa", (torch.bfloat16,), (1536,))
    _expect(w_qb, "w_qb", (torch.bfloat16,), (H * 192, 1536))
    _expect(q_scale_inv, "q_scale_inv", (torch.float32,))
    dev = qkv.device
    if out is None:
        out = torch.empty((B, H, D_QK), dtype=torch.uint8, device=dev)
    _expect(out, "out", (torch.uint8, torch.float8_e4m3fn), (B, H, D_QK))
    params = QueryParams(B, H, width, float(eps))
    need = mla_query_workspace_size(params)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = lib().mla_query(
        ctypes.byref(params), _ptr(qkv), _ptr(w_qa), _ptr(w_qb), _ptr(w_uk), _ptr(q_scale_inv), _ptr(out),
        _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream_handle(stream, dev),
    )
    _check(code, "mla_query")
    return out


def mla_kv_insert(qkv, w_kva, slots, k_scale_inv, kv_cache, *, eps=1e-6, stream=None):
    """KV-cache insert (see include/mla.h).  qkv bf16 [T, >=2112]; w_kva bf16
    [512]; slots int64 [T] (negative: skipped); k_scale_inv float32 [1] on the
    device; kv_cache uint8 / float8_e4m3fn [P, 64, 576], written in place at
    the given slots.  Returns kv_cache."""
    import torch

    _expect(qkv, "qkv", (torch.bfloat16,))
    if qkv.dim() != 2:
        raise ValueError("qkv must be [T, width]")
    T, width = qkv.shape
    _expect(w_kva, "w_kva", (torch.bfloat16,), (D_V,))
    _expect(slots, "slots", (torch.int64,), (T,))
    _expect(k_scale_inv, "k_scale_inv", (torch.float32,), (1,))
    _expect(kv_cache, "kv_cache", (torch.uint8, torch.float8_e4m3fn))
    if kv_cache.dim() != 3 or tuple(kv_cache.shape[1:]) != (PAGE_SIZE, FP8T_ROW_BYTES):
        raise ValueError("kv_cache must be [P, 64, 576]")
    params = InsertParams(T, kv_cache.shape[0], width, float(eps))
    code = lib().mla_kv_insert(
        ctypes.byref(params), _ptr(qkv), _ptr(w_kva), _ptr(slots), _ptr(k_scale_inv), _ptr(kv_cache),
        _stream_handle(stream, qkv.device),
    )
    _check(code, "mla_kv_insert")
    return kv_cache


def insert_to_device(inp: dict, device="cuda"):
    """Move a seeded KV-insert input (numpy raw bits, see synth) to device
    tensors; k_scale_inv becomes a one-element float32 device tensor."""
    import numpy as np
    import torch

    return {
        "qkv": torch.from_numpy(np.ascontiguousarray(inp["qkv"]).view(np.int16)).view(torch.bfloat16).to(device),
        "w_kva": torch.from_numpy(np.ascontiguousarray(inp["w_kva"]).view(np.int16)).view(torch.bfloat16).to(device),
        "cache": torch.from_numpy(np.ascontiguousarray(inp["cache"])).to(device),
        "slots": torch.from_numpy(np.ascontiguousarray(inp["slots"])).to(device),
        "k_scale_inv": torch.tensor([inp["k_scale_inv"]], dtype=torch.float32, device=device),
    }


def to_device(inp: dict, device="cuda"):
    """Move a seeded decode input (numpy raw bits, see synth) to device tensors."""
    import numpy as np
    import torch

    def u16_to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    res = {}
    if inp["q_format"] == "bf16":
        res["q"] = u16_to_bf16(inp["q"])
    else:
        res["q"] = torch.from_numpy(np.ascontiguousarray(inp["q"])).to(device)
    if inp["kv_format"] == "bf16":
        res["kv"] = u16_to_bf16(inp["kv"])
        res["kv_scales"] = None
    else:
        res["kv"] = torch.from_numpy(np.ascontiguousarray(inp["kv"])).to(device)
        res["kv_scales"] = torch.from_numpy(np.ascontiguousarray(inp["kv_scales"])).to(device)
    res["block_table"] = torch.from_numpy(np.ascontiguousarray(inp["block_table"])).to(device)
    res["seqlens"] = torch.from_numpy(np.ascontiguousarray(inp["seqlens"])).to(device)
    res["topk_idx"] = None if inp.get("topk_idx") is None else torch.from_numpy(np.ascontiguousarray(inp["topk_idx"])).to(device)
    return res


def query_to_device(inp: dict, device="cuda"):
    """Move a seeded query-front-end input (numpy raw bits, see synth) to device
    tensors; q_scale_inv becomes a one-element float32 device tensor."""
    import numpy as np
    import torch

    def u16_to_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    return {
        "qkv": u16_to_bf16(inp["qkv"]),
        "w_qa": u16_to_bf16(inp["w_qa"]),
        "w_qb": u16_to_bf16(inp["w_qb"]),
        "w_uk": u16_to_bf16(inp["w_uk"]),
        "q_scale_inv": torch.tensor([inp["q_scale_inv"]], dtype=torch.float32, device=device),
    }
