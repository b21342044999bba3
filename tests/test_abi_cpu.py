"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import mqa_latent_kv_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mla.LIB_PATH):
        from mqa_latent_kv_amd import build

        build.build()
    return mla.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mla_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for name in ("mla_decode", "mla_decode_workspace_size", "mla_query", "mla_query_workspace_size",
                 "mla_kv_insert", "mla_status_string", "mla_version"):
        assert name in fns


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert mla.mla_version() >= 100
    assert mla.mla_status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5):
        assert mla.mla_status_string(code) not in ("ok", "unknown status")
    assert mla.mla_status_string(-99) == "unknown status"


def test_struct_layouts_match_header():
    # all members are 4-byte: the C structs have no padding
    assert ctypes.sizeof(mla.DecodeParams) == 10 * 4
    assert ctypes.sizeof(mla.QueryParams) == 4 * 4
    assert ctypes.sizeof(mla.InsertParams) == 4 * 4


def _params(**kw):
    base = dict(batch=2, heads=128, num_pages=8, max_pages_per_seq=4)
    base.update(kw)
    return mla.decode_params(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _decode(L, p, ws_bytes=1 << 30, **ptrs):
    args = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, topk=None, scales=None, out=FAKE, lse=FAKE, ws=FAKE)
    args.update(ptrs)
    return L.mla_decode(ctypes.byref(p) if p is not None else None, args["q"], args["kv"], args["bt"], args["sl"],
                        args["topk"], args["scales"], args["out"], args["lse"], args["ws"], ctypes.c_size_t(ws_bytes),
                        None)


def _passes_validation(code):
    """A call that passed argument validation stops at the device query (no
    GPU) or at the one-byte workspace (GPU): it never launches on the fake
    pointers."""
    return code in (-5, -3)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(batch=0), -1),
        (dict(heads=0), -1),
        (dict(num_pages=0), -1),
        (dict(max_pages_per_seq=0), -1),
        (dict(topk=-1), -1),
        (dict(softmax_scale=0.0), -1),
        (dict(softmax_scale=float("nan")), -1),
        (dict(heads=7), -2),
        (dict(heads=256), -2),
        (dict(batch=100000), -2),
        (dict(max_pages_per_seq=1 << 26), -2),
    ],
)
def test_decode_param_validation(L, kw, code):
    assert _decode(L, _params(**kw)) == code
    n = ctypes.c_size_t(0)
    assert L.mla_decode_workspace_size(ctypes.byref(_params(**kw)), ctypes.byref(n)) == code


def test_decode_rejects_bad_dtype_enum(L):
    p = _params()
    p.q_dtype = 7
    assert _decode(L, p) == -1
    p = _params()
    p.kv_dtype = 0
    assert _decode(L, p) == -1


def test_decode_null_pointers(L):
    assert _decode(L, None) == -1
    for name in ("q", "kv", "bt", "sl", "out", "lse"):
        assert _decode(L, _params(), **{name: None}) == -1, name
    assert _decode(L, _params(), ws=None) == -3


def test_decode_optional_arguments_must_match_params(L):
    # a top-k list without topk > 0, and topk > 0 without a list
    assert _decode(L, _params(), topk=FAKE) == -1
    assert _decode(L, _params(topk=64)) in (-1, -2)
    # FP8 cache needs scales; a bf16 cache must not get them
    assert _decode(L, _params(kv_format="fp8")) in (-1, -2)
    assert _decode(L, _params(kv_format="fp8_tensor")) == -1
    assert _decode(L, _params(), scales=FAKE) == -1
    # the per-tensor scale is one float: 4-byte alignment is enough
    assert _passes_validation(_decode(L, _params(kv_format="fp8_tensor"), ws_bytes=1, scales=ctypes.c_void_p(0x1004)))
    assert _decode(L, _params(kv_format="fp8_tensor"), scales=ctypes.c_void_p(0x1002)) == -1
    assert _decode(L, _params(kv_format="fp8"), scales=ctypes.c_void_p(0x1004)) == -1
    # the per-tensor layout is a cache format, not a query type
    p = _params()
    p.q_dtype = mla.MLA_DTYPE_FP8_E4M3_TENSOR
    assert _decode(L, p) == -1
    p = _params()
    p.kv_dtype = 4
    assert _decode(L, p, scales=FAKE) == -1


MISALIGNED = ctypes.c_void_p(0x1008)  # 8-byte aligned only


def test_decode_rejects_misaligned_pointers(L):
    # the kernels move q, KV rows, outputs, scales and workspace in 16-byte units
    for name in ("q", "kv", "out", "ws"):
        assert _decode(L, _params(), **{name: MISALIGNED}) == -1, name
    assert _decode(L, _params(kv_format="fp8"), scales=MISALIGNED) == -1
    # int32 tables need only their natural alignment
    assert _passes_validation(_decode(L, _params(), ws_bytes=1, bt=ctypes.c_void_p(0x1004),
                                      sl=ctypes.c_void_p(0x1004)))


def test_decode_tokens_per_seq_bounds(L):
    assert _decode(L, _params(tokens_per_seq=0)) == -1
    assert _decode(L, _params(tokens_per_seq=17)) == -2
    assert _passes_validation(_decode(L, _params(tokens_per_seq=16), ws_bytes=1))
    # B * T * topk entries must stay within 32-bit offsets
    p = _params(batch=4096, topk=(1 << 31) // 8192, tokens_per_seq=2)
    assert _decode(L, p, topk=FAKE) == -2
    p = _params(batch=4096, topk=(1 << 31) // 8192 - 1, tokens_per_seq=2)
    assert _passes_validation(_decode(L, p, ws_bytes=1, topk=FAKE))


def test_decode_rejects_topk_lists_beyond_32_bit_offsets(L):
    p = _params(batch=8192, topk=(1 << 31) // 8192)
    assert _decode(L, p, topk=FAKE) == -2
    n = ctypes.c_size_t(0)
    assert L.mla_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == -2
    p = _params(batch=8192, topk=(1 << 31) // 8192 - 1)
    assert _passes_validation(_decode(L, p, ws_bytes=1, topk=FAKE))


def test_query_validation(L):
    def q(p, ws_bytes=1 << 30, **ptrs):
        a = dict(qkv=FAKE, wqa=FAKE, wqb=FAKE, wuk=FAKE, qsi=FAKE, out=FAKE, ws=FAKE)
        a.update(ptrs)
        return L.mla_query(ctypes.byref(p) if p is not None else None, a["qkv"], a["wqa"], a["wqb"], a["wuk"],
                           a["qsi"], a["out"], a["ws"], ctypes.c_size_t(ws_bytes), None)

    good = mla.QueryParams(64, 8, 1536, 1e-6)
    assert q(None) == -1
    assert q(mla.QueryParams(0, 8, 1536, 1e-6)) == -1
    assert q(mla.QueryParams(64, 8, 1000, 1e-6)) == -1
    assert q(mla.QueryParams(64, 8, 1536, -1.0)) == -1
    assert q(mla.QueryParams(64, 500, 1536, 1e-6)) == -2
    for name in ("qkv", "wqa", "wqb", "wuk", "qsi", "out"):
        assert q(good, **{name: None}) == -1, name
    assert q(good, ws=None) == -3
    # qkv rows are read in 16-byte vectors: the row stride must be a multiple of 8 elements
    assert q(mla.QueryParams(64, 8, 1540, 1e-6)) == -2
    assert q(mla.QueryParams(64, 8, 2112, 1e-6), ws_bytes=1) == -3  # valid up to the workspace size
    for name in ("qkv", "wqa", "wqb", "wuk", "ws"):
        assert q(good, **{name: MISALIGNED}) == -1, name
    # q_scale_inv is one float: 4-byte alignment is required and enough
    assert q(good, qsi=ctypes.c_void_p(0x1002)) == -1
    assert q(good, ws_bytes=1, qsi=ctypes.c_void_p(0x1004)) == -3
    n = ctypes.c_size_t(0)
    assert L.mla_query_workspace_size(ctypes.byref(good), ctypes.byref(n)) == 0 and n.value > 0


def test_kv_insert_validation(L):
    """Every call here fails validation (or has no tokens), so nothing is
    launched and the fake pointers are never used."""
    def ins(p, **ptrs):
        a = dict(qkv=FAKE, w=FAKE, slots=FAKE, ksi=FAKE, cache=FAKE)
        a.update(ptrs)
        return L.mla_kv_insert(ctypes.byref(p) if p is not None else None, a["qkv"], a["w"], a["slots"], a["ksi"],
                               a["cache"], None)

    P = mla.InsertParams
    assert ins(None) == -1
    assert ins(P(-1, 8, 2112, 1e-6)) == -1
    assert ins(P(4, 0, 2112, 1e-6)) == -1
    assert ins(P(4, 8, 2111, 1e-6)) == -1  # the rope key ends at column 2112
    assert ins(P(4, 8, 2112, -1.0)) == -1
    assert ins(P(4, 8, 2116, 1e-6)) == -2  # rows are read in 16-byte vectors
    assert ins(P((1 << 24) + 1, 8, 2112, 1e-6)) == -2
    assert ins(P(4, (1 << 25), 2112, 1e-6)) == -2  # slot rows must fit in 32 bits
    for name in ("qkv", "w", "slots", "ksi", "cache"):
        assert ins(P(4, 8, 2112, 1e-6), **{name: None}) == -1, name
    for name in ("qkv", "w", "cache"):
        assert ins(P(4, 8, 2112, 1e-6), **{name: MISALIGNED}) == -1, name
    assert ins(P(4, 8, 2112, 1e-6), slots=ctypes.c_void_p(0x1004)) == -1  # int64 slots
    assert ins(P(4, 8, 2112, 1e-6), ksi=ctypes.c_void_p(0x1002)) == -1
    # no tokens: a valid call with nothing to launch
    assert ins(P(0, 8, 2112, 1e-6)) == 0
    assert ins(P(0, 8, 2112, 1e-6), slots=ctypes.c_void_p(0x1008), ksi=ctypes.c_void_p(0x1004)) == 0


def test_workspace_size_needs_a_device(L):
    import torch

    n = ctypes.c_size_t(0)
    code = L.mla_decode_workspace_size(ctypes.byref(_params()), ctypes.byref(n))
    if torch.cuda.is_available():
        assert code == 0 and n.value > 0
    else:
        assert code == -5


def test_binding_raises_without_library(monkeypatch):
    monkeypatch.setattr(mla, "_lib", None)
    monkeypatch.setattr(mla, "LIB_PATH", "/nonexistent/libmla.so")
    with pytest.raises(mla.MlaError):
        mla.lib()


def test_query_workspace_sizes_per_form(L):
    """The query's workspace follows its form: up to 8 tokens the bf16 nope
    rows [B][H][128]; from 9 to 128 tokens the bf16 Q_B rows [B][H*192];
    above, the bf16 normalised rows [B][1536] (256-byte aligned) then the
    fp32 Q_B partials [ksplit][B][H*192], with the reduction split in four
    when the 32 x 32 tiles would number under 256."""
    def size(b, h):
        n = ctypes.c_size_t(0)
        assert L.mla_query_workspace_size(ctypes.byref(mla.QueryParams(b, h, 1536, 1e-6)), ctypes.byref(n)) == 0
        return n.value

    def align(x):
        return (x + 255) & ~255

    def tiles(b, h):
        return ((h * 192 + 31) // 32) * ((b + 31) // 32)

    for b, h in [(1, 1), (4, 128), (8, 8)]:
        assert size(b, h) == b * h * 128 * 2 + 256
    for b, h in [(9, 8), (64, 8), (64, 128), (128, 3)]:
        assert size(b, h) == b * h * 192 * 2 + 256, (b, h)
    for b, h in [(129, 1), (129, 128), (8192, 8)]:
        ksplit = 4 if tiles(b, h) < 256 else 1
        assert size(b, h) == align(b * 1536 * 2) + ksplit * b * h * 192 * 4 + 256, (b, h)
    assert tiles(129, 1) < 256 and tiles(129, 128) >= 256  # both forms of the split occur above


def test_lds_dma_assembly_waits_after_writing_m0():
    """Every inline-assembly block of the kernels that writes m0 waits one
    cycle (s_nop) before the instruction that reads it, and names m0 in its
    clobber list: the ISA asks for one wait state between an SALU write of m0
    and a VMEM load to LDS, which the compiler cannot insert inside a block."""
    csrc = os.path.join(os.path.dirname(mla.__file__), "csrc")
    blocks = 0
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".h", ".cpp")):
            continue
        text = open(os.path.join(csrc, name)).read()
        for m in re.finditer(r'asm\s+volatile\s*\((.*?)\);', text, re.S):
            body = m.group(1)
            lead = re.match(r'\s*((?:"(?:[^"\\]|\\.)*"\s*)+)', body)  # the template's string literals
            template = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', lead.group(1))) if lead else ""
            if "m0" not in template:
                continue
            blocks += 1
            insts = [i.strip() for i in template.replace("\\n", "\n").replace("\\t", "").split("\n") if i.strip()]
            for k, inst in enumerate(insts):
                if inst.startswith("s_mov_b32 m0"):
                    assert k + 1 < len(insts) and insts[k + 1].startswith("s_nop"), (name, insts)
            assert '"m0"' in body, (name, "m0 not in the clobber list")
    assert blocks >= 3
