"""Number formats of the MLA decode / query oracle: bf16 and OCP FP8 e4m3fn.

TEST INFRASTRUCTURE ONLY.  This module belongs to the CPU oracle; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The GPU library shares no code with it.

Values are exchanged as raw bit patterns (``uint16`` for bf16, ``uint8`` for
FP8) so that nothing here depends on a framework's own casts; the tests pin
these routines against torch's casts and against brute-force nearest-value
searches.

Formats, as the pages use them:
  * bf16 is the storage type of the latent KV rows, queries and weights, and
    the rounding point after RMSNorm, Q_B and W_UK in the query front end
    (vLLM ``MlaQuery`` API page, class source: every intermediate is cast with
    ``BFloat16(...)``).
  * FP8 is e4m3 of the OCP "fn" flavour: 0x7F/0xFF are NaN and no finite value
    encodes to 0xFF (the ``publish`` docstring on the same page relies on FP8
    bytes never being 0xFF).  Largest finite value 448, smallest subnormal
    2**-9.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------- bf16


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (bf16 is the top half of an f32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _round_to_grid(ax: np.ndarray, min_exp: int, mant_bits: int) -> np.ndarray:
    """Round |x| (f64, finite, >= 0) to the nearest point of a binary float grid
    with ``mant_bits`` explicit mantissa bits and minimum normal exponent
    ``min_exp``; ties go to the even grid point.  No overflow handling."""
    _, e2 = np.frexp(ax)  # ax = m * 2**e2, m in [0.5, 1)
    exp = np.maximum(e2.astype(np.int64) - 1, min_exp)  # floor(log2 ax), clamped for subnormals
    quantum = np.ldexp(1.0, (exp - mant_bits).astype(np.int32))
    # ax / quantum is exact (a power-of-two scaling well inside f64 range) and
    # np.round rounds half to even.
    return np.round(ax / quantum) * quantum


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round f64 values to bf16 (round to nearest, ties to even), directly from
    f64 (no intermediate f32 rounding).  Overflow gives +-inf, NaN gives 0x7FC0."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    finite = np.isfinite(x)
    ax = np.abs(np.where(finite, x, 0.0))
    r = _round_to_grid(ax, -126, 7)
    # The largest finite bf16 is (2 - 2**-7) * 2**127; anything that rounds past
    # it lands exactly on 2**128, which is inf.
    r = np.where(r >= 2.0**128, np.inf, r)
    with np.errstate(over="ignore"):
        mag = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    sign = np.signbit(x).astype(np.uint16) << np.uint16(15)
    out[...] = mag | sign
    out[np.isinf(x)] = np.where(np.signbit(x[np.isinf(x)]), 0xFF80, 0x7F80).astype(np.uint16)
    out[np.isnan(x)] = 0x7FC0
    return out


def bf16_round(x) -> np.ndarray:
    """Value of ``x`` after rounding to bf16 (as f64)."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


# --------------------------------------------------------------------------- e4m3fn

E4M3_MAX = 448.0


def _e4m3_decode_table() -> np.ndarray:
    """All 256 e4m3fn codes by the format's definition: 1 sign bit, 4 exponent
    bits (bias 7), 3 mantissa bits; exponent field 0 is subnormal
    (m/8 * 2**-6); S.1111.111 is NaN; there are no infinities."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * (m / 8.0) * 2.0**-6
        else:
            t[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_TABLE = _e4m3_decode_table()
# Non-negative finite values in code order 0x00..0x7E are strictly increasing.
_E4M3_POS = E4M3_TABLE[:0x7F].copy()


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact value of e4m3fn codes."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def f64_to_e4m3(x) -> np.ndarray:
    """Encode f64 values as e4m3fn codes: round to nearest, ties to even,
    saturating to +-448 (inf saturates too).  NaN encodes as 0x7F, so a finite
    or infinite input never yields 0xFF.  The sign of zero is kept."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    ax = np.abs(np.where(nan, 0.0, x))
    ax = np.minimum(ax, E4M3_MAX)  # saturate before rounding: 448 is a grid point
    r = _round_to_grid(ax, -6, 3)
    r = np.minimum(r, E4M3_MAX)
    idx = np.searchsorted(_E4M3_POS, r)
    assert np.all(_E4M3_POS[idx] == r), "rounded value is not an e4m3 grid point"
    codes = idx.astype(np.uint8) | (np.signbit(x).astype(np.uint8) << np.uint8(7))
    codes = np.where(nan, np.uint8(0x7F), codes).astype(np.uint8)
    return codes


def e4m3_round(x) -> np.ndarray:
    """Value of ``x`` after encoding to e4m3fn (as f64)."""
    return e4m3_to_f64(f64_to_e4m3(x))
