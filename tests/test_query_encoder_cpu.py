"""The query kernels' FP8 encoder, compiled for the host from the kernel
source, against the oracle's encoder on the exact products: every finite bf16
value times a set of scales, bit-exact.

The kernel rounds the exact product v * q (v bf16, q fp32) once, from an fp32
hi/lo split; the oracle rounds the same product computed exactly in float64
(round to nearest even over the finite e4m3fn values, saturating at +-448).
Scales include 0.3 and 1/3, whose fp32 products land on e4m3 midpoints,
powers of two, the 1/8 of the query workload, extremes that saturate or
underflow, and seeded random ones."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.codecs import f64_to_e4m3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "hostsrc", "e4m3_codes.hip")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def encoder_exe(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("enc") / "e4m3_codes")
    cmd = [hipcc, "-O2", "-std=c++17", "--offload-arch=gfx950", f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


def _scales():
    rng = np.random.default_rng(20261202)
    fixed = [0.125, 0.3, 1.0 / 3.0, 1.0, 7.0, 0.5, 3.0, 1e5, 1e-3, 2.5e-5, 448.0 / 3.0, 1e-30, 1e30]
    rand = np.ldexp(1.0 + rng.integers(0, 1 << 23, 40) / float(1 << 23), rng.integers(-20, 21, 40))
    return np.array(fixed + list(rand), dtype=np.float32)


def test_fp8_encoder_matches_oracle_on_every_bf16_product(encoder_exe):
    qs = _scales()
    res = subprocess.run([encoder_exe], input="".join(f"{float(q).hex()}\n" for q in qs).encode(), capture_output=True)
    assert res.returncode == 0
    got = np.frombuffer(res.stdout, dtype=np.uint8)
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    v = bits[np.isfinite(bits)].astype(np.float64)
    assert got.size == v.size * qs.size
    want = np.concatenate([f64_to_e4m3(v * float(q)) for q in qs]).astype(np.uint8)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{bad.size} codes differ; first: v={v[bad[0] % v.size]!r} q={float(qs[bad[0] // v.size])!r} "
                           f"gpu={got[bad[0]]:#04x} oracle={want[bad[0]]:#04x}")
    assert not np.any(got == 0xFF)
