"""Pins of the oracle's half-format decode / round-to-nearest-even encode.

IEEE-754 binary16 and bfloat16 are pinned three ways: every bit pattern decoded
against numpy's float16 and a bit shift of binary32; a table of hand-derived edge
cases (tests/golden/half_rounding.txt); and all 2^32 fp32 inputs against the host
compiler's own _Float16 / __bf16 conversions.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def test_decode_every_fp16_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.half_to_double(O.F16, bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_every_bf16_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32)
    got = O.half_to_double(O.BF16, bits.astype(np.uint16))
    want = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def _golden_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "half_rounding.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            a, b, c = line.split()[:3]
            rows.append((int(a, 16), int(b, 16), int(c, 16)))
    return rows


@pytest.mark.parametrize("x,f16,bf16", _golden_rows())
def test_rounding_golden(x, f16, bf16):
    xf = np.array([x], np.uint32).view(np.float32)
    assert int(O.float_to_half(O.F16, xf)[0]) == f16
    assert int(O.float_to_half(O.BF16, xf)[0]) == bf16


def _clang():
    for c in ("/opt/rocm/llvm/bin/clang", shutil.which("clang") or ""):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def cast_check(tmp_path_factory):
    cc = _clang()
    if cc is None:
        pytest.skip("no clang with _Float16/__bf16 on this host")
    from oracle import build
    so = build.build_oracle(force=False)
    exe = str(tmp_path_factory.mktemp("cast") / "cast_check")
    subprocess.run([cc, "-O2", os.path.join(HERE, "cast_check.c"), so,
                    "-Wl,-rpath," + os.path.dirname(so), "-o", exe], check=True)
    return exe


@pytest.mark.parametrize("dtype", [O.F16, O.BF16], ids=["f16", "bf16"])
def test_rounding_exhaustive_all_fp32(cast_check, dtype):
    """All 2^32 fp32 bit patterns, split over the host's cores."""
    parts = max(1, min(8, os.cpu_count() or 1)) * 4
    step = (1 << 32) // parts
    ranges = [(i * step, (1 << 32) if i == parts - 1 else (i + 1) * step) for i in range(parts)]

    def run(r):
        out = subprocess.run([cast_check, str(dtype), str(r[0]), str(r[1])], check=True,
                             capture_output=True, text=True).stdout.split()
        return int(out[0]), int(out[1])

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        res = list(ex.map(run, ranges))
    bad = [(r, first) for r, (n, first) in zip(ranges, res) if n]
    assert not bad, f"mismatches, first input bits {hex(bad[0][1])}"


def test_nan_becomes_the_quiet_nan_with_its_sign():
    """A NaN casts to the quiet NaN of the half format (all-ones exponent, top mantissa
    bit set), keeping the sign; infinities stay infinities."""
    for dtype, qnan, inf in ((O.F16, 0x7E00, 0x7C00), (O.BF16, 0x7FC0, 0x7F80)):
        x = np.array([np.nan, -np.nan, np.inf, -np.inf], np.float32)
        x[1] = -np.abs(x[1])
        got = O.float_to_half(dtype, x)
        assert [int(v) for v in got] == [qnan, qnan | 0x8000, inf, inf | 0x8000], (dtype, got)
