"""Pins for the oracle's element codecs (CPU only).

Each test ties oracle/codecs.py or the C twin (oracle/nvfp4_ref.c) to something other
than itself: PyTorch's float8_e4m3fn / bfloat16 casts (library routines), the OCP
tables in tests/golden, or the midpoint closed form of round-to-nearest-even on the
E2M1 grid over every fp32 bit pattern.
"""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

from conftest import GOLDEN, ROOT
from oracle import codecs, nvfp4


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_e4m3_decode_exhaustive_vs_torch():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = codecs.e4m3_decode(c)
        if math.isnan(lib[c]):
            assert math.isnan(v), c
        else:
            assert v == lib[c] and math.copysign(1, v) == math.copysign(1, lib[c]), c
    np.testing.assert_array_equal(np.isnan(codecs.E4M3_TABLE), np.isnan(lib))


def test_e4m3_golden_points():
    for code, val in _golden("e4m3fn_points.txt"):
        v = codecs.e4m3_decode(int(code, 16))
        if val == "nan":
            assert math.isnan(v)
        else:
            assert v == float(val) and math.copysign(1, v) == math.copysign(1, float(val)), code


def test_e2m1_decode_golden_table():
    rows = _golden("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        v = codecs.e2m1_decode(int(code, 16))
        assert v == float(val) and math.copysign(1, v) == math.copysign(1, float(val)), code
    assert max(codecs.E2M1_GRID) == codecs.E2M1_MAX == 6.0


def _e4m3_probe_values():
    grid = np.array(codecs.E4M3_GRID)
    mids = (grid[1:] + grid[:-1]) / 2
    pts = np.concatenate([grid, mids]).astype(np.float32)
    nxt_up = np.nextafter(pts, np.float32(np.inf))
    nxt_dn = np.nextafter(pts, np.float32(0))
    rng = np.random.default_rng(7)
    rnd = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)]).astype(np.float32)
    allbf16 = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    vals = np.concatenate([pts, nxt_up, nxt_dn, rnd, allbf16, np.float32([0.0, -0.0, 2.0 ** -10, 464.0])])
    vals = np.concatenate([vals, -vals])
    return vals[np.isfinite(vals) & (np.abs(vals) <= 464.0)]


def test_e4m3_encode_vs_torch_cast():
    """torch's cast is RNE; it agrees with a saturating encoder up to 464 (above that it
    returns NaN), so the comparison covers |x| <= 464."""
    vals = _e4m3_probe_values()
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    py = np.array([codecs.e4m3_encode(float(v)) for v in vals[::7]], dtype=np.uint8)
    np.testing.assert_array_equal(py, ref[::7])
    c = np.array([nvfp4.e4m3_encode_c(float(v)) for v in vals], dtype=np.uint8)
    np.testing.assert_array_equal(c, ref)


def test_e4m3_encode_saturation_and_nan():
    for enc in (codecs.e4m3_encode, nvfp4.e4m3_encode_c):
        assert enc(448.0) == 0x7E and enc(465.0) == 0x7E and enc(1e30) == 0x7E and enc(math.inf) == 0x7E
        assert enc(-1e30) == 0xFE and enc(-math.inf) == 0xFE
        assert enc(math.nan) == 0x7F
        assert enc(-0.0) == 0x80 and enc(0.0) == 0x00
        assert enc(2.0 ** -10) == 0x00          # tie between 0 and 2^-9 -> even (0)
        assert enc(3 * 2.0 ** -10) == 0x02      # tie between 2^-9 and 2^-8 -> even (0x02)


def test_e2m1_encode_examples():
    cases = [(0.0, 0x0), (-0.0, 0x8), (0.25, 0x0), (0.2500001, 0x1), (0.75, 0x2), (0.7499999, 0x1),
             (1.25, 0x2), (1.75, 0x4), (2.5, 0x4), (2.5000002, 0x5), (3.5, 0x6), (5.0, 0x6), (5.0000005, 0x7),
             (6.0, 0x7), (100.0, 0x7), (math.inf, 0x7), (-math.inf, 0xF), (-0.1, 0x8), (-5.5, 0xF), (-2.9, 0xD)]
    for y, code in cases:
        assert codecs.e2m1_encode(y) == code, y
        assert nvfp4.e2m1_encode_c(y) == code, y


@pytest.mark.slow
def test_e2m1_encode_all_fp32_vs_midpoint_closed_form(tmp_path):
    """Every one of the 2^32 fp32 bit patterns (NaNs excluded) through the C twin's E2M1
    encoder equals the closed form of ties-to-even rounding on the grid
    {0, .5, 1, 1.5, 2, 3, 4, 6}: the code counts the midpoints below |y|, a midpoint that
    sits under an odd code being passed only strictly."""
    exe = str(tmp_path / "e2m1_pin")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-o", exe,
                           os.path.join(ROOT, "tests", "pins", "e2m1_midpoints.c"),
                           os.path.join(ROOT, "oracle", "nvfp4_ref.c"), "-lm"])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "mismatches 0" in out.stdout, out.stdout


def test_bf16_rounding_vs_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32)).view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(codecs.bf16_round_bits(x), ref)


def _same_f64(a, b):
    """Equal values with equal signs, NaN at the same positions."""
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    na, nb = np.isnan(a), np.isnan(b)
    np.testing.assert_array_equal(na, nb)
    np.testing.assert_array_equal(a[~na], b[~nb])
    np.testing.assert_array_equal(np.signbit(a[~na]), np.signbit(b[~nb]))


def test_bf16_widening_vs_torch_every_pattern():
    """codecs.bf16_bits_to_f64 and the C twin's bf16 rows -> fp32 widen every one of the 65,536
    bf16 bit patterns exactly as torch's bfloat16 -> float64 / float32 casts do."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    _same_f64(codecs.bf16_bits_to_f64(bits), lib.to(torch.float64).numpy())
    c32 = nvfp4.bf16_rows_to_f32(bits.reshape(-1, 64))
    assert c32.dtype == np.float32
    _same_f64(c32.reshape(-1), lib.to(torch.float32).numpy())


@pytest.mark.parametrize("scale", [1.0, 0.75, 2.0 ** -7, 3.3, 1e-30])
def test_fp8_rows_to_f32_vs_torch_every_code(scale):
    """The write path's FP8 source values fl32(e4m3(code) * src_scale), all 256 codes: torch's
    float8_e4m3fn -> float32 cast times the fp32 scale in one IEEE fp32 multiply."""
    codes = np.tile(np.arange(256, dtype=np.uint8), 3).reshape(-1, 64)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.tensor(np.float32(scale))
    got = nvfp4.fp8_rows_to_f32(codes, scale)
    assert got.dtype == np.float32
    _same_f64(got, ref.numpy())


def test_calibrated_global_scale_rounds_the_exact_quotient():
    """g = amax / (6 * 448) rounded once to the nearest fp32 (ties to even): hand values where the
    quotient is exact, and random amax where the exact rational quotient is rounded here with
    fractions (no floating-point division involved)."""
    from fractions import Fraction
    assert nvfp4.calibrated_global_scale(2688.0) == 1.0
    assert nvfp4.calibrated_global_scale(5376.0) == 2.0
    assert nvfp4.calibrated_global_scale(1344.0) == 0.5
    assert nvfp4.calibrated_global_scale(42.0) == 2.0 ** -6          # 42 * 64 = 2688

    def round_f32(q: Fraction) -> float:
        # nearest fp32 to a positive rational q in the normal range, ties to even
        e = q.numerator.bit_length() - q.denominator.bit_length()
        while Fraction(2) ** e > q:
            e -= 1
        while Fraction(2) ** (e + 1) <= q:
            e += 1
        ulp = Fraction(2) ** (e - 23)
        n, r = divmod(q, ulp)
        if r > ulp / 2 or (r == ulp / 2 and n % 2 == 1):
            n += 1
        return float(n * ulp)
    rng = np.random.default_rng(7)
    for amax in rng.uniform(0.01, 1e4, 500).astype(np.float32):
        want = round_f32(Fraction(float(amax)) / 2688)
        assert nvfp4.calibrated_global_scale(float(amax)) == want, amax
