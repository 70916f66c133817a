"""Pins for the oracle's NVFP4 block quantizer and dequantizer (CPU only).

Anchors: the hand-worked blocks in tests/golden/nvfp4_blocks.txt, the storage arithmetic
the NVFP4 article prints (tests/golden/nvfp4_storage.txt), and properties that follow from
the format alone (idempotence on representable blocks, the largest element mapping to
the largest code, the rounding error bound, block independence).  The last tests plant
plausible mistakes in a copy of the oracle and check that these pins catch them.
"""
import math
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import codecs, nvfp4


def _blocks():
    out = []
    for line in open(os.path.join(GOLDEN, "nvfp4_blocks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, g, xs, sb, packed = [f.strip() for f in line.split("|")]
        out.append((name, float(g), np.array([float(v) for v in xs.split()], dtype=np.float32),
                    int(sb, 16), bytes.fromhex(packed)))
    return out


@pytest.mark.parametrize("case", _blocks(), ids=lambda c: c[0])
def test_worked_blocks_python(case):
    name, g, x, sb, packed = case
    got_sb, codes = nvfp4.quantize_block(x, g)
    assert got_sb == sb
    assert nvfp4.pack_codes(codes) == packed


@pytest.mark.parametrize("case", _blocks(), ids=lambda c: c[0])
def test_worked_blocks_c(case):
    name, g, x, sb, packed = case
    row = np.zeros((1, 576), dtype=np.float32)
    row[0, 16 * 5:16 * 6] = x                       # block 5 of a row
    data, scales = nvfp4.quantize_rows(row, g)
    assert scales[0, 5] == sb
    assert data[0, 40:48].tobytes() == packed
    assert (scales[0, :5] == 0).all() and (data[0, :40] == 0).all()


def test_storage_arithmetic_from_the_page():
    facts = dict(l.split() for l in open(os.path.join(GOLDEN, "nvfp4_storage.txt")) if l.strip() and l[0] != "#")
    per_block = nvfp4.ROW_DATA_BYTES / nvfp4.ROW_BLOCKS + nvfp4.ROW_SCALE_BYTES / nvfp4.ROW_BLOCKS
    assert per_block == float(facts["bytes_per_block"])
    assert nvfp4.BLOCK == int(facts["values_per_block"])
    assert nvfp4.nvfp4_bytes_per_value() * 16 / float(facts["fp8_bytes_per_block"]) == float(facts["fraction_of_fp8"])
    assert round(1 / float(facts["fraction_of_fp8"]), 2) == float(facts["capacity_ratio"])
    assert nvfp4.ROW_DATA_BYTES + nvfp4.ROW_SCALE_BYTES == 324 and nvfp4.ROW_DIMS == 512 + 64


def test_scale_bytes_follow_block_magnitude():
    """Block k holds +-6 * 2^(k%8 - 4): its scale is exactly 2^(k%8 - 4), i.e. e4m3 byte
    (k%8 + 3) << 3, and every element maps to code 7 (with its sign).  Catches wrong block
    boundaries and wrong scale positions."""
    row = np.empty((1, 576), dtype=np.float32)
    for k in range(36):
        mag = 6.0 * 2.0 ** (k % 8 - 4)
        row[0, 16 * k:16 * k + 16] = [mag if i % 3 else -mag for i in range(16)]
    data, scales = nvfp4.quantize_rows(row, 1.0)
    for k in range(36):
        assert scales[0, k] == (k % 8 + 3) << 3
        codes = [(data[0, 8 * k + j // 2] >> (4 * (j % 2))) & 0xF for j in range(16)]
        assert codes == [0x7 if i % 3 else 0xF for i in range(16)]
    assert (nvfp4.quantize_row_py(row[0], 1.0)[1] == scales[0].tobytes())


def test_special_blocks():
    nan_blk = np.zeros(16, np.float32)
    nan_blk[3] = np.nan
    assert nvfp4.quantize_block(nan_blk, 1.0) == (0x7F, [0] * 16)
    assert nvfp4.quantize_block(np.zeros(16, np.float32), 1.0) == (0x00, [0] * 16)
    neg0 = np.zeros(16, np.float32)
    neg0[0], neg0[1] = 1.0, -0.0
    sb, codes = nvfp4.quantize_block(neg0, 1.0)
    assert codes[1] == 0x8 and codes[0] == 0x7
    inf_blk = np.ones(16, np.float32)
    inf_blk[2] = -np.inf
    sb, codes = nvfp4.quantize_block(inf_blk, 1.0)
    assert sb == 0x7E and codes[2] == 0xF


def _random_blocks(n, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 16)).astype(np.float32)
    if outliers:
        x[rng.random((n, 16)) < 0.01] *= 8
    x *= np.float32(2.0) ** rng.integers(-6, 6, (n, 1)).astype(np.float32)
    return x


def test_python_and_c_agree_on_random_rows():
    x = _random_blocks(36 * 60, 11).reshape(60, 576)
    data, scales = nvfp4.quantize_rows(x, 1.0)
    for r in range(0, 60, 7):
        d, s = nvfp4.quantize_row_py(x[r], 1.0)
        assert d == data[r].tobytes() and s == scales[r].tobytes()
    g = nvfp4.calibrated_global_scale(float(np.abs(x).max()))
    data, scales = nvfp4.quantize_rows(x, g)
    for r in range(0, 60, 13):
        d, s = nvfp4.quantize_row_py(x[r], g)
        assert d == data[r].tobytes() and s == scales[r].tobytes()


def _normal_scale(sb):
    return 0x08 <= (sb & 0x7F) <= 0x7E


def test_largest_element_takes_largest_code_and_error_bound():
    """With a normal scale byte, RNE on E4M3 changes (amax/6) by at most 1/16 relative, so
    amax / sd lies in [5.64, 6.4] and rounds to 6 (code 7).  Every element is within half the
    local E2M1 spacing times sd of its dequantized value (and saturated ones within sd * 0.4)."""
    x = _random_blocks(36 * 84, 5)
    grid = np.array(codecs.E2M1_GRID)
    for g in (1.0, nvfp4.calibrated_global_scale(float(np.abs(x).max()))):
        data, scales = nvfp4.quantize_rows(x.reshape(-1, 576), g)
        deq = nvfp4.dequant_nvfp4_f64(data, scales, g).reshape(-1, 16)
        for i, (blk, sb) in enumerate(zip(x, scales.reshape(-1))):
            if not _normal_scale(int(sb)):
                continue
            sd = float(np.float32(np.float32(codecs.e4m3_decode(int(sb))) * np.float32(g)))
            k = int(np.argmax(np.abs(blk)))
            assert abs(deq[i, k]) == 6 * codecs.e4m3_decode(int(sb)) * float(np.float32(g))
            y = np.abs(blk.astype(np.float64)) / sd
            idx = np.clip(np.searchsorted(grid, y), 1, 7)
            half_gap = (grid[idx] - grid[idx - 1]) / 2
            err = np.abs(np.abs(deq[i]) - np.abs(blk.astype(np.float64))) / sd
            assert (err <= half_gap + 1e-6).all() or (y > 6).any()
            assert np.all(np.sign(deq[i]) * np.sign(blk) >= 0)


def test_idempotent_on_representable_blocks():
    """Blocks that are already NVFP4 values (code * scale, with a code 7 present) quantize
    back to the same bytes at g = 1."""
    rng = np.random.default_rng(9)
    for _ in range(2000):
        sb = int(rng.integers(0x08, 0x7F))
        codes = rng.integers(0, 16, 16)
        codes[rng.integers(0, 16)] = 0x7 | (int(rng.integers(0, 2)) << 3)
        x = np.array([codecs.e2m1_decode(int(c)) * codecs.e4m3_decode(sb) for c in codes], dtype=np.float32)
        got_sb, got = nvfp4.quantize_block(x, 1.0)
        assert got_sb == sb
        assert [c & 0x7 for c in got] == [int(c) & 0x7 for c in codes]
        assert all((g & 8) == (int(c) & 8) for g, c in zip(got, codes) if (int(c) & 7) != 0)


def test_dequant_products_exact_in_bf16_and_fp16():
    """Every finite E2M1 x E4M3 product fits bf16 and fp16 exactly, so a dequantized value
    is a single rounding-free number in either 16-bit type."""
    import torch
    prods = np.array([codecs.e2m1_decode(c) * codecs.e4m3_decode(s) for c in range(16) for s in range(256)
                      if not math.isnan(codecs.e4m3_decode(s))])
    t = torch.from_numpy(prods)
    assert (t.to(torch.bfloat16).double() == t).all()
    assert (t.to(torch.float16).double() == t).all()


# ---------------------------------------------------------------- planted mistakes


def _worked_blocks_pass(qblock):
    for name, g, x, sb, packed in _blocks():
        got_sb, codes = qblock(x, g)
        if got_sb != sb or nvfp4.pack_codes(codes) != packed:
            return False
    return True


def test_pins_catch_planted_mistakes(monkeypatch):
    f32 = np.float32

    def swapped_nibbles(codes):
        return bytes((codes[2 * j + 1] & 0xF) | ((codes[2 * j] & 0xF) << 4) for j in range(8))

    # 1. nibble order swapped
    monkeypatch.setattr(nvfp4, "pack_codes", swapped_nibbles)
    assert not _worked_blocks_pass(nvfp4.quantize_block)
    monkeypatch.undo()

    # 2. block scale rounded up instead of to nearest
    def ceil_scale(x, g):
        x = np.asarray(x, np.float32)
        sf = f32(f32(f32(np.max(np.abs(x))) / f32(6)) / f32(g))
        sb = next(c for c in range(0x7F) if codecs.e4m3_decode(c) >= sf)
        sd = f32(f32(codecs.e4m3_decode(sb)) * f32(g))
        return sb, [codecs.e2m1_encode(float(f32(v / sd))) for v in x]
    assert not _worked_blocks_pass(ceil_scale)

    # 3. reciprocal multiply instead of division
    def recip(x, g):
        x = np.asarray(x, np.float32)
        sf = f32(f32(f32(np.max(np.abs(x))) / f32(6)) / f32(g))
        sb = codecs.e4m3_encode(float(sf))
        sd = f32(f32(codecs.e4m3_decode(sb)) * f32(g))
        r = f32(f32(1) / sd)
        return sb, [codecs.e2m1_encode(float(f32(v * r))) for v in x]
    assert not _worked_blocks_pass(recip)

    # 4. sign dropped on values that round to zero
    def no_neg_zero(x, g):
        sb, codes = nvfp4.quantize_block(x, g)
        return sb, [0 if c == 8 else c for c in codes]
    assert not _worked_blocks_pass(no_neg_zero)

    # 5. global scale applied on the wrong side (multiplying instead of dividing)
    def g_wrong(x, g):
        return nvfp4.quantize_block(np.asarray(x, np.float32), 1.0 / g)
    assert not _worked_blocks_pass(g_wrong)

    # 6. ties away from zero in the E2M1 rounding
    def ties_away(x, g):
        sb, _ = nvfp4.quantize_block(x, g)
        sd = f32(f32(codecs.e4m3_decode(sb)) * f32(g))
        out = []
        for v in np.asarray(x, np.float32):
            a = abs(float(f32(v / sd)))
            k = int(np.argmin([abs(a - q) - 1e-12 * q for q in codecs.E2M1_GRID]))
            out.append((8 if math.copysign(1, v) < 0 else 0) | k)
        return sb, out
    assert not _worked_blocks_pass(ties_away)


def test_fp32_dequant_matches_fp64_definition():
    """At g = 1 (and any power of two) fl32(fl32(e2m1 * e4m3) * g) is exact, so it equals the
    fp64 dequantization; the e4m3 re-encode of those values agrees with torch's cast."""
    import torch
    x = _random_blocks(36 * 20, 21).reshape(20, 576)
    for g in (1.0, 0.25, 8.0):
        data, scales = nvfp4.quantize_rows(x, g)
        f32 = nvfp4.dequant_nvfp4_f32(data, scales, g)
        np.testing.assert_array_equal(f32.astype(np.float64), nvfp4.dequant_nvfp4_f64(data, scales, g))
        small = f32[np.abs(f32) <= 464]
        ref = torch.from_numpy(small).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(nvfp4.e4m3_encode_array(small), ref)
