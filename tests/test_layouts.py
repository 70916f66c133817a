"""Host checks of the extend attention kernel's LDS tile layout (no GPU): the swizzle table is
read out of the kernel source, then every (row, 16-byte chunk) slot of the fp16 tile must be
distinct and inside the tile, and each lane group the LDS serves in one pass (16-byte accesses:
lanes 8i .. 8i+7 with 8i+32 .. 8i+39; 8-byte transposed reads: 32 consecutive lanes) must touch
each of the 64 four-byte banks at most once, for the K-operand reads, the transposed V reads
and the tile writes, with the lane -> (row, chunk) maps the kernel uses."""
import os
import re

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "quantized_kv_paged_amd", "csrc", "extend_attn.hip")


def _constant(name):
    m = re.search(r"constexpr int %s = (\d+);" % name, open(SRC).read())
    assert m, name
    return int(m.group(1))


def _swizzle_table():
    m = re.search(r"int xswz\(int r\) \{ return \(int\)\(\((0x[0-9a-f]+)u >> \(4 \* \(r & 7\)\)\) & 15u\); \}", open(SRC).read())
    assert m, "swizzle table not found in the kernel source"
    word = int(m.group(1), 16)
    return [(word >> (4 * r)) & 15 for r in range(8)]


ROW_B = _constant("kXRowB")
ROWS = _constant("kXRows")
THREADS = 64 * 2 * _constant("kXT")
S = _swizzle_table()


def xoff(r, c):
    s = S[r & 7]
    return r * ROW_B + 16 * (((c & ~15) | ((c & 15) ^ s)) if c < 64 else 64 + ((c & 7) ^ (s & 7)))


G16 = [list(range(i, i + 8)) + list(range(i + 32, i + 40)) for i in (0, 8, 16, 24)]
G8 = [list(range(0, 32)), list(range(32, 64))]


def _max_bank_load(addrs, nbytes, groups):
    worst = 0
    for g in groups:
        banks = {}
        for lane in g:
            if addrs[lane] is None:      # an idle lane does not access the LDS
                continue
            for k in range(0, nbytes, 4):
                dw = (addrs[lane] + k) // 4
                banks.setdefault(dw % 64, set()).add(dw)
        worst = max(worst, max((len(v) for v in banks.values()), default=0))
    return worst


def test_tile_slots_distinct_and_inside():
    assert ROW_B == 1152 and ROWS == 32
    slots = {xoff(r, c) for r in range(ROWS) for c in range(72)}
    assert len(slots) == ROWS * 72
    assert min(slots) >= 0 and max(slots) + 16 <= ROWS * ROW_B


@pytest.mark.parametrize("dh", [0, 1])
def test_operand_reads_conflict_free(dh):
    for tb in range(2):
        for kb in range(9):   # K operands: lane (g, l16) reads row l16 + 16 tb at one chunk
            a = []
            for lane in range(64):
                g, l16 = lane >> 4, lane & 15
                c = 32 * dh + 8 * (kb >> 1) + 2 * g + (kb & 1) if kb < 8 else 64 + 4 * dh + g
                a.append(xoff(l16 + 16 * tb, c))
            assert _max_bank_load(a, 16, G16) == 1, (tb, kb)
    for hi in range(2):
        for nt in range(16):  # transposed V operands: 8 bytes of row 4g + l16 / 4 (+16)
            a = []
            for lane in range(64):
                g, l16 = lane >> 4, lane & 15
                q4, vrow = l16 & 3, 4 * g + (l16 >> 2)
                byte = 2 * (256 * dh + 16 * nt + 4 * q4)
                a.append(xoff(vrow + 16 * hi, byte // 16) + byte % 16)
            assert _max_bank_load(a, 8, G8) == 1, (hi, nt)


def test_tile_writes_conflict_free():
    for w in range(THREADS // 64):
        for j in range((1152 + THREADS - 1) // THREADS):
            units = [64 * w + lane + THREADS * j for lane in range(64)]
            if all(u >= 1152 for u in units):
                continue
            for half in range(2):
                a = [xoff(u & 31, 2 * (u >> 5) + half) if u < 1152 else None for u in units]
                assert _max_bank_load(a, 16, G16) == 1, (w, j, half)
