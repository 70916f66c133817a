"""Host checks of the extend attention kernel's LDS layouts (no GPU): the swizzle tables are
read out of the kernel source, then every (row, 16-byte chunk) slot of the fp16 tile and of a
wave's query area must be distinct and inside its area, and each lane group the LDS serves in
one pass (16-byte accesses: lanes 8i .. 8i+7 with 8i+32 .. 8i+39; 8-byte transposed reads: 32
consecutive lanes) must touch each of the 64 four-byte banks at most once, for the K-operand
reads, the query reads, the transposed V reads and the tile writes, with the lane -> (row,
chunk) maps the kernel uses."""
import os
import re

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "quantized_kv_paged_amd", "csrc", "extend_attn.hip")


def _constant(name):
    m = re.search(r"constexpr int %s = (\d+);" % name, open(SRC).read())
    assert m, name
    return int(m.group(1))


def _swizzle_table(fn, var):
    m = re.search(r"int %s\(int %s\) \{ return \(int\)\(\((0x[0-9a-f]+)u >> \(4 \* \(%s & 7\)\)\) & 15u\); \}" % (fn, var, var),
                  open(SRC).read())
    assert m, fn + " table not found in the kernel source"
    word = int(m.group(1), 16)
    return [(word >> (4 * r)) & 15 for r in range(8)]


ROW_B = _constant("kXRowB")
ROWS = _constant("kXRows")
QL = _constant("kXQL")
THREADS = 64 * _constant("kXT")
S = _swizzle_table("xswz", "r")
F = _swizzle_table("qswz", "h")


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


def qoff(h, c):
    return h * 64 * QL + 16 * ((c & ~15) | ((c & 15) ^ F[h & 7]))


def test_tile_and_query_slots_distinct_and_inside():
    assert ROW_B == 1152 and ROWS == 32 and QL % 4 == 0
    slots = {xoff(r, c) for r in range(ROWS) for c in range(72)}
    assert len(slots) == ROWS * 72
    assert min(slots) >= 0 and max(slots) + 16 <= ROWS * ROW_B
    q = {qoff(h, c) for h in range(16) for c in range(4 * QL)}
    assert len(q) == 16 * 4 * QL and min(q) >= 0 and max(q) + 16 <= 16 * 64 * QL


def test_operand_reads_conflict_free():
    for tb in range(2):
        for kb in range(18):  # K operands: lane (g, l16) reads row l16 + 16 tb at one chunk
            a = []
            for lane in range(64):
                g, l16 = lane >> 4, lane & 15
                a.append(xoff(l16 + 16 * tb, 4 * kb + g if kb < 16 else 64 + 4 * (kb - 16) + g))
            assert _max_bank_load(a, 16, G16) == 1, (tb, kb)
    for kb in range(QL):      # query operands from LDS: lane (g, head l16), chunk 4kb + g
        a = [qoff(lane & 15, 4 * kb + (lane >> 4)) for lane in range(64)]
        assert _max_bank_load(a, 16, G16) == 1, kb
    for hi in range(2):
        for nt in range(32):  # transposed V operands: 8 bytes of row 4g + l16 / 4 (+16)
            a = []
            for lane in range(64):
                g, l16 = lane >> 4, lane & 15
                q4, vrow = l16 & 3, 4 * g + (l16 >> 2)
                byte = 2 * (16 * nt + 4 * q4)
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
