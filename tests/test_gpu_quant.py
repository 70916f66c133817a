"""GPU parity of the NVFP4 quantize-on-write and of kv_dequantize: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import synth
from conftest import GOLDEN
from oracle import codecs
from oracle import nvfp4 as onv

pytestmark = pytest.mark.gpu
POISON = 0xA5


def _qk():
    import quantized_kv_paged_amd as qk
    return qk


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _quantize_gpu(src, fmt, slots, pool_tokens, g, src_scale=1.0):
    qk = _qk()
    data = torch.full((pool_tokens, 288), POISON, dtype=torch.uint8, device="cuda")
    scales = torch.full((pool_tokens, 36), POISON, dtype=torch.uint8, device="cuda")
    s = _t(src.view(np.int16)).view(torch.bfloat16) if fmt == qk.MLAQ_BF16 else _t(src)
    qk.kv_quantize_nvfp4(s, fmt, src_scale, _t(slots.astype(np.int64)), data, scales, g)
    torch.cuda.synchronize()
    return data.cpu().numpy(), scales.cpu().numpy()


def _check_scatter(data, scales, slots, ref_d, ref_s, pool_tokens):
    written = np.zeros(pool_tokens, bool)
    ok = (slots >= 0) & (slots < pool_tokens)
    written[slots[ok]] = True
    np.testing.assert_array_equal(data[slots[ok]], ref_d[ok])
    np.testing.assert_array_equal(scales[slots[ok]], ref_s[ok])
    assert (data[~written] == POISON).all() and (scales[~written] == POISON).all()


def _special_fp8_rows(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 576)).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 8
    x *= np.float32(2.0) ** rng.integers(-8, 6, (n, 36, 1)).repeat(16, 2).reshape(n, 576).astype(np.float32)
    codes = synth.to_fp8_bytes(x)
    codes[0, :16] = 0x7E                # all 448
    codes[1, 16:32] = 0x00              # all zero -> scale 0
    codes[1, 32:48] = np.arange(16)     # subnormals only
    codes[2, 48:64] = 0x80              # -0
    codes[3, 0] = 0x7F                  # NaN block
    codes[4, :] = np.arange(256).repeat(3)[:576].astype(np.uint8)   # every code
    return codes


@pytest.mark.parametrize("g", [1.0, "calibrated", 0.37, 3.0])
def test_quantize_fp8_source_bit_exact(g):
    n, pool = 700, 1500
    src = _special_fp8_rows(n, 31)
    rng = np.random.default_rng(32)
    slots = rng.permutation(pool)[:n].astype(np.int64)
    slots[5], slots[9] = -1, pool + 7          # skipped rows
    if g == "calibrated":
        x = onv.fp8_rows_to_f32(src, 1.0)
        g = onv.calibrated_global_scale(float(np.nanmax(np.abs(x))))
    data, scales = _quantize_gpu(src, _qk().MLAQ_FP8_E4M3, slots, pool, g)
    ref_d, ref_s = onv.quantize_fp8_rows(src, 1.0, g)
    _check_scatter(data, scales, slots, ref_d, ref_s, pool)


def test_quantize_fp8_source_scale():
    n = 64
    src = _special_fp8_rows(n, 33)
    slots = np.arange(n, dtype=np.int64)
    data, scales = _quantize_gpu(src, _qk().MLAQ_FP8_E4M3, slots, n, 1.0, src_scale=0.8125)
    ref_d, ref_s = onv.quantize_fp8_rows(src, 0.8125, 1.0)
    _check_scatter(data, scales, slots, ref_d, ref_s, n)


def test_quantize_bf16_source_bit_exact_with_specials():
    n = 300
    rng = np.random.default_rng(34)
    x = rng.standard_normal((n, 576)).astype(np.float32) * np.float32(3.0)
    bits = codecs.bf16_round_bits(x)
    bits[0, 3] = 0x7F80          # +inf
    bits[1, 17] = 0xFF80         # -inf
    bits[2, 40] = 0x7FC0         # NaN
    bits[3, :16] = 0x8000        # -0
    bits[4, 16:32] = 0x0001      # tiny subnormal
    slots = np.arange(n, dtype=np.int64)[::-1].copy()
    data, scales = _quantize_gpu(bits, _qk().MLAQ_BF16, slots, n, 1.0)
    ref_d, ref_s = onv.quantize_bf16_rows(bits, 1.0)
    _check_scatter(data, scales, slots, ref_d, ref_s, n)


def test_quantize_every_bf16_value_in_range():
    """The device E2M1 and E4M3 encoders over every bf16 value: blocks whose first element
    is 6 (scale 1.0) and whose other 15 elements sweep all bf16 values of magnitude <= 6, and
    blocks whose largest element sweeps every positive finite bf16 value (scale byte)."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_bits_to_f64(allb)
    small = allb[np.abs(v) <= 6]
    pad = (-len(small)) % 15
    small = np.concatenate([small, np.zeros(pad, np.uint16)]).reshape(-1, 15)
    blocks = np.concatenate([np.full((small.shape[0], 1), 0x40C0, np.uint16), small], 1)   # 6.0 first
    pos = allb[(v > 0) & np.isfinite(v)]
    pad = (-len(pos)) % 16
    pos_blocks = np.concatenate([pos, np.zeros(pad, np.uint16)]).reshape(-1, 16)
    allblocks = np.concatenate([blocks, pos_blocks])
    pad = (-allblocks.shape[0]) % 36
    allblocks = np.concatenate([allblocks, np.zeros((pad, 16), np.uint16)]).reshape(-1, 576)
    n = allblocks.shape[0]
    for g in (1.0, 0.37):
        data, scales = _quantize_gpu(allblocks, _qk().MLAQ_BF16, np.arange(n, dtype=np.int64), n, g)
        ref_d, ref_s = onv.quantize_bf16_rows(allblocks, g)
        np.testing.assert_array_equal(scales, ref_s)
        np.testing.assert_array_equal(data, ref_d)


def test_worked_blocks_through_the_gpu():
    """The hand-worked NVFP4 blocks (inputs rounded to bf16 keep every code) give the golden bytes."""
    import os
    for line in open(os.path.join(GOLDEN, "nvfp4_blocks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, g, xs, sb, packed = [f.strip() for f in line.split("|")]
        row = np.zeros((1, 576), np.float32)
        row[0, 32:48] = [float(v) for v in xs.split()]
        bits = codecs.bf16_round_bits(row)
        data, scales = _quantize_gpu(bits, _qk().MLAQ_BF16, np.array([0], np.int64), 1, float(g))
        assert scales[0, 2] == int(sb, 16), name
        assert data[0, 16:24].tobytes() == bytes.fromhex(packed), name


def test_write_path_workload_bit_exact():
    """8,192-token FP8 chunk (bf16-rounded N(0,1)) into 128 scattered spare pages of the 1M pool layout."""
    w = synth.WORKLOADS["nvfp4_1m"]
    pt = synth.page_table(w)
    slots = synth.slot_mapping(w, pt)
    src = synth.write_source_fp8(w)
    assert src.shape == (8192, 576) and slots.max() < w.pool_tokens
    qk = _qk()
    data = torch.full((w.pool_tokens, 288), POISON, dtype=torch.uint8, device="cuda")
    scales = torch.full((w.pool_tokens, 36), POISON, dtype=torch.uint8, device="cuda")
    qk.kv_quantize_nvfp4(_t(src), qk.MLAQ_FP8_E4M3, 1.0, _t(slots), data, scales, 1.0)
    torch.cuda.synchronize()
    ref_d, ref_s = onv.quantize_fp8_rows(src, 1.0, 1.0)
    ts = torch.from_numpy(slots).cuda()
    np.testing.assert_array_equal(data[ts].cpu().numpy(), ref_d)
    np.testing.assert_array_equal(scales[ts].cpu().numpy(), ref_s)
    mask = torch.ones(w.pool_tokens, dtype=torch.bool, device="cuda")
    mask[ts] = False
    assert bool((data[mask] == POISON).all()) and bool((scales[mask] == POISON).all())


def _nan_mask(bits, fmt):
    qk = _qk()
    if fmt == qk.MLAQ_FP32:
        return (bits & 0x7FFFFFFF) > 0x7F800000
    if fmt == qk.MLAQ_BF16:
        return (bits & 0x7FFF) > 0x7F80
    return (bits & 0x7F) == 0x7F


def _assert_equal_nan_as_class(got, ref, fmt):
    """Bit-exact, except that a NaN's sign and payload are not specified: NaN positions must
    match and every other element must be identical."""
    gm, rm = _nan_mask(got, fmt), _nan_mask(ref, fmt)
    np.testing.assert_array_equal(gm, rm)
    np.testing.assert_array_equal(got[~gm], ref[~rm])


@pytest.mark.parametrize("g", [1.0, 0.37])
def test_dequantize_nvfp4_bit_exact(g):
    qk = _qk()
    rng = np.random.default_rng(41)
    n = 400
    x = rng.standard_normal((n, 576)).astype(np.float32) * 4
    d_np, s_np = onv.quantize_rows(x, g)
    s_np[7, 3] = 0x7F                                   # NaN scale
    d, s = _t(d_np), _t(s_np)
    rows = rng.integers(0, n, 250).astype(np.int64)
    rows[10] = n + 3                                     # out of range -> NaN row
    f32 = onv.dequant_nvfp4_f32(d_np, s_np, g)
    for fmt in (qk.MLAQ_FP32, qk.MLAQ_BF16, qk.MLAQ_FP8_E4M3):
        out_all = qk.kv_dequantize(qk.MLAQ_NVFP4, d, s, g, fmt)
        out_rows = qk.kv_dequantize(qk.MLAQ_NVFP4, d, s, g, fmt, rows=_t(rows))
        torch.cuda.synchronize()
        if fmt == qk.MLAQ_FP32:
            ref = f32.view(np.uint32)
            got = out_all.cpu().numpy().view(np.uint32)
            got_r = out_rows.cpu().numpy().view(np.uint32)
        elif fmt == qk.MLAQ_BF16:
            ref = codecs.bf16_round_bits(f32)
            got = out_all.view(torch.int16).cpu().numpy().view(np.uint16)
            got_r = out_rows.view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            ref = onv.e4m3_encode_array(f32)
            got = out_all.cpu().numpy()
            got_r = out_rows.cpu().numpy()
        _assert_equal_nan_as_class(got, ref, fmt)
        ok = rows < n
        _assert_equal_nan_as_class(got_r[ok], ref[rows[ok]], fmt)
    assert np.isnan(qk.kv_dequantize(qk.MLAQ_NVFP4, d, s, g, qk.MLAQ_FP32, rows=_t(rows)).cpu().numpy()[10]).all()


@pytest.mark.parametrize("g", [1.0, 1.02])
def test_dequantize_nvfp4_to_fp8_saturates_bit_exact(g):
    """FP8 output of values past the e4m3 range, byte for byte as the oracle's encoder gives them:
    rows of magnitude up to about 700 dequantize to values above 464, which saturate to +-448
    (0x7E / 0xFE); at g = 1.02 products such as 448 g = 456.96 land in (448, 464], which round to
    448; a NaN block scale gives the NaN code 0x7F in all 16 bytes of its block."""
    qk = _qk()
    rng = np.random.default_rng(47)
    n = 64
    x = (rng.standard_normal((n, 576)) * 150).astype(np.float32)
    x[7, 64:80] = 0.0
    x[7, 64:66] = [685.44, 457.0]   # block scale 685.44 / 6 / 1.02 = 112; 457 codes as 4: 448 g
    d_np, s_np = onv.quantize_rows(x, g)
    s_np[5, 2] = 0x7F                                    # NaN scale: dims 32 .. 47 of row 5
    f32 = onv.dequant_nvfp4_f32(d_np, s_np, g)
    ref = onv.e4m3_encode_array(f32)
    out = qk.kv_dequantize(qk.MLAQ_NVFP4, _t(d_np), _t(s_np), g, qk.MLAQ_FP8_E4M3)
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got, ref)
    assert (got == 0x7E).any() and (got == 0xFE).any()   # saturated codes were produced
    assert (got[5, 32:48] == 0x7F).all()
    if g != 1.0:
        a = np.abs(f32[~np.isnan(f32)])
        assert ((a > 448) & (a <= 464)).any()            # the round-to-448 interval was reached


def test_dequantize_fp8_bit_exact():
    qk = _qk()
    codes = np.tile(np.arange(256, dtype=np.uint8), 9 * 40).reshape(160, 576)
    for scale in (1.0, 0.3):
        f32 = onv.fp8_rows_to_f32(codes, scale)
        out = qk.kv_dequantize(qk.MLAQ_FP8_E4M3, _t(codes), None, scale, qk.MLAQ_FP32)
        _assert_equal_nan_as_class(out.cpu().numpy().view(np.uint32), f32.view(np.uint32), qk.MLAQ_FP32)
        out = qk.kv_dequantize(qk.MLAQ_FP8_E4M3, _t(codes), None, scale, qk.MLAQ_BF16)
        _assert_equal_nan_as_class(out.view(torch.int16).cpu().numpy().view(np.uint16), codecs.bf16_round_bits(f32),
                                   qk.MLAQ_BF16)


@pytest.mark.parametrize("scale", [1.0, 0.3])
def test_dequantize_fp8_row_list_bit_exact(scale):
    """FP8 source through a row list (the gather of the pages' first fix): every listed row, in list
    order and with repeats, is fl32(e4m3 * scale) (fp32) or its bf16 rounding; rows outside the pool
    (past the end, negative) give NaN rows."""
    qk = _qk()
    rng = np.random.default_rng(43)
    n = 300
    codes = rng.integers(0, 256, (n, 576), dtype=np.uint8)
    rows = rng.integers(0, n, 500).astype(np.int64)
    rows[[7, 123]] = [n, n + 1000]
    rows[200] = -1
    f32 = onv.fp8_rows_to_f32(codes, scale)
    bad = (rows < 0) | (rows >= n)
    for fmt in (qk.MLAQ_FP32, qk.MLAQ_BF16):
        out = qk.kv_dequantize(qk.MLAQ_FP8_E4M3, _t(codes), None, scale, fmt, rows=_t(rows))
        torch.cuda.synchronize()
        if fmt == qk.MLAQ_FP32:
            got, ref = out.cpu().numpy().view(np.uint32), f32.view(np.uint32)
        else:
            got, ref = out.view(torch.int16).cpu().numpy().view(np.uint16), codecs.bf16_round_bits(f32)
        _assert_equal_nan_as_class(got[~bad], ref[rows[~bad]], fmt)
        assert _nan_mask(got[bad], fmt).all()


@pytest.mark.parametrize("kv_scale", [1.0, 0.3])
def test_gather_then_cast_baseline_end_to_end(kv_scale):
    """The pages' intermediate fix: the active rows of an FP8 pool gathered and cast to a dense BF16
    workspace (kv_dequantize with the page table's row list), then the BF16 decode over an identity
    page table into that workspace.  The workspace is checked bit for bit, the attention against the
    oracle over the same bf16 values (ragged requests, an empty one, pages of 16 tokens)."""
    import synth
    from cases import assert_parity, build_case, oracle_decode, Case
    from oracle import attention
    qk = _qk()
    lens = [700, 0, 33, 1500, 64]
    P = 16
    c = build_case("fp8", lens, P, seed=44, sigma=0.5, kv_scale=kv_scale)
    # active rows of each request, in token order, each request padded to whole pages of the workspace
    rows, indptr, table = [], [0], []
    for b, L in enumerate(lens):
        r = attention.gather_rows(c.pt.kv_indptr, c.pt.kv_indices, P, b, L) if L else np.zeros(0, np.int64)
        npg = -(-L // P)
        pad = np.full(npg * P - L, int(r[-1]) if L else 0, dtype=np.int64)
        base = sum(len(x) for x in rows)
        rows.append(np.concatenate([r.astype(np.int64), pad]))
        table.extend(range(base // P, base // P + npg))
        indptr.append(indptr[-1] + npg)
    rows = np.concatenate(rows)
    ws = qk.kv_dequantize(qk.MLAQ_FP8_E4M3, _t(c.fp8_pool), None, kv_scale, qk.MLAQ_BF16, rows=_t(rows))
    torch.cuda.synchronize()
    ref_bits = codecs.bf16_round_bits(onv.fp8_rows_to_f32(c.fp8_pool, kv_scale))[rows]
    np.testing.assert_array_equal(ws.view(torch.int16).cpu().numpy().view(np.uint16), ref_bits)
    q = torch.from_numpy(c.q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    ind, ptr = _t(np.array(table, np.int32)), _t(np.array(indptr, np.int32))
    lens_t = _t(np.array(lens, np.int32))
    # the oracle over the dense bf16 workspace through the same identity table
    none = np.zeros(0, np.int32)
    dense = Case("bf16", c.w, synth.PageTable(np.array(indptr, np.int32), np.array(table, np.int32),
                                              np.array(lens, np.int32), none, none),
                 c.q_bits, c.fp8_pool, bf16_pool=ref_bits, max_kv_len=max(lens))
    ref_out, ref_lse = oracle_decode(dense)
    for s in (0, 1, 3):
        out, lse = qk.mla_decode_bf16(q, ws, ptr, ind, lens_t, P, max(lens), c.w.sm_scale, num_splits=s)
        torch.cuda.synchronize()
        mx, rel = assert_parity(out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_out, ref_lse,
                                tag=f"gather-cast scale={kv_scale} splits={s}")
        print(f"[gather-cast kv_scale={kv_scale}] splits={s} max-abs {mx:.2e} rel-L2 {rel:.2e}", flush=True)
    # and, at the per-tensor scale of the pages (1.0, where the cast is exact), the oracle over the FP8 pool
    if kv_scale == 1.0:
        fo, fl = oracle_decode(c)
        np.testing.assert_array_equal(fo, ref_out)
