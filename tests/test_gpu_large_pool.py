"""Pools larger than 4 GiB: every row offset is 64-bit.  The case's pages are moved, half of
them, past the 4 GiB byte offset of a large zero-filled pool (the other half stay at their low
ids, so one request reads both ends), and every call must give bit for bit what it gives on
the small pool: decode (pages of 64 and of 1 token), the fused append, extend with its chunk
write, quantize-on-write to high slots and dequantize from high rows.  Decode is also checked
against the oracle, to the parity bar."""
import numpy as np
import pytest
import torch

import synth
from cases import Device, assert_parity, build_case, gpu_decode, oracle_decode

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


def _lift(c, row_bytes):
    """Page ids past 4 GiB of row data for the even pages; returns (new indices, pool pages)."""
    P = c.w.page_size
    base = -(-(GIB4 + (1 << 26)) // (P * row_bytes))          # first page wholly past 4 GiB + 64 MiB
    old = c.pt.kv_indices
    new = np.where(old % 2 == 0, old + base, old).astype(np.int32)
    return new, base + c.w.pool_pages


def _big(small, P, old, new, pages):
    """Zero-filled device pool of `pages` pages holding small's pages `old` at ids `new`."""
    W = small.shape[1]
    big = torch.zeros((pages * P, W), dtype=torch.uint8, device="cuda")
    o = torch.from_numpy(old.astype(np.int64)).cuda()
    n = torch.from_numpy(new.astype(np.int64)).cuda()
    big.view(pages, P, W)[n] = small.view(-1, P, W)[o]
    return big


def _hi_device(c, d, new):
    d2 = Device.__new__(Device)
    d2.__dict__.update(d.__dict__)
    d2.indices = torch.from_numpy(new).cuda()
    return d2


@pytest.mark.parametrize("page_size", [64, 1])
def test_fp8_decode_past_4gib(page_size):
    lens = [700, 1, 2000] if page_size == 64 else [300, 1, 257]
    c = build_case("fp8", lens, page_size, seed=91, extra_pages=4)
    d = Device(c)
    new, pages = _lift(c, 576)
    d2 = _hi_device(c, d, new)
    d2.fp8 = _big(d.fp8, page_size, c.pt.kv_indices, new, pages)
    assert d2.fp8.numel() > GIB4 and int(new.max()) * page_size * 576 > GIB4
    ref_out, ref_lse = oracle_decode(c)
    for s in (0, 1, 3):
        o1, l1 = gpu_decode(c, d, num_splits=s)
        o2, l2 = gpu_decode(c, d2, num_splits=s)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), f"splits {s}"
        assert_parity(o2, l2, ref_out, ref_lse, tag=f"fp8 P{page_size} past 4 GiB splits={s}")


def test_nvfp4_decode_and_append_past_4gib():
    import quantized_kv_paged_amd as qk
    c = build_case("nvfp4", [900, 64, 65], 64, seed=93, extra_pages=4)
    d = Device(c)
    new, pages = _lift(c, 288)
    d2 = _hi_device(c, d, new)
    d2.nv_data = _big(d.nv_data, 64, c.pt.kv_indices, new, pages)
    d2.nv_scales = _big(d.nv_scales, 64, c.pt.kv_indices, new, pages)
    assert d2.nv_data.numel() > GIB4
    ref_out, ref_lse = oracle_decode(c)
    for s in (0, 2):
        o1, l1 = gpu_decode(c, d, num_splits=s)
        o2, l2 = gpu_decode(c, d2, num_splits=s)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), f"splits {s}"
        assert_parity(o2, l2, ref_out, ref_lse, tag=f"nvfp4 past 4 GiB splits={s}")
    # fused append: the new row of every request lands in its last token's row
    B = len(c.pt.kv_lens)
    rows = _t8(synth.to_fp8_bytes(synth.new_token_rows(93, B)))
    res = []
    for dd in (d, d2):
        out, lse = qk.mla_decode_nvfp4_append(dd.q, rows, qk.MLAQ_FP8_E4M3, 1.0, dd.nv_data, dd.nv_scales, c.scale,
                                              dd.indptr, dd.indices, dd.lens, 64, c.max_kv_len, c.w.sm_scale)
        torch.cuda.synchronize()
        res.append((out.cpu(), lse.cpu()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    lo_rows, hi_rows = _last_rows(c, c.pt.kv_indices), _last_rows(c, new)
    assert torch.equal(d.nv_data[lo_rows], d2.nv_data[hi_rows])
    assert torch.equal(d.nv_scales[lo_rows], d2.nv_scales[hi_rows])


def _t8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _last_rows(c, indices):
    P = c.w.page_size
    r = []
    for b, L in enumerate(c.pt.kv_lens):
        j = int(L) - 1
        r.append(int(indices[c.pt.kv_indptr[b] + j // P]) * P + j % P)
    return torch.tensor(r, dtype=torch.int64, device="cuda")


def test_quantize_and_dequantize_past_4gib():
    import quantized_kv_paged_amd as qk
    n = 1000
    src = _t8(synth.to_fp8_bytes(synth.extend_chunk_rows(95, n)))
    lo = torch.arange(n, dtype=torch.int64, device="cuda") * 7
    hi_base = -(-(GIB4 + (1 << 26)) // 288)
    hi = lo + hi_base
    pool_rows = hi_base + 7 * n
    small_d = torch.zeros((7 * n, 288), dtype=torch.uint8, device="cuda")
    small_s = torch.zeros((7 * n, 36), dtype=torch.uint8, device="cuda")
    big_d = torch.zeros((pool_rows, 288), dtype=torch.uint8, device="cuda")
    big_s = torch.zeros((pool_rows, 36), dtype=torch.uint8, device="cuda")
    assert big_d.numel() > GIB4
    qk.kv_quantize_nvfp4(src, qk.MLAQ_FP8_E4M3, 1.0, lo, small_d, small_s, 0.5)
    qk.kv_quantize_nvfp4(src, qk.MLAQ_FP8_E4M3, 1.0, hi, big_d, big_s, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(small_d[lo], big_d[hi]) and torch.equal(small_s[lo], big_s[hi])
    assert int(big_d[hi].ne(0).sum()) > 0
    for fmt in (qk.MLAQ_FP32, qk.MLAQ_BF16, qk.MLAQ_FP8_E4M3):
        a = qk.kv_dequantize(qk.MLAQ_NVFP4, small_d, small_s, 0.5, fmt, rows=lo)
        b = qk.kv_dequantize(qk.MLAQ_NVFP4, big_d, big_s, 0.5, fmt, rows=hi)
        torch.cuda.synchronize()
        assert torch.equal(a, b), fmt
    del big_d, big_s
    fp8_big = torch.zeros((-(-(GIB4 + (1 << 26)) // 576) + n, 576), dtype=torch.uint8, device="cuda")
    hi8 = torch.arange(n, dtype=torch.int64, device="cuda") + (fp8_big.shape[0] - n)
    fp8_big[hi8] = src
    b = qk.kv_dequantize(qk.MLAQ_FP8_E4M3, fp8_big, None, 1.0, qk.MLAQ_FP32, rows=hi8)
    a = qk.kv_dequantize(qk.MLAQ_FP8_E4M3, src, None, 1.0, qk.MLAQ_FP32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_extend_past_4gib():
    import quantized_kv_paged_amd as qk
    from oracle import attention
    prefix, chunk = np.array([0, 700, 130], np.int32), np.array([40, 64, 9], np.int32)
    c = build_case("nvfp4", prefix + chunk, 64, seed=97, extra_pages=4)
    d = Device(c)
    new, pages = _lift(c, 288)
    qo = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    nq = int(qo[-1])
    q = _t8(synth.q_bits(97, nq, 16).view(np.int16)).view(torch.bfloat16)
    ckv = _t8(synth.to_fp8_bytes(synth.extend_chunk_rows(97, nq)))
    mp, mc = int(prefix.max()), int(chunk.max())

    def slots(indices):
        return _t8(np.concatenate([attention.gather_rows(c.pt.kv_indptr, indices, 64, b,
                                                         int(prefix[b] + chunk[b]))[prefix[b]:]
                                   for b in range(len(prefix))]).astype(np.int64))
    pools = [(d.nv_data.clone(), d.nv_scales.clone(), c.pt.kv_indices),
             (_big(d.nv_data, 64, c.pt.kv_indices, new, pages), _big(d.nv_scales, 64, c.pt.kv_indices, new, pages),
              new)]
    assert pools[1][0].numel() > GIB4
    res = []
    for data, scales, idx in pools:
        sl = slots(idx)
        out, lse = qk.mla_extend_nvfp4(q, _t8(qo), ckv, 1.0, data, scales, c.scale, d.indptr, _t8(idx), _t8(prefix),
                                       sl, 64, mp, mc, c.w.sm_scale, num_splits=3)
        torch.cuda.synchronize()
        res.append((out.cpu(), lse.cpu(), data[sl].cpu(), scales[sl].cpu()))
    for k in range(4):
        assert torch.equal(res[0][k], res[1][k]), k
    assert torch.isfinite(res[1][0]).all()
