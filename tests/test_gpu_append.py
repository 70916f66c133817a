"""Fused append-then-attend over an NVFP4 pool, through the C ABI, against the oracle.

The last of each request's kv_lens tokens is the new token.  The call must write that token's
pool row with exactly the bytes of the oracle's quantizer (O-5) for the new source row and
leave every other row unchanged (bit-exact), and return the attention of the oracle (O-8)
over all kv_lens tokens of the updated pool within the decode tolerances."""
import numpy as np
import pytest
import torch

import synth
from cases import assert_parity, build_case, Device, gpu_decode, oracle_decode
from oracle import attention
from oracle import nvfp4 as onv

pytestmark = pytest.mark.gpu


def _qk():
    import quantized_kv_paged_amd as qk
    return qk


def _case(lens, page_size, seed, src_fmt, g=1.0, heads=16):
    c = build_case("nvfp4", lens, page_size, seed, heads=heads, outlier_p=0.01, g=g)
    x = synth.new_token_rows(seed, len(lens))
    if src_fmt == "bf16":
        src = synth.to_bf16_bits(x)
        ref_d, ref_s = onv.quantize_bf16_rows(src, c.scale)
    else:
        src = synth.to_fp8_bytes(x)
        ref_d, ref_s = onv.quantize_fp8_rows(src, 1.0, c.scale)
    rows = np.array([attention.gather_rows(c.pt.kv_indptr, c.pt.kv_indices, page_size, b, int(L))[-1]
                     if L > 0 else -1 for b, L in enumerate(lens)], dtype=np.int64)
    return c, src, ref_d, ref_s, rows


def _updated(c, ref_d, ref_s, rows):
    d, s = c.nv_data.copy(), c.nv_scales.copy()
    ok = rows >= 0
    d[rows[ok]], s[rows[ok]] = ref_d[ok], ref_s[ok]
    return d, s


def _append_gpu(c, src, src_fmt, num_splits):
    qk = _qk()
    dev = Device(c)
    if src_fmt == "bf16":
        s = torch.from_numpy(src.view(np.int16)).cuda().view(torch.bfloat16)
        fmt = qk.MLAQ_BF16
    else:
        s = torch.from_numpy(src).cuda()
        fmt = qk.MLAQ_FP8_E4M3
    out, lse = qk.mla_decode_nvfp4_append(dev.q, s, fmt, 1.0, dev.nv_data, dev.nv_scales, c.scale, dev.indptr,
                                          dev.indices, dev.lens, c.w.page_size, c.max_kv_len, c.w.sm_scale,
                                          num_splits=num_splits)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy(), dev.nv_data.cpu().numpy(), \
        dev.nv_scales.cpu().numpy()


def _check(lens, page_size, seed, src_fmt, splits, g=1.0, heads=16):
    c, src, ref_d, ref_s, rows = _case(lens, page_size, seed, src_fmt, g=g, heads=heads)
    upd_d, upd_s = _updated(c, ref_d, ref_s, rows)
    c_ref = build_case("nvfp4", lens, page_size, seed, heads=heads, outlier_p=0.01, g=g)
    c_ref.nv_data, c_ref.nv_scales = upd_d, upd_s
    ref_out, ref_lse = oracle_decode(c_ref)
    for s in splits:
        out, lse, pool_d, pool_s = _append_gpu(c, src, src_fmt, s)
        np.testing.assert_array_equal(pool_d, upd_d)
        np.testing.assert_array_equal(pool_s, upd_s)
        mx, rel = assert_parity(out, lse, ref_out, ref_lse, tag=f"append {src_fmt} splits={s}")
        print(f"[append {src_fmt} P{page_size} g={c.scale:.4g}] splits={s} max-abs {mx:.2e} rel-L2 {rel:.2e}",
              flush=True)
    return c, src


def test_append_bf16_source_ragged():
    """Contexts of 1 (the new token alone), 2, tile and page edges, and a long one; one and several splits."""
    _check([1, 2, 33, 64, 65, 700, 2049], 64, seed=41, src_fmt="bf16", splits=(0, 1, 3))


@pytest.mark.parametrize("g", [None, 0.37])
def test_append_fp8_source_global_scale(g):
    _check([129, 1000, 31], 64, seed=42, src_fmt="fp8", splits=(0, 2), g=g)


def test_append_row_by_row_pages_and_heads():
    """Pages shorter than a tile (rows gathered per lane) and 32 heads (two head groups)."""
    _check([17, 100, 1, 48], 16, seed=43, src_fmt="bf16", splits=(0, 1))
    _check([257, 40], 16, seed=44, src_fmt="fp8", splits=(0, 3), heads=32)


def test_append_equals_quantize_then_decode():
    """The fused call and kv_quantize_nvfp4 + mla_decode_nvfp4 write the same bytes and agree
    within the fp16-probability rounding of the decode kernel."""
    qk = _qk()
    lens = [300, 77, 1]
    c, src, ref_d, ref_s, rows = _case(lens, 64, 45, "bf16")
    out_f, lse_f, pool_d, pool_s = _append_gpu(c, src, "bf16", 0)
    dev = Device(c)
    s = torch.from_numpy(src.view(np.int16)).cuda().view(torch.bfloat16)
    qk.kv_quantize_nvfp4(s, qk.MLAQ_BF16, 1.0, torch.from_numpy(rows).cuda(), dev.nv_data, dev.nv_scales, c.scale)
    out_s, lse_s = qk.mla_decode_nvfp4(dev.q, dev.nv_data, dev.nv_scales, c.scale, dev.indptr, dev.indices,
                                       dev.lens, 64, c.max_kv_len, c.w.sm_scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev.nv_data.cpu().numpy(), pool_d)
    np.testing.assert_array_equal(dev.nv_scales.cpu().numpy(), pool_s)
    o2 = out_s.double().cpu().numpy()
    assert np.abs(out_f - o2).max() <= 1e-3 * max(1.0, np.abs(o2).max())
    assert np.abs(lse_f - lse_s.double().cpu().numpy()).max() <= 1e-4


def test_append_nan_row_and_empty_request():
    """A NaN in a new row is stored as the NaN scale and gives NaN for that request only; a
    request with kv_len 0 has no new token: NaN out and lse, nothing written."""
    lens = [50, 0, 80]
    c, src, ref_d, ref_s, rows = _case(lens, 64, 46, "bf16")
    x = synth.new_token_rows(46, 3)
    x[0, 7] = np.nan
    src = synth.to_bf16_bits(x)
    ref_d, ref_s = onv.quantize_bf16_rows(src, c.scale)
    assert ref_s[0, 0] == 0x7F
    out, lse, pool_d, pool_s = _append_gpu(c, src, "bf16", 0)
    upd_d, upd_s = _updated(c, ref_d, ref_s, rows)
    np.testing.assert_array_equal(pool_d, upd_d)
    np.testing.assert_array_equal(pool_s, upd_s)
    assert np.isnan(out[0]).all() and np.isnan(lse[0]).all()
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    c_ref = build_case("nvfp4", lens, 64, 46, outlier_p=0.01)
    c_ref.nv_data, c_ref.nv_scales = upd_d, upd_s
    ref_out, ref_lse = oracle_decode(c_ref, requests=[2])
    assert_parity(out, lse, ref_out, ref_lse, requests=[2], tag="append nan")


@pytest.mark.parametrize("ctx, splits", [(262144, 0), (32768, 1024)])
def test_append_with_the_most_splits(ctx, splits):
    """A fused append at batch 1 where the split count reaches MLAQ_MAX_SPLITS (1,024): by the
    automatic plan at 256K context, forced at 32K. The merge then reduces 1,025 partial slots per
    request, the new token's being the last."""
    qk = _qk()
    lens = [ctx]
    c, src, ref_d, ref_s, rows = _case(lens, 64, seed=47, src_fmt="bf16")
    p = qk.decode_params(1, 16, 64, ctx, c.nv_data.shape[0], c.w.sm_scale, splits)
    assert qk.mlaq_decode_num_splits(p, qk.MLAQ_NVFP4) == 1024
    _check(lens, 64, seed=47, src_fmt="bf16", splits=(splits,))
