"""GPU parity of the decode kernels against the fp64 oracle, through the C ABI.

Bar: max-abs error <= 1e-2 and relative L2 error <= 5e-3 of the [B, H, 512] output
(lse within 2e-3); bitwise equality where the arithmetic is identical by construction
(page placement, FP8 vs NVFP4 holding the same values)."""
import numpy as np
import pytest
import torch

import cases
from cases import assert_parity, build_case, gpu_decode, oracle_decode, Device

pytestmark = pytest.mark.gpu


def _run(c, splits=(0,), tag=""):
    d = Device(c)
    ref_out, ref_lse = oracle_decode(c)
    res = {}
    for s in splits:
        out, lse = gpu_decode(c, d, num_splits=s)
        print(f"[{tag}] splits={s} ", end="")
        mx, rel = assert_parity(out, lse, ref_out, ref_lse, tag=f"{tag} splits={s}")
        print(f"max-abs {mx:.2e} rel-L2 {rel:.2e}", flush=True)
        res[s] = (out, lse)
    return res


def test_tiny_fp8_workload():
    """batch 1, 16 heads, context 512, page 16 over a 1024-token pool, auto splits and one split."""
    import synth
    w = synth.WORKLOADS["tiny_fp8"]
    c = build_case("fp8", [w.kv_len], w.page_size, w.seed, extra_pages=w.pool_pages - w.kv_len // w.page_size)
    assert c.fp8_pool.shape[0] == w.pool_tokens
    _run(c, splits=(0, 1), tag="tiny")


@pytest.mark.parametrize("splits", [1, 2, 7, 32])
def test_fp8_ragged_lengths_and_splits(splits):
    c = build_case("fp8", [0, 1, 17, 64, 1000, 15, 16, 65], 16, seed=11)
    _run(c, splits=(splits,), tag="ragged")


@pytest.mark.parametrize("page_size", [1, 16, 64, 128])
def test_page_sizes(page_size):
    c = build_case("fp8", [100, 333, 64], page_size, seed=12)
    _run(c, splits=(0, 3), tag=f"P{page_size}")


@pytest.mark.parametrize("g", [1.0, None, 0.37])
def test_nvfp4_parity(g):
    c = build_case("nvfp4", [129, 700, 2048], 64, seed=13, outlier_p=0.01, g=g)
    _run(c, splits=(0, 1, 5), tag=f"nvfp4 g={c.scale}")


def test_bf16_parity():
    c = build_case("bf16", [65, 500, 1], 16, seed=14)
    _run(c, splits=(0, 1), tag="bf16")


def test_fp8_kv_scale():
    c = build_case("fp8", [300, 77], 16, seed=15, sigma=0.5, kv_scale=0.75)
    _run(c, splits=(0, 2), tag="kv_scale")


def test_32_heads():
    c = build_case("fp8", [257, 40], 16, seed=16, heads=32)
    _run(c, splits=(0, 1), tag="H32")
    c = build_case("nvfp4", [190], 64, seed=17, heads=64, outlier_p=0.01)
    _run(c, splits=(0, 3), tag="H64 nvfp4")


def test_limits_128_heads_1024_page_1024_splits():
    """The largest shapes the ABI accepts: 128 heads (8 head groups), 1,024-token pages, 1,024 splits."""
    c = build_case("fp8", [300, 77], 16, seed=18, heads=128)
    _run(c, splits=(0, 2), tag="H128")
    c = build_case("nvfp4", [3000, 1500], 1024, seed=19, outlier_p=0.01, extra_pages=1)
    _run(c, splits=(0, 1), tag="P1024 nvfp4")
    c = build_case("nvfp4", [40000], 64, seed=20, outlier_p=0.01, extra_pages=1)
    _run(c, splits=(1024,), tag="1024 splits")


def test_page_placement_is_bitwise_invariant():
    """The same logical KV under two different physical page layouts gives identical bits."""
    c1 = build_case("fp8", [700, 130], 16, seed=21, extra_pages=9)
    c2 = build_case("fp8", [700, 130], 16, seed=21, extra_pages=9)
    rng = np.random.default_rng(5)
    perm = rng.permutation(c2.w.pool_pages).astype(np.int32)
    new_idx = perm[c1.pt.kv_indices]
    pool2 = np.zeros_like(c1.fp8_pool)
    P = c1.w.page_size
    for old, new in zip(c1.pt.kv_indices, new_idx):
        pool2[new * P:(new + 1) * P] = c1.fp8_pool[old * P:(old + 1) * P]
    c2.pt.kv_indices = new_idx
    c2.fp8_pool = pool2
    for s in (0, 1, 4):
        o1, l1 = gpu_decode(c1, Device(c1), num_splits=s)
        o2, l2 = gpu_decode(c2, Device(c2), num_splits=s)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), s


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_request_order_is_bitwise_invariant(fmt):
    """A request's result depends on nothing but its own query, length and rows: reversing the
    batch order (queries, lengths and page-table segments together) reverses the outputs bit
    for bit, with the automatic split count and with forced ones."""
    c = build_case(fmt, [333, 0, 1500, 64, 17], 64, seed=23)
    d = Device(c)
    B = len(c.pt.kv_lens)
    seg = [c.pt.kv_indices[c.pt.kv_indptr[b]:c.pt.kv_indptr[b + 1]] for b in range(B)]
    order = list(range(B))[::-1]
    d2 = Device(c)
    d2.q = d.q[order].contiguous()
    d2.lens = d.lens[order].contiguous()
    d2.indices = torch.from_numpy(np.concatenate([seg[b] for b in order]).astype(np.int32)).cuda()
    d2.indptr = torch.from_numpy(np.concatenate([[0], np.cumsum([len(seg[b]) for b in order])]).astype(np.int32)).cuda()
    for s in (0, 1, 3):
        o1, l1 = gpu_decode(c, d, num_splits=s)
        o2, l2 = gpu_decode(c, d2, num_splits=s)
        assert np.array_equal(o1[order], o2) and np.array_equal(l1[order], l2), s


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_head_groups_are_independent(fmt):
    """With 64 heads, each 16-head group gives bit for bit what a 16-head call on the same
    query rows gives (same forced split count): the head groups share nothing but the rows."""
    c = build_case(fmt, [900, 5, 260], 64, seed=25, heads=64)
    d = Device(c)
    for s in (1, 4):
        o_all, l_all = gpu_decode(c, d, num_splits=s)
        for hg in range(4):
            d16 = Device(c)
            d16.q = d.q[:, 16 * hg:16 * (hg + 1)].contiguous()
            o, l = gpu_decode(c, d16, num_splits=s)
            assert np.array_equal(o, o_all[:, 16 * hg:16 * (hg + 1)]), (s, hg)
            assert np.array_equal(l, l_all[:, 16 * hg:16 * (hg + 1)]), (s, hg)


def test_fp8_and_nvfp4_agree_on_shared_values():
    """An FP8 pool and an NVFP4 pool (all block scales 1.0, global scale 1.0) holding the same
    E2M1 values dequantize to the same fp16 operands.  The two formats run different workgroup
    shapes (two softmax streams per workgroup for FP8, one for NVFP4), so probabilities are
    rounded to fp16 against different running maxima and sums are grouped differently: the
    outputs must agree to that rounding (about 2^-11 relative), far inside the oracle
    tolerance.  The softmax sums add the rounded probabilities (each within 2^-12 of the
    exact one), so the two lse agree to 2^-12 in the sum, about 2.4e-4 in the log."""
    c = build_case("fp8", [333, 1024], 64, seed=22)
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 16, size=c.fp8_pool.shape, dtype=np.uint8)
    from oracle import codecs
    vals = codecs.e2m1_decode_np(codes).astype(np.float32)
    import synth
    c.fp8_pool = synth.to_fp8_bytes(vals)
    nv = build_case("nvfp4", [333, 1024], 64, seed=22)
    nv.nv_data = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    nv.nv_scales = np.full((codes.shape[0], 36), 0x38, np.uint8)
    nv.scale = 1.0
    for s in (0, 1):
        o1, l1 = gpu_decode(c, Device(c), num_splits=s)
        o2, l2 = gpu_decode(nv, Device(nv), num_splits=s)
        assert np.abs(o1 - o2).max() <= 1e-3 * max(1.0, np.abs(o1).max()), s
        assert np.abs(l1 - l2).max() <= 5e-4, s
    ref_out, ref_lse = oracle_decode(nv)
    assert_parity(o2, l2, ref_out, ref_lse, tag="shared values")


def test_bad_device_inputs_give_nan_not_faults():
    """A page id outside the pool, a length above max_kv_len, a negative length and a
    length beyond the request's pages poison only that request's outputs with NaN."""
    c = build_case("fp8", [200, 300, 100, 50, 80], 16, seed=23, extra_pages=4)
    ref_out, ref_lse = oracle_decode(c)
    c.pt.kv_indices = c.pt.kv_indices.copy()
    c.pt.kv_indices[c.pt.kv_indptr[1] + 3] = c.w.pool_pages + 5        # request 1: page out of range
    c.pt.kv_lens = c.pt.kv_lens.copy()
    c.pt.kv_lens[2] = -4                                                 # request 2: negative length
    c.pt.kv_lens[3] = (c.pt.kv_indptr[4] - c.pt.kv_indptr[3]) * 16 + 1  # request 3: beyond its pages
    for s in (0, 1):
        out, lse = gpu_decode(c, Device(c), num_splits=s, max_kv_len=300)
        assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
        assert np.isnan(out[2]).all() and np.isnan(out[3]).all()
        assert_parity(out, lse, ref_out, ref_lse, requests=[0, 4], tag="good requests")
    c.pt.kv_lens[4] = 301                                                # above max_kv_len
    out, lse = gpu_decode(c, Device(c), num_splits=0, max_kv_len=300)
    assert np.isnan(out[4]).all()


def test_nan_in_kv_propagates_to_its_request():
    c = build_case("fp8", [100, 90], 16, seed=24)
    rows = cases.attention.gather_rows(c.pt.kv_indptr, c.pt.kv_indices, 16, 1, 90)
    c.fp8_pool = c.fp8_pool.copy()
    c.fp8_pool[rows[40], 530] = 0x7F                                     # NaN in a rope dim
    ref_out, ref_lse = oracle_decode(c)
    assert np.isnan(ref_out[1]).all()
    out, lse = gpu_decode(c, Device(c))
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    assert_parity(out, lse, ref_out, ref_lse, requests=[0], tag="nan")


def test_lse_optional_and_empty_batch():
    import quantized_kv_paged_amd as qk
    c = build_case("fp8", [64, 0], 16, seed=25)
    out, lse = gpu_decode(c, Device(c), want_lse=False)
    assert lse is None
    assert (out[1] == 0).all()
    ref_out, _ = oracle_decode(c)
    assert np.abs(out - ref_out).max() <= cases.TOL_MAX_ABS
    d = Device(c)
    q0 = d.q[:0]
    o, l_ = qk.mla_decode_fp8(q0, d.fp8, 1.0, d.indptr, d.indices, d.lens, 16, 64, 0.07)
    assert o.shape == (0, 16, 512)


def test_full_pool_cast_baseline_matches():
    """The comparison path of the pages (whole FP8 pool -> BF16, then a 16-bit decode) gives
    the oracle's answer too."""
    import quantized_kv_paged_amd as qk
    c = build_case("fp8", [500, 260], 64, seed=26, extra_pages=20)
    d = Device(c)
    pool_bf16 = qk.kv_dequantize(qk.MLAQ_FP8_E4M3, d.fp8, None, 1.0, qk.MLAQ_BF16)
    out, lse = qk.mla_decode_bf16(d.q, pool_bf16, d.indptr, d.indices, d.lens, 64, c.max_kv_len, c.w.sm_scale)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_decode(c)
    assert_parity(out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_out, ref_lse, tag="cast baseline")


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_peaked_softmax_with_long_tail(fmt):
    """Probabilities enter the PV products as fp16 relative to the running maximum, so a tail far
    below one dominant token sits on the fp16 subnormal grid.  One sink token about 20 log2 units
    above a 64K-token tail that still holds several percent of the weight: automatic splits and the
    fewest splits the per-split token cap (MLAQ_MAX_SPLIT_TOKENS) admits must match the oracle, and a
    count below that cap is rejected before any launch."""
    import quantized_kv_paged_amd as qk
    from oracle import attention, codecs
    from oracle import nvfp4 as onv
    L = 65536
    c = build_case("fp8", [L], 64, seed=31, sigma=0.5, extra_pages=1)
    rng = np.random.default_rng(31)
    u = rng.standard_normal(576)
    qf = u[None, :] + 0.3 * rng.standard_normal((16, 576))
    c.q_bits = codecs.bf16_round_bits(qf.astype(np.float32))[None]
    rows = attention.gather_rows(c.pt.kv_indptr, c.pt.kv_indices, 64, 0, L)
    sink = int(rows[40000])
    c.fp8_pool[sink] = torch.from_numpy((0.33 * u).astype(np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    if fmt == "nvfp4":
        c.fmt = "nvfp4"
        c.nv_data, c.nv_scales = onv.quantize_fp8_rows(c.fp8_pool, 1.0, 1.0)
        c.scale = 1.0
    # the regime: gap of the sink over the tail's typical score, and the tail's share of the weight
    x = cases.dequant_rows(c, rows)
    s = codecs.bf16_bits_to_f64(c.q_bits[0]) @ x.T * c.w.sm_scale / np.log(2)      # log2 units [16, L]
    gap = s[:, 40000] - np.median(np.delete(s, 40000, axis=1), axis=1)
    w_ = np.exp2(s - s.max(axis=1, keepdims=True))
    tail = 1.0 - w_[:, 40000] / w_.sum(axis=1)
    assert 17 <= gap.min() and gap.max() <= 25 and tail.min() > 0.02, (gap, tail)
    ref_out, ref_lse = oracle_decode(c)
    d = Device(c)
    fcode = qk.MLAQ_FP8_E4M3 if fmt == "fp8" else qk.MLAQ_NVFP4
    p = qk.decode_params(1, 16, 64, L, c.fp8_pool.shape[0], c.w.sm_scale, 0)
    least = -(-L // (1 << 14))
    for splits in (0, least):
        out, lse = gpu_decode(c, d, num_splits=splits)
        mx, rel = assert_parity(out, lse, ref_out, ref_lse, tag=f"sink {fmt} splits={splits}")
        print(f"[sink {fmt}] gap {gap.min():.1f}-{gap.max():.1f} log2, tail weight {tail.min():.3f}-{tail.max():.3f}; "
              f"splits={splits or qk.mlaq_decode_num_splits(p, fcode)} max-abs {mx:.2e} rel-L2 {rel:.2e}", flush=True)
    with pytest.raises(qk.MlaqError) as e:
        gpu_decode(c, d, num_splits=least - 1)
    assert e.value.status == 2


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_page_tiles_at_the_pool_edge(fmt):
    """Pages that hold whole tiles (64 tokens): the pool ends 40 rows into its last page.  A request
    whose last page is that partial page and whose rows stay inside the pool is exact; one that
    reads past the pool's end, one with a page id just past the pool and one with a negative page
    id give NaN, in single-split and automatic-split launches."""
    P = 64
    c = build_case(fmt, [64 * 3 + 38, 64 * 2 + 50, 64 * 4, 64 * 2 + 7, 64 * 5], P, seed=41, extra_pages=4)
    n_pages = c.w.pool_tokens // P
    last = n_pages - 1
    T = last * P + 40                                    # pool rows: the last page holds 40
    idx = c.pt.kv_indices.copy()
    ip = c.pt.kv_indptr
    free = [p for p in range(n_pages) if p not in set(idx.tolist()) and p != last]
    for k in np.nonzero(idx == last)[0]:                 # only requests 0 and 1 use the partial page
        idx[k] = free.pop()
    idx[ip[1] - 1] = last                                # request 0: 38 of its 40 rows
    idx[ip[2] - 1] = last                                # request 1: 50 rows, 10 past the pool's end
    idx[ip[2] + 1] = n_pages                             # request 2: a page id past the pool
    idx[ip[3]] = -1                                      # request 3: a negative page id
    c.pt.kv_indices = idx
    ref_out, ref_lse = oracle_decode(c, requests=[0, 4])
    d = Device(c)
    if fmt == "fp8":
        d.fp8 = d.fp8[:T].contiguous()
    else:
        d.nv_data, d.nv_scales = d.nv_data[:T].contiguous(), d.nv_scales[:T].contiguous()
    for s in (1, 0):
        out, lse = gpu_decode(c, d, num_splits=s)
        for b in (1, 2, 3):
            assert np.isnan(out[b]).all() and np.isnan(lse[b]).all(), (s, b)
        assert_parity(out, lse, ref_out, ref_lse, requests=[0, 4], tag=f"pool edge {fmt} splits={s}")
