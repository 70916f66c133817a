"""The allocation-free NVFP4 decode (mla_decode_nvfp4_noalloc) against mla_decode_nvfp4 with a
caller workspace, through the C ABI.  Calls follow one another on the same device, each on a smaller
input than the one before, so every call meets the scratch holding the previous call's partials.
Where the automatic plan fits the scratch the two calls agree bit for bit; where it does not, the
allocation-free call takes the largest split count that fits and agrees bit for bit with the
workspace call forced to that count; both are also checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

from cases import assert_parity, build_case, Device, gpu_decode, oracle_decode

pytestmark = pytest.mark.gpu
SCRATCH = 48 << 20
SLOT = 16 * 512 * 4 + 32 * 4       # bytes of one (request, split, 16-head group) partial


def _noalloc(c, d, max_kv_len, num_splits=0):
    import quantized_kv_paged_amd as qk
    out, lse = qk.mla_decode_nvfp4_noalloc(d.q, d.nv_data, d.nv_scales, c.scale, d.indptr, d.indices, d.lens,
                                           c.w.page_size, max_kv_len, c.w.sm_scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def _same(a, b):
    np.testing.assert_array_equal(np.isnan(a), np.isnan(b))
    np.testing.assert_array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_noalloc_matches_the_workspace_call():
    import quantized_kv_paged_amd as qk
    rng = np.random.default_rng(60)
    # (lengths, page size, max_kv_len, forced splits): the first case's automatic plan (15 splits x 129
    # requests, 63.7 MB of partials) outgrows the scratch, so the call runs the largest count that
    # fits (11); then a multi-split case at the automatic plan, a forced count, and a one-split case
    cases = [(list(rng.integers(0, 1500, 129)), 64, 32768, 0), ([3000, 1500, 0, 700], 64, 3000, 0),
             ([2048, 5], 64, 2048, 7), ([300, 17], 16, 300, 1)]
    for i, (lens, P, mk, splits) in enumerate(cases):
        c = build_case("nvfp4", lens, P, seed=61 + i, outlier_p=0.01)
        d = Device(c)
        p = qk.decode_params(len(lens), 16, P, mk, c.nv_data.shape[0], c.w.sm_scale, splits)
        planned = qk.mlaq_decode_num_splits(p, qk.MLAQ_NVFP4)
        fits = len(lens) * planned * SLOT <= SCRATCH or planned == 1
        used = planned if fits else min(SCRATCH // (len(lens) * SLOT), 1024)
        ref_o, ref_l = gpu_decode(c, d, num_splits=used, max_kv_len=mk)
        o, l = _noalloc(c, d, mk, splits)
        _same(o, ref_o)
        _same(l, ref_l)
        ro, rl = oracle_decode(c)
        mx, rel = assert_parity(o, l, ro, rl, tag=f"noalloc case {i}")
        print(f"[noalloc case {i}] batch {len(lens)}, plan {planned} splits, ran {used}: bitwise equal to the "
              f"workspace call; vs oracle max-abs {mx:.2e} rel-L2 {rel:.2e}", flush=True)


def test_noalloc_rejects_what_does_not_fit():
    import quantized_kv_paged_amd as qk
    c = build_case("nvfp4", [100, 50], 64, seed=70)
    d = Device(c)
    with pytest.raises(qk.MlaqError) as e:                 # forced: 1,000 splits x 2 requests = 66 MB
        _noalloc(c, d, 32768, 1000)
    assert e.value.status == 5 and "scratch" in str(e.value)
    o, l = _noalloc(c, d, 100, 0)                          # the device is still usable afterwards
    ro, rl = oracle_decode(c)
    assert_parity(o, l, ro, rl, tag="after rejection")
