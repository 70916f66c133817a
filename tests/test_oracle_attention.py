"""Pins for the oracle's paged gather and fp64 attention (CPU only).

Anchors: PyTorch's scaled_dot_product_attention in float64 on the CPU (a library
routine), scipy's logsumexp, closed forms (one token, identical rows, zero query, two
tokens), a hand-built page table, and planted mistakes that these pins must catch.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention

H, D, DV = 16, 576, 512


def _case(L, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((H, D)), rng.standard_normal((L, D)), float(1 / np.sqrt(192))


@pytest.mark.parametrize("L", [1, 2, 17, 300])
def test_decode_vs_torch_sdpa_fp64(L):
    q, x, sm = _case(L, L)
    out, lse = attention.decode_dense(q, x, sm)
    qt = torch.from_numpy(q)[None, :, None, :]                     # [1, H, 1, D]
    k = torch.from_numpy(x)[None, None].expand(1, H, L, D)
    v = torch.from_numpy(x[:, :DV])[None, None].expand(1, H, L, DV)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=sm)[0, :, 0].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, logsumexp(sm * x @ q.T, axis=0), rtol=1e-13, atol=1e-13)


def test_closed_forms():
    q, x, sm = _case(5, 1)
    out, lse = attention.decode_dense(q, x[:1], sm)                 # one token
    np.testing.assert_array_equal(out, np.broadcast_to(x[0, :DV], (H, DV)))
    np.testing.assert_allclose(lse, sm * x[0] @ q.T, rtol=1e-14)
    same = np.repeat(x[:1], 7, axis=0)                              # identical rows
    out, lse = attention.decode_dense(q, same, sm)
    np.testing.assert_allclose(out, np.broadcast_to(x[0, :DV], (H, DV)), rtol=1e-14)
    np.testing.assert_allclose(lse, sm * x[0] @ q.T + np.log(7), rtol=1e-13)
    out, lse = attention.decode_dense(np.zeros((H, D)), x, sm)      # zero query -> mean
    np.testing.assert_allclose(out, np.broadcast_to(x[:, :DV].mean(0), (H, DV)), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, np.log(5), rtol=1e-14)
    out, _ = attention.decode_dense(q, x[:2], sm)                   # two tokens: logistic weights
    s = sm * x[:2] @ q.T
    w1 = 1 / (1 + np.exp(s[1] - s[0]))
    np.testing.assert_allclose(out, w1[:, None] * x[0, :DV] + (1 - w1)[:, None] * x[1, :DV], rtol=1e-12, atol=1e-14)


def test_empty_and_nan():
    q, x, sm = _case(3, 2)
    out, lse = attention.decode_dense(q, x[:0], sm)
    assert (out == 0).all() and np.isneginf(lse).all()
    x = x.copy()
    x[1, 530] = np.nan                                              # NaN in a rope dim
    out, lse = attention.decode_dense(q, x, sm)
    assert np.isnan(out).all() and np.isnan(lse).all()


def test_gather_hand_built_table():
    indptr = np.array([0, 2, 3], np.int32)
    indices = np.array([3, 0, 2], np.int32)
    np.testing.assert_array_equal(attention.gather_rows(indptr, indices, 2, 0, 3), [6, 7, 0])
    np.testing.assert_array_equal(attention.gather_rows(indptr, indices, 2, 1, 2), [4, 5])
    np.testing.assert_array_equal(attention.gather_rows(indptr, indices, 2, 0, 3, start=1, count=2), [7, 0])


def test_chunked_equals_dense_and_page_layout_invariance():
    q, x, sm = _case(1000, 4)
    out, lse = attention.decode_dense(q, x, sm)
    chunks = lambda: [x[i:i + 137] for i in range(0, 1000, 137)]
    out2, lse2 = attention.decode_head_block(q, chunks, sm)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)
    # the same logical rows under two physical page layouts gather identically
    P, L = 8, 1000
    pages = -(-L // P)
    pool_pages = pages + 5
    for seed in (0, 1):
        perm = np.random.default_rng(seed).permutation(pool_pages)[:pages]
        pool = np.zeros((pool_pages * P, D))
        rows = attention.gather_rows(np.array([0, pages]), perm, P, 0, L)
        pool[rows] = x
        o, l_ = attention.decode_dense(q, pool[rows], sm)
        np.testing.assert_array_equal(o, out)


def test_merge_partials_vs_logsumexp():
    q, x, sm = _case(600, 6)
    out, lse = attention.decode_dense(q, x, sm)
    cuts = [0, 1, 250, 251, 600]
    parts = [attention.decode_dense(q, x[a:b], sm) for a, b in zip(cuts[:-1], cuts[1:])]
    o = np.stack([p[0] for p in parts])
    ls = np.stack([p[1] for p in parts])
    mo, ml = attention.merge_partials(o, ls)
    np.testing.assert_allclose(ml, logsumexp(ls, axis=0), rtol=1e-13)
    np.testing.assert_allclose(mo, out, rtol=1e-11, atol=1e-13)
    empty = attention.decode_dense(q, x[:0], sm)
    mo2, ml2 = attention.merge_partials(np.concatenate([o, empty[0][None]]), np.concatenate([ls, empty[1][None]]))
    np.testing.assert_allclose(mo2, out, rtol=1e-11, atol=1e-13)


def _pins_hold(decode):
    """The SDPA, one-token, zero-query and logsumexp pins, run against `decode`."""
    q, x, sm = _case(17, 3)
    out, lse = decode(q, x, sm)
    qt = torch.from_numpy(q)[None, :, None, :]
    k = torch.from_numpy(x)[None, None].expand(1, H, 17, D)
    v = torch.from_numpy(x[:, :DV])[None, None].expand(1, H, 17, DV)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=sm)[0, :, 0].numpy()
    ok = out.shape == ref.shape and np.allclose(out, ref, rtol=1e-10, atol=1e-12)
    ok &= np.allclose(lse, logsumexp(sm * x @ q.T, axis=0), rtol=1e-12)
    o1, _ = decode(q, x[:1], sm)
    ok &= o1.shape == (H, DV) and np.array_equal(o1, np.broadcast_to(x[0, :DV], (H, DV)))
    return bool(ok)


def _variant(v_slice=slice(0, DV), scale_twice=False, log2=False, normalise=True, transpose_q=False):
    def decode(q, x, sm):
        s = sm * (x @ q.T)
        if scale_twice:
            s = sm * s
        if transpose_q:
            s = sm * (x[:, ::-1] @ q.T)
        m = s.max(axis=0)
        w = np.exp(s - m)
        z = w.sum(axis=0)
        out = w.T @ x[:, v_slice]
        if normalise:
            out = out / z[:, None]
        lse = m + (np.log2(z) if log2 else np.log(z))
        return out, lse
    return decode


def test_pins_catch_planted_mistakes():
    assert _pins_hold(attention.decode_dense)
    assert _pins_hold(_variant())                       # the unmutated copy passes
    assert not _pins_hold(_variant(v_slice=slice(64, D)))
    assert not _pins_hold(_variant(scale_twice=True))
    assert not _pins_hold(_variant(log2=True))
    assert not _pins_hold(_variant(normalise=False))
    assert not _pins_hold(_variant(transpose_q=True))
