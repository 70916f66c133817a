"""Pins of the extend oracle (oracle/extend.py) against things other than itself: PyTorch's
fp64 scaled-dot-product attention with an explicit causal mask (a library routine), closed
forms, and the separately pinned scalar E4M3 encoder for the FP8 workspace bytes."""
import numpy as np
import pytest
import torch

from oracle import codecs, extend
from oracle import nvfp4 as onv


def _ws(rng, n, lo=0, hi=0x7E):
    codes = rng.integers(lo, hi, (n, 576)).astype(np.uint8)
    return codes | (rng.integers(0, 2, (n, 576)).astype(np.uint8) << 7)


@pytest.mark.parametrize("P,C", [(0, 5), (7, 1), (13, 6)])
def test_causal_extend_matches_torch_sdpa(P, C):
    rng = np.random.default_rng(P * 31 + C)
    H, sm = 16, 0.0721688
    ws = _ws(rng, P + C, hi=0x60)                      # moderate magnitudes
    q = rng.standard_normal((C, H, 576))
    out, lse = extend.extend_request(q, ws, P, 1.0, sm)
    x = torch.from_numpy(codecs.e4m3_decode_np(ws))   # fp64 [P + C, 576]
    qt = torch.from_numpy(q).permute(1, 0, 2)          # [H, C, 576]
    mask = torch.arange(P + C)[None, :] <= (P + torch.arange(C))[:, None]   # [C, P + C]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, x[None].expand(H, -1, -1).contiguous(),
                                                           x[None, :, :512].expand(H, -1, -1).contiguous(),
                                                           attn_mask=mask, scale=sm)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    s = sm * torch.einsum("hcd,nd->hcn", qt, x).masked_fill(~mask[None], float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).T.numpy(), rtol=1e-12, atol=1e-12)


def test_single_token_closed_form():
    """Prefix 0, chunk 1: the token sees only itself, so out = its value dims, lse = its score."""
    rng = np.random.default_rng(3)
    ws = _ws(rng, 1)
    q = rng.standard_normal((1, 16, 576))
    out, lse = extend.extend_request(q, ws, 0, 0.5, 0.1)
    x = codecs.e4m3_decode_np(ws)[0] * 0.5
    np.testing.assert_array_equal(out[0], np.broadcast_to(x[:512], (16, 512)))
    np.testing.assert_allclose(lse[0], 0.1 * (q[0] @ x), rtol=1e-13)


def test_workspace_prefix_bytes_follow_the_scalar_encoder():
    """Every workspace byte is e4m3(fl32(fl32(fl32(e2m1*e4m3)*g)/chunk_scale)), checked against the
    pure-Python encoder on each value, including products that need rounding (6 significant bits)."""
    rng = np.random.default_rng(5)
    data = rng.integers(0, 256, (4, 288)).astype(np.uint8)
    scales = rng.integers(0x20, 0x48, (4, 36)).astype(np.uint8)
    for g, cs in [(1.0, 1.0), (0.37, 1.0), (1.0, 0.75)]:
        ws = extend.workspace_prefix(data, scales, g, cs)
        vals = onv.dequant_nvfp4_f64(data, scales, 1.0)            # exact products
        f32 = np.float32
        for r in range(4):
            for d in range(0, 576, 7):
                x = f32(f32(vals[r, d]) * f32(g))
                assert ws[r, d] == codecs.e4m3_encode(float(f32(x / f32(cs)))), (g, cs, r, d)
    # a product with 5 significant bits (1.5 * 1.875 = 2.8125) rounds to the nearest e4m3 (2.75)
    d1 = np.zeros((1, 288), np.uint8)
    d1[0, 0] = 0x3                                     # code 3 = 1.5 in dim 0
    s1 = np.full((1, 36), 0x3F, np.uint8)              # e4m3 0x3F = 1.875
    assert codecs.e4m3_decode(int(extend.workspace_prefix(d1, s1, 1.0, 1.0)[0, 0])) == 2.75
