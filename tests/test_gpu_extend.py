"""Extend (chunked prefill) over an NVFP4 cache, through the C ABI, against the oracle.

Checked per call: the FP8 workspace rows the gather kernel builds (prefix dequantized to e4m3
in the chunk's scale, chunk rows appended) are bit-exact; the attention of every chunk token
over the rows it may see is within the decode tolerances; the chunk's rows are written to the
cache bit-exactly and no other cache row changes."""
import numpy as np
import pytest
import torch

import synth
from cases import assert_parity, build_case
from oracle import attention, codecs, extend
from oracle import nvfp4 as onv

pytestmark = pytest.mark.gpu


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(prefix, chunk, page_size, seed, splits=(0,), g=1.0, chunk_scale=1.0, heads=16, prefix_lens_dev=None):
    import quantized_kv_paged_amd as qk
    prefix, chunk = np.asarray(prefix, np.int32), np.asarray(chunk, np.int32)
    B = len(prefix)
    c = build_case("nvfp4", prefix + chunk, page_size, seed, heads=heads, outlier_p=0.01, g=g)
    qo = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    nq = int(qo[-1])
    q_bits = synth.q_bits(seed + 100, nq, heads)
    ckv = synth.to_fp8_bytes(synth.extend_chunk_rows(seed, nq) / np.float32(chunk_scale))
    slots = np.concatenate([attention.gather_rows(c.pt.kv_indptr, c.pt.kv_indices, page_size, b,
                                                  int(prefix[b] + chunk[b]))[prefix[b]:] for b in range(B)])
    # oracle: workspace bytes, attention, cache after the write
    ws_ref, out_ref, lse_ref = [], np.zeros((nq, heads, 512)), np.zeros((nq, heads))
    q64 = codecs.bf16_bits_to_f64(q_bits)
    for b in range(B):
        rows = attention.gather_rows(c.pt.kv_indptr, c.pt.kv_indices, page_size, b, int(prefix[b]))
        ws = np.concatenate([extend.workspace_prefix(c.nv_data[rows], c.nv_scales[rows], c.scale, chunk_scale),
                             ckv[qo[b]:qo[b + 1]]])
        ws_ref.append(ws)
        out_ref[qo[b]:qo[b + 1]], lse_ref[qo[b]:qo[b + 1]] = extend.extend_request(
            q64[qo[b]:qo[b + 1]], ws, int(prefix[b]), chunk_scale, c.w.sm_scale)
    new_d, new_s = onv.quantize_fp8_rows(ckv, chunk_scale, c.scale)
    pool_d, pool_s = c.nv_data.copy(), c.nv_scales.copy()
    pool_d[slots], pool_s[slots] = new_d, new_s
    mp, mc = int(prefix.max()), int(chunk.max())
    region = -(-(mp + mc) // 64) * 64
    for s in splits:
        data, scales = _t(c.nv_data), _t(c.nv_scales)
        p = qk.extend_params(B, heads, page_size, data.shape[0], nq, mp, mc, c.w.sm_scale, s)
        ws = torch.zeros(qk.mlaq_extend_workspace_bytes(p), dtype=torch.uint8, device="cuda")
        pl = _t(prefix if prefix_lens_dev is None else prefix_lens_dev)
        out, lse = qk.mla_extend_nvfp4(_t(q_bits.view(np.int16)).view(torch.bfloat16), _t(qo), _t(ckv), chunk_scale,
                                       data, scales, c.scale, _t(c.pt.kv_indptr), _t(c.pt.kv_indices), pl,
                                       _t(slots.astype(np.int64)), page_size, mp, mc, c.w.sm_scale, num_splits=s,
                                       workspace=ws)
        torch.cuda.synchronize()
        out, lse = out.double().cpu().numpy(), lse.double().cpu().numpy()
        wsh = ws.cpu().numpy()
        if prefix_lens_dev is None:
            for b in range(B):
                n = int(prefix[b] + chunk[b])
                got = wsh[b * region * 576:(b * region + n) * 576].reshape(n, 576)
                np.testing.assert_array_equal(got, ws_ref[b], err_msg=f"workspace request {b}")
            mx, rel = assert_parity(out, lse, out_ref, lse_ref, tag=f"extend splits={s}")
            print(f"[extend P{page_size} g={c.scale:.4g} cs={chunk_scale}] splits={s} max-abs {mx:.2e} rel-L2 {rel:.2e}",
                  flush=True)
        np.testing.assert_array_equal(data.cpu().numpy(), pool_d)
        np.testing.assert_array_equal(scales.cpu().numpy(), pool_s)
    return out, lse, out_ref, lse_ref, qo


def test_extend_ragged_prefixes_and_chunks():
    """Empty prefix, prefixes and chunks across page and tile edges; one and several splits."""
    _run([0, 100, 700], [5, 64, 33], 64, seed=51, splits=(0, 1, 3))


@pytest.mark.parametrize("g,cs", [(None, 1.0), (0.37, 0.75)])
def test_extend_scales(g, cs):
    _run([129, 40], [17, 1], 16, seed=52, splits=(0, 2), g=g, chunk_scale=cs)


def test_extend_request_with_empty_chunk():
    """A request with no chunk tokens (prefix only) between two that have some: it owns no
    query rows, and the others' results and cache writes are unaffected."""
    _run([100, 50, 0], [3, 0, 7], 64, seed=58, splits=(0, 2))


def test_prefill_many_blocks_32_heads():
    """Causal prompts of unequal lengths with more token blocks than CUs (600 workgroups),
    32 heads, one and two KV splits."""
    _run([0, 0, 0, 0], [300, 257, 64, 1], 64, seed=59, splits=(0, 2), heads=32)


def test_extend_many_blocks_128_heads():
    """Long chunks over a cached prefix with eight head groups (528 workgroups), KV splits."""
    _run([300, 40], [130, 129], 64, seed=60, splits=(0, 3), heads=128)


@pytest.mark.parametrize("page_size", [1, 32, 128])
def test_extend_page_sizes(page_size):
    """The workspace gather and the chunk write at other page sizes, one-token pages included;
    chunks start mid-page and cross page edges."""
    _run([0, 130, 75], [9, 40, 64], page_size, seed=61 + page_size, splits=(0, 2))


def test_extend_32_heads():
    _run([300], [20], 64, seed=53, heads=32)


def test_extend_128_heads_and_splits():
    """Eight 16-head groups, each its own workgroups over the shared rows; one and several KV
    splits (the merge kernel then reads the per-group partials)."""
    _run([190, 0], [9, 6], 64, seed=56, splits=(0, 1, 3), heads=128)


def test_bad_prefix_nan_with_64_heads():
    """Tokens of an invalid request get NaN in every head group, with one split (the view builder
    writes them) and with several (the merge kernel does)."""
    prefix, chunk = [30, 70], [5, 2]
    bad = np.asarray([30, -3], np.int32)
    for s in (1, 2):
        out, lse, out_ref, lse_ref, qo = _run(prefix, chunk, 64, seed=57, splits=(s,), heads=64, prefix_lens_dev=bad)
        assert np.isnan(out[qo[1]:qo[2]]).all() and np.isnan(lse[qo[1]:qo[2]]).all()
        assert_parity(out[:qo[1]], lse[:qo[1]], out_ref[:qo[1]], lse_ref[:qo[1]], tag=f"64 heads splits={s}")


def test_extend_bad_prefix_length_gives_nan_for_its_tokens():
    prefix, chunk = [50, 80], [4, 3]
    bad = np.asarray([50, 10 ** 6], np.int32)                 # above max_prefix_len
    out, lse, out_ref, lse_ref, qo = _run(prefix, chunk, 64, seed=54, prefix_lens_dev=bad)
    assert np.isnan(out[qo[1]:qo[2]]).all() and np.isnan(lse[qo[1]:qo[2]]).all()
    assert_parity(out[:qo[1]], lse[:qo[1]], out_ref[:qo[1]], lse_ref[:qo[1]], tag="extend good request")


def test_initial_prefill_is_extend_with_empty_prefix():
    """The initial-prefill path of the pages (attention over the chunk's own FP8 KV, then the NVFP4
    write; no cache read) is extend with every prefix empty: causal attention inside each prompt."""
    _run([0, 0, 0], [1, 70, 257], 64, seed=55, splits=(0, 2))


@pytest.mark.parametrize("kind", ["extend", "prefill"])
def test_benchmark_shapes(kind):
    """The launch configurations the benchmark times, on 32K NVFP4 contexts (g = 1): extend = 4
    requests x a 256-token chunk after a 32,512-token prefix; prefill = 4 prompts of 2,048 tokens
    (empty prefixes).  Every request's FP8 workspace region is checked bit for bit, the cache after
    the chunk write bit for bit (written rows and every other row), and the attention of the first,
    the last and every 16th chunk token of every request (all heads) against the oracle."""
    import dataclasses
    import quantized_kv_paged_amd as qk
    w = dataclasses.replace(synth.WORKLOADS["nvfp4_32k"], name="extend_bench", batch=4, pool_tokens=4 * 32768)
    pt = synth.page_table(w)
    host = synth.build_fp8_pool(w, pt)
    data_np, scales_np = onv.quantize_fp8_rows(host, 1.0, 1.0)
    del host
    B, P, H = 4, w.page_size, w.heads
    C, PF, qseed, kseed = (256, w.kv_len - 256, w.seed + 7, w.seed) if kind == "extend" else \
        (2048, 0, w.seed + 8, w.seed + 1)
    nq = B * C
    tok = np.arange(PF, PF + C, dtype=np.int64)
    slots = np.concatenate([pt.kv_indices[pt.kv_indptr[b] + tok // P].astype(np.int64) * P + tok % P
                            for b in range(B)])
    q_bits = synth.q_bits(qseed, nq, H)
    ckv = synth.to_fp8_bytes(synth.extend_chunk_rows(kseed, nq))
    qo = (np.arange(B + 1) * C).astype(np.int32)
    p = qk.extend_params(B, H, P, w.pool_tokens, nq, PF, C, w.sm_scale)
    print(f"[{kind}] {B} x ({PF} prefix + {C} chunk), {qk._lib.mlaq_extend_num_splits(__import__('ctypes').byref(p))}"
          f" KV splits", flush=True)
    ws = torch.zeros(qk.mlaq_extend_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    data, scales = _t(data_np), _t(scales_np)
    out, lse = qk.mla_extend_nvfp4(_t(q_bits.view(np.int16)).view(torch.bfloat16), _t(qo), _t(ckv), 1.0, data,
                                   scales, 1.0, _t(pt.kv_indptr), _t(pt.kv_indices),
                                   _t(np.full(B, PF, np.int32)), _t(slots), P, PF, C, w.sm_scale, workspace=ws)
    torch.cuda.synchronize()
    out, lse, wsh = out.double().cpu().numpy(), lse.double().cpu().numpy(), ws.cpu().numpy()
    region = -(-(PF + C) // 64) * 64
    q64 = codecs.bf16_bits_to_f64(q_bits)
    picks = sorted(set([0, C - 1] + list(range(0, C, 16))))
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for b in range(B):
        rows = attention.gather_rows(pt.kv_indptr, pt.kv_indices, P, b, PF)
        ws_ref = np.concatenate([extend.workspace_prefix(data_np[rows], scales_np[rows], 1.0, 1.0),
                                 ckv[b * C:(b + 1) * C]])
        np.testing.assert_array_equal(wsh[b * region * 576:(b * region + PF + C) * 576].reshape(PF + C, 576), ws_ref,
                                      err_msg=f"{kind} workspace request {b}")
        x = extend.workspace_values(ws_ref, 1.0)
        for i in picks:
            o, l_ = attention.decode_dense(q64[b * C + i], x[:PF + i + 1], w.sm_scale)
            ref_o.append(o), ref_l.append(l_), got_o.append(out[b * C + i]), got_l.append(lse[b * C + i])
    mx, rel = assert_parity(np.stack(got_o), np.stack(got_l), np.stack(ref_o), np.stack(ref_l), tag=kind)
    print(f"[{kind}] {len(got_o)} sampled chunk tokens x {H} heads: max-abs {mx:.2e} rel-L2 {rel:.2e}", flush=True)
    new_d, new_s = onv.quantize_fp8_rows(ckv, 1.0, 1.0)
    data_np[slots], scales_np[slots] = new_d, new_s
    np.testing.assert_array_equal(data.cpu().numpy(), data_np)
    np.testing.assert_array_equal(scales.cpu().numpy(), scales_np)
