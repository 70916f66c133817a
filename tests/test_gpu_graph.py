"""The calls allocate nothing, never synchronise and never read device memory on the host, so
they can be captured in a HIP graph.  Each test captures one call, then replays the graph
several times with eager work in between (new query values written in place, synchronised),
and checks every replay bit for bit against an eager call on the same inputs."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from cases import build_case

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _new_q(q, rep):
    bits = synth.q_bits(1000 + rep, q.shape[0], q.shape[1])
    q.copy_(_t(bits.view(np.int16)).view(torch.bfloat16))


def _replay_and_check(q, graph, out_g, lse_g, eager):
    for rep in range(REPLAYS):
        _new_q(q, rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out_e, lse_e = eager()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: out differs from the eager call"
        assert torch.equal(lse_g, lse_e), f"replay {rep}: lse differs from the eager call"
        assert torch.isfinite(out_g).all()


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_decode_replays_in_a_graph(fmt):
    import quantized_kv_paged_amd as qk
    c = build_case(fmt, [700, 1, 3000, 64], 64, seed=81)
    pt = c.pt
    q = _t(c.q_bits.view(np.int16)).view(torch.bfloat16)
    indptr, indices, lens = _t(pt.kv_indptr), _t(pt.kv_indices), _t(pt.kv_lens)
    B, H = q.shape[0], q.shape[1]
    out_g = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse_g = torch.empty((B, H), dtype=torch.float32, device="cuda")
    if fmt == "fp8":
        kv = _t(c.fp8_pool)
        call = lambda out, lse, ws: qk.mla_decode_fp8(q, kv, c.scale, indptr, indices, lens, 64, c.max_kv_len,
                                                      c.w.sm_scale, out=out, lse=lse, workspace=ws)
        fcode = qk.MLAQ_FP8_E4M3
    else:
        data, scales = _t(c.nv_data), _t(c.nv_scales)
        call = lambda out, lse, ws: qk.mla_decode_nvfp4(q, data, scales, c.scale, indptr, indices, lens, 64,
                                                        c.max_kv_len, c.w.sm_scale, out=out, lse=lse, workspace=ws)
        fcode = qk.MLAQ_NVFP4
    p = qk.decode_params(B, H, 64, c.max_kv_len, c.fp8_pool.shape[0], c.w.sm_scale)
    assert qk.mlaq_decode_num_splits(p, fcode) > 1          # the merge kernel is captured too
    ws_g = qk.alloc_workspace(p, fcode)
    ws_e = qk.alloc_workspace(p, fcode)
    call(out_g, lse_g, ws_g)                                  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out_g, lse_g, ws_g)

    def eager():
        return call(None, None, ws_e)
    _replay_and_check(q, graph, out_g, lse_g, eager)


def test_fused_append_replays_in_a_graph():
    """The append call also writes the new row into the pool; every replay writes the same
    bytes, so the eager call after it sees the same pool."""
    import quantized_kv_paged_amd as qk
    c = build_case("nvfp4", [300, 65, 1200], 64, seed=83)
    pt = c.pt
    q = _t(c.q_bits.view(np.int16)).view(torch.bfloat16)
    indptr, indices, lens = _t(pt.kv_indptr), _t(pt.kv_indices), _t(pt.kv_lens)
    data, scales = _t(c.nv_data), _t(c.nv_scales)
    B, H = q.shape[0], q.shape[1]
    new_rows = _t(synth.to_fp8_bytes(synth.new_token_rows(83, B)))
    out_g = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse_g = torch.empty((B, H), dtype=torch.float32, device="cuda")
    p = qk.decode_params(B, H, 64, c.max_kv_len, data.shape[0], c.w.sm_scale)
    n = qk._lib.mlaq_decode_nvfp4_append_workspace_bytes(ctypes.byref(p))
    ws_g = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws_e = torch.empty(n, dtype=torch.uint8, device="cuda")

    def call(out, lse, ws):
        return qk.mla_decode_nvfp4_append(q, new_rows, qk.MLAQ_FP8_E4M3, 1.0, data, scales, c.scale, indptr, indices,
                                          lens, 64, c.max_kv_len, c.w.sm_scale, out=out, lse=lse, workspace=ws)
    call(out_g, lse_g, ws_g)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out_g, lse_g, ws_g)
    _replay_and_check(q, graph, out_g, lse_g, lambda: call(None, None, ws_e))


def test_extend_replays_in_a_graph():
    """Extend: workspace gather, per-token views, tiled attention with KV splits and merge, and
    the chunk's write into the cache, all in one captured call."""
    import quantized_kv_paged_amd as qk
    from oracle import attention
    prefix, chunk = np.array([0, 700, 130], np.int32), np.array([40, 64, 9], np.int32)
    c = build_case("nvfp4", prefix + chunk, 64, seed=85)
    qo = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    nq = int(qo[-1])
    q = _t(synth.q_bits(85, nq, 16).view(np.int16)).view(torch.bfloat16)
    ckv = _t(synth.to_fp8_bytes(synth.extend_chunk_rows(85, nq)))
    slots = _t(np.concatenate([attention.gather_rows(c.pt.kv_indptr, c.pt.kv_indices, 64, b,
                                                     int(prefix[b] + chunk[b]))[prefix[b]:]
                               for b in range(len(prefix))]).astype(np.int64))
    data, scales = _t(c.nv_data), _t(c.nv_scales)
    indptr, indices, pl, qo_t = _t(c.pt.kv_indptr), _t(c.pt.kv_indices), _t(prefix), _t(qo)
    mp, mc = int(prefix.max()), int(chunk.max())
    p = qk.extend_params(len(prefix), 16, 64, data.shape[0], nq, mp, mc, c.w.sm_scale, 3)
    assert qk._lib.mlaq_extend_num_splits(ctypes.byref(p)) == 3
    n = qk.mlaq_extend_workspace_bytes(p)
    ws_g = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws_e = torch.empty(n, dtype=torch.uint8, device="cuda")
    out_g = torch.empty((nq, 16, 512), dtype=torch.float32, device="cuda")
    lse_g = torch.empty((nq, 16), dtype=torch.float32, device="cuda")

    def call(out, lse, ws):
        return qk.mla_extend_nvfp4(q, qo_t, ckv, 1.0, data, scales, c.scale, indptr, indices, pl, slots, 64, mp, mc,
                                   c.w.sm_scale, num_splits=3, out=out, lse=lse, workspace=ws)
    call(out_g, lse_g, ws_g)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out_g, lse_g, ws_g)
    _replay_and_check(q, graph, out_g, lse_g, lambda: call(None, None, ws_e))
