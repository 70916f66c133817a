"""Full-size workloads, in the launch configuration the benchmark times (automatic split plan),
with sampled requests checked against the fp64 oracle (all 16 heads x 512 dims of each
sampled request).  Pools are generated on the host (FP8 from synth.py, NVFP4 by the
oracle's encoder), so nothing the oracle reads comes from the GPU path."""
import numpy as np
import pytest
import torch

import synth
from cases import TOL_LSE, TOL_MAX_ABS, TOL_REL_L2, errors
from oracle import attention, codecs
from oracle import nvfp4 as onv

pytestmark = pytest.mark.gpu
CH = 65536


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _oracle_request(w, pt, b, dequant):
    """fp64 oracle for request b, dequantizing its rows chunk by chunk."""
    L = int(pt.kv_lens[b])
    q = codecs.bf16_bits_to_f64(synth.q_bits(w.seed, w.batch, w.heads))[b]

    def chunks():
        for c0 in range(0, L, CH):
            rows = attention.gather_rows(pt.kv_indptr, pt.kv_indices, w.page_size, b, L, c0, min(CH, L - c0))
            yield dequant(rows)
    return attention.decode_head_block(q, chunks, w.sm_scale)


def _check(out, lse, ref_out, ref_lse, tag):
    mx, rel = errors(out, ref_out)
    dl = float(np.abs(lse - ref_lse).max())
    print(f"[{tag}] max-abs {mx:.2e} rel-L2 {rel:.2e} lse {dl:.2e}", flush=True)
    assert mx <= TOL_MAX_ABS and rel <= TOL_REL_L2 and dl <= TOL_LSE, tag


def _setup(name):
    import quantized_kv_paged_amd as qk
    w = synth.WORKLOADS[name]
    pt = synth.page_table(w)
    host = synth.build_fp8_pool(w, pt)
    d = dict(q=_dev(synth.q_bits(w.seed, w.batch, w.heads).view(np.int16)).view(torch.bfloat16),
             indptr=_dev(pt.kv_indptr), indices=_dev(pt.kv_indices), lens=_dev(pt.kv_lens))
    p = qk.decode_params(w.batch, w.heads, w.page_size, w.kv_len, w.pool_tokens, w.sm_scale)
    fmt = qk.MLAQ_NVFP4 if w.fmt == "nvfp4" else qk.MLAQ_FP8_E4M3
    print(f"[{name}] pool {host.shape}, {qk.mlaq_decode_num_splits(p, fmt)} splits", flush=True)
    return qk, w, pt, host, d


def _decode_nvfp4(qk, w, d, data, scales, g):
    out, lse = qk.mla_decode_nvfp4(d["q"], _dev(data), _dev(scales), g, d["indptr"], d["indices"], d["lens"],
                                   w.page_size, w.kv_len, w.sm_scale)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def test_fp8_32k_pool_of_the_pages():
    qk, w, pt, host, d = _setup("fp8_32k")
    out, lse = qk.mla_decode_fp8(d["q"], _dev(host), 1.0, d["indptr"], d["indices"], d["lens"], w.page_size,
                                 w.kv_len, w.sm_scale)
    torch.cuda.synchronize()
    out, lse = out.double().cpu().numpy(), lse.double().cpu().numpy()
    for b in (0, 5):
        ro, rl = _oracle_request(w, pt, b, lambda rows: onv.dequant_fp8_f64(host[rows], 1.0))
        _check(out[b], lse[b], ro, rl, f"fp8_32k b={b}")


@pytest.mark.parametrize("calibrated", [False, True])
def test_nvfp4_32k(calibrated):
    qk, w, pt, host, d = _setup("nvfp4_32k")
    x = onv.fp8_rows_to_f32(host, 1.0)
    g = onv.calibrated_global_scale(float(np.abs(x).max())) if calibrated else 1.0
    data, scales = onv.quantize_rows(x, g)
    del x
    out, lse = _decode_nvfp4(qk, w, d, data, scales, g)
    for b in ((0, 43) if not calibrated else (17,)):
        ro, rl = _oracle_request(w, pt, b, lambda rows: onv.dequant_nvfp4_f64(data[rows], scales[rows], g))
        _check(out[b], lse[b], ro, rl, f"nvfp4_32k g={g} b={b}")


def test_nvfp4_160k_and_fp8_same_batch():
    qk, w, pt, host, d = _setup("nvfp4_160k")
    data, scales = onv.quantize_fp8_rows(host, 1.0, 1.0)
    out, lse = _decode_nvfp4(qk, w, d, data, scales, 1.0)
    b = 9
    ro, rl = _oracle_request(w, pt, b, lambda rows: onv.dequant_nvfp4_f64(data[rows], scales[rows], 1.0))
    _check(out[b], lse[b], ro, rl, f"nvfp4_160k b={b}")
    out8, lse8 = qk.mla_decode_fp8(d["q"], _dev(host), 1.0, d["indptr"], d["indices"], d["lens"], w.page_size,
                                   w.kv_len, w.sm_scale)
    torch.cuda.synchronize()
    ro, rl = _oracle_request(w, pt, b, lambda rows: onv.dequant_fp8_f64(host[rows], 1.0))
    _check(out8[b].double().cpu().numpy(), lse8[b].double().cpu().numpy(), ro, rl, f"fp8 at 160k b={b}")


def test_nvfp4_1m():
    qk, w, pt, host, d = _setup("nvfp4_1m")
    data, scales = onv.quantize_fp8_rows(host, 1.0, 1.0)
    del host
    out, lse = _decode_nvfp4(qk, w, d, data, scales, 1.0)
    b = 1
    ro, rl = _oracle_request(w, pt, b, lambda rows: onv.dequant_nvfp4_f64(data[rows], scales[rows], 1.0))
    _check(out[b], lse[b], ro, rl, f"nvfp4_1m b={b}")
