"""Seeded decode cases shared by the GPU parity tests.

Inputs come from synth.py; NVFP4 pools are quantized by the oracle's encoder, so every
byte the oracle reads was produced on the CPU by the generator or by the oracle itself.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import synth
from oracle import attention, codecs
from oracle import nvfp4 as onv

TOL_MAX_ABS = 1e-2
TOL_REL_L2 = 5e-3
TOL_LSE = 2e-3


@dataclasses.dataclass
class Case:
    fmt: str                  # fp8 | nvfp4 | bf16
    w: synth.Workload
    pt: synth.PageTable
    q_bits: np.ndarray        # uint16 [B, H, 576]
    fp8_pool: np.ndarray      # uint8 [pool, 576] (source / FP8 pool)
    nv_data: np.ndarray | None = None
    nv_scales: np.ndarray | None = None
    bf16_pool: np.ndarray | None = None
    scale: float = 1.0        # kv_scale (fp8) or global scale (nvfp4)
    max_kv_len: int = 0


def build_case(fmt: str, lens, page_size: int, seed: int, heads: int = 16, extra_pages: int = 3,
               sigma: float = 1.0, outlier_p: float = 0.0, g: float | None = 1.0, kv_scale: float = 1.0) -> Case:
    lens = np.asarray(lens, dtype=np.int32)
    pages = int(sum(-(-int(L) // page_size) for L in lens))
    pool_tokens = (pages + extra_pages) * page_size
    src_fmt = "nvfp4" if fmt == "nvfp4" else "fp8"
    w = synth.Workload("case", src_fmt, len(lens), heads, int(lens.max(initial=0)), page_size, pool_tokens, sigma,
                       outlier_p, 8.0, synth.SM_SCALE, seed)
    pt = synth.page_table(w, kv_lens=lens)
    pool = synth.build_fp8_pool(w, pt)
    c = Case(fmt, w, pt, synth.q_bits(seed, len(lens), heads), pool, max_kv_len=int(lens.max(initial=0)))
    if fmt == "nvfp4":
        x = onv.fp8_rows_to_f32(pool, 1.0)
        if g is None:
            g = onv.calibrated_global_scale(float(np.abs(x).max()))
        c.nv_data, c.nv_scales = onv.quantize_rows(x, g)
        c.scale = g
    elif fmt == "bf16":
        c.bf16_pool = codecs.bf16_round_bits(onv.fp8_rows_to_f32(pool, 1.0))
    else:
        c.scale = kv_scale
    return c


def dequant_rows(c: Case, rows: np.ndarray) -> np.ndarray:
    if c.fmt == "fp8":
        return onv.dequant_fp8_f64(c.fp8_pool[rows], c.scale)
    if c.fmt == "nvfp4":
        return onv.dequant_nvfp4_f64(c.nv_data[rows], c.nv_scales[rows], c.scale)
    return codecs.bf16_bits_to_f64(c.bf16_pool[rows])


def oracle_decode(c: Case, requests=None) -> tuple[np.ndarray, np.ndarray]:
    B, H = c.q_bits.shape[:2]
    requests = range(B) if requests is None else requests
    out = np.zeros((B, H, 512))
    lse = np.zeros((B, H))
    q = codecs.bf16_bits_to_f64(c.q_bits)
    for b in requests:
        L = int(c.pt.kv_lens[b])
        rows = attention.gather_rows(c.pt.kv_indptr, c.pt.kv_indices, c.w.page_size, b, L)
        x = dequant_rows(c, rows)
        out[b], lse[b] = attention.decode_dense(q[b], x, c.w.sm_scale)
    return out, lse


class Device:
    """Device copies of a case."""

    def __init__(self, c: Case, dev="cuda"):
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.q = t(c.q_bits.view(np.int16)).view(torch.bfloat16)
        self.indptr, self.indices, self.lens = t(c.pt.kv_indptr), t(c.pt.kv_indices), t(c.pt.kv_lens)
        self.fp8 = t(c.fp8_pool) if c.fmt == "fp8" else None
        self.nv_data = t(c.nv_data) if c.nv_data is not None else None
        self.nv_scales = t(c.nv_scales) if c.nv_scales is not None else None
        self.bf16 = t(c.bf16_pool.view(np.int16)).view(torch.bfloat16) if c.bf16_pool is not None else None


def gpu_decode(c: Case, d: Device, num_splits: int = 0, want_lse: bool = True, max_kv_len=None):
    import quantized_kv_paged_amd as qk
    mk = c.max_kv_len if max_kv_len is None else max_kv_len
    args = (d.indptr, d.indices, d.lens, c.w.page_size, mk, c.w.sm_scale)
    if c.fmt == "fp8":
        out, lse = qk.mla_decode_fp8(d.q, d.fp8, c.scale, *args, num_splits=num_splits, want_lse=want_lse)
    elif c.fmt == "nvfp4":
        out, lse = qk.mla_decode_nvfp4(d.q, d.nv_data, d.nv_scales, c.scale, *args, num_splits=num_splits,
                                       want_lse=want_lse)
    else:
        out, lse = qk.mla_decode_bf16(d.q, d.bf16, *args, num_splits=num_splits, want_lse=want_lse)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), (lse.double().cpu().numpy() if lse is not None else None)


def errors(out: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    diff = out - ref
    return float(np.abs(diff).max(initial=0.0)), float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30))


def assert_parity(out, lse, ref_out, ref_lse, requests=None, tag=""):
    if requests is not None:
        out, lse, ref_out, ref_lse = out[requests], lse[requests], ref_out[requests], ref_lse[requests]
    mx, rel = errors(out, ref_out)
    assert mx <= TOL_MAX_ABS and rel <= TOL_REL_L2, f"{tag} max-abs {mx:.3g} rel-L2 {rel:.3g}"
    if lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(lse)), tag
        assert np.array_equal(ref_lse[~fin], lse[~fin]), tag
        assert np.abs(lse[fin] - ref_lse[fin]).max(initial=0.0) <= TOL_LSE, tag
    return mx, rel
