"""Python binding of libmlaq (paged MLA decode over FP8 / NVFP4 latent KV on MI355X).

Argument marshalling only: every step of decode, quantize-on-write and dequantization
runs in the HIP kernels of libmlaq.so, called through its C ABI (include/mlaq.h).
PyTorch provides device memory and the current stream.  Importing this package fails
loudly when the built library is missing; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmlaq.so")

MLAQ_BF16, MLAQ_FP8_E4M3, MLAQ_NVFP4, MLAQ_FP32 = 0, 1, 2, 3
HEAD_DIM, LATENT_DIM, ROPE_DIM = 576, 512, 64
NVFP4_DATA_BYTES, NVFP4_SCALE_BYTES = 288, 36
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_ALIGN", 4: "ERR_UNSUPPORTED", 5: "ERR_WORKSPACE",
          6: "ERR_LAUNCH", 7: "ERR_VALUE"}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python quantized_kv_paged_amd/build.py` "
                      "(or __graft_entry__.build()); there is no fallback implementation")


class DecodeParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("pool_tokens", ctypes.c_int64), ("max_kv_len", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class ExtendParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("pool_tokens", ctypes.c_int64), ("num_q", ctypes.c_int32), ("max_prefix_len", ctypes.c_int32),
                ("max_chunk_len", ctypes.c_int32), ("num_splits", ctypes.c_int32), ("sm_scale", ctypes.c_float)]


_lib = ctypes.CDLL(LIB_PATH)
_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_pp = ctypes.POINTER(DecodeParams)
_ep = ctypes.POINTER(ExtendParams)
_SIGS = {
    "mlaq_decode_num_splits": ([_pp, ctypes.c_int], _i32),
    "mlaq_decode_workspace_bytes": ([_pp], _sz),
    "mlaq_decode_format_workspace_bytes": ([_pp, ctypes.c_int], _sz),
    "mla_decode_fp8": ([_pp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "mla_decode_nvfp4": ([_pp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "mla_decode_bf16": ([_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "mla_decode_nvfp4_noalloc": ([_pp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mlaq_decode_nvfp4_append_workspace_bytes": ([_pp], _sz),
    "mla_decode_nvfp4_append": ([_pp, _vp, _vp, ctypes.c_int, _f32, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _sz, _vp], ctypes.c_int),
    "mlaq_extend_workspace_bytes": ([_ep], _sz),
    "mlaq_extend_num_splits": ([_ep], _i32),
    "mla_extend_nvfp4": ([_ep, _vp, _vp, _vp, _f32, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                         ctypes.c_int),
    "kv_quantize_nvfp4": ([_vp, ctypes.c_int, _f32, _i64, _vp, _vp, _vp, _i64, _f32, _vp], ctypes.c_int),
    "kv_dequantize": ([ctypes.c_int, _vp, _vp, _f32, _vp, _i64, _i64, ctypes.c_int, _vp, _vp], ctypes.c_int),
    "mlaq_set_profile_events": ([_vp, _vp, _vp, _vp], ctypes.c_int),
    "mlaq_read_probe": ([_vp, _i64, _vp, _i32, _vp], ctypes.c_int),
    "mlaq_last_error": ([], ctypes.c_char_p),
    "mlaq_version": ([], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes, _fn.restype = _args, _res

EXPORTS = tuple(_SIGS)


class MlaqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(status: int) -> None:
    if status != 0:
        raise MlaqError(status, _lib.mlaq_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None


def mlaq_set_profile_events(split_start, split_end, merge_start=None, merge_end=None) -> None:
    """Raw hipEvent_t handles (ints or None) recorded at the start and end of the kernels of the
    next decode call on this thread."""
    _check(_lib.mlaq_set_profile_events(split_start, split_end, merge_start, merge_end))


def version() -> str:
    return _lib.mlaq_version().decode()


def last_error() -> str:
    return _lib.mlaq_last_error().decode()


def decode_params(batch, num_heads, page_size, max_kv_len, pool_tokens, sm_scale, num_splits=0) -> DecodeParams:
    return DecodeParams(batch=batch, num_heads=num_heads, page_size=page_size, pool_tokens=pool_tokens,
                        max_kv_len=max_kv_len, num_splits=num_splits, sm_scale=sm_scale)


def mlaq_decode_num_splits(p: DecodeParams, kv_format: int) -> int:
    return _lib.mlaq_decode_num_splits(ctypes.byref(p), kv_format)


def mlaq_decode_workspace_bytes(p: DecodeParams, kv_format: int | None = None) -> int:
    """Workspace bytes of a decode with params p: for one KV format, or (kv_format None) the size
    that serves every decode format."""
    if kv_format is None:
        n = _lib.mlaq_decode_workspace_bytes(ctypes.byref(p))
    else:
        n = _lib.mlaq_decode_format_workspace_bytes(ctypes.byref(p), kv_format)
    if n == ctypes.c_size_t(-1).value:
        raise MlaqError(2, last_error())
    return n


def alloc_workspace(p: DecodeParams, kv_format: int | None = None, device="cuda") -> torch.Tensor | None:
    n = mlaq_decode_workspace_bytes(p, kv_format)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _decode_outputs(q, out, lse, want_lse):
    B, H = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((B, H, LATENT_DIM), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    return out, lse


def _params_for(q, page_size, max_kv_len, pool_tokens, sm_scale, num_splits):
    return decode_params(q.shape[0], q.shape[1], page_size, max_kv_len, pool_tokens, sm_scale, num_splits)


def mla_decode_fp8(q, kv, kv_scale, kv_indptr, kv_indices, kv_lens, page_size, max_kv_len, sm_scale, *,
                   num_splits=0, out=None, lse=None, want_lse=True, workspace=None, stream=None):
    """q: bf16 [B, H, 576]; kv: uint8 e4m3fn [pool, 576]; page table int32 tensors; returns (out, lse)."""
    p = _params_for(q, page_size, max_kv_len, kv.shape[0], sm_scale, num_splits)
    out, lse = _decode_outputs(q, out, lse, want_lse)
    if workspace is None:
        workspace = alloc_workspace(p, MLAQ_FP8_E4M3, q.device)
    _check(_lib.mla_decode_fp8(ctypes.byref(p), _ptr(q), _ptr(kv), kv_scale, _ptr(kv_indptr), _ptr(kv_indices),
                               _ptr(kv_lens), _ptr(out), _ptr(lse), _ptr(workspace),
                               0 if workspace is None else workspace.numel(), _stream(stream)))
    return out, lse


def mla_decode_nvfp4(q, kv_data, kv_scales, global_scale, kv_indptr, kv_indices, kv_lens, page_size, max_kv_len,
                     sm_scale, *, num_splits=0, out=None, lse=None, want_lse=True, workspace=None, stream=None):
    """q: bf16 [B, H, 576]; kv_data uint8 [pool, 288]; kv_scales uint8 [pool, 36]; returns (out, lse)."""
    p = _params_for(q, page_size, max_kv_len, kv_data.shape[0], sm_scale, num_splits)
    out, lse = _decode_outputs(q, out, lse, want_lse)
    if workspace is None:
        workspace = alloc_workspace(p, MLAQ_NVFP4, q.device)
    _check(_lib.mla_decode_nvfp4(ctypes.byref(p), _ptr(q), _ptr(kv_data), _ptr(kv_scales), global_scale,
                                 _ptr(kv_indptr), _ptr(kv_indices), _ptr(kv_lens), _ptr(out), _ptr(lse),
                                 _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream)))
    return out, lse


def mla_decode_nvfp4_noalloc(q, kv_data, kv_scales, global_scale, kv_indptr, kv_indices, kv_lens, page_size,
                             max_kv_len, sm_scale, *, num_splits=0, out=None, lse=None, want_lse=True, stream=None):
    """mla_decode_nvfp4 without a workspace: the split partials live in the library's per-device
    scratch (calls on one device must not overlap).  Returns (out, lse)."""
    p = _params_for(q, page_size, max_kv_len, kv_data.shape[0], sm_scale, num_splits)
    out, lse = _decode_outputs(q, out, lse, want_lse)
    _check(_lib.mla_decode_nvfp4_noalloc(ctypes.byref(p), _ptr(q), _ptr(kv_data), _ptr(kv_scales), global_scale,
                                         _ptr(kv_indptr), _ptr(kv_indices), _ptr(kv_lens), _ptr(out), _ptr(lse),
                                         _stream(stream)))
    return out, lse


def mla_decode_nvfp4_append(q, new_kv, new_kv_format, src_scale, kv_data, kv_scales, global_scale, kv_indptr,
                            kv_indices, kv_lens, page_size, max_kv_len, sm_scale, *, num_splits=0, out=None,
                            lse=None, want_lse=True, workspace=None, stream=None):
    """Fused append-then-attend: quantizes new_kv [B, 576] (e4m3fn bytes or bf16) into the pool row of
    token kv_lens[b] - 1 of each request and decodes over all kv_lens[b] tokens; returns (out, lse)."""
    p = _params_for(q, page_size, max_kv_len, kv_data.shape[0], sm_scale, num_splits)
    out, lse = _decode_outputs(q, out, lse, want_lse)
    if workspace is None:
        n = _lib.mlaq_decode_nvfp4_append_workspace_bytes(ctypes.byref(p))
        if n == ctypes.c_size_t(-1).value:
            raise MlaqError(2, last_error())
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    _check(_lib.mla_decode_nvfp4_append(ctypes.byref(p), _ptr(q), _ptr(new_kv), new_kv_format, src_scale,
                                        _ptr(kv_data), _ptr(kv_scales), global_scale, _ptr(kv_indptr),
                                        _ptr(kv_indices), _ptr(kv_lens), _ptr(out), _ptr(lse), _ptr(workspace),
                                        0 if workspace is None else workspace.numel(), _stream(stream)))
    return out, lse


def mla_decode_bf16(q, kv, kv_indptr, kv_indices, kv_lens, page_size, max_kv_len, sm_scale, *,
                    num_splits=0, out=None, lse=None, want_lse=True, workspace=None, stream=None):
    """q: bf16 [B, H, 576]; kv: bf16 [pool, 576]; returns (out, lse)."""
    p = _params_for(q, page_size, max_kv_len, kv.shape[0], sm_scale, num_splits)
    out, lse = _decode_outputs(q, out, lse, want_lse)
    if workspace is None:
        workspace = alloc_workspace(p, MLAQ_BF16, q.device)
    _check(_lib.mla_decode_bf16(ctypes.byref(p), _ptr(q), _ptr(kv), _ptr(kv_indptr), _ptr(kv_indices),
                                _ptr(kv_lens), _ptr(out), _ptr(lse), _ptr(workspace),
                                0 if workspace is None else workspace.numel(), _stream(stream)))
    return out, lse


def extend_params(batch, num_heads, page_size, pool_tokens, num_q, max_prefix_len, max_chunk_len, sm_scale,
                  num_splits=0) -> ExtendParams:
    return ExtendParams(batch, num_heads, page_size, pool_tokens, num_q, max_prefix_len, max_chunk_len, num_splits,
                        sm_scale)


def mlaq_extend_workspace_bytes(p: ExtendParams) -> int:
    n = _lib.mlaq_extend_workspace_bytes(ctypes.byref(p))
    if n == ctypes.c_size_t(-1).value:
        raise MlaqError(2, last_error())
    return n


def mla_extend_nvfp4(q, qo_indptr, chunk_kv, chunk_scale, kv_data, kv_scales, global_scale, kv_indptr, kv_indices,
                     prefix_lens, slot_mapping, page_size, max_prefix_len, max_chunk_len, sm_scale, *,
                     num_splits=0, out=None, lse=None, want_lse=True, workspace=None, stream=None):
    """Extend (chunked prefill) over an NVFP4 cache: q bf16 [num_q, H, 576], chunk_kv uint8 e4m3fn
    [num_q, 576], qo_indptr / prefix_lens int32, slot_mapping int64 [num_q]; the chunk is written into
    kv_data / kv_scales after the attention.  Returns (out, lse)."""
    B = qo_indptr.shape[0] - 1
    p = extend_params(B, q.shape[1], page_size, kv_data.shape[0], q.shape[0], max_prefix_len, max_chunk_len,
                      sm_scale, num_splits)
    out, lse = _decode_outputs(q, out, lse, want_lse)
    if workspace is None:
        workspace = torch.empty(max(mlaq_extend_workspace_bytes(p), 256), dtype=torch.uint8, device=q.device)
    _check(_lib.mla_extend_nvfp4(ctypes.byref(p), _ptr(q), _ptr(qo_indptr), _ptr(chunk_kv), chunk_scale,
                                 _ptr(kv_data), _ptr(kv_scales), global_scale, _ptr(kv_indptr), _ptr(kv_indices),
                                 _ptr(prefix_lens), _ptr(slot_mapping), _ptr(out), _ptr(lse), _ptr(workspace),
                                 workspace.numel(), _stream(stream)))
    return out, lse


def kv_quantize_nvfp4(src, src_format, src_scale, slot_mapping, kv_data, kv_scales, global_scale, *, stream=None):
    """src: uint8 e4m3fn or bf16 [n, 576]; slot_mapping int64 [n]; writes kv_data / kv_scales rows in place."""
    n = src.shape[0]
    _check(_lib.kv_quantize_nvfp4(_ptr(src), src_format, src_scale, n, _ptr(slot_mapping), _ptr(kv_data),
                                  _ptr(kv_scales), kv_data.shape[0], global_scale, _stream(stream)))


def kv_dequantize(src_format, kv_data, kv_scales, scale, dst_format, *, rows=None, num_rows=None, dst=None,
                  stream=None):
    """Dequantize pool rows (all rows when rows is None) into dst [num_rows, 576]."""
    if num_rows is None:
        num_rows = rows.shape[0] if rows is not None else kv_data.shape[0]
    if dst is None:
        dt = {MLAQ_BF16: torch.bfloat16, MLAQ_FP32: torch.float32, MLAQ_FP8_E4M3: torch.uint8}[dst_format]
        dst = torch.empty((num_rows, HEAD_DIM), dtype=dt, device=kv_data.device)
    _check(_lib.kv_dequantize(src_format, _ptr(kv_data), _ptr(kv_scales), scale, _ptr(rows), num_rows,
                              kv_data.shape[0], dst_format, _ptr(dst), _stream(stream)))
    return dst


def read_probe(buf, num_blocks=2048, partials=None, stream=None):
    """Streaming read of the device tensor buf (a measurement aid).  Returns the uint8
    [num_blocks, 16] per-block XORs of the 16-byte words read."""
    if partials is None:
        partials = torch.empty((num_blocks, 16), dtype=torch.uint8, device=buf.device)
    _check(_lib.mlaq_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(partials), num_blocks,
                                _stream(stream)))
    return partials


__all__ = ["mla_decode_fp8", "mla_decode_nvfp4", "mla_decode_nvfp4_noalloc", "mla_decode_nvfp4_append", "mla_decode_bf16", "mla_extend_nvfp4",
           "extend_params", "mlaq_extend_workspace_bytes", "kv_quantize_nvfp4", "kv_dequantize",
           "mlaq_decode_num_splits", "mlaq_decode_workspace_bytes", "decode_params", "alloc_workspace",
           "read_probe", "MlaqError", "version", "last_error", "EXPORTS", "LIB_PATH"]
