"""Extend (chunked prefill) over an NVFP4 cache (oracle).

Test infrastructure (see oracle/__init__.py).

Source: the NVFP4 article (aitop.news), section "SGLang implementation: three attention
paths", item 2: for a chunk of new tokens, the cached prefix is gathered and dequantized into
an FP8 workspace shared across layers, the chunk's own KV is concatenated to it, attention
runs over the concatenation, and afterwards the chunk is quantized into the NVFP4 cache.

Readings (listed in the design doc):
  * the workspace holds e4m3fn bytes; a prefix value is e4m3(fl32(x / chunk_scale)) with
    x = fl32(fl32(e2m1 * e4m3) * g) its fp32 dequantized value (O-6), so prefix and chunk rows
    share the chunk's per-tensor scale (with chunk_scale 1.0 this is the pages' path);
  * attention is the decode attention (O-8) of each chunk token's query rows over the
    workspace rows it may see: the prefix, the chunk tokens before it and itself (causal
    inside the chunk, as a prefill is);
  * the chunk is written to the cache with the write path (O-5) from its FP8 rows.
"""
from __future__ import annotations

import numpy as np

from . import attention, codecs
from . import nvfp4 as onv


def workspace_prefix(data: np.ndarray, scales: np.ndarray, g: float, chunk_scale: float) -> np.ndarray:
    """e4m3fn bytes [n, 576] of the prefix rows (NVFP4 codes + scales) in the chunk's scale domain."""
    x = onv.dequant_nvfp4_f32(data, scales, g)                     # fp32, exact products times g
    y = (x / np.float32(chunk_scale)).astype(np.float32)           # one fp32 division per value
    return onv.e4m3_encode_array(y)


def workspace_values(ws_bytes: np.ndarray, chunk_scale: float) -> np.ndarray:
    """fp64 values of workspace bytes: e4m3 * chunk_scale."""
    return onv.dequant_fp8_f64(ws_bytes, chunk_scale)


def extend_request(q: np.ndarray, ws_bytes: np.ndarray, prefix_len: int, chunk_scale: float, sm_scale: float
                   ) -> tuple[np.ndarray, np.ndarray]:
    """q: fp64 [C, H, 576] (the chunk's query rows); ws_bytes: e4m3fn [prefix_len + C, 576]
    (prefix then chunk).  Chunk token i attends workspace rows 0 .. prefix_len + i.
    Returns out [C, H, 512], lse [C, H]."""
    C, H = q.shape[0], q.shape[1]
    x = workspace_values(ws_bytes, chunk_scale)
    out = np.zeros((C, H, attention.DV))
    lse = np.zeros((C, H))
    for i in range(C):
        out[i], lse[i] = attention.decode_dense(q[i], x[:prefix_len + i + 1], sm_scale)
    return out, lse


def q_from_bits(bits: np.ndarray) -> np.ndarray:
    return codecs.bf16_bits_to_f64(bits)
