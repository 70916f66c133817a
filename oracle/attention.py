"""Paged gather and fp64 softmax attention for single-token MLA decode (oracle).

Test infrastructure (see oracle/__init__.py).

Sources ("The Smoking Gun: Tracing the FP8-to-BF16 KV Cache Cast", sections "Message
Overview" and "The Investigation Leading to This Message"):
  * the decode plan takes CSR page-table arrays (qo/kv indptr, kv indices, kv lengths),
    the head count, kv_lora_rank, qk_rope_head_dim, a page size, causal = False and
    sm_scale;
  * the pool is [495552, 1, 576]: one shared latent KV head, 576 = kv_lora_rank 512 +
    qk_rope_head_dim 64.
Readings (listed in the design doc): scores use all 576 dims; the value is the first 512
(latent) dims of the same row; no mask, window, sink or cap; lse in natural log; an
empty context gives out = 0, lse = -inf; NaN propagates.
"""
from __future__ import annotations

from typing import Callable, Iterable

import numpy as np

D = 576
DV = 512


def gather_rows(kv_indptr: np.ndarray, kv_indices: np.ndarray, page_size: int, b: int, kv_len: int,
                start: int = 0, count: int | None = None) -> np.ndarray:
    """Pool rows of logical tokens j in [start, start+count) of request b:
    row(b, j) = kv_indices[kv_indptr[b] + j // P] * P + j % P."""
    if count is None:
        count = kv_len - start
    j = np.arange(start, start + count, dtype=np.int64)
    page = np.asarray(kv_indices, dtype=np.int64)[int(kv_indptr[b]) + j // page_size]
    return page * page_size + j % page_size


def decode_head_block(q: np.ndarray, chunks: Callable[[], Iterable[np.ndarray]], sm_scale: float
                      ) -> tuple[np.ndarray, np.ndarray]:
    """Attention of the H query rows q (fp64 [H, 576]) over the dequantized KV rows of
    one request, given as a re-iterable source of fp64 [n, 576] chunks in token order.

    s_j = sm_scale * q . x_j ; out = sum_j softmax(s)_j * x_j[:512] ; lse = log sum_j exp(s_j).
    Two passes (scores first, then the weighted sum) so that any context length fits.
    """
    q = np.asarray(q, dtype=np.float64)
    H = q.shape[0]
    scores = []
    for x in chunks():
        scores.append(sm_scale * (x @ q.T))          # [n, H]
    if not scores or sum(s.shape[0] for s in scores) == 0:
        return np.zeros((H, DV)), np.full(H, -np.inf)
    s = np.concatenate(scores, axis=0)                # [L, H]
    m = s.max(axis=0)                                 # propagates NaN
    w = np.exp(s - m)                                 # [L, H]
    z = w.sum(axis=0)
    out = np.zeros((H, DV))
    pos = 0
    for x in chunks():
        n = x.shape[0]
        out += w[pos:pos + n].T @ x[:, :DV]
        pos += n
    return out / z[:, None], m + np.log(z)


def decode_dense(q: np.ndarray, x: np.ndarray, sm_scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Same as decode_head_block for a context held as one fp64 array x [L, 576]."""
    return decode_head_block(q, lambda: [x], sm_scale)


def merge_partials(o: np.ndarray, lse: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Combine normalized partial outputs o_s [S, H, DV] with their log-sum-exps lse_s [S, H]
    over disjoint token sets: out = sum_s exp(lse_s - LSE) o_s, LSE = log sum_s exp(lse_s)."""
    mx = np.max(lse, axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lse - safe)
    tot = w.sum(axis=0)
    out = np.einsum("sh,shd->hd", w, o) / np.where(tot > 0, tot, 1.0)[:, None]
    return out, np.where(tot > 0, safe + np.log(tot), -np.inf)
