"""Seeded synthetic inputs for paged MLA decode over a low-precision latent KV pool.

This module is shared by the tests, the benchmark and the CPU oracle.  It draws
random numbers and lays them out (queries, latent KV rows, page tables, slot
mappings); it holds none of the decode or NVFP4 arithmetic.  Casting the drawn
fp32 values to the storage types (bf16 for queries, FP8 e4m3fn for the source KV)
uses torch's CPU casts, i.e. library routines, so that neither the oracle nor the
GPU library supplies its own inputs.

Workload shapes follow the pages:
  * latent row = 576 dims: kv_lora_rank 512 followed by qk_rope_head_dim 64
    ("The Smoking Gun: Tracing the FP8-to-BF16 KV Cache Cast", section "The
    Investigation Leading to This Message": pool [495552, 1, 576]).
  * context lengths 32K / 160K / 1M with 44 / 10 / 1-2 requests (aitop.news
    NVFP4 KV cache article, performance section).

Every stream is a numpy PCG64 generator keyed by a tuple, so any chunk of rows can be
regenerated independently (the oracle re-draws only the rows it needs):
  q                    -> (seed, 0)
  KV rows of request b -> (seed, 1, b, c) for chunk c of CHUNK rows, outlier mask (seed, 2, b, c)
  page permutation     -> (seed, 3)
  write-path source    -> (seed, 4)
  appended decode rows -> (seed, 6)
  extend chunk rows    -> (seed, 7)
  rows owned by no request (filler) -> (seed, 5, c)
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

D_LATENT = 512
D_ROPE = 64
D = D_LATENT + D_ROPE
CHUNK = 65536


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    fmt: str            # "fp8" or "nvfp4"
    batch: int
    heads: int
    kv_len: int
    page_size: int
    pool_tokens: int    # rows in the pool (multiple of page_size)
    sigma: float        # std of the source KV values
    outlier_p: float    # per-element probability of an outlier
    outlier_x: float    # outlier multiplier
    sm_scale: float
    seed: int
    write_tokens: int = 0   # tokens quantized on write (NVFP4 only)
    write_pages: int = 0    # spare pool pages that receive them

    @property
    def pool_pages(self) -> int:
        return self.pool_tokens // self.page_size

    @property
    def pages_per_req(self) -> int:
        return -(-self.kv_len // self.page_size)


SM_SCALE = float(1.0 / np.sqrt(192.0))

# The five workloads (tiny FP8; FP8 32K with the pool of the pages; NVFP4 at 32K / 160K / 1M).
WORKLOADS = {
    "tiny_fp8": Workload("tiny_fp8", "fp8", 1, 16, 512, 16, 1024, 1.0, 0.0, 1.0, SM_SCALE, 1),
    "fp8_32k": Workload("fp8_32k", "fp8", 8, 16, 32768, 64, 495552, 0.5, 0.0, 1.0, SM_SCALE, 2),
    "nvfp4_32k": Workload("nvfp4_32k", "nvfp4", 44, 16, 32768, 64, 44 * 32768, 1.0, 0.01, 8.0, SM_SCALE, 3),
    "nvfp4_160k": Workload("nvfp4_160k", "nvfp4", 10, 16, 163840, 64, 10 * 163840, 1.0, 0.01, 8.0, SM_SCALE, 4),
    "nvfp4_1m": Workload("nvfp4_1m", "nvfp4", 2, 16, 1048576, 64, 2 * 1048576 + 128 * 64, 1.0, 0.01, 8.0,
                         SM_SCALE, 5, write_tokens=8192, write_pages=128),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(key)))


def q_fp32(seed: int, batch: int, heads: int) -> np.ndarray:
    """Absorbed latent queries, standard normal, fp32 [batch, heads, 576]."""
    return _rng(seed, 0).standard_normal((batch, heads, D), dtype=np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (torch's round-to-nearest-even cast), returned as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_fp32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_fp8_bytes(x: np.ndarray) -> np.ndarray:
    """fp32 -> FP8 e4m3fn bytes with torch's cast (values clamped to the finite range first)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def q_bits(seed: int, batch: int, heads: int) -> np.ndarray:
    """bf16 query bits [batch, heads, 576]."""
    return to_bf16_bits(q_fp32(seed, batch, heads))


def _chunk_fp32(w: Workload, b: int, c: int) -> np.ndarray:
    x = _rng(w.seed, 1, b, c).standard_normal((CHUNK, D), dtype=np.float32)
    if w.sigma != 1.0:
        x *= np.float32(w.sigma)
    if w.outlier_p > 0.0:
        mask = _rng(w.seed, 2, b, c).random((CHUNK, D), dtype=np.float32) < w.outlier_p
        x[mask] *= np.float32(w.outlier_x)
    return x


def kv_fp32(w: Workload, b: int, start: int, count: int) -> np.ndarray:
    """Logical KV source rows [start, start+count) of request b, fp32 [count, 576]."""
    out = np.empty((count, D), dtype=np.float32)
    pos = 0
    while pos < count:
        t = start + pos
        c, off = divmod(t, CHUNK)
        n = min(CHUNK - off, count - pos)
        out[pos:pos + n] = _chunk_fp32(w, b, c)[off:off + n]
        pos += n
    return out


def kv_fp8(w: Workload, b: int, start: int, count: int) -> np.ndarray:
    """Logical KV rows of request b as FP8 e4m3fn bytes [count, 576].

    FP8 workloads cast the fp32 source directly; NVFP4 workloads follow the write path
    of the pages (bf16 activations stored as FP8 before NVFP4 quantization), so their
    source is rounded to bf16 first.
    """
    x = kv_fp32(w, b, start, count)
    if w.fmt == "nvfp4":
        x = bf16_bits_to_fp32(to_bf16_bits(x))
    return to_fp8_bytes(x)


def filler_fp8(w: Workload, page: int) -> np.ndarray:
    """FP8 rows for a pool page that no request owns."""
    x = _rng(w.seed, 5, page).standard_normal((w.page_size, D), dtype=np.float32) * np.float32(w.sigma)
    return to_fp8_bytes(x)


@dataclasses.dataclass
class PageTable:
    kv_indptr: np.ndarray    # int32 [B+1]
    kv_indices: np.ndarray   # int32 [sum pages]
    kv_lens: np.ndarray      # int32 [B]
    write_pages: np.ndarray  # int32 [write_pages] spare pages for the write path
    free_pages: np.ndarray   # int32 pages owned by nobody


def page_table(w: Workload, kv_lens: np.ndarray | None = None) -> PageTable:
    """Requests take consecutive blocks of a seeded permutation of the pool pages; the
    write path takes the next `write_pages` pages of the permutation."""
    perm = _rng(w.seed, 3).permutation(w.pool_pages).astype(np.int32)
    lens = np.full(w.batch, w.kv_len, dtype=np.int32) if kv_lens is None else np.asarray(kv_lens, np.int32)
    ppr = -(-lens.astype(np.int64) // w.page_size)
    indptr = np.zeros(w.batch + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(ppr)
    used = int(indptr[-1])
    if used + w.write_pages > w.pool_pages:
        raise ValueError("pool too small for the page table")
    return PageTable(indptr, perm[:used].copy(), lens, perm[used:used + w.write_pages].copy(),
                     perm[used + w.write_pages:].copy())


def slot_mapping(w: Workload, pt: PageTable) -> np.ndarray:
    """Destination pool rows (int64) of the write-path tokens: token t -> page t // P of the spare pages."""
    t = np.arange(w.write_tokens, dtype=np.int64)
    return pt.write_pages[t // w.page_size].astype(np.int64) * w.page_size + t % w.page_size


def write_source_fp8(w: Workload) -> np.ndarray:
    """Write-path chunk: bf16-rounded N(0,1) tokens cast to FP8 e4m3fn bytes [write_tokens, 576]."""
    x = _rng(w.seed, 4).standard_normal((w.write_tokens, D), dtype=np.float32)
    return to_fp8_bytes(bf16_bits_to_fp32(to_bf16_bits(x)))


def new_token_rows(seed: int, batch: int) -> np.ndarray:
    """Source rows of the tokens appended by a decode step: N(0,1) fp32 [batch, 576]."""
    return _rng(seed, 6).standard_normal((batch, D), dtype=np.float32)


def extend_chunk_rows(seed: int, n: int) -> np.ndarray:
    """KV rows of an extend chunk (n tokens over all requests): N(0,1) fp32 [n, 576]."""
    return _rng(seed, 7).standard_normal((n, D), dtype=np.float32)


def build_fp8_pool(w: Workload, pt: PageTable, threads: int = 16) -> np.ndarray:
    """Whole FP8 pool [pool_tokens, 576] uint8 in host memory: request rows scattered by the
    page table, free pages filled from the filler stream, write pages zero."""
    pool = np.zeros((w.pool_tokens, D), dtype=np.uint8)
    P = w.page_size

    def fill_chunk(task) -> None:
        b, c0 = task
        n = min(CHUNK, int(pt.kv_lens[b]) - c0)
        pages = pt.kv_indices[pt.kv_indptr[b]:pt.kv_indptr[b + 1]]
        rows = kv_fp8(w, b, c0, n)
        j = np.arange(c0, c0 + n)
        pool[pages[j // P].astype(np.int64) * P + j % P] = rows

    tasks = [(b, c0) for b in range(w.batch) for c0 in range(0, int(pt.kv_lens[b]), CHUNK)]
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill_chunk, tasks))
        list(ex.map(lambda p: pool.__setitem__(slice(int(p) * P, int(p) * P + P), filler_fp8(w, int(p))),
                    pt.free_pages))
    return pool


def build_bf16_source_pool(w: Workload, pt: PageTable, threads: int = 16) -> np.ndarray:
    """The requests' KV source rows rounded to bf16 (torch's cast), as uint16 bits [pool_tokens, 576],
    at the same pool rows as build_fp8_pool; rows no request owns are zero.  For NVFP4 workloads this
    is the bf16 tensor the FP8 rows were cast from."""
    pool = np.zeros((w.pool_tokens, D), dtype=np.uint16)
    P = w.page_size

    def fill_chunk(task) -> None:
        b, c0 = task
        n = min(CHUNK, int(pt.kv_lens[b]) - c0)
        pages = pt.kv_indices[pt.kv_indptr[b]:pt.kv_indptr[b + 1]]
        j = np.arange(c0, c0 + n)
        pool[pages[j // P].astype(np.int64) * P + j % P] = to_bf16_bits(kv_fp32(w, b, c0, n))

    tasks = [(b, c0) for b in range(w.batch) for c0 in range(0, int(pt.kv_lens[b]), CHUNK)]
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill_chunk, tasks))
    return pool
