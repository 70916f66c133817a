#!/usr/bin/env python3
"""Benchmark of paged MLA decode over FP8 / NVFP4 latent KV on one MI355X.

One step = one decode call over the whole batch: the split-KV kernel (page-table gather,
in-register dequantization, QK^T and PV on MFMA, online softmax, split partials) and the
merge kernel, i.e. one layer of one decode step for every request; in the 1M workload the
step also runs the NVFP4 quantize-on-write of an 8,192-token chunk into scattered pages.
Inputs are synthetic (synth.py) and resident in HBM before any timed region.  Consecutive
steps cycle through several copies of the pool ("layers") at different addresses, so that
the 256 MB Infinity Cache cannot serve a step from the previous one.

Headline (default --workload nvfp4_1m): NVFP4, batch 2 x 16 heads, 1,048,576-token contexts,
page 64, plus the 8,192-token write, the largest of the workloads and the one the NVFP4
article's long-context gain is quoted on.  The same run measures FP8 at the same batch and
context, the write path alone, and (unless --no-extras) the other workloads: fp8_32k (with
NVFP4 at its batch, the whole-pool cast baseline and the gather-then-cast baseline),
nvfp4_32k (with a calibrated global scale and the quantization effect of both scales,
the fused append, extend and initial prefill), nvfp4_160k (with FP8 at its batch).

Prints ONE JSON line.  `value` = KV bytes read per step / measured time per step (GB/s).
"""
from __future__ import annotations

import argparse
import dataclasses
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode KV-read GB/s (% of HBM peak) and decode-attn steps/s, FP8 vs NVFP4"
HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_FLOPS = 2.5e15
FP8_ROW, NV_ROW, BF16_ROW = 576, 324, 1152
ROW_BYTES = {"fp8": FP8_ROW, "nvfp4": NV_ROW, "bf16": BF16_ROW}
WORKLOADS = ("fp8_32k", "nvfp4_32k", "nvfp4_160k", "nvfp4_1m")


def _hip():
    """The HIP runtime already loaded by torch (one runtime per process)."""
    path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
    lib = ctypes.CDLL(path)
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


class Events:
    def __init__(self, hip, n):
        self.hip = hip
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e.value)

    def ms(self, a, b):
        """Elapsed ms between two recorded events; None if either was never recorded."""
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) != 0:
            self.hip.hipGetLastError()   # clear the runtime's sticky error so the next call does not report it
            return None
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def src_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "device_common.h", "mlaq_kernels.h"):
        h.update(open(os.path.join(ROOT, "quantized_kv_paged_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel_tag: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were taken on
    the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel_tag}_pmc.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("src_hash") != src_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Bench:
    """Device state shared by the legs: the library, the launch stream, events."""

    def __init__(self, steps, warmup):
        import torch
        import quantized_kv_paged_amd as qk
        self.torch, self.qk, self.L = torch, qk, qk._lib
        torch.cuda.set_device(0)
        self.hip = _hip()
        self.stream = torch.cuda.current_stream().cuda_stream
        self.steps, self.warmup = steps, warmup

    def dev(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def check(self, st):
        if st != 0:
            raise RuntimeError(self.qk.last_error())

    @staticmethod
    def layers_for(live_bytes):
        """Pool copies cycled through: at least 600 MB of live KV over all copies (over twice the
        256 MB Infinity Cache) and at least two."""
        return max(2, int(np.ceil(600e6 / live_bytes)))

    def inputs(self, w):
        """Page table, host FP8 pool and the device copies of q and the page table."""
        import synth
        t0 = time.perf_counter()
        pt = synth.page_table(w)
        host = synth.build_fp8_pool(w, pt)
        d = {"indptr": self.dev(pt.kv_indptr), "indices": self.dev(pt.kv_indices), "lens": self.dev(pt.kv_lens),
             "q": self.dev(synth.q_bits(w.seed, w.batch, w.heads).view(np.int16)).view(self.torch.bfloat16)}
        log(f"{w.name}: host pool {host.shape} in {time.perf_counter() - t0:.1f} s")
        return pt, host, d

    def nvfp4_layers(self, fp8_dev, n, g=1.0):
        """n copies of the NVFP4 pool made from the device FP8 pool by the library's quantize-on-write."""
        torch = self.torch
        rows = fp8_dev.shape[0]
        data = torch.empty((rows, 288), dtype=torch.uint8, device="cuda")
        scales = torch.empty((rows, 36), dtype=torch.uint8, device="cuda")
        slots = torch.arange(rows, dtype=torch.int64, device="cuda")
        self.qk.kv_quantize_nvfp4(fp8_dev, self.qk.MLAQ_FP8_E4M3, 1.0, slots, data, scales, g)
        del slots
        return [(data, scales)] + [(data.clone(), scales.clone()) for _ in range(n - 1)]

    def decode_step(self, fmt, p, d, layers, out, lse, ws, scale=1.0, write=None, stream=None):
        """One decode step on layer l: fmt 'fp8' (layers = FP8 pools), 'nvfp4' (layers = (data,
        scales)) or 'bf16'; `write` = (src, slots, n, pool_rows) adds the NVFP4 quantize-on-write."""
        L, strm = self.L, self.stream if stream is None else stream
        pp = ctypes.byref(p)
        com = (d["indptr"].data_ptr(), d["indices"].data_ptr(), d["lens"].data_ptr(), out.data_ptr(),
               lse.data_ptr(), ws.data_ptr(), ws.numel(), strm)
        qp, chk = d["q"].data_ptr(), self.check
        if fmt == "fp8":
            ptrs = [t.data_ptr() for t in layers]
            return lambda l: chk(L.mla_decode_fp8(pp, qp, ptrs[l], scale, *com))
        if fmt == "bf16":
            ptrs = [t.data_ptr() for t in layers]
            return lambda l: chk(L.mla_decode_bf16(pp, qp, ptrs[l], *com))
        ptrs = [(a.data_ptr(), s.data_ptr()) for a, s in layers]
        if write is None:
            return lambda l: chk(L.mla_decode_nvfp4(pp, qp, ptrs[l][0], ptrs[l][1], scale, *com))
        src, slots, n, rows = write

        def step(l):
            chk(L.kv_quantize_nvfp4(src.data_ptr(), self.qk.MLAQ_FP8_E4M3, 1.0, n, slots.data_ptr(), ptrs[l][0],
                                    ptrs[l][1], rows, scale, strm))
            chk(L.mla_decode_nvfp4(pp, qp, ptrs[l][0], ptrs[l][1], scale, *com))
        return step

    def settle(self, ms=150.0):
        """Bring the GPU out of idle before a timed leg: streaming reads (the library's read probe
        over a 1 GiB buffer) for about `ms` milliseconds.  The pools of a leg are generated on the
        host first, and the seconds the GPU spends idle meanwhile drop its clocks; a few warmup
        steps of a sub-millisecond kernel do not bring them back."""
        torch = self.torch
        if getattr(self, "_settle_buf", None) is None:
            self._settle_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
            self._settle_parts = torch.empty((32768, 16), dtype=torch.uint8, device="cuda")
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(32):
                self.qk.read_probe(self._settle_buf, 32768, self._settle_parts)
            torch.cuda.synchronize()

    def timed(self, step, n_layers, steps=None, warmup=None, kernels=True, dist=False):
        """Clock settling (see settle), warmup, then: region 1 launches `steps` steps as they run in
        use (ms per step, the headline); with dist, region 2 records an event between consecutive
        steps (per-step median / p10 / p90); with kernels, region 3 launches the steps with HIP
        events recorded at each kernel's own start and end (mlaq_set_profile_events) and gives the
        split and merge kernels' mean durations.  Times in microseconds."""
        torch, qk = self.torch, self.qk
        steps = self.steps if steps is None else steps
        warmup = self.warmup if warmup is None else warmup
        self.settle()
        for i in range(warmup):
            step(i % n_layers)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            step(i % n_layers)
        end.record()
        torch.cuda.synchronize()
        r = {"step_us": start.elapsed_time(end) / steps * 1e3}
        if dist:
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            evs[0].record()
            for i in range(steps):
                step(i % n_layers)
                evs[i + 1].record()
            torch.cuda.synchronize()
            per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]) * 1e3
            r["p10_us"], r["p50_us"], r["p90_us"] = (float(x) for x in np.percentile(per, [10, 50, 90]))
        if kernels:
            ev = Events(self.hip, 4 * steps)
            start.record()
            for i in range(steps):
                qk.mlaq_set_profile_events(*ev.ev[4 * i:4 * i + 4])
                step(i % n_layers)
            end.record()
            torch.cuda.synchronize()
            r["step_with_kernel_events_us"] = start.elapsed_time(end) / steps * 1e3
            r["split_us"] = float(np.mean([ev.ms(4 * i, 4 * i + 1) for i in range(steps)])) * 1e3
            merges = [m for m in (ev.ms(4 * i + 2, 4 * i + 3) for i in range(steps)) if m is not None]
            r["merge_us"] = float(np.mean(merges)) * 1e3 if merges else 0.0
            ev.close()
        return r


def summary(t, kv_bytes, splits):
    """Per-leg figures: step time and rate, KV GB/s per step, the split kernel's rate and roofline
    fraction, the merge kernel."""
    s = {"num_splits": splits, "step_us": round(t["step_us"], 2), "steps_per_s": round(1e6 / t["step_us"], 1),
         "kv_gbs": round(kv_bytes / t["step_us"] / 1e3, 1),
         "frac_of_hbm_peak": round(kv_bytes / t["step_us"] / 1e3 / HBM_PEAK_GBS, 4)}
    if "split_us" in t:
        s.update({"split_kernel_us": round(t["split_us"], 2),
                  "split_kernel_gbs": round(kv_bytes / t["split_us"] / 1e3, 1),
                  "split_kernel_frac": round(kv_bytes / t["split_us"] / 1e3 / HBM_PEAK_GBS, 4),
                  "merge_us": round(t["merge_us"], 2)})
    if "p50_us" in t:
        s.update({k: round(t[k], 2) for k in ("p10_us", "p50_us", "p90_us")})
    return s


PROBE_BYTES = 4 << 30                # 16x the 256 MB Infinity Cache: every pass streams from HBM
PROBE_BLOCKS = (16384, 32768, 65536)  # 256-thread workgroups per launch; the best is reported


def read_probe(bn, reps=10):
    """Measured HBM read ceiling: the library's streaming-read probe over a 4 GiB buffer, for
    each block count reps back-to-back passes after 3 untimed ones; the best rate is reported."""
    torch, qk = bn.torch, bn.qk
    buf = torch.empty(PROBE_BYTES, dtype=torch.uint8, device="cuda")
    best = None
    for blocks in PROBE_BLOCKS:
        parts = torch.empty((blocks, 16), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            qk.read_probe(buf, blocks, parts)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            qk.read_probe(buf, blocks, parts)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        if best is None or ms < best[0]:
            best = (ms, blocks)
    del buf
    ms, blocks = best
    gbs = PROBE_BYTES / (ms * 1e-3) / 1e9
    return {"bytes": PROBE_BYTES, "blocks": blocks, "ms_per_pass": round(ms, 4), "gbs": round(gbs, 1),
            "frac_of_nominal": round(gbs / HBM_PEAK_GBS, 4)}


def graph_steps(bn, make_step, n_layers, steps, kv_bytes):
    """The same steps replayed from a HIP graph: one graph holds one step per pool copy, captured
    on a side stream, and is replayed until about `steps` steps have run."""
    torch = bn.torch
    gs = torch.cuda.Stream()
    gstep = make_step(gs.cuda_stream)
    with torch.cuda.stream(gs):
        for l in range(n_layers):
            gstep(l)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        for l in range(n_layers):
            gstep(l)
    reps = max(1, steps // n_layers)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(gs):
        start.record()
        for _ in range(reps):
            g.replay()
        end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / (reps * n_layers) * 1e3
    return {"step_us": round(us, 2), "steps": reps * n_layers, "kv_gbs": round(kv_bytes / us / 1e3, 1)}


def decode_config(bn, w, primary, headline=False, extras=True):
    """One workload: its own format (primary) and the other format at the same batch, context and
    page tables (FP8 pools are the workload's FP8 rows; NVFP4 pools are those rows quantized by the
    library's write path with g = 1).  Returns (result dict, context for the config's extra legs)."""
    import synth
    torch, qk = bn.torch, bn.qk
    pt, host, d = bn.inputs(w)
    p = qk.decode_params(w.batch, w.heads, w.page_size, w.kv_len, w.pool_tokens, w.sm_scale)
    need = max(qk.mlaq_decode_workspace_bytes(p), qk._lib.mlaq_decode_nvfp4_append_workspace_bytes(ctypes.byref(p)))
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device="cuda")
    fp8_dev = bn.dev(host)
    write = None
    if w.write_tokens:
        write = (bn.dev(synth.write_source_fp8(w)), bn.dev(synth.slot_mapping(w, pt)), w.write_tokens, w.pool_tokens)
    res, ctx = {}, {"pt": pt, "host": host, "d": d, "p": p, "ws": ws, "out": out, "lse": lse, "fp8": fp8_dev}
    for fmt in ([primary] + ([f for f in ("fp8", "nvfp4") if f != primary] if extras else [])):
        kv_bytes = w.batch * w.kv_len * ROW_BYTES[fmt]
        n = bn.layers_for(kv_bytes)
        if fmt == "fp8":
            layers = [fp8_dev] + [fp8_dev.clone() for _ in range(n - 1)]
        else:
            layers = bn.nvfp4_layers(fp8_dev, n)
        torch.cuda.synchronize()
        wr = write if (fmt == "nvfp4" and write is not None) else None
        step = bn.decode_step(fmt, p, d, layers, out, lse, ws, write=wr)
        fcode = qk.MLAQ_FP8_E4M3 if fmt == "fp8" else qk.MLAQ_NVFP4
        t = bn.timed(step, n, dist=headline and fmt == primary)
        s = summary(t, kv_bytes, qk.mlaq_decode_num_splits(p, fcode))
        s.update({"kv_bytes_per_step": kv_bytes, "layers_cycled": n})
        if wr is not None:
            s["includes_write_tokens"] = w.write_tokens
        if fmt == primary:
            res["primary"] = (s, t, kv_bytes, n)
            if headline and extras:
                res["graph"] = graph_steps(bn, lambda strm: bn.decode_step(fmt, p, d, layers, out, lse, ws, write=wr,
                                                                            stream=strm), n, bn.steps, kv_bytes)
            if fmt == "nvfp4":
                ctx["nv_layers"] = layers
        else:
            res["other"] = (fmt, s)
            del layers
        log(f"{w.name} {fmt}: step {s['step_us']} us, split kernel {s.get('split_kernel_us')} us")
    if not extras or primary != "nvfp4":
        ctx.pop("nv_layers", None)
    torch.cuda.empty_cache()
    return res, ctx


def split_sweep(bn, w, fmt, counts):
    """The workload's decode step (without the write path) in one format at forced split counts:
    one JSON line per count with the step, split-kernel and merge times (the planner's choice is
    marked).  A measurement aid for the split planner; not part of the benchmark line."""
    torch, qk = bn.torch, bn.qk
    pt, host, d = bn.inputs(w)
    fp8_dev = bn.dev(host)
    kv_bytes = w.batch * w.kv_len * ROW_BYTES[fmt]
    n = bn.layers_for(kv_bytes)
    layers = [fp8_dev] + [fp8_dev.clone() for _ in range(n - 1)] if fmt == "fp8" else bn.nvfp4_layers(fp8_dev, n)
    out = torch.empty((w.batch, w.heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device="cuda")
    fcode = qk.MLAQ_FP8_E4M3 if fmt == "fp8" else qk.MLAQ_NVFP4
    planned = qk.mlaq_decode_num_splits(qk.decode_params(w.batch, w.heads, w.page_size, w.kv_len,
                                                         w.pool_tokens, w.sm_scale), fcode)
    for c in counts:
        p = qk.decode_params(w.batch, w.heads, w.page_size, w.kv_len, w.pool_tokens, w.sm_scale, num_splits=c)
        ws = torch.zeros(max(qk.mlaq_decode_workspace_bytes(p, fcode), 256), dtype=torch.uint8, device="cuda")
        t = bn.timed(bn.decode_step(fmt, p, d, layers, out, lse, ws), n)
        line = {"sweep": w.name, "kv_format": fmt, "batch": w.batch, "kv_len": w.kv_len, "planned": c == planned,
                **summary(t, kv_bytes, c)}
        print(json.dumps(line), flush=True)
        del ws


def write_path_leg(bn, w, ctx):
    """The quantize-on-write of the workload's write chunk on its own (FP8 source -> NVFP4 rows in
    scattered pages): microseconds per call, tokens/s and GB/s of algorithmic bytes (source read,
    slots read, rows written)."""
    import synth
    layers = ctx["nv_layers"]
    src = bn.dev(synth.write_source_fp8(w))
    slots = bn.dev(synth.slot_mapping(w, ctx["pt"]))
    ptrs = [(a.data_ptr(), s.data_ptr()) for a, s in layers]
    L = bn.L

    def step(l):
        bn.check(L.kv_quantize_nvfp4(src.data_ptr(), bn.qk.MLAQ_FP8_E4M3, 1.0, w.write_tokens, slots.data_ptr(),
                                     ptrs[l][0], ptrs[l][1], w.pool_tokens, 1.0, bn.stream))
    t = bn.timed(step, len(layers), kernels=False, dist=True)
    moved = w.write_tokens * (FP8_ROW + 8 + NV_ROW)
    return {"tokens": w.write_tokens, "call_us": round(t["step_us"], 2), "p50_us": round(t["p50_us"], 2),
            "tokens_per_s": round(w.write_tokens / t["step_us"] * 1e6, 1),
            "gbs": round(moved / t["step_us"] / 1e3, 1), "bytes_moved_per_call": moved}


def fp8_32k_legs(bn, w, ctx, fp8_step_us):
    """The pages' own path (whole-pool cast to BF16 every layer, then a BF16 decode) and their
    intermediate fix (cast only the active rows, then a BF16 decode over them)."""
    torch, qk, L = bn.torch, bn.qk, bn.L
    pt, d, out, lse, ws, p = ctx["pt"], ctx["d"], ctx["out"], ctx["lse"], ctx["ws"], ctx["p"]
    fp8 = ctx["fp8"]
    n = bn.layers_for(w.batch * w.kv_len * FP8_ROW)
    layers = [fp8] + [fp8.clone() for _ in range(n - 1)]
    fp8p = [t.data_ptr() for t in layers]
    pp, strm, chk = ctypes.byref(p), bn.stream, bn.check
    common = (d["indptr"].data_ptr(), d["indices"].data_ptr(), d["lens"].data_ptr(), out.data_ptr(),
              lse.data_ptr(), ws.data_ptr(), ws.numel(), strm)
    qp = d["q"].data_ptr()
    bf = torch.empty((w.pool_tokens, 576), dtype=torch.bfloat16, device="cuda")

    def cstep(l):
        chk(L.kv_dequantize(qk.MLAQ_FP8_E4M3, fp8p[l], None, 1.0, None, w.pool_tokens, w.pool_tokens, qk.MLAQ_BF16,
                            bf.data_ptr(), strm))
        chk(L.mla_decode_bf16(pp, qp, bf.data_ptr(), *common))
    t = bn.timed(cstep, n, steps=max(20, bn.steps // 4), warmup=5, kernels=False)
    res = {"cast_baseline": {"step_us": round(t["step_us"], 2), "steps_per_s": round(1e6 / t["step_us"], 1),
                             "bytes_moved_per_step": w.pool_tokens * (FP8_ROW + BF16_ROW) + w.batch * w.kv_len * BF16_ROW,
                             "speedup_of_fp8_path": round(t["step_us"] / fp8_step_us, 2)}}
    del bf
    P = w.page_size
    tok = np.arange(w.kv_len, dtype=np.int64)
    rows_h = np.concatenate([pt.kv_indices[pt.kv_indptr[b] + tok // P].astype(np.int64) * P + tok % P
                             for b in range(w.batch)])
    rows = bn.dev(rows_h)
    n_act = rows_h.shape[0]
    gbf = torch.empty((n_act, 576), dtype=torch.bfloat16, device="cuda")
    gind = torch.arange(n_act // P, dtype=torch.int32, device="cuda")
    gptr = torch.arange(w.batch + 1, dtype=torch.int32, device="cuda") * (w.kv_len // P)
    gp = qk.decode_params(w.batch, w.heads, P, w.kv_len, n_act, w.sm_scale)
    gpp = ctypes.byref(gp)
    gcommon = (gptr.data_ptr(), gind.data_ptr(), d["lens"].data_ptr(), out.data_ptr(), lse.data_ptr(),
               ws.data_ptr(), ws.numel(), strm)

    def gstep(l):
        chk(L.kv_dequantize(qk.MLAQ_FP8_E4M3, fp8p[l], None, 1.0, rows.data_ptr(), n_act, w.pool_tokens,
                            qk.MLAQ_BF16, gbf.data_ptr(), strm))
        chk(L.mla_decode_bf16(gpp, qp, gbf.data_ptr(), *gcommon))
    t = bn.timed(gstep, n, steps=max(20, bn.steps // 4), warmup=20, kernels=False)
    res["gather_cast_baseline"] = {"step_us": round(t["step_us"], 2), "steps_per_s": round(1e6 / t["step_us"], 1),
                                   "bytes_moved_per_step": n_act * (FP8_ROW + 8 + 2 * BF16_ROW),
                                   "speedup_of_fp8_path": round(t["step_us"] / fp8_step_us, 2)}
    return res


def nvfp4_32k_legs(bn, w, ctx):
    """Calibrated global scale (timed) and the quantization effect of both scales; the fused
    append; extend and initial prefill over the cache."""
    import synth
    torch, qk, L = bn.torch, bn.qk, bn.L
    pt, d, out, lse, ws, p, fp8 = ctx["pt"], ctx["d"], ctx["out"], ctx["lse"], ctx["ws"], ctx["p"], ctx["fp8"]
    res = {}
    # ---- calibrated g = fl32(amax / (6 * 448)) over the source pool (host formula, fp32 division)
    amax = float(fp8.view(torch.float8_e4m3fn).float().abs().max())
    g = float(np.float32(amax) / np.float32(2688.0))
    kv_bytes = w.batch * w.kv_len * NV_ROW
    n = bn.layers_for(kv_bytes)
    cal = bn.nvfp4_layers(fp8, n, g)
    t = bn.timed(bn.decode_step("nvfp4", p, d, cal, out, lse, ws, scale=g), n)
    res["calibrated_scale"] = dict(summary(t, kv_bytes, qk.mlaq_decode_num_splits(p, qk.MLAQ_NVFP4)),
                                   global_scale=g, amax=amax)
    # ---- quantization effect (informational): each format's output against the same decode over
    #      the bf16 source rows the FP8 rows were cast from (the library's BF16 decode, parity-tested
    #      within 5e-3 of the oracle, far below the effects measured here)
    bf = bn.dev(synth.build_bf16_source_pool(w, pt).view(np.int16)).view(torch.bfloat16)
    outs = {}
    for name, fmt, layers, sc in (("bf16_source", "bf16", [bf], 1.0), ("fp8", "fp8", [fp8], 1.0),
                                  ("nvfp4_g1", "nvfp4", ctx["nv_layers"][:1], 1.0),
                                  ("nvfp4_calibrated", "nvfp4", cal[:1], g)):
        bn.decode_step(fmt, p, d, layers, out, lse, ws, scale=sc)(0)
        torch.cuda.synchronize()
        outs[name] = out.double().clone()
    ref = outs["bf16_source"]
    res["quantization_effect_rel_l2"] = {
        k: round(float(torch.linalg.vector_norm(v - ref) / torch.linalg.vector_norm(ref)), 5)
        for k, v in outs.items() if k != "bf16_source"}
    res["quantization_effect_rel_l2"]["reference"] = "BF16 decode over the bf16 source rows, whole [44, 16, 512] output"
    del bf, cal, outs
    torch.cuda.empty_cache()
    nv = ctx["nv_layers"]
    nvp = [(a.data_ptr(), s.data_ptr()) for a, s in nv]
    n = len(nv)
    strm, chk, pp = bn.stream, bn.check, ctypes.byref(p)
    common = (d["indptr"].data_ptr(), d["indices"].data_ptr(), d["lens"].data_ptr(), out.data_ptr(),
              lse.data_ptr(), ws.data_ptr(), ws.numel(), strm)
    qp = d["q"].data_ptr()
    # ---- fused append-then-attend against a quantize launch for the B new rows + the decode
    P = w.page_size
    last = w.kv_len - 1
    arows = bn.dev(np.array([int(pt.kv_indices[pt.kv_indptr[b] + last // P]) * P + last % P for b in range(w.batch)],
                            dtype=np.int64))
    nsrc = bn.dev(synth.to_bf16_bits(synth.new_token_rows(w.seed, w.batch)).view(np.int16))

    def fstep(l):
        chk(L.mla_decode_nvfp4_append(pp, qp, nsrc.data_ptr(), qk.MLAQ_BF16, 1.0, nvp[l][0], nvp[l][1], 1.0, *common))

    def sstep(l):
        chk(L.kv_quantize_nvfp4(nsrc.data_ptr(), qk.MLAQ_BF16, 1.0, w.batch, arows.data_ptr(), nvp[l][0], nvp[l][1],
                                w.pool_tokens, 1.0, strm))
        chk(L.mla_decode_nvfp4(pp, qp, nvp[l][0], nvp[l][1], 1.0, *common))
    tf = bn.timed(fstep, n, warmup=50, kernels=False)
    ts = bn.timed(sstep, n, warmup=50, kernels=False)
    res["append_fused"] = {"step_us": round(tf["step_us"], 2), "separate_step_us": round(ts["step_us"], 2),
                           "new_tokens_per_step": w.batch, "speedup_vs_separate": round(ts["step_us"] / tf["step_us"], 3)}
    # ---- extend: the first 4 requests take a 256-token chunk after a prefix of the rest of their
    #      context; initial prefill: 4 prompts of 2,048 tokens with empty prefixes
    for kind, EC, EP, qseed, kseed in (("extend", 256, w.kv_len - 256, w.seed + 7, w.seed),
                                       ("prefill", 2048, 0, w.seed + 8, w.seed + 1)):
        EB = min(4, w.batch)
        nq = EB * EC
        tok = np.arange(EP, EP + EC, dtype=np.int64)
        eslots = bn.dev(np.concatenate([pt.kv_indices[pt.kv_indptr[b] + tok // P].astype(np.int64) * P + tok % P
                                        for b in range(EB)]))
        eqo = torch.arange(EB + 1, dtype=torch.int32, device="cuda") * EC
        epl = torch.full((EB,), EP, dtype=torch.int32, device="cuda")
        eq = bn.dev(synth.q_bits(qseed, nq, w.heads).view(np.int16))
        eckv = bn.dev(synth.to_fp8_bytes(synth.extend_chunk_rows(kseed, nq)))
        ep = qk.extend_params(EB, w.heads, P, w.pool_tokens, nq, EP, EC, w.sm_scale)
        ews = torch.empty(qk.mlaq_extend_workspace_bytes(ep), dtype=torch.uint8, device="cuda")
        eout = torch.empty((nq, w.heads, 512), dtype=torch.float32, device="cuda")
        else_ = torch.empty((nq, w.heads), dtype=torch.float32, device="cuda")

        def estep(l, ep=ep, eq=eq, eqo=eqo, eckv=eckv, epl=epl, eslots=eslots, eout=eout, else_=else_, ews=ews):
            chk(L.mla_extend_nvfp4(ctypes.byref(ep), eq.data_ptr(), eqo.data_ptr(), eckv.data_ptr(), 1.0, nvp[l][0],
                                   nvp[l][1], 1.0, d["indptr"].data_ptr(), d["indices"].data_ptr(), epl.data_ptr(),
                                   eslots.data_ptr(), eout.data_ptr(), else_.data_ptr(), ews.data_ptr(), ews.numel(),
                                   strm))
        # 20 warm-up calls (about 40 ms of MFMA-bound work) bring the clocks to where a sustained
        # run holds them; 3 left the first timed calls up to 10 % slow
        t = bn.timed(estep, n, steps=20, warmup=20)
        flops = EB * sum(2 * w.heads * (EP + i + 1) * (576 + 512) for i in range(EC))
        attn_us = t["split_us"] + t["merge_us"]
        res[kind] = {"requests": EB, "prefix_tokens": EP, "chunk_tokens": EC, "call_us": round(t["step_us"], 1),
                     "kv_splits": qk._lib.mlaq_extend_num_splits(ctypes.byref(ep)),
                     "chunk_tokens_per_s": round(nq / t["step_us"] * 1e6, 1),
                     "attention_kernel_us": round(t["split_us"], 1), "merge_us": round(t["merge_us"], 1),
                     "attention_tflops": round(flops / attn_us / 1e6, 1),
                     "frac_of_fp16_mfma_peak": round(flops / attn_us / 1e6 / (FP16_MFMA_PEAK_FLOPS / 1e12), 4)}
        del ews, eout, else_
    return res


def cpu_baseline(w, pt, pool_fp8, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the workload, on the host's cores (BLAS
    threads set to os.cpu_count()): whole request chunks of up to 128K tokens, cycling over the
    batch, until about budget_s seconds of timed gather + fp64 dequant + fp64 attention (NVFP4
    chunks are first encoded by the oracle, untimed).  With a write chunk in the workload, the
    oracle's encoder is also timed on it: the C twin on all of it, the scalar Python encoder on
    its first 32 tokens."""
    from threadpoolctl import threadpool_limits
    from oracle import attention, codecs
    from oracle import nvfp4 as onv
    import synth
    cores = os.cpu_count()
    nvfp4 = w.fmt == "nvfp4"
    chunk = 131072
    with threadpool_limits(limits=cores):
        q_all = codecs.bf16_bits_to_f64(synth.q_bits(w.seed, w.batch, w.heads))
        samples = [(b, s0, min(chunk, int(pt.kv_lens[b]) - s0)) for b in range(w.batch)
                   for s0 in range(0, int(pt.kv_lens[b]), chunk)]
        row = NV_ROW if nvfp4 else FP8_ROW
        timed, tokens, done, k = 0.0, 0, 0, 0
        encoded = {}
        while done == 0 or timed < budget_s:
            b, s0, n = samples[k % len(samples)]
            if nvfp4 and k % len(samples) not in encoded:
                all_rows = attention.gather_rows(pt.kv_indptr, pt.kv_indices, w.page_size, b, s0 + n)
                encoded[k % len(samples)] = onv.quantize_fp8_rows(pool_fp8[all_rows[s0:]], 1.0, 1.0)
            t0 = time.perf_counter()
            rows = attention.gather_rows(pt.kv_indptr, pt.kv_indices, w.page_size, b, s0 + n)[s0:]
            if nvfp4:
                nv_data, nv_scales = encoded[k % len(samples)]
                x = onv.dequant_nvfp4_f64(nv_data, nv_scales, 1.0)
            else:
                x = onv.dequant_fp8_f64(pool_fp8[rows], 1.0)
            attention.decode_dense(q_all[b], x, w.sm_scale)
            timed += time.perf_counter() - t0
            tokens += n
            done += 1
            k += 1
            del x
        step_tokens = w.batch * w.kv_len
        res = {"value": round(tokens * row / timed / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{done} request chunks of up to {chunk} tokens, cycling over the batch ({tokens} tokens, "
                         f"{tokens / step_tokens:.3f} steps' worth): gather + fp64 dequant + fp64 attention, "
                         f"{timed:.1f} s timed, BLAS threads {cores} (numpy's element-wise steps run on one)",
               "steps_per_s": round(tokens / step_tokens / timed, 6)}
        if w.write_tokens:
            src = synth.write_source_fp8(w)
            t0 = time.perf_counter()
            onv.quantize_fp8_rows(src, 1.0, 1.0)
            tc = time.perf_counter() - t0
            ns = 32
            x = onv.fp8_rows_to_f32(src[:ns], 1.0)
            t0 = time.perf_counter()
            for r in range(ns):
                onv.quantize_row_py(x[r], 1.0)
            tp = time.perf_counter() - t0
            res["write_path"] = {"tokens": w.write_tokens, "c_encoder_s": round(tc, 4),
                                 "c_encoder_tokens_per_s": round(w.write_tokens / tc, 1),
                                 "c_encoder_threads": int(os.environ.get("OMP_NUM_THREADS", cores)),
                                 "python_encoder_tokens_per_s": round(ns / tp, 2),
                                 "python_encoder_sample_tokens": ns}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first (clocks and memory settle over the first tens of ms)")
    ap.add_argument("--workload", default="nvfp4_1m", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split-sweep", default=None,
                    help="comma-separated split counts: time the workload's decode at each (one JSON line "
                         "per count) instead of the benchmark line")
    ap.add_argument("--sweep-format", default=None, choices=("fp8", "nvfp4"),
                    help="the format of --split-sweep (default: the workload's own)")
    ap.add_argument("--sweep-shape", default=None,
                    help="BATCH:CONTEXT for --split-sweep: the workload's distributions and page size at "
                         "another batch and context (pool = batch x context)")
    ap.add_argument("--no-extras", action="store_true", help="the headline workload's own format only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import synth
    bn = Bench(args.steps, args.warmup)
    torch = bn.torch
    w = synth.WORKLOADS[args.workload]
    if args.split_sweep:
        if args.sweep_shape:
            sb, sl = (int(x) for x in args.sweep_shape.split(":"))
            w = dataclasses.replace(w, name=f"{w.name}@{sb}x{sl}", batch=sb, kv_len=sl, pool_tokens=sb * sl,
                                    write_tokens=0, write_pages=0)
        split_sweep(bn, w, args.sweep_format or w.fmt, [int(x) for x in args.split_sweep.split(",")])
        return
    extras = not args.no_extras
    # the read probe first: it is reported, and it brings the clocks up before any timed region
    probe = read_probe(bn) if extras else None
    head, ctx = decode_config(bn, w, w.fmt, headline=True, extras=extras)
    s, t, kv_bytes, n_layers = head["primary"]
    achieved = kv_bytes / t["split_us"] / 1e3
    value = kv_bytes / t["step_us"] / 1e3
    kernel_tag = f"mla_decode_kernel_{w.name}"
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t["step_us"] / 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.fmt.upper()} paged MLA decode, batch {w.batch} x {w.heads} heads, "
                               f"context {w.kv_len}, page {w.page_size}, pool {w.pool_tokens} x 576"
                               + (f", plus NVFP4 quantize-on-write of {w.write_tokens} tokens per step"
                                  if w.write_tokens else ""),
                   "kv_format": w.fmt, "batch": w.batch, "heads": w.heads, "kv_len": w.kv_len,
                   "page_size": w.page_size, "pool_tokens": w.pool_tokens, "num_splits": s["num_splits"],
                   "layers_cycled": n_layers, "kv_bytes_per_step": kv_bytes},
        "steps_per_s": s["steps_per_s"], "frac_of_hbm_peak": s["frac_of_hbm_peak"],
        "step_us": {"mean": s["step_us"], "p10": s["p10_us"], "p50": s["p50_us"], "p90": s["p90_us"],
                    "steps_per_s_at_p50": round(1e6 / s["p50_us"], 1)},
        "kernels_us": {"split": s["split_kernel_us"], "merge": s["merge_us"],
                       "step_with_kernel_events": round(t["step_with_kernel_events_us"], 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": pmc_traffic(kernel_tag),
                     "kernel": "mla_decode_kernel", "bytes_per_launch": kv_bytes},
    }
    if extras:
        probe["split_kernel_frac_of_probe"] = round(achieved / probe["gbs"], 4)
        res["read_probe"] = probe
        res["graph"] = head["graph"]
        fmt2, s2 = head["other"]
        res[f"{fmt2}_same_batch"] = s2
        res["nvfp4_speedup_vs_fp8"] = round((s2["step_us"] / s["step_us"]) if fmt2 == "fp8"
                                            else (s["step_us"] / s2["step_us"]), 3)
        if w.write_tokens:
            res["write_path"] = write_path_leg(bn, w, ctx)
    if args.copy_calibration:
        # a plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE per dispatch give the
        # counters' bytes-per-byte scale
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, ctx["pt"], ctx["host"])
    del ctx
    torch.cuda.empty_cache()
    if extras:
        # the other workloads: the same two formats at their batch, context and page tables, plus
        # their own comparison legs
        res["configs"] = {}
        for name in WORKLOADS:
            if name == w.name:
                continue
            wo = synth.WORKLOADS[name]
            r, c = decode_config(bn, wo, wo.fmt, headline=False, extras=True)
            so = r["primary"][0]
            entry = {"kv_format": wo.fmt, "batch": wo.batch, "kv_len": wo.kv_len, **so}
            fo, sf = r["other"]
            entry[f"{fo}_same_batch"] = sf
            entry["nvfp4_speedup_vs_fp8"] = round((sf["step_us"] / so["step_us"]) if fo == "fp8"
                                                  else (so["step_us"] / sf["step_us"]), 3)
            if name == "fp8_32k":
                entry.update(fp8_32k_legs(bn, wo, c, so["step_us"]))
            if name == "nvfp4_32k":
                entry.update(nvfp4_32k_legs(bn, wo, c))
            res["configs"][name] = entry
            del r, c
            torch.cuda.empty_cache()
    print(json.dumps(res))


if __name__ == "__main__":
    main()
