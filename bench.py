#!/usr/bin/env python3
"""Benchmark of paged MLA decode over FP8 / NVFP4 latent KV on one MI355X.

One step = one decode call over the whole batch: the split-KV kernel (page-table gather,
in-register dequantization, QK^T and PV on MFMA, online softmax, split partials) and the
merge kernel, i.e. one layer of one decode step for every request.  Inputs are synthetic
(synth.py) and resident in HBM before the timed region.  Consecutive steps cycle through
several copies of the pool ("layers") at different addresses, so that the 256 MB
Infinity Cache cannot serve a step from the previous one.

Default workload: FP8 pool of the pages (495,552 tokens x 576), batch 8, 32K context, page 64.
Other workloads (--workload): nvfp4_32k, nvfp4_160k, nvfp4_1m (the last one adds the
8,192-token NVFP4 quantize-on-write to every step).

Prints ONE JSON line.  `value` = KV bytes read per step / measured time per step (GB/s).
"""
from __future__ import annotations

import argparse
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
FP8_ROW, NV_ROW, BF16_ROW = 576, 324, 1152


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


def timed_steps(step, n_layers, steps, warmup, hip, torch, profile=True):
    """Warmup, then two timed regions of `steps` steps each.  Region 1 launches the steps as
    they run in use and gives ms per step (the headline).  Region 2 (profile=True) launches
    the same steps with HIP events recorded at each kernel's own start and end (on the launch
    stream) and gives the split kernel's and the merge kernel's mean durations.  Returns
    (ms per step, split-kernel ms, merge ms, ms per step of region 2)."""
    import quantized_kv_paged_amd as qk
    for i in range(warmup):
        step(i % n_layers)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(i % n_layers)
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end) / steps
    if not profile:
        return total, None, None, None
    ev = Events(hip, 4 * steps)
    start.record()
    for i in range(steps):
        qk.mlaq_set_profile_events(*ev.ev[4 * i:4 * i + 4])
        step(i % n_layers)
    end.record()
    torch.cuda.synchronize()
    total2 = start.elapsed_time(end) / steps
    split = float(np.mean([ev.ms(4 * i, 4 * i + 1) for i in range(steps)]))
    merges = [m for m in (ev.ms(4 * i + 2, 4 * i + 3) for i in range(steps)) if m is not None]
    merge = float(np.mean(merges)) if merges else 0.0
    ev.close()
    return total, split, merge, total2


PROBE_BYTES = 4 << 30                # 16x the 256 MB Infinity Cache: every pass streams from HBM
PROBE_BLOCKS = (16384, 32768, 65536)  # 256-thread workgroups per launch; the best is reported


def read_probe(qk, torch, split_gbs, reps=10):
    """Measured HBM read ceiling: the library's streaming-read probe over a 4 GiB buffer, for
    each block count reps back-to-back passes after 3 untimed ones; the best rate is reported
    and the split kernel's KV-read rate is also given as a fraction of it."""
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
            "frac_of_nominal": round(gbs / HBM_PEAK_GBS, 4),
            "split_kernel_frac_of_probe": round(split_gbs / gbs, 4)}


def graph_steps(make_step, n_layers, steps, torch, kv_bytes):
    """The same steps replayed from a HIP graph: one graph holds one step per pool copy, captured
    on a side stream, and is replayed until about `steps` steps have run; gives ms per step
    without per-launch host work."""
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
    ms = start.elapsed_time(end) / (reps * n_layers)
    return {"ms_per_step": round(ms, 5), "steps": reps * n_layers,
            "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1)}


def pmc_traffic(kernel_tag: str, launches_bytes: float):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were taken on
    the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel_tag}_pmc.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("src_hash") != src_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, pt, pool_fp8, nvfp4=False, budget_s=10.0):
    """The oracle, as it stands, on a bounded sample of the workload: whole requests (chunks of at
    most 128K tokens for longer contexts) in order, cycling, until about budget_s seconds of
    timed work.  For NVFP4 workloads each chunk's rows are first quantized by the oracle's
    encoder (untimed), so the timed part is the decode the GPU step performs: gather, dequantize,
    attention."""
    from oracle import attention, codecs
    from oracle import nvfp4 as onv
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    chunk = 131072
    q_all = codecs.bf16_bits_to_f64(synth.q_bits(w.seed, w.batch, w.heads))
    samples = [(b, s0, min(chunk, int(pt.kv_lens[b]) - s0)) for b in range(w.batch)
               for s0 in range(0, int(pt.kv_lens[b]), chunk)]
    row = NV_ROW if nvfp4 else FP8_ROW
    timed, tokens, done, k = 0.0, 0, 0, 0
    encoded = {}
    while done == 0 or timed < budget_s:
        b, s0, n = samples[k % len(samples)]
        if nvfp4:
            if k % len(samples) not in encoded:
                all_rows = attention.gather_rows(pt.kv_indptr, pt.kv_indices, w.page_size, b, s0 + n)
                encoded[k % len(samples)] = onv.quantize_fp8_rows(pool_fp8[all_rows[s0:]], 1.0, 1.0)
            nv_data, nv_scales = encoded[k % len(samples)]
        t0 = time.perf_counter()
        rows = attention.gather_rows(pt.kv_indptr, pt.kv_indices, w.page_size, b, s0 + n)[s0:]
        x = onv.dequant_nvfp4_f64(nv_data, nv_scales, 1.0) if nvfp4 else onv.dequant_fp8_f64(pool_fp8[rows], 1.0)
        attention.decode_dense(q_all[b], x, w.sm_scale)
        timed += time.perf_counter() - t0
        tokens += n
        done += 1
        k += 1
        del x
    step_tokens = w.batch * w.kv_len
    return {"value": round(tokens * row / timed / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} request chunks of up to {chunk} tokens, cycling over the batch ({tokens} tokens, "
                      f"{tokens / step_tokens:.2f} steps' worth): gather + fp64 dequant + fp64 attention, "
                      f"{timed:.1f} s timed",
            "steps_per_s": round(tokens / step_tokens / timed, 6)}


def build_pools(w, torch, qk, n_layers, fmt):
    """Device pools for n_layers layers (copies at distinct addresses) + page table + q."""
    import synth
    t0 = time.perf_counter()
    pt = synth.page_table(w)
    host = synth.build_fp8_pool(w, pt)
    t1 = time.perf_counter()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    d = {"indptr": dev(pt.kv_indptr), "indices": dev(pt.kv_indices), "lens": dev(pt.kv_lens),
         "q": dev(synth.q_bits(w.seed, w.batch, w.heads).view(np.int16)).view(torch.bfloat16)}
    fp8 = dev(host)
    d["fp8"] = [fp8] + [fp8.clone() for _ in range(n_layers - 1)] if fmt == "fp8" else [fp8]
    if fmt == "nvfp4":
        data = torch.empty((w.pool_tokens, 288), dtype=torch.uint8, device="cuda")
        scales = torch.empty((w.pool_tokens, 36), dtype=torch.uint8, device="cuda")
        slots = torch.arange(w.pool_tokens, dtype=torch.int64, device="cuda")
        qk.kv_quantize_nvfp4(fp8, qk.MLAQ_FP8_E4M3, 1.0, slots, data, scales, 1.0)
        d["nv"] = [(data, scales)] + [(data.clone(), scales.clone()) for _ in range(n_layers - 1)]
        del slots
    torch.cuda.synchronize()
    d["gen_s"] = round(t1 - t0, 1)
    return pt, host, d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first (clocks and memory settle over the first tens of ms)")
    ap.add_argument("--workload", default="fp8_32k", choices=["fp8_32k", "nvfp4_32k", "nvfp4_160k", "nvfp4_1m"])
    ap.add_argument("--layers", type=int, default=0, help="pool copies cycled through (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the comparison legs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_kv_paged_amd as qk
    import synth
    torch.cuda.set_device(0)
    hip = _hip()
    w = synth.WORKLOADS[args.workload]
    fmt = w.fmt
    live = w.batch * w.kv_len * (FP8_ROW if fmt == "fp8" else NV_ROW)
    n_layers = args.layers or max(2, int(np.ceil(600e6 / live)))
    print(f"[bench] {w.name}: building {n_layers} layer pools", file=sys.stderr, flush=True)
    pt, host, d = build_pools(w, torch, qk, n_layers, fmt)
    print(f"[bench] pools ready (host generation {d['gen_s']} s)", file=sys.stderr, flush=True)

    p = qk.decode_params(w.batch, w.heads, w.page_size, w.kv_len, w.pool_tokens, w.sm_scale)
    fcode = qk.MLAQ_FP8_E4M3 if fmt == "fp8" else qk.MLAQ_NVFP4
    splits = qk.mlaq_decode_num_splits(p, fcode)
    # one workspace large enough for every format run on this shape (the comparison legs)
    need = max([qk.mlaq_decode_workspace_bytes(p)] +
               [qk._lib.mlaq_decode_nvfp4_append_workspace_bytes(ctypes.byref(p))])
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    pp = ctypes.byref(p)
    L = qk._lib
    common = (d["indptr"].data_ptr(), d["indices"].data_ptr(), d["lens"].data_ptr(), out.data_ptr(),
              lse.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    qp = d["q"].data_ptr()

    def check(st):
        if st != 0:
            raise RuntimeError(qk.last_error())

    def make_step(strm):
        """One step (layer l) launched on the HIP stream handle strm."""
        com = common[:-1] + (strm,)
        if fmt == "fp8":
            fp8p = [t.data_ptr() for t in d["fp8"]]
            return lambda l: check(L.mla_decode_fp8(pp, qp, fp8p[l], 1.0, *com))
        nvp = [(a.data_ptr(), s.data_ptr()) for a, s in d["nv"]]
        if w.write_tokens:
            def wstep(l):
                check(L.kv_quantize_nvfp4(wsrc.data_ptr(), qk.MLAQ_FP8_E4M3, 1.0, w.write_tokens,
                                          wslots.data_ptr(), nvp[l][0], nvp[l][1], w.pool_tokens, 1.0, strm))
                check(L.mla_decode_nvfp4(pp, qp, nvp[l][0], nvp[l][1], 1.0, *com))
            return wstep
        return lambda l: check(L.mla_decode_nvfp4(pp, qp, nvp[l][0], nvp[l][1], 1.0, *com))

    if fmt == "fp8":
        kv_bytes = w.batch * w.kv_len * FP8_ROW
    else:
        nvp = [(a.data_ptr(), s.data_ptr()) for a, s in d["nv"]]
        if w.write_tokens:
            wsrc = torch.from_numpy(synth.write_source_fp8(w)).cuda()
            wslots = torch.from_numpy(synth.slot_mapping(w, pt)).cuda()
        kv_bytes = w.batch * w.kv_len * NV_ROW
    step = make_step(stream)

    ms, split_ms, merge_ms, ms_ev = timed_steps(step, n_layers, args.steps, args.warmup, hip, torch)
    achieved = kv_bytes / (split_ms * 1e-3) / 1e9
    value = kv_bytes / (ms * 1e-3) / 1e9
    kernel_tag = f"mla_decode_kernel_{w.name}"
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {fmt.upper()} paged MLA decode, batch {w.batch} x {w.heads} heads, "
                               f"context {w.kv_len}, page {w.page_size}, pool {w.pool_tokens} x 576"
                               + (f", plus quantize-on-write of {w.write_tokens} tokens" if w.write_tokens else ""),
                   "kv_format": fmt, "batch": w.batch, "heads": w.heads, "kv_len": w.kv_len,
                   "page_size": w.page_size, "pool_tokens": w.pool_tokens, "num_splits": splits,
                   "layers_cycled": n_layers, "kv_bytes_per_step": kv_bytes},
        "steps_per_s": round(1000.0 / ms, 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "kernels_us": {"split": round(split_ms * 1e3, 2), "merge": round(merge_ms * 1e3, 2),
                       "step_with_kernel_events": round(ms_ev * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": pmc_traffic(kernel_tag, kv_bytes), "kernel": "mla_decode_kernel",
                     "bytes_per_launch": kv_bytes},
    }

    if not args.no_extras:
        res["read_probe"] = read_probe(qk, torch, achieved)
        res["graph"] = graph_steps(make_step, n_layers, args.steps, torch, kv_bytes)

    if args.copy_calibration:
        # a plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE per dispatch give the
        # counters' bytes-per-byte scale
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_extras and fmt == "fp8":
        # the same batch, requantized to NVFP4 with the library's own write path
        nv_live = w.batch * w.kv_len * NV_ROW
        nl = max(2, int(np.ceil(600e6 / nv_live)))
        data = torch.empty((w.pool_tokens, 288), dtype=torch.uint8, device="cuda")
        scales = torch.empty((w.pool_tokens, 36), dtype=torch.uint8, device="cuda")
        slots = torch.arange(w.pool_tokens, dtype=torch.int64, device="cuda")
        qk.kv_quantize_nvfp4(d["fp8"][0], qk.MLAQ_FP8_E4M3, 1.0, slots, data, scales, 1.0)
        nvs = [(data, scales)] + [(data.clone(), scales.clone()) for _ in range(nl - 1)]
        nvp = [(a.data_ptr(), s.data_ptr()) for a, s in nvs]
        nstep = lambda l: check(L.mla_decode_nvfp4(pp, qp, nvp[l][0], nvp[l][1], 1.0, *common))
        nms, nsplit, nmerge, _ = timed_steps(nstep, nl, args.steps, args.warmup, hip, torch)
        res["nvfp4_same_batch"] = {"ms_per_step": round(nms, 5), "steps_per_s": round(1000 / nms, 1),
                                   "num_splits": qk.mlaq_decode_num_splits(p, qk.MLAQ_NVFP4),
                                   "kv_gbs": round(nv_live / (nms * 1e-3) / 1e9, 1),
                                   "split_kernel_gbs": round(nv_live / (nsplit * 1e-3) / 1e9, 1),
                                   "speedup_vs_fp8": round(ms / nms, 3)}
        del nvs, data, scales
        # the pages' path: cast the whole FP8 pool to BF16 every layer, then a 16-bit decode
        bf = torch.empty((w.pool_tokens, 576), dtype=torch.bfloat16, device="cuda")
        fp8p = [t.data_ptr() for t in d["fp8"]]

        def cstep(l):
            check(L.kv_dequantize(qk.MLAQ_FP8_E4M3, fp8p[l], None, 1.0, None, w.pool_tokens, w.pool_tokens,
                                  qk.MLAQ_BF16, bf.data_ptr(), stream))
            check(L.mla_decode_bf16(pp, qp, bf.data_ptr(), *common))
        cms, _, _, _ = timed_steps(cstep, n_layers, max(20, args.steps // 4), 5, hip, torch, profile=False)
        res["cast_baseline"] = {"ms_per_step": round(cms, 5), "steps_per_s": round(1000 / cms, 1),
                                "bytes_moved_per_step": w.pool_tokens * (FP8_ROW + BF16_ROW) + w.batch * w.kv_len * BF16_ROW,
                                "speedup_of_fp8_path": round(cms / ms, 2)}
        del bf
        # the pages' intermediate fix: gather and cast only the active rows to a dense BF16
        # workspace, then a 16-bit decode over it (identity page table into the workspace)
        P = w.page_size
        tok = np.arange(w.kv_len, dtype=np.int64)
        rows_h = np.concatenate([pt.kv_indices[pt.kv_indptr[b] + tok // P].astype(np.int64) * P + tok % P
                                 for b in range(w.batch)])
        rows = torch.from_numpy(rows_h).cuda()
        n_act = rows_h.shape[0]
        gbf = torch.empty((n_act, 576), dtype=torch.bfloat16, device="cuda")
        gind = torch.arange(n_act // P, dtype=torch.int32, device="cuda")
        gptr = torch.arange(w.batch + 1, dtype=torch.int32, device="cuda") * (w.kv_len // P)
        gp = qk.decode_params(w.batch, w.heads, P, w.kv_len, n_act, w.sm_scale)
        gpp = ctypes.byref(gp)
        gcommon = (gptr.data_ptr(), gind.data_ptr(), d["lens"].data_ptr(), out.data_ptr(), lse.data_ptr(),
                   ws.data_ptr(), ws.numel(), stream)

        def gstep(l):
            check(L.kv_dequantize(qk.MLAQ_FP8_E4M3, fp8p[l], None, 1.0, rows.data_ptr(), n_act, w.pool_tokens,
                                  qk.MLAQ_BF16, gbf.data_ptr(), stream))
            check(L.mla_decode_bf16(gpp, qp, gbf.data_ptr(), *gcommon))
        gms, _, _, _ = timed_steps(gstep, n_layers, max(20, args.steps // 4), 20, hip, torch, profile=False)
        res["gather_cast_baseline"] = {"ms_per_step": round(gms, 5), "steps_per_s": round(1000 / gms, 1),
                                       "bytes_moved_per_step": n_act * (FP8_ROW + 8 + 2 * BF16_ROW),
                                       "speedup_of_fp8_path": round(gms / ms, 2)}
        del gbf, rows

    if not args.no_extras and fmt == "nvfp4":
        # one new token per request and step: the fused append-then-attend call against a
        # quantize-on-write launch for the B new rows followed by the decode
        P = w.page_size
        last = w.kv_len - 1
        rows_h = np.array([int(pt.kv_indices[pt.kv_indptr[b] + last // P]) * P + last % P for b in range(w.batch)],
                          dtype=np.int64)
        arows = torch.from_numpy(rows_h).cuda()
        nsrc = torch.from_numpy(synth.to_bf16_bits(synth.new_token_rows(w.seed, w.batch)).view(np.int16)).cuda()

        def fstep(l):
            check(L.mla_decode_nvfp4_append(pp, qp, nsrc.data_ptr(), qk.MLAQ_BF16, 1.0, nvp[l][0], nvp[l][1], 1.0,
                                            *common))

        def sstep(l):
            check(L.kv_quantize_nvfp4(nsrc.data_ptr(), qk.MLAQ_BF16, 1.0, w.batch, arows.data_ptr(), nvp[l][0],
                                      nvp[l][1], w.pool_tokens, 1.0, stream))
            check(L.mla_decode_nvfp4(pp, qp, nvp[l][0], nvp[l][1], 1.0, *common))
        fms, _, _, _ = timed_steps(fstep, n_layers, args.steps, 50, hip, torch, profile=False)
        sms, _, _, _ = timed_steps(sstep, n_layers, args.steps, 50, hip, torch, profile=False)
        res["append_fused"] = {"ms_per_step": round(fms, 5), "separate_ms_per_step": round(sms, 5),
                               "new_tokens_per_step": w.batch, "speedup_vs_separate": round(sms / fms, 3)}

        # extend (chunked prefill) over the cache: the first 4 requests take a 256-token chunk
        # after a prefix of the rest of their context (prefix dequantized to an FP8 workspace,
        # per-token causal views attended by the FP8 decode kernels, chunk written back)
        EB, EC = min(4, w.batch), 256
        EP = w.kv_len - EC
        nq = EB * EC
        tok = np.arange(EP, w.kv_len, dtype=np.int64)
        eslots = torch.from_numpy(np.concatenate(
            [pt.kv_indices[pt.kv_indptr[b] + tok // P].astype(np.int64) * P + tok % P for b in range(EB)])).cuda()
        eqo = torch.arange(EB + 1, dtype=torch.int32, device="cuda") * EC
        epl = torch.full((EB,), EP, dtype=torch.int32, device="cuda")
        eq = torch.from_numpy(synth.q_bits(w.seed + 7, nq, w.heads).view(np.int16)).cuda()
        eckv = torch.from_numpy(synth.to_fp8_bytes(synth.extend_chunk_rows(w.seed, nq))).cuda()
        ep = qk.extend_params(EB, w.heads, P, w.pool_tokens, nq, EP, EC, w.sm_scale)
        ews = torch.empty(qk.mlaq_extend_workspace_bytes(ep), dtype=torch.uint8, device="cuda")
        eout = torch.empty((nq, w.heads, 512), dtype=torch.float32, device="cuda")
        else_ = torch.empty((nq, w.heads), dtype=torch.float32, device="cuda")

        def estep(l):
            check(L.mla_extend_nvfp4(ctypes.byref(ep), eq.data_ptr(), eqo.data_ptr(), eckv.data_ptr(), 1.0,
                                     nvp[l][0], nvp[l][1], 1.0, d["indptr"].data_ptr(), d["indices"].data_ptr(),
                                     epl.data_ptr(), eslots.data_ptr(), eout.data_ptr(), else_.data_ptr(),
                                     ews.data_ptr(), ews.numel(), stream))
        ems, esplit, emerge, _ = timed_steps(estep, n_layers, 10, 3, hip, torch)
        eflops = EB * sum(2 * w.heads * (EP + i + 1) * (576 + 512) for i in range(EC))
        res["extend"] = {"requests": EB, "prefix_tokens": EP, "chunk_tokens": EC, "ms_per_call": round(ems, 4),
                         "chunk_tokens_per_s": round(nq / (ems * 1e-3), 1),
                         "attention_kernel_ms": round(esplit + emerge, 4),
                         "attention_tflops": round(eflops / ((esplit + emerge) * 1e-3) / 1e12, 1),
                         "frac_of_fp16_mfma_peak": round(eflops / ((esplit + emerge) * 1e-3) / 2.5e15, 4),
                         "workspace_rows_read_per_call_gb": round(
                             EB * sum(EP + i + 1 for i in range(EC)) * FP8_ROW / 1e9, 2)}

        # initial prefill (the same call with empty prefixes): 4 prompts of 2,048 tokens, causal
        # attention over their own FP8 rows, then the NVFP4 write of all 8,192 rows
        PB, PC = min(4, w.batch), 2048
        pn = PB * PC
        ptok = np.arange(PC, dtype=np.int64)
        pslots = torch.from_numpy(np.concatenate(
            [pt.kv_indices[pt.kv_indptr[b] + ptok // P].astype(np.int64) * P + ptok % P for b in range(PB)])).cuda()
        pqo = torch.arange(PB + 1, dtype=torch.int32, device="cuda") * PC
        ppl = torch.zeros((PB,), dtype=torch.int32, device="cuda")
        pq = torch.from_numpy(synth.q_bits(w.seed + 8, pn, w.heads).view(np.int16)).cuda()
        pkv = torch.from_numpy(synth.to_fp8_bytes(synth.extend_chunk_rows(w.seed + 1, pn))).cuda()
        pp_ = qk.extend_params(PB, w.heads, P, w.pool_tokens, pn, 0, PC, w.sm_scale)
        pws = torch.empty(qk.mlaq_extend_workspace_bytes(pp_), dtype=torch.uint8, device="cuda")
        pout = torch.empty((pn, w.heads, 512), dtype=torch.float32, device="cuda")
        plse = torch.empty((pn, w.heads), dtype=torch.float32, device="cuda")

        def pstep(l):
            check(L.mla_extend_nvfp4(ctypes.byref(pp_), pq.data_ptr(), pqo.data_ptr(), pkv.data_ptr(), 1.0,
                                     nvp[l][0], nvp[l][1], 1.0, d["indptr"].data_ptr(), d["indices"].data_ptr(),
                                     ppl.data_ptr(), pslots.data_ptr(), pout.data_ptr(), plse.data_ptr(),
                                     pws.data_ptr(), pws.numel(), stream))
        pms, psplit, pmerge, _ = timed_steps(pstep, n_layers, 10, 3, hip, torch)
        pflops = PB * sum(2 * w.heads * (i + 1) * (576 + 512) for i in range(PC))
        res["prefill"] = {"requests": PB, "prompt_tokens": PC, "ms_per_call": round(pms, 4),
                          "prompt_tokens_per_s": round(pn / (pms * 1e-3), 1),
                          "attention_kernel_ms": round(psplit + pmerge, 4),
                          "attention_tflops": round(pflops / ((psplit + pmerge) * 1e-3) / 1e12, 1),
                          "frac_of_fp16_mfma_peak": round(pflops / ((psplit + pmerge) * 1e-3) / 2.5e15, 4)}

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, pt, host, nvfp4=(fmt == "nvfp4"))
    print(json.dumps(res))


if __name__ == "__main__":
    main()
