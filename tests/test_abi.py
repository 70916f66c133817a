"""C-ABI checks that need no GPU: the library loads, exports every function include/mlaq.h
declares, rejects bad arguments with the documented status before any launch, and plans
splits / workspace on the host."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from conftest import ROOT

qk = pytest.importorskip("quantized_kv_paged_amd")
from quantized_kv_paged_amd import DecodeParams, MlaqError  # noqa: E402

HEADER = os.path.join(ROOT, "include", "mlaq.h")
ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_VALUE = 1, 2, 3, 4, 5, 7


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_functions_are_exported():
    names = _declared_functions()
    assert {"mla_decode_fp8", "mla_decode_nvfp4", "kv_quantize_nvfp4", "kv_dequantize"} <= set(names)
    lib = ctypes.CDLL(qk.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", qk.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, flags=re.M), n
    assert set(qk.EXPORTS) == set(names)


def _declarations():
    """{name: (return type, [parameter types])} of every function the header declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for ret, name, args in re.findall(r"^\s*((?:const\s+)?[a-z_0-9]+\s*\**)\s*([a-z_0-9]+)\s*\(([^;{]*?)\)\s*;",
                                      text, flags=re.M | re.S):
        types = []
        for a in " ".join(args.split()).split(","):
            a = a.strip()
            if a in ("", "void"):
                continue
            t = re.sub(r"\s*\b[a-z_0-9]+$", "", a)          # drop the parameter name
            types.append(re.sub(r"\s*\*", "*", t))
        out[name] = (re.sub(r"\s*\*", "*", ret.strip()), types)
    return out


# The calls of the boundary as the hot-path scope table writes them (plan() inputs, separate q and
# KV formats, pool rows of 576, global scale as a scalar), with the documented deviations applied:
# kv_dequantize takes pool_tokens after num_rows so that a device-resident row list can be
# range-checked without a fault.
_BOUNDARY = {
    "mlaq_decode_workspace_bytes": ("size_t", ["const mlaq_decode_params*"]),
    "mla_decode_fp8": ("mlaq_status", ["const mlaq_decode_params*", "const uint16_t*", "const uint8_t*", "float",
                                       "const int32_t*", "const int32_t*", "const int32_t*", "float*", "float*",
                                       "void*", "size_t", "hipStream_t"]),
    "mla_decode_nvfp4": ("mlaq_status", ["const mlaq_decode_params*", "const uint16_t*", "const uint8_t*",
                                         "const uint8_t*", "float", "const int32_t*", "const int32_t*",
                                         "const int32_t*", "float*", "float*", "void*", "size_t", "hipStream_t"]),
    "mla_decode_bf16": ("mlaq_status", ["const mlaq_decode_params*", "const uint16_t*", "const uint16_t*",
                                        "const int32_t*", "const int32_t*", "const int32_t*", "float*", "float*",
                                        "void*", "size_t", "hipStream_t"]),
    "kv_quantize_nvfp4": ("mlaq_status", ["const void*", "mlaq_format", "float", "int64_t", "const int64_t*",
                                          "uint8_t*", "uint8_t*", "int64_t", "float", "hipStream_t"]),
    "kv_dequantize": ("mlaq_status", ["mlaq_format", "const uint8_t*", "const uint8_t*", "float", "const int64_t*",
                                      "int64_t", "int64_t", "mlaq_format", "void*", "hipStream_t"]),
    "mlaq_last_error": ("const char*", []),
}
# Calls beyond the table, each documented in the header: the per-format sizes and split counts,
# the fused append, extend / prefill, the allocation-free decode, and the measurement aids.
_ADDED = {"mlaq_decode_format_workspace_bytes", "mlaq_decode_num_splits", "mla_decode_nvfp4_append",
          "mlaq_decode_nvfp4_append_workspace_bytes", "mla_extend_nvfp4", "mlaq_extend_workspace_bytes",
          "mlaq_extend_num_splits", "mlaq_set_profile_events", "mlaq_read_probe", "mlaq_version",
          "mla_decode_nvfp4_noalloc"}


def test_boundary_signatures():
    decl = _declarations()
    for name, sig in _BOUNDARY.items():
        assert decl.get(name) == sig, (name, decl.get(name))
    extra = set(decl) - set(_BOUNDARY)
    assert extra <= _ADDED, extra - _ADDED


def test_params_layout_and_status_codes():
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} mlaq_decode_params;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"([a-z_0-9]+)\s+([a-z_0-9]+)\s*;", body)
    assert fields == [("int32_t", "batch"), ("int32_t", "num_heads"), ("int32_t", "page_size"),
                      ("int64_t", "pool_tokens"), ("int32_t", "max_kv_len"), ("int32_t", "num_splits"),
                      ("float", "sm_scale")]
    assert [f for f, _ in DecodeParams._fields_] == [n for _, n in fields]
    # the binding's layout is the C compiler's
    src = ("#include <stdio.h>\n#include <stddef.h>\n#include \"mlaq.h\"\nint main(void) { printf(\"%zu"
           + " %zu" * len(fields) + "\\n\", sizeof(mlaq_decode_params)"
           + "".join(f", offsetof(mlaq_decode_params, {n})" for _, n in fields) + "); return 0; }\n")
    import tempfile
    with tempfile.TemporaryDirectory() as td:
        c, exe = os.path.join(td, "l.c"), os.path.join(td, "l")
        open(c, "w").write(src)
        r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                            "-I", "/opt/rocm/include", c, "-o", exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    assert got == [ctypes.sizeof(DecodeParams)] + [getattr(DecodeParams, n).offset for _, n in fields]
    codes = dict((n, int(v)) for n, v in re.findall(r"(MLAQ_(?:OK|ERR_[A-Z]+))\s*=\s*(\d+)", text))
    assert codes == {"MLAQ_OK": 0, "MLAQ_ERR_NULL": 1, "MLAQ_ERR_SHAPE": 2, "MLAQ_ERR_ALIGN": 3,
                     "MLAQ_ERR_UNSUPPORTED": 4, "MLAQ_ERR_WORKSPACE": 5, "MLAQ_ERR_LAUNCH": 6, "MLAQ_ERR_VALUE": 7}


def _p(**kw):
    d = dict(batch=2, num_heads=16, page_size=64, max_kv_len=4096, pool_tokens=1 << 16, num_splits=0,
             sm_scale=0.07)
    d.update(kw)
    return DecodeParams(**d)


FAKE = 1 << 20  # a 256-byte aligned fake device address; never dereferenced on these paths


def _fp8(p, q=FAKE, kv=FAKE, scale=1.0, indptr=FAKE, indices=FAKE, lens=FAKE, out=FAKE, lse=FAKE, ws=FAKE,
         ws_bytes=1 << 30):
    return qk._lib.mla_decode_fp8(ctypes.byref(p), q, kv, scale, indptr, indices, lens, out, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=8), ERR_SHAPE), (dict(num_heads=24), ERR_SHAPE), (dict(num_heads=144), ERR_SHAPE),
    (dict(page_size=0), ERR_SHAPE), (dict(page_size=2048), ERR_SHAPE), (dict(page_size=48), ERR_SHAPE),
    (dict(batch=-1), ERR_SHAPE),
    (dict(batch=70000), ERR_SHAPE), (dict(max_kv_len=-5), ERR_SHAPE), (dict(pool_tokens=0), ERR_SHAPE),
    (dict(num_splits=2000), ERR_SHAPE), (dict(sm_scale=float("nan")), ERR_VALUE),
])
def test_param_validation(kw, status):
    assert _fp8(_p(**kw)) == status
    assert qk.last_error() != ""


def test_pointer_and_value_validation():
    p = _p()
    assert qk._lib.mla_decode_fp8(None, FAKE, FAKE, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == ERR_NULL
    assert _fp8(p, q=None) == ERR_NULL
    assert _fp8(p, kv=None) == ERR_NULL
    assert _fp8(p, indices=None) == ERR_NULL
    assert _fp8(p, out=None) == ERR_NULL
    assert _fp8(p, q=FAKE + 8) == ERR_ALIGN
    assert _fp8(p, kv=FAKE + 4) == ERR_ALIGN
    assert _fp8(p, lens=FAKE + 2) == ERR_ALIGN
    assert _fp8(p, scale=0.0) == ERR_VALUE
    assert _fp8(p, scale=float("inf")) == ERR_VALUE
    assert _fp8(p, ws=None) == ERR_NULL
    need = qk.mlaq_decode_workspace_bytes(p, qk.MLAQ_FP8_E4M3)
    assert need > 0 and qk.mlaq_decode_workspace_bytes(p) >= need
    assert _fp8(p, ws_bytes=need - 1) == ERR_WORKSPACE
    assert _fp8(p, ws=FAKE + 16) == ERR_ALIGN
    assert "workspace" in qk.last_error()
    assert _fp8(_p(batch=0)) == 0                       # empty batch is a no-op
    st = qk._lib.mla_decode_nvfp4(ctypes.byref(p), FAKE, FAKE, None, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  1 << 30, None)
    assert st == ERR_NULL
    st = qk._lib.mla_decode_nvfp4(ctypes.byref(p), FAKE, FAKE, FAKE + 2, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  1 << 30, None)
    assert st == ERR_ALIGN


def test_quantize_and_dequantize_validation():
    L = qk._lib
    assert L.kv_quantize_nvfp4(FAKE, 3, 1.0, 8, FAKE, FAKE, FAKE, 64, 1.0, None) == ERR_UNSUPPORTED
    assert L.kv_quantize_nvfp4(FAKE, 2, 1.0, 8, FAKE, FAKE, FAKE, 64, 1.0, None) == ERR_UNSUPPORTED
    assert L.kv_quantize_nvfp4(FAKE, 1, 1.0, 8, FAKE, FAKE, FAKE, 64, 0.0, None) == ERR_VALUE
    assert L.kv_quantize_nvfp4(FAKE, 1, float("nan"), 8, FAKE, FAKE, FAKE, 64, 1.0, None) == ERR_VALUE
    assert L.kv_quantize_nvfp4(None, 1, 1.0, 8, FAKE, FAKE, FAKE, 64, 1.0, None) == ERR_NULL
    assert L.kv_quantize_nvfp4(FAKE + 4, 1, 1.0, 8, FAKE, FAKE, FAKE, 64, 1.0, None) == ERR_ALIGN
    assert L.kv_quantize_nvfp4(FAKE, 1, 1.0, -1, FAKE, FAKE, FAKE, 64, 1.0, None) == ERR_SHAPE
    assert L.kv_quantize_nvfp4(FAKE, 1, 1.0, 0, None, None, None, 64, 1.0, None) == 0
    assert L.kv_dequantize(0, FAKE, None, 1.0, None, 4, 64, 0, FAKE, None) == ERR_UNSUPPORTED
    assert L.kv_dequantize(1, FAKE, None, 1.0, None, 4, 64, 1, FAKE, None) == ERR_UNSUPPORTED  # FP8 -> FP8
    assert L.kv_dequantize(1, FAKE, FAKE, 1.0, None, 4, 64, 0, FAKE, None) == ERR_UNSUPPORTED  # scales w/ FP8
    assert L.kv_dequantize(2, FAKE, None, 1.0, None, 4, 64, 0, FAKE, None) == ERR_NULL
    assert L.kv_dequantize(2, FAKE, FAKE, -1.0, None, 4, 64, 0, FAKE, None) == ERR_VALUE
    assert L.kv_dequantize(2, FAKE, FAKE, 1.0, None, 65, 64, 0, FAKE, None) == ERR_SHAPE
    assert L.kv_dequantize(2, FAKE, FAKE, 1.0, None, 4, 64, 0, FAKE + 8, None) == ERR_ALIGN
    with pytest.raises(MlaqError) as e:
        qk._check(L.kv_dequantize(2, FAKE, FAKE, 1.0, None, 65, 64, 0, FAKE, None))
    assert e.value.status == ERR_SHAPE and "num_rows" in str(e.value)


def test_read_probe_validation():
    L = qk._lib
    assert L.mlaq_read_probe(FAKE, 24, FAKE, 8, None) == ERR_SHAPE      # not whole 16-byte words
    assert L.mlaq_read_probe(FAKE, -16, FAKE, 8, None) == ERR_SHAPE
    assert L.mlaq_read_probe(FAKE, 64, FAKE, 0, None) == ERR_SHAPE
    assert L.mlaq_read_probe(None, 64, FAKE, 8, None) == ERR_NULL
    assert L.mlaq_read_probe(FAKE, 64, None, 8, None) == ERR_NULL
    assert L.mlaq_read_probe(FAKE + 8, 64, FAKE, 8, None) == ERR_ALIGN


def test_split_planning_and_workspace():
    import synth
    # (FP8 plan, NVFP4 plan): FP8 workgroups stream 64-token tiles, two per CU; NVFP4
    # workgroups stream 32-token tiles, four per CU
    expect = {"tiny_fp8": (8, 16), "fp8_32k": (64, 128), "nvfp4_32k": (11, 23), "nvfp4_160k": (51, 101),
              "nvfp4_1m": (256, 512)}
    for name, w in synth.WORKLOADS.items():
        p = _p(batch=w.batch, num_heads=w.heads, page_size=w.page_size, max_kv_len=w.kv_len,
               pool_tokens=w.pool_tokens)
        for fmt, want in zip((qk.MLAQ_FP8_E4M3, qk.MLAQ_NVFP4), expect[name]):
            s = qk.mlaq_decode_num_splits(p, fmt)
            assert s == want, (name, fmt, s)
            ws = qk.mlaq_decode_workspace_bytes(p, fmt)
            slots = w.batch * s * (w.heads // 16)
            assert ws == ((slots * (16 * 512 * 4 + 32 * 4) + 255) // 256) * 256
        assert qk.mlaq_decode_num_splits(p, qk.MLAQ_BF16) == expect[name][0]
        slots = w.batch * expect[name][0] * (w.heads // 16)
        assert qk.mlaq_decode_workspace_bytes(p, qk.MLAQ_BF16) == ((slots * (16 * 512 * 4 + 32 * 4) + 255) // 256) * 256
    for fmt in (qk.MLAQ_FP8_E4M3, qk.MLAQ_NVFP4, qk.MLAQ_BF16):
        assert qk.mlaq_decode_num_splits(_p(max_kv_len=32), fmt) == 1
        assert qk.mlaq_decode_workspace_bytes(_p(max_kv_len=32), fmt) == 0
        assert qk.mlaq_decode_num_splits(_p(num_splits=7), fmt) == 7
        assert qk.mlaq_decode_num_splits(_p(num_heads=20), fmt) == 0
        with pytest.raises(MlaqError):
            qk.mlaq_decode_workspace_bytes(_p(num_heads=20), fmt)
    assert qk.mlaq_decode_num_splits(_p(), qk.MLAQ_FP32) == 0          # not a decode KV format
    with pytest.raises(MlaqError):
        qk.mlaq_decode_workspace_bytes(_p(), qk.MLAQ_FP32)
    # the format-free size serves every format
    for name, w in synth.WORKLOADS.items():
        p = _p(batch=w.batch, num_heads=w.heads, page_size=w.page_size, max_kv_len=w.kv_len,
               pool_tokens=w.pool_tokens)
        assert qk.mlaq_decode_workspace_bytes(p) == max(
            qk.mlaq_decode_workspace_bytes(p, f) for f in (qk.MLAQ_FP8_E4M3, qk.MLAQ_NVFP4, qk.MLAQ_BF16))
    with pytest.raises(MlaqError):
        qk.mlaq_decode_workspace_bytes(_p(num_heads=20))


def test_split_planning_follows_the_measured_sweep():
    # forced-split sweeps of the decode step (split kernel + merge) on MI355X, recorded in
    # profiles/mla_decode_kernel_split_counts.md: the fastest count at each shape (at 16 x 4K the
    # plan's 32 was 3 % behind 43).  Small batches run fastest on one workgroup per CU with a few
    # tiles each, large ones on every slot filled once.
    fastest = {("nvfp4", 8, 32768): 128, ("nvfp4", 44, 32768): 23, ("nvfp4", 10, 163840): 101,
               ("nvfp4", 2, 1048576): 512, ("fp8", 8, 32768): 64, ("fp8", 2, 1048576): 256,
               ("nvfp4", 8, 4096): 32, ("nvfp4", 1, 32768): 256, ("nvfp4", 4, 8192): 64,
               ("nvfp4", 2, 16384): 128, ("nvfp4", 16, 4096): 32, ("nvfp4", 32, 1024): 8}
    for (fmt, batch, ctx), want in fastest.items():
        p = _p(batch=batch, max_kv_len=ctx, pool_tokens=batch * ctx, page_size=64)
        code = qk.MLAQ_NVFP4 if fmt == "nvfp4" else qk.MLAQ_FP8_E4M3
        assert qk.mlaq_decode_num_splits(p, code) == want, (fmt, batch, ctx)


def test_split_token_cap():
    """No split covers more than MLAQ_MAX_SPLIT_TOKENS tokens: forced counts below
    ceil(max_kv_len / cap) are rejected before any launch, and the automatic plan never goes there."""
    cap = 1 << 14
    for L in (cap, cap + 1, 65536, 1 << 20, 1 << 24):
        need = -(-L // cap)
        for fmt in (qk.MLAQ_FP8_E4M3, qk.MLAQ_NVFP4, qk.MLAQ_BF16):
            for b in (1, 2, 64):
                s = qk.mlaq_decode_num_splits(_p(batch=b, max_kv_len=L), fmt)
                assert s >= need and -(-L // s) <= cap, (L, fmt, b, s)
        if need > 1:
            assert _fp8(_p(max_kv_len=L, num_splits=need - 1)) == ERR_SHAPE
            assert "splits" in qk.last_error()
            assert qk.mlaq_decode_num_splits(_p(max_kv_len=L, num_splits=need - 1), qk.MLAQ_NVFP4) == 0
        assert qk.mlaq_decode_num_splits(_p(max_kv_len=L, num_splits=need), qk.MLAQ_NVFP4) == need
    assert _fp8(_p(max_kv_len=(1 << 24) + 1)) == ERR_SHAPE              # above MLAQ_MAX_KV_LEN
    # extend: rows seen per split are capped the same way
    big = _ext_p(max_prefix_len=65536 - 32, max_chunk_len=32)
    assert qk._lib.mlaq_extend_num_splits(ctypes.byref(big)) >= 4
    assert _ext(_ext_p(max_prefix_len=65536 - 32, max_chunk_len=32, num_splits=3)) == ERR_SHAPE
    assert qk._lib.mlaq_extend_num_splits(ctypes.byref(_ext_p(max_prefix_len=65536 - 32, max_chunk_len=32,
                                                              num_splits=4))) == 4


def _app(p, new_kv=FAKE, fmt=0, src_scale=1.0, data=FAKE, scales=FAKE, g=1.0, ws=FAKE, ws_bytes=1 << 30):
    return qk._lib.mla_decode_nvfp4_append(ctypes.byref(p), FAKE, new_kv, fmt, src_scale, data, scales, g, FAKE,
                                           FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_append_validation_and_workspace():
    p = _p()
    assert _app(p, fmt=qk.MLAQ_NVFP4) == ERR_UNSUPPORTED
    assert _app(p, fmt=qk.MLAQ_FP32) == ERR_UNSUPPORTED
    assert _app(p, fmt=qk.MLAQ_FP8_E4M3, src_scale=0.0) == ERR_VALUE
    assert _app(p, new_kv=None) == ERR_NULL
    assert _app(p, new_kv=FAKE + 8) == ERR_ALIGN
    assert _app(p, scales=None) == ERR_NULL
    assert _app(p, g=float("nan")) == ERR_VALUE
    assert _app(_p(num_heads=24)) == ERR_SHAPE
    assert _app(_p(batch=0), new_kv=None) == 0          # empty batch is a no-op
    # the merge pass always runs and every request has one more partial slot (its new token):
    # even one split needs the workspace
    slot = 16 * 512 * 4 + 32 * 4
    one = _p(max_kv_len=32)
    assert qk.mlaq_decode_num_splits(one, qk.MLAQ_NVFP4) == 1
    need = qk._lib.mlaq_decode_nvfp4_append_workspace_bytes(ctypes.byref(one))
    assert need == ((2 * 2 * slot + 255) // 256) * 256
    assert _app(one, ws=None) == ERR_NULL
    assert _app(one, ws_bytes=need - 1) == ERR_WORKSPACE
    many = _p()
    s = qk.mlaq_decode_num_splits(many, qk.MLAQ_NVFP4)
    assert s > 1
    assert qk._lib.mlaq_decode_nvfp4_append_workspace_bytes(ctypes.byref(many)) == ((2 * (s + 1) * slot + 255) // 256) * 256
    assert qk._lib.mlaq_decode_nvfp4_append_workspace_bytes(ctypes.byref(_p(num_heads=20))) == ctypes.c_size_t(-1).value


def _ext_p(**kw):
    d = dict(batch=2, num_heads=16, page_size=64, pool_tokens=1 << 16, num_q=64, max_prefix_len=4096,
             max_chunk_len=32, num_splits=0, sm_scale=0.07)
    d.update(kw)
    return qk.extend_params(d["batch"], d["num_heads"], d["page_size"], d["pool_tokens"], d["num_q"],
                            d["max_prefix_len"], d["max_chunk_len"], d["sm_scale"], d["num_splits"])


def _ext(p, q=FAKE, qo=FAKE, ckv=FAKE, cs=1.0, data=FAKE, scales=FAKE, g=1.0, slots=FAKE, out=FAKE, ws=FAKE,
         ws_bytes=1 << 34):
    return qk._lib.mla_extend_nvfp4(ctypes.byref(p), q, qo, ckv, cs, data, scales, g, FAKE, FAKE, FAKE, slots, out,
                                    FAKE, ws, ws_bytes, None)


def test_extend_validation_and_workspace():
    p = _ext_p()
    assert _ext(_ext_p(num_heads=8)) == ERR_SHAPE
    assert _ext(_ext_p(num_q=70000)) == ERR_SHAPE
    assert _ext(_ext_p(max_prefix_len=-1)) == ERR_SHAPE
    assert _ext(_ext_p(max_chunk_len=0)) == ERR_SHAPE              # num_q > 0 needs a chunk
    assert _ext(_ext_p(page_size=48)) == ERR_SHAPE
    assert _ext(_ext_p(pool_tokens=0)) == ERR_SHAPE
    assert _ext(_ext_p(num_q=65535, max_prefix_len=1 << 25, max_chunk_len=1 << 25)) == ERR_SHAPE   # int32 views
    assert _ext(p, cs=0.0) == ERR_VALUE
    assert _ext(p, g=float("inf")) == ERR_VALUE
    assert _ext(p, q=None) == ERR_NULL
    assert _ext(p, slots=None) == ERR_NULL
    assert _ext(p, ckv=FAKE + 8) == ERR_ALIGN
    assert _ext(p, slots=FAKE + 4) == ERR_ALIGN
    assert _ext(p, ws=None) == ERR_NULL
    need = qk.mlaq_extend_workspace_bytes(p)
    assert _ext(p, ws_bytes=need - 1) == ERR_WORKSPACE
    assert _ext(p, ws=FAKE + 16) == ERR_ALIGN
    assert _ext(_ext_p(num_q=0), q=None, qo=None, ckv=None) == 0    # nothing to do
    # workspace: one FP8 region of round_up(prefix + chunk, 64) rows per request, the per-token
    # lengths and page offsets, then the partials of the KV splits per 16-head group
    region = -(-(4096 + 32) // 64) * 64
    a256 = lambda x: -(-x // 256) * 256
    base = a256(2 * region * 576) + a256(64 * 4) + a256(65 * 4)
    for heads in (16, 64):
        ph = _ext_p(num_heads=heads)
        s = qk._lib.mlaq_extend_num_splits(ctypes.byref(ph))
        assert s >= 1
        assert qk.mlaq_extend_workspace_bytes(ph) == base + (
            a256(64 * s * (heads // 16) * (16 * 512 * 4 + 32 * 4)) if s > 1 else 0)
    assert need == qk.mlaq_extend_workspace_bytes(_ext_p(num_heads=16))
    assert qk._lib.mlaq_extend_workspace_bytes(ctypes.byref(_ext_p(num_heads=20))) == ctypes.c_size_t(-1).value


def test_product_path_never_loads_the_oracle():
    """Importing the package (and the benchmark's helpers it needs) loads libmlaq.so and
    nothing from oracle/: no CPU path stands behind the calls.  The package source names no
    oracle module either."""
    code = ("import sys; import quantized_kv_paged_amd as qk; "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "print(qk.LIB_PATH); assert not bad, bad")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().endswith("libmlaq.so")
    pkg = os.path.join(ROOT, "quantized_kv_paged_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\bimport\s+oracle|\bfrom\s+oracle\b", text), f


def test_oracle_shares_nothing_with_the_hip_path():
    """oracle/ imports, includes and links nothing from the GPU package (its C twin is built
    from its own source only)."""
    odir = os.path.join(ROOT, "oracle")
    for f in os.listdir(odir):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(odir, f)).read()
            assert not re.search(r"import\s+quantized_kv_paged_amd|from\s+quantized_kv_paged_amd|libmlaq|csrc/|mlaq\.h",
                                 text), f


def test_noalloc_validation():
    """The allocation-free decode rejects, before any launch or device query, what the workspace call
    rejects and plans whose partials do not fit its 48 MiB scratch."""
    L = qk._lib

    def na(p, q=FAKE, data=FAKE, scales=FAKE, g=1.0):
        return L.mla_decode_nvfp4_noalloc(ctypes.byref(p), q, data, scales, g, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert na(_p(num_heads=24)) == ERR_SHAPE
    assert na(_p(max_kv_len=65536, num_splits=1)) == ERR_SHAPE          # per-split token cap
    assert na(_p(batch=4, max_kv_len=32768, num_splits=512)) == ERR_WORKSPACE   # forced: 4 x 512 slots
    assert "scratch" in qk.last_error()
    assert na(_p(batch=2000, max_kv_len=1 << 20)) == ERR_WORKSPACE      # 64 splits at least: 4.2 GB
    assert na(_p(batch=0)) == 0
