"""NVFP4 block quantizer and dequantizer (oracle).

Test infrastructure (see oracle/__init__.py).

Format (NVFP4 article, section "NVFP4 format: two-level scaling"): values are E2M1,
each block of 16 values carries one E4M3 scale, and the tensor carries one FP32
global scale; 16 values occupy 8 bytes of codes plus 1 scale byte.  The write path
(implementation item 1) quantizes FP8 KV to NVFP4 when it is stored; the accuracy
section runs with the global scale left at 1.0.

The pages give the format but not the quantizer's arithmetic.  Readings taken here
(each listed in the design doc):
  * a block is 16 consecutive dims of one 576-dim row (36 blocks per row);
  * block scale = E4M3(RNE, saturating) of (amax / 6) / g, all in fp32;
  * effective divisor sd = decoded scale * g (fp32); codes = E2M1(RNE, saturating)
    of x / sd in fp32 (true division, no fused multiply-add);
  * sd == 0 -> all codes 0; a NaN anywhere in the block -> scale byte 0x7F, codes 0;
  * packed byte j of a row = code(2j) | code(2j+1) << 4 (even dim in the low nibble);
  * the global scale g multiplies on dequantization: x = e2m1 * e4m3 * g.

Two implementations of the same steps: `quantize_block` (pure Python, for small cases
and the pins) and the C file nvfp4_ref.c (for pool-sized inputs), loaded here with
ctypes.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import codecs

BLOCK = 16
ROW_DIMS = 576
ROW_BLOCKS = ROW_DIMS // BLOCK          # 36
ROW_DATA_BYTES = ROW_DIMS // 2          # 288
ROW_SCALE_BYTES = ROW_BLOCKS            # 36

_f32 = np.float32


def quantize_block(x: list[float] | np.ndarray, g: float) -> tuple[int, list[int]]:
    """One 16-value block (fp32 values) -> (scale byte, 16 E2M1 codes)."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape == (BLOCK,)
    g32 = _f32(g)
    if np.isnan(x).any():
        return 0x7F, [0] * BLOCK
    a = _f32(np.max(np.abs(x)))
    sf = _f32(_f32(a / _f32(6.0)) / g32)
    sb = codecs.e4m3_encode(float(sf))
    sd = _f32(_f32(codecs.e4m3_decode(sb)) * g32)
    if sd == 0:
        return sb, [0] * BLOCK
    codes = []
    for v in x:
        y = _f32(v / sd)
        codes.append(codecs.e2m1_encode(float(y)))
    return sb, codes


def pack_codes(codes: list[int]) -> bytes:
    """Pairs of codes -> bytes, even position in the low nibble."""
    return bytes((codes[2 * j] & 0xF) | ((codes[2 * j + 1] & 0xF) << 4) for j in range(len(codes) // 2))


def quantize_row_py(row: np.ndarray, g: float) -> tuple[bytes, bytes]:
    """One 576-value fp32 row -> (288 packed bytes, 36 scale bytes), pure Python."""
    data, scales = b"", b""
    for k in range(ROW_BLOCKS):
        sb, codes = quantize_block(row[k * BLOCK:(k + 1) * BLOCK], g)
        data += pack_codes(codes)
        scales += bytes([sb])
    return data, scales


def dequant_nvfp4_f64(data: np.ndarray, scales: np.ndarray, g: float) -> np.ndarray:
    """fp64 values of NVFP4 rows: x[d] = e2m1(code d) * e4m3(scale of block d // 16) * g."""
    data = np.asarray(data, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lo = codecs.e2m1_decode_np(data & 0xF)
    hi = codecs.e2m1_decode_np(data >> 4)
    vals = np.empty(data.shape[:-1] + (data.shape[-1] * 2,), dtype=np.float64)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    s = np.repeat(codecs.e4m3_decode_np(scales), BLOCK, axis=-1)
    return vals * s * float(np.float32(g))


def dequant_fp8_f64(codes: np.ndarray, scale: float) -> np.ndarray:
    """fp64 values of FP8 rows: e4m3(code) * per-tensor scale."""
    return codecs.e4m3_decode_np(codes) * float(np.float32(scale))


# ---------------------------------------------------------------- C twin (large inputs)

_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_nvfp4_ref.so")


def build_c(force: bool = False) -> str:
    """Compile nvfp4_ref.c with gcc (plain IEEE fp32: no fast-math, no contraction)."""
    src = os.path.join(_HERE, "nvfp4_ref.c")
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(src):
        import subprocess
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math", "-o", tmp, src, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        _LIB = ctypes.CDLL(build_c())
        _LIB.oracle_nvfp4_quantize_f32_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                                        ctypes.c_void_p, ctypes.c_void_p]
        _LIB.oracle_fp8_rows_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
        _LIB.oracle_bf16_rows_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        _LIB.oracle_e2m1_encode_f32.argtypes = [ctypes.c_float]
        _LIB.oracle_e2m1_encode_f32.restype = ctypes.c_int
        _LIB.oracle_e4m3_encode_f32.argtypes = [ctypes.c_float]
        _LIB.oracle_e4m3_encode_f32.restype = ctypes.c_int
        _LIB.oracle_e4m3_encode_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        _LIB.oracle_nvfp4_dequant_f32_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                       ctypes.c_float, ctypes.c_void_p]
    return _LIB


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def fp8_rows_to_f32(codes: np.ndarray, src_scale: float) -> np.ndarray:
    """FP8 source rows -> fp32 values fl32(e4m3(code) * src_scale) (write-path input)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float32)
    _lib().oracle_fp8_rows_to_f32(_ptr(codes), codes.size, src_scale, _ptr(out))
    return out


def bf16_rows_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    _lib().oracle_bf16_rows_to_f32(_ptr(bits), bits.size, _ptr(out))
    return out


def quantize_rows(x: np.ndarray, g: float) -> tuple[np.ndarray, np.ndarray]:
    """fp32 rows [n, 576] -> (codes uint8 [n, 288], scales uint8 [n, 36]) with the C twin."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.ndim == 2 and x.shape[1] == ROW_DIMS
    n = x.shape[0]
    data = np.empty((n, ROW_DATA_BYTES), dtype=np.uint8)
    scales = np.empty((n, ROW_SCALE_BYTES), dtype=np.uint8)
    _lib().oracle_nvfp4_quantize_f32_rows(_ptr(x), n, g, _ptr(data), _ptr(scales))
    return data, scales


def quantize_fp8_rows(codes: np.ndarray, src_scale: float, g: float) -> tuple[np.ndarray, np.ndarray]:
    """The write path from an FP8 source: decode with the per-tensor scale, then quantize."""
    return quantize_rows(fp8_rows_to_f32(codes, src_scale), g)


def quantize_bf16_rows(bits: np.ndarray, g: float) -> tuple[np.ndarray, np.ndarray]:
    return quantize_rows(bf16_rows_to_f32(bits), g)


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    """Element-wise e4m3fn encode (nearest, ties to even, saturating) of an fp32 array."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _lib().oracle_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def dequant_nvfp4_f32(data: np.ndarray, scales: np.ndarray, g: float) -> np.ndarray:
    """fp32 dequantized rows: fl32(fl32(e2m1 * e4m3) * g) (the product itself is exact)."""
    data = np.ascontiguousarray(data, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n = data.shape[0]
    out = np.empty((n, ROW_DIMS), dtype=np.float32)
    _lib().oracle_nvfp4_dequant_f32_rows(_ptr(data), _ptr(scales), n, g, _ptr(out))
    return out


def e2m1_encode_c(y: float) -> int:
    return _lib().oracle_e2m1_encode_f32(y)


def e4m3_encode_c(x: float) -> int:
    return _lib().oracle_e4m3_encode_f32(x)


def calibrated_global_scale(amax: float) -> float:
    """g = amax / (6 * 448) in fp32 (the calibrated NVFP4 workload)."""
    return float(_f32(_f32(amax) / _f32(2688.0)))


def nvfp4_bytes_per_value() -> float:
    return (BLOCK / 2 + 1) / BLOCK

