"""fp64 CPU oracle (ctypes wrapper over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the bench's CPU-baseline leg, never by the product package.  It shares no
code with the HIP path; inputs come from ``synth`` (seeded, no method
arithmetic) and every definition here is written out from the pages in
``oracle.c``.
"""
from __future__ import annotations

import ctypes
import functools
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle.so")

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_d = ctypes.c_double
_f = ctypes.c_float


@functools.lru_cache(maxsize=1)
def lib():
    if not os.path.exists(LIB):
        raise ImportError(f"{LIB} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    sig = {
        "orc_bf16_to_f64": ([ctypes.c_uint16], _d),
        "orc_f64_to_bf16": ([_d], ctypes.c_uint16),
        "orc_round_bf16": ([_p, _i64, _p], None),
        "orc_bf16_array_to_f64": ([_p, _i64, _p], None),
        "orc_yarn_table": ([_d, _i32, _d, _i64, _i64, _d, _d, _d, _p, _p, _p, _p], _i32),
        "orc_rope": ([_p, _i64, _i32, _i32, _i64, _i32, _p, _p, _d, _p], None),
        "orc_rope_bf16": ([_p, _i64, _i32, _i32, _i64, _i32, _p, _p, _d, _p], None),
        "orc_gather_paged": ([_p, _i64, _i32, _i32, _i64, _p, _i64, _p], _i32),
        "orc_e2m1_value": ([_i32], _d),
        "orc_e4m3_value": ([_i32], _d),
        "orc_nvfp4_tensor_scale": ([_p, _i64], _f),
        "orc_nvfp4_quantize": ([_p, _i64, _i32, _i32, _f, _p, _p], None),
        "orc_nvfp4_pack": ([_p, _i64, _p], None),
        "orc_nvfp4_dequantize": ([_p, _p, _i64, _i32, _i32, _f, _p], None),
        "orc_f16_value": ([ctypes.c_uint16], _d),
        "orc_f64_to_f16_sat": ([_d], ctypes.c_uint16),
        "orc_int8_quantize": ([_p, _i64, _i32, _i32, _p, _p], None),
        "orc_int8_dequantize": ([_p, _p, _i64, _i32, _i32, _p], None),
        "orc_decode_attention": ([_p, _i32, _i32, _i32, _i64, _i32, _p, _p, _p, _p, _f, _f, _d,
                                  _p, _p], _i32),
        "orc_prefill_attention": ([_p, _p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _f, _f,
                                   _d, _p], _i32),
        "orc_num_threads": ([], _i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


# --- bf16 helpers -----------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    a, p = _c(bits, np.uint16)
    out = np.empty(a.shape, dtype=np.float64)
    lib().orc_bf16_array_to_f64(p, a.size, out.ctypes.data)
    return out


def round_bf16(x) -> np.ndarray:
    a, p = _c(x, np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_round_bf16(p, a.size, out.ctypes.data)
    return out


# --- C1 / C2 -------------------------------------------------------------------

class YarnTable:
    def __init__(self, inv_freq, mscale, low, high):
        self.inv_freq, self.mscale, self.low, self.high = inv_freq, mscale, low, high


def yarn_table(rope_theta=1e7, rotary_dim=64, factor=4.0, original_max_position=262144,
               correction_max_position=0, beta_fast=32.0, beta_slow=1.0,
               mscale=0.0) -> YarnTable:
    inv = np.empty(rotary_dim // 2, dtype=np.float64)
    ms, lo, hi = _d(), _i32(), _i32()
    rc = lib().orc_yarn_table(rope_theta, rotary_dim, factor, original_max_position,
                              correction_max_position, beta_fast, beta_slow, mscale,
                              inv.ctypes.data, ctypes.byref(ms), ctypes.byref(lo),
                              ctypes.byref(hi))
    if rc:
        raise ValueError("yarn parameters outside the definition's domain")
    return YarnTable(inv, ms.value, lo.value, hi.value)


def rope(x_bits, positions, table: YarnTable, rotary_dim=64, bf16_out=False):
    """x_bits: uint16 [T, H, D]; positions: [T].  fp64 [T, H, D] or bf16 bits."""
    x, px = _c(x_bits, np.uint16)
    T, H, D = x.shape
    pos, pp = _c(positions, np.int64)
    assert pos.shape == (T,)
    inv, pi = _c(table.inv_freq, np.float64)
    if bf16_out:
        y = np.empty((T, H, D), dtype=np.uint16)
        lib().orc_rope_bf16(px, T, H, D, H * D, rotary_dim, pp, pi, table.mscale, y.ctypes.data)
    else:
        y = np.empty((T, H, D), dtype=np.float64)
        lib().orc_rope(px, T, H, D, H * D, rotary_dim, pp, pi, table.mscale, y.ctypes.data)
    return y


# --- C3 -------------------------------------------------------------------------

def gather_paged(pool_bytes: np.ndarray, num_blocks, nheads, block_size, row_bytes, table, ntok):
    pool, pp = _c(pool_bytes, np.uint8)
    tab, pt = _c(table, np.int32)
    out = np.empty((ntok, nheads, row_bytes), dtype=np.uint8)
    rc = lib().orc_gather_paged(pp, num_blocks, nheads, block_size, row_bytes, pt, ntok,
                                out.ctypes.data)
    if rc:
        raise IndexError("block table entry outside the pool")
    return out


# --- C4 -------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def nvfp4_tensor_scale(x_bits) -> np.float32:
    x, p = _c(x_bits, np.uint16)
    return np.float32(lib().orc_nvfp4_tensor_scale(p, x.size))


def nvfp4_quantize(x_bits, S):
    """x_bits uint16 [T, H, D] -> (codes uint8 [T, H, D], scales uint8 [T, H, D/16])."""
    x, p = _c(x_bits, np.uint16)
    T, H, D = x.shape
    codes = np.empty((T, H, D), dtype=np.uint8)
    scales = np.empty((T, H, D // 16), dtype=np.uint8)
    lib().orc_nvfp4_quantize(p, T, H, D, float(S), codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def nvfp4_pack(codes) -> np.ndarray:
    c, p = _c(codes, np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] // 2,), dtype=np.uint8)
    lib().orc_nvfp4_pack(p, c.size // 2, out.ctypes.data)
    return out


def nvfp4_dequantize(codes, scales, S) -> np.ndarray:
    c, pc = _c(codes, np.uint8)
    s, ps = _c(scales, np.uint8)
    T, H, D = c.shape
    out = np.empty((T, H, D), dtype=np.float64)
    lib().orc_nvfp4_dequantize(pc, ps, T, H, D, float(S), out.ctypes.data)
    return out


def f16_value(bits: int) -> float:
    return lib().orc_f16_value(bits)


def f64_to_f16_sat(x: float) -> int:
    """Non-negative x -> nearest binary16 bit pattern, ties to even, saturating at 65504."""
    return int(lib().orc_f64_to_f16_sat(x))


def int8_quantize(x_bits):
    """INT8 group-64: x_bits uint16 [T, H, D] -> (codes int8 [T, H, D], scales
    uint16 binary16 bits [T, H, D/64])."""
    x, p = _c(x_bits, np.uint16)
    T, H, D = x.shape
    codes = np.empty((T, H, D), dtype=np.int8)
    scales = np.empty((T, H, D // 64), dtype=np.uint16)
    lib().orc_int8_quantize(p, T, H, D, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def int8_dequantize(codes, scales) -> np.ndarray:
    c, pc = _c(codes, np.int8)
    s, ps = _c(scales, np.uint16)
    T, H, D = c.shape
    out = np.empty((T, H, D), dtype=np.float64)
    lib().orc_int8_dequantize(pc, ps, T, H, D, out.ctypes.data)
    return out


# --- C5 / C6 --------------------------------------------------------------------

def _kv_args(k, v, nvfp4, int8):
    """(kind, k array, v array, k scales, v scales, kS, vS) for the C oracle."""
    if nvfp4 is not None:
        return (1, _c(k, np.uint8), _c(v, np.uint8), _c(nvfp4[0], np.uint8),
                _c(nvfp4[1], np.uint8), float(nvfp4[2]), float(nvfp4[3]))
    if int8 is not None:
        return (2, _c(k, np.int8), _c(v, np.int8), _c(int8[0], np.uint16), _c(int8[1], np.uint16),
                1.0, 1.0)
    return 0, _c(k, np.uint16), _c(v, np.uint16), (None, None), (None, None), 1.0, 1.0


def decode_attention(q, k, v, scale=None, nvfp4=None, int8=None, with_lse=False):
    """q: fp64 [Hq, D] (roped).  bf16 cache: k, v uint16 [N, Hkv, D].
    NVFP4 cache: nvfp4=(k_scales, v_scales, kS, vS) and k, v are codes [N, Hkv, D].
    INT8 cache: int8=(k_scales, v_scales) (binary16 bits [N, Hkv, D/64]) and
    k, v are int8 codes [N, Hkv, D]."""
    qa, pq = _c(q, np.float64)
    Hq, D = qa.shape
    kind, (ka, pk), (va, pv), (_, pks), (_, pvs), kS, vS = _kv_args(k, v, nvfp4, int8)
    N, Hkv, _ = ka.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((Hq, D), dtype=np.float64)
    lse = np.empty(Hq, dtype=np.float64)
    rc = lib().orc_decode_attention(pq, Hq, Hkv, D, N, kind, pk, pv, pks, pvs, kS, vS, scale,
                                    out.ctypes.data, lse.ctypes.data)
    if rc:
        raise ValueError("bad decode_attention arguments")
    return (out, lse) if with_lse else out


def prefill_attention(q, positions, k, v, scale=None, nvfp4=None, int8=None):
    """q fp64 [R, Hq, D]; row r attends to cached tokens 0..positions[r]."""
    qa, pq = _c(q, np.float64)
    R, Hq, D = qa.shape
    pos, pp = _c(positions, np.int64)
    kind, (ka, pk), (va, pv), (_, pks), (_, pvs), kS, vS = _kv_args(k, v, nvfp4, int8)
    Hkv = ka.shape[1]
    assert ka.shape[0] >= int(pos.max()) + 1
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((R, Hq, D), dtype=np.float64)
    rc = lib().orc_prefill_attention(pq, pp, R, Hq, Hkv, D, kind, pk, pv, pks, pvs, kS, vS, scale,
                                     out.ctypes.data)
    if rc:
        raise ValueError("bad prefill_attention arguments")
    return out


def num_threads() -> int:
    """Threads the oracle's parallel loops run on."""
    return int(lib().orc_num_threads())


def kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_element, batch=1):
    """KV bytes per token: layers x batch x 2 (K and V) x kv_heads x head_dim x bytes."""
    return layers * batch * 2 * kv_heads * head_dim * bytes_per_element
