"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no attention, rope or quantisation arithmetic: it maps
(seed, stream, element index) to bf16 bit patterns through the counter form of
SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) and a 65,536-entry table of
N(0,1) quantiles, plus the seeded integer structure of the workloads (block
permutations, outlier channel sets, needle positions).  ``synth_host.c`` and
``synth_dev.hip`` implement the same element definition for the host and the
device; tests compare the two on sampled slices.
"""
from __future__ import annotations

import ctypes
import functools
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

# Streams within one seed: tensor id + 64 * layer (or session).
Q, K, V, K_OUTLIER, V_OUTLIER, Q_OUTLIER = 0, 1, 2, 3, 4, 5


def stream_id(layer: int, tensor: int) -> int:
    return 64 * int(layer) + int(tensor)


def outlier_threshold(p: float) -> int:
    """Bernoulli(p) as an integer test on the top 24 bits of a draw."""
    return int(round(p * (1 << 24)))


@functools.lru_cache(maxsize=1)
def normal_table() -> np.ndarray:
    """bf16 bit patterns of the N(0,1) quantiles at (i + 0.5) / 65536.

    fp64 quantile (scipy ndtri) -> fp32 (RNE) -> bf16 (RNE).  It is a table
    definition, used identically by both sides.
    """
    from scipy.special import ndtri

    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    f = ndtri(p).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


@functools.lru_cache(maxsize=1)
def _host():
    if not os.path.exists(HOST_LIB):
        raise ImportError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(HOST_LIB)
    lib.synth_draws.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                ctypes.c_void_p]
    lib.synth_draws.restype = None
    lib.synth_fill_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                    ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p]
    lib.synth_fill_bf16.restype = None
    return lib


@functools.lru_cache(maxsize=1)
def _dev():
    if not os.path.exists(DEV_LIB):
        raise ImportError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
    import torch  # noqa: F401  (bind to the HIP runtime torch already loaded)
    lib = ctypes.CDLL(DEV_LIB)
    lib.synth_dev_fill_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                        ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.synth_dev_fill_bf16.restype = ctypes.c_int
    return lib


def draws(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    _host().synth_draws(seed, stream, start, count, out.ctypes.data)
    return out


def host_fill(seed, stream, token0, ntok, nheads, dim, chan_mul=None, outlier_stream=0,
              outlier_p=0.0, outlier_mul=1.0) -> np.ndarray:
    """bf16 bit patterns [ntok, nheads, dim] for logical tokens token0.. of one tensor."""
    out = np.empty((ntok, nheads, dim), dtype=np.uint16)
    tab = normal_table()
    cm = None
    if chan_mul is not None:
        cm = np.ascontiguousarray(chan_mul, dtype=np.float32).reshape(nheads * dim)
    _host().synth_fill_bf16(seed, stream, token0, ntok, nheads, dim, tab.ctypes.data,
                            cm.ctypes.data if cm is not None else None, outlier_stream,
                            outlier_threshold(outlier_p), outlier_mul, out.ctypes.data)
    return out


_dev_tables = {}


def dev_fill(out, seed, stream, token0, ntok, nheads, dim, chan_mul=None, outlier_stream=0,
             outlier_p=0.0, outlier_mul=1.0):
    """Device twin of host_fill, writing into ``out`` (a CUDA tensor of 2-byte elements)."""
    import torch

    dev = out.device
    if dev not in _dev_tables:
        _dev_tables[dev] = torch.from_numpy(normal_table().view(np.int16)).to(dev)
    tab = _dev_tables[dev]
    cm = None
    if chan_mul is not None:
        cm = torch.as_tensor(np.ascontiguousarray(chan_mul, dtype=np.float32).reshape(-1),
                             device=dev)
    assert out.is_contiguous() and out.element_size() == 2
    assert out.numel() >= ntok * nheads * dim
    rc = _dev().synth_dev_fill_bf16(seed, stream, token0, ntok, nheads, dim, tab.data_ptr(),
                                    cm.data_ptr() if cm is not None else None, outlier_stream,
                                    outlier_threshold(outlier_p), outlier_mul, out.data_ptr(),
                                    torch.cuda.current_stream(dev).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill_bf16 failed (status {rc})")
    return out


def block_permutation(seed: int, num_blocks: int) -> np.ndarray:
    """A seeded permutation of pool block ids (int32)."""
    rng = np.random.Generator(np.random.PCG64([seed, 0x5EED]))
    return rng.permutation(num_blocks).astype(np.int32)


def outlier_channels(seed: int, layer: int, tensor: int, nheads: int, dim: int, count: int,
                     mul: float) -> np.ndarray:
    """Per-head multipliers [nheads, dim]: ``count`` seeded channels per head get ``mul``."""
    rng = np.random.Generator(np.random.PCG64([seed, layer, tensor, 0xC4A7]))
    m = np.ones((nheads, dim), dtype=np.float32)
    for h in range(nheads):
        m[h, rng.choice(dim, size=count, replace=False)] = mul
    return m


def needle_position(seed: int, layer: int, n_ctx: int) -> int:
    rng = np.random.Generator(np.random.PCG64([seed, layer, 0x0EED1E]))
    return int(rng.integers(0, n_ctx))
