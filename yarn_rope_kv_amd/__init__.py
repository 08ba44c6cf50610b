"""YaRN-roped, GQA, paged long-context attention for MI355X (gfx950).

A thin ctypes binding over ``libyrk.so`` (C ABI in ``include/yrk.h``).  The
functions here only marshal arguments: torch tensors provide device memory
and the current HIP stream; every step of the computation runs in the HIP
kernels behind the C ABI.  There is no CPU fallback: importing this package
fails if the library is not built.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libyrk.so")

OK, EINVAL, ERANGE, ENOTSUP, ENOSPC, EDEVICE = 0, -1, -2, -3, -4, -5
DEVERR_BLOCK_ID, DEVERR_POSITION = 1, 2
KV_BF16, KV_NVFP4, KV_INT8 = 0, 1, 2
OUT_BF16, OUT_F32 = 0, 1
HEAD_DIM, BLOCK_SIZE = 256, 16

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build()); "
                      "there is no fallback path")
# torch brings its own HIP runtime.  Load it before libyrk so that libyrk's
# libamdhip64 dependency resolves to that same, already-loaded runtime: two
# HIP runtimes in one process do not share devices, memory or streams.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


class YrkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.yrk_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


class _YarnParamsC(ctypes.Structure):
    _fields_ = [("rope_theta", ctypes.c_double), ("head_dim", ctypes.c_int32),
                ("rotary_dim", ctypes.c_int32), ("factor", ctypes.c_double),
                ("original_max_position", ctypes.c_int64),
                ("correction_max_position", ctypes.c_int64), ("beta_fast", ctypes.c_double),
                ("beta_slow", ctypes.c_double), ("mscale", ctypes.c_double)]


class _KvLayerC(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("paged", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("k_tensor_scale_dev", ctypes.c_void_p), ("v_tensor_scale_dev", ctypes.c_void_p)]


_P = ctypes.c_void_p
_i32, _i64, _f = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIGS = {
    "yrk_abi_version": ([], ctypes.c_int),
    "yrk_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "yrk_yarn_table": ([ctypes.POINTER(_YarnParamsC), _P, _P, _P, _P], ctypes.c_int),
    "yrk_yarn_rope_apply": ([ctypes.POINTER(_YarnParamsC), _P, _i64, _i32, _i64, _P, _P, _P],
                            ctypes.c_int),
    "yrk_nvfp4_tensor_scale": ([_P, _i64, _P, _P], ctypes.c_int),
    "yrk_kv_append_quantize": ([ctypes.POINTER(_KvLayerC), _P, _P, _i64, _P, _i64, _P, _P, _P],
                               ctypes.c_int),
    "yrk_rope_append": ([ctypes.POINTER(_KvLayerC), ctypes.POINTER(_YarnParamsC), _P, _i32, _i64,
                         _P, _P, _i64, _P, _i64, _P, _P, _P], ctypes.c_int),
    "yrk_decode_workspace_size": ([_i32, _i32, _i32, _i32, _i64], ctypes.c_size_t),
    "yrk_decode_attention": ([ctypes.POINTER(_KvLayerC), _P, _i32, _i32, _P, _i64, _P, _i64, _f,
                              _P, _i32, _P, ctypes.c_size_t, _P, _P], ctypes.c_int),
    "yrk_decode_attention_noalloc": ([ctypes.POINTER(_KvLayerC), _P, _i32, _i32, _P, _i64, _P,
                                      _i64, _f, _P, _i32, _P, _P], ctypes.c_int),
    "yrk_verify_workspace_size": ([_i32, _i32, _i32, _i32, _i32, _i64], ctypes.c_size_t),
    "yrk_verify_attention": ([ctypes.POINTER(_KvLayerC), _P, _i32, _i32, _i32, _P, _i64, _P, _i64,
                              _f, _P, _i32, _P, ctypes.c_size_t, _P, _P], ctypes.c_int),
    "yrk_prefill_workspace_size": ([_i64, _i32, _i32], ctypes.c_size_t),
    "yrk_prefill_attention": ([ctypes.POINTER(_KvLayerC), _P, _i64, _i32, _i64, _P, _i64, _f, _P,
                               _P, ctypes.c_size_t, _P, _P], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


def exported_symbols():
    return sorted(_SIGS)


def _check(status, where):
    if status != OK:
        raise YrkError(status, where)


def _nbytes(t):
    return t.numel() * t.element_size()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


@dataclasses.dataclass
class YarnParams:
    """YaRN parameters (see yrk_yarn_params in include/yrk.h)."""
    rope_theta: float = 1e7
    head_dim: int = 256
    rotary_dim: int = 64
    factor: float = 4.0
    original_max_position: int = 262144
    correction_max_position: int = 0
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 0.0

    def c(self):
        return _YarnParamsC(**dataclasses.asdict(self))


def yarn_table(params: YarnParams):
    """(inv_freq[rotary_dim/2] fp64, mscale, corr_low, corr_high) from the library."""
    inv = np.empty(params.rotary_dim // 2, dtype=np.float64)
    ms = ctypes.c_double()
    lo, hi = ctypes.c_int32(), ctypes.c_int32()
    cp = params.c()
    _check(_lib.yrk_yarn_table(ctypes.byref(cp), inv.ctypes.data, ctypes.byref(ms),
                               ctypes.byref(lo), ctypes.byref(hi)), "yrk_yarn_table")
    return inv, ms.value, lo.value, hi.value


def yarn_rope_apply(params: YarnParams, x, positions, err=None):
    """Rotate x in place.  x: bf16 [T, H, head_dim] (token stride x.stride(0)),
    positions: int32 [T] on the same device; err: optional uint32 device word."""
    T, H, D = x.shape
    assert x.stride(2) == 1 and x.stride(1) == D, "heads must be contiguous rows"
    cp = params.c()
    _check(_lib.yrk_yarn_rope_apply(ctypes.byref(cp), x.data_ptr(), T, H, x.stride(0),
                                    positions.data_ptr(), _ptr(err), _stream(x)),
           "yrk_yarn_rope_apply")
    return x


def nvfp4_tensor_scale(x, out):
    """out (fp32 [1], device) = amax(|x|) / 2688, or 1 when x is all zero."""
    _check(_lib.yrk_nvfp4_tensor_scale(x.data_ptr(), x.numel(), out.data_ptr(), _stream(x)),
           "yrk_nvfp4_tensor_scale")
    return out


class KVLayer:
    """One layer's cache in torch-owned device memory (layouts in include/yrk.h)."""

    def __init__(self, dtype, num_kv_heads, num_blocks, paged, k, v, k_scale=None,
                 v_scale=None, k_tensor_scale=None, v_tensor_scale=None):
        self.dtype, self.num_kv_heads, self.num_blocks, self.paged = (dtype, num_kv_heads,
                                                                      num_blocks, paged)
        self.k, self.v = k, v
        self.k_scale, self.v_scale = k_scale, v_scale
        self.k_tensor_scale, self.v_tensor_scale = k_tensor_scale, v_tensor_scale

    @classmethod
    def allocate(cls, dtype, num_kv_heads, num_blocks, paged=True, device="cuda"):
        import torch
        shape = (num_blocks, num_kv_heads, BLOCK_SIZE) if paged else \
            (num_blocks * BLOCK_SIZE, num_kv_heads)
        if dtype == KV_BF16:
            k = torch.empty(shape + (HEAD_DIM,), dtype=torch.bfloat16, device=device)
            v = torch.empty_like(k)
            return cls(dtype, num_kv_heads, num_blocks, paged, k, v)
        if dtype == KV_INT8:
            k = torch.empty(shape + (HEAD_DIM,), dtype=torch.int8, device=device)
            v = torch.empty_like(k)
            ks = torch.empty(shape + (HEAD_DIM // 64,), dtype=torch.float16, device=device)
            vs = torch.empty_like(ks)
            return cls(dtype, num_kv_heads, num_blocks, paged, k, v, ks, vs)
        k = torch.empty(shape + (HEAD_DIM // 2,), dtype=torch.uint8, device=device)
        v = torch.empty_like(k)
        ks = torch.empty(shape + (HEAD_DIM // 16,), dtype=torch.uint8, device=device)
        vs = torch.empty_like(ks)
        kts = torch.ones(1, dtype=torch.float32, device=device)
        vts = torch.ones(1, dtype=torch.float32, device=device)
        return cls(dtype, num_kv_heads, num_blocks, paged, k, v, ks, vs, kts, vts)

    def c(self):
        return _KvLayerC(self.dtype, self.num_kv_heads, HEAD_DIM, BLOCK_SIZE, self.num_blocks,
                         1 if self.paged else 0, 0, _ptr(self.k), _ptr(self.v),
                         _ptr(self.k_scale), _ptr(self.v_scale), _ptr(self.k_tensor_scale),
                         _ptr(self.v_tensor_scale))


def kv_append_quantize(layer: KVLayer, k, v, block_table, positions, err=None):
    """Append k, v (bf16 [T, Hkv, 256], contiguous) at positions (int32 [T])."""
    T = k.shape[0]
    lc = layer.c()
    bt_len = block_table.numel() if block_table is not None else 0
    _check(_lib.yrk_kv_append_quantize(ctypes.byref(lc), k.data_ptr(), v.data_ptr(), T,
                                       _ptr(block_table), bt_len, positions.data_ptr(),
                                       _ptr(err), _stream(k)), "yrk_kv_append_quantize")


def rope_append(layer: KVLayer, params: YarnParams, q, k, v, block_table, positions, err=None):
    """One pass: q (bf16 [T, Hq, 256] or a strided view of rows, or None) roped
    in place at positions; k (not yet roped) and v (bf16 [T, Hkv, 256]) roped
    and appended at the same positions."""
    T = k.shape[0]
    lc, pc = layer.c(), params.c()
    if q is not None:
        if q.stride(2) != 1 or q.stride(1) != HEAD_DIM:
            raise YrkError(EINVAL, "rope_append: q heads must be contiguous rows")
        q_ptr, hq, q_stride = q.data_ptr(), q.shape[1], q.stride(0)
    else:
        q_ptr, hq, q_stride = None, 0, 0
    bt_len = block_table.numel() if block_table is not None else 0
    _check(_lib.yrk_rope_append(ctypes.byref(lc), ctypes.byref(pc), q_ptr, hq, q_stride,
                                k.data_ptr(), v.data_ptr(), T, _ptr(block_table), bt_len,
                                positions.data_ptr(), _ptr(err), _stream(k)), "yrk_rope_append")


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, max_seq_len, head_dim=HEAD_DIM):
    return int(_lib.yrk_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              max_seq_len))


def decode_attention(layer: KVLayer, q, block_tables, seq_lens, max_seq_len, out, workspace,
                     softmax_scale=0.0, err=None):
    """q: bf16 [S, Hq, 256]; block_tables: int32 [S, stride] (or None, contiguous);
    seq_lens: int32 [S]; out: bf16 or fp32 [S, Hq, 256]; workspace: uint8 tensor."""
    import torch
    S, Hq, _ = q.shape
    lc = layer.c()
    bt_stride = block_tables.shape[1] if block_tables is not None else 0
    out_dtype = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    _check(_lib.yrk_decode_attention(ctypes.byref(lc), q.data_ptr(), S, Hq, _ptr(block_tables),
                                     bt_stride, seq_lens.data_ptr(), max_seq_len,
                                     softmax_scale, out.data_ptr(), out_dtype,
                                     workspace.data_ptr(), _nbytes(workspace), _ptr(err),
                                     _stream(q)), "yrk_decode_attention")
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_attention_noalloc(layer: KVLayer, q, block_tables, seq_lens, max_seq_len, out,
                             softmax_scale=0.0, err=None):
    """decode_attention with the partials in the library's device scratch
    (no workspace, no allocation); calls on one GPU must not overlap."""
    import torch
    S, Hq, _ = q.shape
    lc = layer.c()
    bt_stride = block_tables.shape[1] if block_tables is not None else 0
    out_dtype = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    _check(_lib.yrk_decode_attention_noalloc(ctypes.byref(lc), q.data_ptr(), S, Hq,
                                             _ptr(block_tables), bt_stride, seq_lens.data_ptr(),
                                             max_seq_len, softmax_scale, out.data_ptr(),
                                             out_dtype, _ptr(err), _stream(q)),
           "yrk_decode_attention_noalloc")
    return out


def verify_workspace_size(num_seqs, num_queries, num_q_heads, num_kv_heads, max_seq_len,
                          head_dim=HEAD_DIM):
    return int(_lib.yrk_verify_workspace_size(num_seqs, num_queries, num_q_heads, num_kv_heads,
                                              head_dim, max_seq_len))


def verify_attention(layer: KVLayer, q, block_tables, seq_lens, max_seq_len, out, workspace,
                     softmax_scale=0.0, err=None):
    """q: bf16 [S, Q, Hq, 256], the last Q cached tokens of each sequence (query
    i at position seq_lens[s] - Q + i); block_tables: int32 [S, stride] (or
    None, contiguous); seq_lens: int32 [S]; out: bf16 or fp32 [S, Q, Hq, 256];
    workspace: uint8 tensor of verify_workspace_size() bytes."""
    import torch
    S, Q, Hq, _ = q.shape
    lc = layer.c()
    bt_stride = block_tables.shape[1] if block_tables is not None else 0
    out_dtype = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    _check(_lib.yrk_verify_attention(ctypes.byref(lc), q.data_ptr(), S, Q, Hq, _ptr(block_tables),
                                     bt_stride, seq_lens.data_ptr(), max_seq_len,
                                     softmax_scale, out.data_ptr(), out_dtype,
                                     workspace.data_ptr(), _nbytes(workspace), _ptr(err),
                                     _stream(q)), "yrk_verify_attention")
    return out


def prefill_workspace_size(num_q_tokens, num_q_heads, head_dim=HEAD_DIM):
    return int(_lib.yrk_prefill_workspace_size(num_q_tokens, num_q_heads, head_dim))


def prefill_attention(layer: KVLayer, q, q_start_position, block_table, out, workspace=None,
                      softmax_scale=0.0, err=None):
    """q: bf16 [T, Hq, 256] at positions q_start_position + i; out: bf16 like q.
    workspace: device buffer of prefill_workspace_size(T, Hq) bytes (allocated
    here when not given)."""
    T, Hq, _ = q.shape
    if workspace is None and T > 0:
        workspace = torch.empty(max(prefill_workspace_size(T, Hq), 4), dtype=torch.uint8,
                                device=q.device)
    lc = layer.c()
    bt_len = block_table.numel() if block_table is not None else 0
    _check(_lib.yrk_prefill_attention(ctypes.byref(lc), q.data_ptr(), T, Hq, q_start_position,
                                      _ptr(block_table), bt_len, softmax_scale, out.data_ptr(),
                                      _ptr(workspace),
                                      _nbytes(workspace) if workspace is not None else 0,
                                      _ptr(err), _stream(q)), "yrk_prefill_attention")
    return out
