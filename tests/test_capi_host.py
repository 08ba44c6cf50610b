"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, computes the host-only YaRN table like the oracle, and rejects bad
arguments before enqueueing anything (no GPU needed: none of these calls
reaches a launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import yarn_rope_kv_amd as Y

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "yrk.h")


def test_every_declared_symbol_is_exported():
    text = open(HEADER).read()
    declared = set(re.findall(r"^(?:int|size_t|const char\*)\s+(yrk_\w+)\(", text, re.M))
    assert len(declared) >= 10
    assert declared == set(Y.exported_symbols())
    for name in declared:
        assert hasattr(Y._lib, name)
    assert Y._lib.yrk_abi_version() == 2


@pytest.mark.parametrize("orig,corr,factor", [(262144, 0, 4.0), (262144, 1048576, 4.0),
                                              (1024, 0, 4.0), (4096, 0, 1.0), (32768, 0, 16.0)])
def test_library_table_matches_oracle(orig, corr, factor):
    p = Y.YarnParams(original_max_position=orig, correction_max_position=corr, factor=factor)
    inv, ms, lo, hi = Y.yarn_table(p)
    t = O.yarn_table(original_max_position=orig, correction_max_position=corr, factor=factor)
    assert (lo, hi) == (t.low, t.high)
    assert ms == pytest.approx(t.mscale, rel=1e-15)
    assert np.allclose(inv, t.inv_freq, rtol=4e-16, atol=0)


@pytest.mark.parametrize("base", [1.0000001, 1.001])
def test_library_table_matches_oracle_near_base_one(base):
    """Correction-range ends far outside the int range: the same table."""
    inv, _, lo, hi = Y.yarn_table(Y.YarnParams(rope_theta=base))
    t = O.yarn_table(rope_theta=base)
    assert np.allclose(inv, t.inv_freq, rtol=4e-16, atol=0)
    assert hi == t.high


def _rope(p, x=0x1000, T=1, H=24, stride=24 * 256, pos=0x2000, err=None):
    cp = p.c()
    return Y._lib.yrk_yarn_rope_apply(ctypes.byref(cp), x, T, H, stride, pos, err, None)


@pytest.mark.parametrize("kw", [dict(factor=0.5), dict(factor=65.0), dict(factor=float("nan")),
                                dict(rotary_dim=63), dict(rotary_dim=258), dict(rope_theta=1.0),
                                dict(original_max_position=0), dict(beta_fast=0.5),
                                dict(mscale=float("inf"))])
def test_rope_rejects_bad_params(kw):
    assert _rope(Y.YarnParams(**kw)) == Y.EINVAL


@pytest.mark.parametrize("d", [258, 512, 8192])
def test_rotary_tables_beyond_the_library_are_refused(d):
    """head_dim = rotary_dim past the 128-pair table (and, for the fused pass,
    past 64 dims): ENOTSUP, returned before the table is built, with the
    process alive (these once overran a stack array)."""
    p = Y.YarnParams(head_dim=d, rotary_dim=d)
    assert _rope(p, stride=24 * d) == Y.ENOTSUP
    L = _layer()
    pc = p.c()
    assert Y._lib.yrk_rope_append(ctypes.byref(L), ctypes.byref(pc), 0x8000, 24, 24 * 256,
                                  0x100, 0x200, 4, 0x400, 4, 0x300, None, None) == Y.ENOTSUP


def test_rope_rejects_bad_shapes_and_nulls():
    p = Y.YarnParams()
    assert _rope(p, stride=24 * 256 - 1) == Y.EINVAL
    assert _rope(p, x=None) == Y.EINVAL
    assert _rope(p, pos=None) == Y.EINVAL
    assert _rope(p, T=-1) == Y.EINVAL
    assert _rope(p, x=None, T=0) == Y.OK   # nothing to do, nothing touched


def _layer(**kw):
    base = dict(dtype=Y.KV_BF16, num_kv_heads=4, head_dim=256, block_size=16, num_blocks=64,
                paged=1, reserved=0, k=0x10000, v=0x20000, k_scale=None, v_scale=None,
                k_tensor_scale_dev=None, v_tensor_scale_dev=None)
    base.update(kw)
    return Y._KvLayerC(**base)


def _decode(layer, S=1, Hq=24, bt=0x3000, stride=64, lens=0x4000, max_len=1024, out=0x5000,
            out_dtype=Y.OUT_BF16, ws=0x6000, ws_bytes=1 << 30, q=0x7000, scale=0.0):
    return Y._lib.yrk_decode_attention(ctypes.byref(layer), q, S, Hq, bt, stride, lens, max_len,
                                       scale, out, out_dtype, ws, ws_bytes, None, None)


def test_decode_validation():
    L = _layer()
    assert _decode(_layer(head_dim=128)) == Y.ENOTSUP
    assert _decode(_layer(block_size=32)) == Y.ENOTSUP
    assert _decode(_layer(dtype=7)) == Y.EINVAL
    assert _decode(_layer(reserved=1)) == Y.EINVAL
    assert _decode(_layer(dtype=Y.KV_NVFP4)) == Y.EINVAL     # scale planes missing
    assert _decode(_layer(dtype=Y.KV_INT8)) == Y.EINVAL      # group-scale planes missing
    assert _decode(_layer(dtype=Y.KV_INT8, k_scale=0x1, v_scale=None)) == Y.EINVAL
    assert _decode(_layer(dtype=3)) == Y.EINVAL
    assert _decode(L, Hq=22) == Y.EINVAL                     # not a multiple of KV heads
    assert _decode(L, Hq=40) == Y.ENOTSUP                    # group of 10
    assert _decode(L, max_len=64 * 16 + 1) == Y.ERANGE       # beyond the block table
    assert _decode(L, q=0x7001) == Y.EINVAL                  # misaligned
    assert _decode(L, out_dtype=5) == Y.EINVAL
    assert _decode(L, scale=-1.0) == Y.EINVAL
    assert _decode(L, bt=None) == Y.EINVAL
    assert _decode(L, ws_bytes=16) == Y.ENOSPC
    assert _decode(_layer(paged=0), S=2, bt=None) == Y.EINVAL   # contiguous needs one sequence
    assert _decode(_layer(paged=0), bt=None, max_len=64 * 16 + 1) == Y.ERANGE
    # every plane the kernels read with wide loads must be aligned
    assert _decode(_layer(k=0x10008)) == Y.EINVAL
    assert _decode(_layer(v=0x20004)) == Y.EINVAL
    nv = dict(dtype=Y.KV_NVFP4, k_scale=0x40000, v_scale=0x50000, k_tensor_scale_dev=0x60000,
              v_tensor_scale_dev=0x70000)
    assert _decode(_layer(**nv), ws_bytes=16) == Y.ENOSPC            # aligned: reaches the end
    assert _decode(_layer(**dict(nv, k_scale=0x40004))) == Y.EINVAL
    assert _decode(_layer(**dict(nv, v_tensor_scale_dev=0x70002))) == Y.EINVAL
    assert _decode(_layer(dtype=Y.KV_INT8, k_scale=0x40000, v_scale=0x50008)) == Y.EINVAL
    # shapes beyond the launch grid, and pools whose block ids do not fit int32
    assert _decode(L, S=70000, stride=64) == Y.ENOTSUP
    assert _decode(_layer(num_blocks=1 << 31)) == Y.ERANGE
    # a table stride whose token count overflows int64 is no error by itself
    assert _decode(L, stride=(1 << 63) - 1, ws_bytes=16) == Y.ENOSPC


def test_decode_workspace_size_is_stable():
    a = Y.decode_workspace_size(1, 24, 4, 1048576)
    assert a == Y.decode_workspace_size(1, 24, 4, 1048576) > 0
    assert Y.decode_workspace_size(0, 24, 4, 1048576) == 0
    assert Y.decode_workspace_size(1, 24, 4, 1048576, head_dim=128) == 0
    # partial outputs grow with the number of sequences, never below one split each
    assert Y.decode_workspace_size(15, 24, 4, 131072) >= 15 * 24 * 257 * 4
    # an empty longest sequence still plans one split (this once divided by zero)
    assert Y.decode_workspace_size(2, 24, 4, 0) >= 2 * 24 * 257 * 4


def _verify(layer, S=1, nq=4, Hq=24, bt=0x3000, stride=64, lens=0x4000, max_len=1024,
            out=0x5000, out_dtype=Y.OUT_BF16, ws=0x6000, ws_bytes=1 << 30, q=0x7000, scale=0.0):
    return Y._lib.yrk_verify_attention(ctypes.byref(layer), q, S, nq, Hq, bt, stride, lens,
                                       max_len, scale, out, out_dtype, ws, ws_bytes, None, None)


def test_verify_validation():
    L = _layer()
    assert _verify(_layer(head_dim=128)) == Y.ENOTSUP
    assert _verify(_layer(dtype=Y.KV_NVFP4, k_scale=0x40000, v_scale=0x50000,
                          k_tensor_scale_dev=0x60000, v_tensor_scale_dev=0x70000)) == Y.ENOTSUP
    # INT8 is accepted: the call gets as far as the workspace check
    assert _verify(_layer(dtype=Y.KV_INT8, k_scale=0x40000, v_scale=0x50000),
                   ws_bytes=16) == Y.ENOSPC
    assert _verify(_layer(dtype=Y.KV_NVFP4)) == Y.EINVAL     # scale planes missing
    assert _verify(L, nq=0) == Y.EINVAL
    assert _verify(L, nq=9) == Y.ENOTSUP                     # 9 x 6 = 54 rows > 48
    # 12 x 4 = 48 rows is accepted: the call gets as far as the workspace check
    assert _verify(L, nq=12, Hq=16, ws_bytes=16) == Y.ENOSPC
    assert _verify(L, Hq=22) == Y.EINVAL
    assert _verify(L, Hq=40) == Y.ENOTSUP
    assert _verify(L, max_len=64 * 16 + 1) == Y.ERANGE
    assert _verify(L, q=0x7008) == Y.EINVAL                  # misaligned
    assert _verify(L, out_dtype=5) == Y.EINVAL
    assert _verify(L, scale=float("nan")) == Y.EINVAL
    assert _verify(L, bt=None) == Y.EINVAL
    assert _verify(L, ws_bytes=16) == Y.ENOSPC
    assert _verify(_layer(paged=0), S=2, bt=None) == Y.EINVAL


def test_verify_workspace_size():
    a = Y.verify_workspace_size(1, 6, 24, 4, 1048576)
    assert a > 0 and a == Y.verify_workspace_size(1, 6, 24, 4, 1048576)
    assert Y.verify_workspace_size(1, 9, 24, 4, 1048576) == 0     # 54 rows per KV head
    assert Y.verify_workspace_size(1, 0, 24, 4, 1048576) == 0
    assert Y.verify_workspace_size(1, 2, 24, 5, 1048576) == 0     # 24 heads over 5 KV heads
    # one partial (256 + 1 floats) per (sequence, query, head, split), at least one split
    assert Y.verify_workspace_size(3, 6, 24, 4, 64) >= 3 * 6 * 24 * 257 * 4
    assert Y.verify_workspace_size(1, 2, 24, 4, 0) >= 2 * 24 * 257 * 4


def test_append_validation():
    L = _layer()
    f = Y._lib.yrk_kv_append_quantize
    assert f(ctypes.byref(L), 0x100, 0x200, 4, None, 0, 0x300, None, None) == Y.EINVAL
    assert f(ctypes.byref(L), 0x100, 0x200, -1, 0x400, 4, 0x300, None, None) == Y.EINVAL
    assert f(ctypes.byref(L), 0x101, 0x200, 4, 0x400, 4, 0x300, None, None) == Y.EINVAL
    assert f(ctypes.byref(L), None, None, 0, 0x400, 4, None, None, None) == Y.OK
    assert f(ctypes.byref(_layer(head_dim=64)), 0x100, 0x200, 4, 0x400, 4, 0x300, None,
             None) == Y.ENOTSUP
    # INT8 needs both group-scale planes, not the NVFP4 tensor scales
    assert f(ctypes.byref(_layer(dtype=Y.KV_INT8)), 0x100, 0x200, 4, 0x400, 4, 0x300, None,
             None) == Y.EINVAL
    i8 = _layer(dtype=Y.KV_INT8, k_scale=0x40000, v_scale=0x50000)
    assert f(ctypes.byref(i8), None, None, 0, 0x400, 4, None, None, None) == Y.OK


def test_rope_append_validation():
    L = _layer()
    p = Y.YarnParams()
    f = Y._lib.yrk_rope_append

    def call(layer=L, params=p, q=0x8000, hq=24, qs=24 * 256, k=0x100, v=0x200, T=4, bt=0x400,
             bt_len=4, pos=0x300):
        lc, pc = layer, params.c()
        return f(ctypes.byref(lc), ctypes.byref(pc), q, hq, qs, k, v, T, bt, bt_len, pos, None,
                 None)

    assert call(params=Y.YarnParams(factor=0.5)) == Y.EINVAL
    assert call(params=Y.YarnParams(rotary_dim=32)) == Y.ENOTSUP   # fused pass: 64 of 256
    assert call(params=Y.YarnParams(head_dim=128, rotary_dim=64)) == Y.ENOTSUP
    assert call(qs=24 * 256 - 4) == Y.EINVAL                        # rows overlap
    assert call(qs=24 * 256 + 2) == Y.EINVAL                        # stride not a multiple of 4
    assert call(q=0x8004) == Y.EINVAL                               # q not 8-byte aligned
    assert call(hq=0) == Y.EINVAL
    assert call(k=0x108) == Y.EINVAL                                # k not 16-byte aligned
    assert call(T=-1) == Y.EINVAL
    assert call(bt=None) == Y.EINVAL
    assert call(layer=_layer(dtype=Y.KV_INT8)) == Y.EINVAL          # scale planes missing
    assert call(T=0) == Y.OK                                        # nothing enqueued
    assert call(q=None, hq=0, qs=0, T=0) == Y.OK


def test_prefill_validation():
    L = _layer()
    f = Y._lib.yrk_prefill_attention
    args = lambda **kw: dict(dict(q=0x100, T=64, Hq=24, start=0, bt=0x400, bt_len=64, out=0x800),
                             **kw)

    def call(**kw):
        a = args(**kw)
        return f(ctypes.byref(kw.get("layer", L)), a["q"], a["T"], a["Hq"], a["start"], a["bt"],
                 a["bt_len"], 0.0, a["out"], kw.get("ws", 0x1000), kw.get("ws_bytes", 1 << 20),
                 None, None)

    assert call(start=64 * 16 - 63) == Y.ERANGE
    # chunks ending within two 32-key tiles of 2^31 are refused (int32 key bounds)
    # (the accepted call stops at its workspace size, before any launch)
    big = (1 << 31) // 16
    short = Y.prefill_workspace_size(64, 24) - 1
    assert call(start=(1 << 31) - 65 - 64, bt_len=big, ws_bytes=short) == Y.ENOSPC
    assert call(start=(1 << 31) - 64 - 64, bt_len=big, ws_bytes=short) == Y.ERANGE
    assert call(start=(1 << 63) - 1) == Y.ERANGE
    assert call(bt=None) == Y.EINVAL
    assert call(Hq=8) == Y.ENOTSUP
    assert call(T=-1) == Y.EINVAL
    assert call(layer=_layer(dtype=Y.KV_NVFP4, k_scale=0x40000, v_scale=0x50000,
                             k_tensor_scale_dev=0x10, v_tensor_scale_dev=0x10)) == Y.ENOTSUP
    assert call(layer=_layer(dtype=Y.KV_INT8, k_scale=0x40000, v_scale=0x50000)) == Y.ENOTSUP
    assert call(T=0, q=None, out=None) == Y.OK
    # the workspace holds one flag word per wave of the launch grid
    assert call(ws=None) == Y.EINVAL
    assert call(ws=0x1002) == Y.EINVAL
    need = Y.prefill_workspace_size(64, 24)
    assert need == 8 * 4 * 4      # 2 row tiles of 192 rows, 2 XCDs per KV head
    assert call(ws_bytes=need - 1) == Y.ENOSPC
    assert Y.prefill_workspace_size(8192, 24) == 1024 * 4 * 4
    assert Y.prefill_workspace_size(0, 24) == 0


def test_tensor_scale_validation():
    f = Y._lib.yrk_nvfp4_tensor_scale
    assert f(0x100, -1, 0x200, None) == Y.EINVAL
    assert f(0x100, 10, None, None) == Y.EINVAL
    assert f(0x100, 10, 0x201, None) == Y.EINVAL


def test_status_strings():
    for s in (Y.OK, Y.EINVAL, Y.ERANGE, Y.ENOTSUP, Y.ENOSPC, Y.EDEVICE):
        assert Y._lib.yrk_status_string(s)
