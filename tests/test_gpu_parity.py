"""GPU parity: every kernel behind the C ABI against the fp64 oracle on the
same seeded inputs.  Bit-exact for indexing, paging and NVFP4 codes/scales;
attention within max |err| <= 1e-2 (bf16 output, fp32 accumulation)."""
import json
import os
import sys

import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ATOL = 1e-2
STATS = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out",
                     "parity_stats.jsonl")


def _say(msg):
    print(f"[parity] {msg}", file=sys.stderr, flush=True)


def _record(case, **kw):
    if os.path.isdir(os.path.dirname(STATS)):
        with open(STATS, "a") as f:
            f.write(json.dumps(dict(case=case, **kw)) + "\n")


@pytest.fixture(scope="module")
def Y():
    import yarn_rope_kv_amd
    return yarn_rope_kv_amd


@pytest.fixture(scope="module")
def W():
    import workloads
    return workloads


DEV = "cuda:0"


def _bits(t):
    """A bf16 CUDA tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _f64(t):
    if t.dtype == torch.bfloat16:
        return O.bf16_to_f64(_bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def _oracle_table(w):
    return O.yarn_table(rope_theta=1e7, rotary_dim=64, factor=4.0, original_max_position=w.orig)


def _bf16_spacing(x):
    """Distance between consecutive bf16 values at |x| (one bf16 step)."""
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _compare_attention(case, gpu, ref, atol=ATOL, bf16_out=True):
    """Element-wise bound: |gpu - ref| <= atol.  For a bf16 output the stored
    value alone can be half a bf16 step from the exact result, and a bf16 step
    exceeds 1e-2 once |o| >= 2.56, so there the bound is one bf16 step."""
    err = np.abs(gpu - ref)
    ref_b = O.bf16_to_f64(O.round_bf16(ref))
    spacing = _bf16_spacing(ref)
    tol = np.maximum(atol, spacing) if bf16_out else np.full_like(ref, atol)
    stats = dict(max_abs_err=float(err.max()), rel_l2=float(np.linalg.norm(gpu - ref) /
                                                           max(np.linalg.norm(ref), 1e-300)),
                 rel_l2_bf16_oracle=float(np.linalg.norm(ref_b - ref) /
                                          max(np.linalg.norm(ref), 1e-300)),
                 max_err_in_bf16_spacings=float((np.abs(gpu - ref_b) / spacing).max()),
                 ref_rms=float(np.sqrt(np.mean(ref ** 2))),
                 max_ref=float(np.abs(ref).max()), bound_ok=bool(np.all(err <= tol)))
    _say(f"{case}: {stats}")
    _record(case, **stats)
    assert stats["bound_ok"], stats
    return stats


# -- generator ------------------------------------------------------------------

def test_device_generator_matches_host():
    w_tensor = torch.empty((300, 4, 256), dtype=torch.bfloat16, device=DEV)
    mul = synth.outlier_channels(1002, 0, synth.K, 4, 256, 4, 8.0)
    synth.dev_fill(w_tensor, 1002, 7, 1000, 300, 4, 256, chan_mul=mul, outlier_stream=9,
                   outlier_p=0.01, outlier_mul=20.0)
    host = synth.host_fill(1002, 7, 1000, 300, 4, 256, chan_mul=mul, outlier_stream=9,
                           outlier_p=0.01, outlier_mul=20.0)
    assert np.array_equal(_bits(w_tensor), host)


# -- rope -------------------------------------------------------------------------

@pytest.mark.parametrize("orig,corr,factor", [(262144, 0, 4.0), (1024, 0, 4.0),
                                              (262144, 1048576, 4.0), (4096, 0, 1.0)])
def test_rope_matches_oracle(Y, orig, corr, factor):
    _say(f"rope orig={orig} corr={corr} factor={factor}")
    rng = np.random.default_rng(orig + corr)
    pos = np.concatenate([[0, 1, 4095, 4096, 262143, 262144, 1048575, 1048576],
                          rng.integers(0, 1 << 20, 56)]).astype(np.int64)
    T = len(pos)
    for H, stream in ((24, synth.Q), (4, synth.K)):
        raw = synth.host_fill(77, stream, 0, T, H, 256)
        x = torch.from_numpy(raw.view(np.int16)).to(DEV).view(torch.bfloat16)
        p = Y.YarnParams(original_max_position=orig, correction_max_position=corr, factor=factor)
        Y.yarn_rope_apply(p, x, torch.from_numpy(pos.astype(np.int32)).to(DEV))
        got = _bits(x)
        t = O.yarn_table(original_max_position=orig, correction_max_position=corr, factor=factor)
        ref = O.rope(raw, pos, t, bf16_out=True)
        diff = got != ref
        _record("rope", orig=orig, corr=corr, factor=factor, heads=H, mismatches=int(diff.sum()),
                elements=int(diff.size))
        # the only allowed difference is one bf16 step from fp64 noise at a rounding tie
        assert np.all(np.abs(got.astype(np.int32) - ref.astype(np.int32))[diff] <= 1)
        assert diff.sum() <= max(1, diff.size // 100000)
        assert np.array_equal(got[..., 64:], raw[..., 64:])


def test_rope_negative_positions_are_flagged_and_left_unchanged(Y):
    """A negative position is an error only the device sees: that token is
    left as it is and the position bit is set; the others are roped."""
    pos = np.array([5, -1, 262144, -(1 << 31), 1048575, -7], dtype=np.int64)
    raw = synth.host_fill(79, synth.Q, 0, len(pos), 24, 256)
    x = torch.from_numpy(raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.yarn_rope_apply(Y.YarnParams(), x, torch.from_numpy(pos.astype(np.int32)).to(DEV), err=err)
    got = _bits(x)
    bad = pos < 0
    assert int(err.item()) == Y.DEVERR_POSITION
    assert np.array_equal(got[bad], raw[bad])
    ref = O.rope(raw[~bad], pos[~bad], O.yarn_table(), bf16_out=True)
    assert np.array_equal(got[~bad], ref)
    # no negative position: the word stays clear
    err.zero_()
    Y.yarn_rope_apply(Y.YarnParams(), x[:1], torch.tensor([3], dtype=torch.int32, device=DEV),
                      err=err)
    assert int(err.item()) == 0


def test_rope_on_strided_rows(Y):
    """q heads inside a wider per-token row (a fused projection output)."""
    T, H = 9, 24
    buf = torch.zeros((T, 40 * 256), dtype=torch.bfloat16, device=DEV)
    raw = synth.host_fill(78, synth.Q, 0, T, H, 256)
    buf[:, 256 * 8: 256 * 32] = torch.from_numpy(raw.view(np.int16)).to(DEV).view(
        torch.bfloat16).reshape(T, -1)
    view = buf[:, 256 * 8: 256 * 32].view(T, H, 256)
    pos = np.arange(1040000, 1040000 + T)
    Y.yarn_rope_apply(Y.YarnParams(), view, torch.from_numpy(pos.astype(np.int32)).to(DEV))
    ref = O.rope(raw, pos, O.yarn_table(), bf16_out=True)
    got = _bits(buf)
    assert np.sum(_bits(view) != ref) <= 1
    assert np.all(got[:, : 256 * 8] == 0) and np.all(got[:, 256 * 32:] == 0)


# -- append -----------------------------------------------------------------------

def test_append_bf16_paged_and_contiguous_bit_exact(Y):
    T, pages = 200, 32
    k_raw = synth.host_fill(90, 1, 0, T, 4, 256)
    v_raw = synth.host_fill(90, 2, 0, T, 4, 256)
    k = torch.from_numpy(k_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    v = torch.from_numpy(v_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    table = synth.block_permutation(90, pages)
    pos = np.arange(T, dtype=np.int32)
    L = Y.KVLayer.allocate(Y.KV_BF16, 4, pages, paged=True, device=DEV)
    L.k.zero_(), L.v.zero_()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.kv_append_quantize(L, k, v, torch.from_numpy(table).to(DEV), torch.from_numpy(pos).to(DEV),
                         err=err)
    for pool, raw in ((L.k, k_raw), (L.v, v_raw)):
        got = O.gather_paged(_bits(pool).view(np.uint8), pages, 4, 16, 512, table, T)
        assert np.array_equal(got.view(np.uint16).reshape(T, 4, 256), raw)
    assert int(err.item()) == 0
    C = Y.KVLayer.allocate(Y.KV_BF16, 4, pages, paged=False, device=DEV)
    perm = np.random.default_rng(1).permutation(T).astype(np.int32)   # out-of-order positions
    Y.kv_append_quantize(C, k[perm], v[perm], None, torch.from_numpy(perm).to(DEV))
    assert np.array_equal(_bits(C.k)[:T], k_raw) and np.array_equal(_bits(C.v)[:T], v_raw)


def test_append_flags_bad_positions_and_pages(Y):
    pages = 4
    L = Y.KVLayer.allocate(Y.KV_BF16, 4, pages, paged=True, device=DEV)
    L.k.zero_(), L.v.zero_()
    table = torch.tensor([0, 1, 7, 3], dtype=torch.int32, device=DEV)   # page 2 -> 7: outside
    k = torch.ones((3, 4, 256), dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    pos = torch.tensor([5, 40, 70], dtype=torch.int32, device=DEV)      # 70 is beyond the table
    Y.kv_append_quantize(L, k, k, table, pos, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == Y.DEVERR_BLOCK_ID | Y.DEVERR_POSITION
    assert float(L.k.float().sum()) == 4 * 256                          # only position 5 written


def test_tensor_scale_bit_exact(Y):
    out = torch.empty(1, dtype=torch.float32, device=DEV)
    for seed, rows, cut in ((3, 1 << 17, 0), (4, 1543, 3), (5, 1, 7)):
        raw = synth.host_fill(seed, 1, 0, rows, 1, 8, outlier_stream=3, outlier_p=0.01,
                              outlier_mul=20.0).reshape(-1)
        raw = raw[: raw.size - cut]           # odd lengths exercise the tail loop
        x = torch.from_numpy(raw.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
        Y.nvfp4_tensor_scale(x, out)
        assert out.item() == float(O.nvfp4_tensor_scale(raw))
    z = torch.zeros(100, dtype=torch.bfloat16, device=DEV)
    Y.nvfp4_tensor_scale(z, out)
    assert out.item() == 1.0


@pytest.mark.parametrize("paged", [True, False])
def test_append_nvfp4_bit_exact(Y, paged):
    T, pages = 300, 32
    k_raw = synth.host_fill(91, 1, 0, T, 4, 256, outlier_stream=3, outlier_p=0.01,
                            outlier_mul=20.0)
    v_raw = synth.host_fill(91, 2, 0, T, 4, 256, outlier_stream=4, outlier_p=0.01,
                            outlier_mul=20.0)
    v_raw[5, 1, :16] = 0            # an all-zero block
    v_raw[6, 2, 3] = 0x8000         # -0
    k = torch.from_numpy(k_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    v = torch.from_numpy(v_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    L = Y.KVLayer.allocate(Y.KV_NVFP4, 4, pages, paged=paged, device=DEV)
    Y.nvfp4_tensor_scale(k, L.k_tensor_scale)
    Y.nvfp4_tensor_scale(v, L.v_tensor_scale)
    table = synth.block_permutation(91, pages)
    pos = np.arange(T, dtype=np.int32)
    Y.kv_append_quantize(L, k, v, torch.from_numpy(table).to(DEV) if paged else None,
                         torch.from_numpy(pos).to(DEV))
    for raw, codes_t, scales_t, S_t in ((k_raw, L.k, L.k_scale, L.k_tensor_scale),
                                        (v_raw, L.v, L.v_scale, L.v_tensor_scale)):
        S = O.nvfp4_tensor_scale(raw)
        assert S_t.item() == float(S)
        c_ref, s_ref = O.nvfp4_quantize(raw, S)
        packed_ref = O.nvfp4_pack(c_ref)
        cb = codes_t.cpu().numpy()
        sb = scales_t.cpu().numpy()
        if paged:
            got_c = O.gather_paged(cb.reshape(-1), pages, 4, 16, 128, table, T)
            got_s = O.gather_paged(sb.reshape(-1), pages, 4, 16, 16, table, T)
        else:
            got_c, got_s = cb[:T], sb[:T]
        assert np.array_equal(got_s.reshape(s_ref.shape), s_ref)
        assert np.array_equal(got_c.reshape(packed_ref.shape), packed_ref)


@pytest.mark.parametrize("paged", [True, False])
def test_append_int8_bit_exact(Y, paged):
    T, pages = 300, 32
    k_raw = synth.host_fill(92, 1, 0, T, 4, 256, outlier_stream=3, outlier_p=0.01,
                            outlier_mul=20.0)
    v_raw = synth.host_fill(92, 2, 0, T, 4, 256, outlier_stream=4, outlier_p=0.01,
                            outlier_mul=20.0)
    v_raw[5, 1, :64] = 0                       # an all-zero group
    v_raw[6, 2, 3] = 0x8000                    # -0
    # a group 2^-16 smaller (binary16-subnormal scale) and one 2^24 larger
    # (the scale saturates at 65504 and the codes clamp at +-127)
    for raw, e in ((k_raw, -16), (v_raw, 24)):
        x = (raw[7, 0, 64:128].astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** e)
        raw[7, 0, 64:128] = (x.view(np.uint32) >> 16).astype(np.uint16)
    k = torch.from_numpy(k_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    v = torch.from_numpy(v_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    L = Y.KVLayer.allocate(Y.KV_INT8, 4, pages, paged=paged, device=DEV)
    table = synth.block_permutation(92, pages)
    pos = np.arange(T, dtype=np.int32)
    Y.kv_append_quantize(L, k, v, torch.from_numpy(table).to(DEV) if paged else None,
                         torch.from_numpy(pos).to(DEV))
    for raw, codes_t, scales_t in ((k_raw, L.k, L.k_scale), (v_raw, L.v, L.v_scale)):
        c_ref, s_ref = O.int8_quantize(raw)
        cb = codes_t.cpu().numpy().view(np.uint8)
        sb = scales_t.cpu().numpy().view(np.uint8)
        if paged:
            got_c = O.gather_paged(cb.reshape(-1), pages, 4, 16, 256, table, T)
            got_s = O.gather_paged(sb.reshape(-1), pages, 4, 16, 8, table, T)
        else:
            got_c, got_s = cb[:T], sb[:T]
        assert np.array_equal(got_s.reshape(-1).view(np.uint16).reshape(s_ref.shape), s_ref)
        assert np.array_equal(got_c.reshape(-1).view(np.int8).reshape(c_ref.shape), c_ref)
    assert 0 < O.f16_value(int(O.int8_quantize(k_raw[7:8])[1][0, 0, 1])) < 2.0 ** -14
    assert O.int8_quantize(v_raw[7:8])[1][0, 0, 1] == 0x7BFF


# -- decode -----------------------------------------------------------------------

def _host_case(W, w, u, N=None):
    """The oracle side of one layer / session: roped q (bits), roped K, V."""
    N = w.n_ctx if N is None else N
    t = _oracle_table(w)
    q_raw = synth.host_fill(w.seed, synth.stream_id(u, synth.Q), 0, 1, w.hq, 256)
    q = O.rope(q_raw, [N], t, bf16_out=True)[0]
    kw = {}
    if w.elem_outlier_p:
        kw = dict(outlier_p=w.elem_outlier_p, outlier_mul=20.0)
    k_raw = synth.host_fill(w.seed, synth.stream_id(u, synth.K), 0, N, w.hkv, 256,
                            chan_mul=W.chan_mul(w, u, synth.K),
                            outlier_stream=synth.stream_id(u, synth.K_OUTLIER), **kw)
    k = O.rope(k_raw, np.arange(N), t, bf16_out=True)
    del k_raw
    v = synth.host_fill(w.seed, synth.stream_id(u, synth.V), 0, N, w.hkv, 256,
                        chan_mul=W.chan_mul(w, u, synth.V),
                        outlier_stream=synth.stream_id(u, synth.V_OUTLIER), **kw)
    p_star = -1
    if w.needle:
        p_star = synth.needle_position(w.seed, u, N)
        for g in range(w.hkv):
            k[p_star, g] = O.round_bf16(2.0 * O.bf16_to_f64(q[w.group * g]))
    return q, k, v, p_star


def _raw_full(W, w, u, tensor, N, token0=0):
    """Raw (un-roped) K or V rows [N, hkv, 256] of one layer at full size,
    drawn by the seeded generator's device twin and copied to the host (the
    twins are bit-identical: checked here on three slices against host_fill,
    and on a whole tensor by test_device_generator_matches_host).  No
    attention kernel is involved in drawing them."""
    ostream = synth.K_OUTLIER if tensor == synth.K else synth.V_OUTLIER
    t = torch.empty((N, w.hkv, 256), dtype=torch.bfloat16, device=DEV)
    W.gen_kv(w, u, tensor, N, t, token0=token0)
    raw = _bits(t)
    del t
    kw = dict(outlier_p=w.elem_outlier_p, outlier_mul=20.0) if w.elem_outlier_p else {}
    for a in (0, N // 2, max(N - 64, 0)):
        n = min(64, N - a)
        host = synth.host_fill(w.seed, synth.stream_id(u, tensor), token0 + a, n, w.hkv, 256,
                               chan_mul=W.chan_mul(w, u, tensor),
                               outlier_stream=synth.stream_id(u, ostream), **kw)
        assert np.array_equal(raw[a:a + n], host)
    return raw


def _host_case_full(W, w, u):
    """_host_case at full size with the raw K and V from _raw_full."""
    N = w.n_ctx
    t = _oracle_table(w)
    q_raw = synth.host_fill(w.seed, synth.stream_id(u, synth.Q), 0, 1, w.hq, 256)
    q = O.rope(q_raw, [N], t, bf16_out=True)[0]
    k = O.rope(_raw_full(W, w, u, synth.K, N), np.arange(N), t, bf16_out=True)
    v = _raw_full(W, w, u, synth.V, N)
    p_star = -1
    if w.needle:
        p_star = synth.needle_position(w.seed, u, N)
        for g in range(w.hkv):
            k[p_star, g] = O.round_bf16(2.0 * O.bf16_to_f64(q[w.group * g]))
    return q, k, v, p_star


def _decode_gpu(W, dl, w):
    out, ws = W.decode_outputs(w, dl, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    W.run_decode(dl, out, ws, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return out


def test_decode_tiny_contiguous_f32(Y, W):
    w = W.WORKLOADS["tiny"]
    _say("decode tiny")
    dl = W.build_decode_layer(w, 0, device=DEV, keep_raw=True)
    out = _decode_gpu(W, dl, w)
    q, k, v, _ = _host_case(W, w, 0)
    assert np.array_equal(_bits(dl.q)[0], q)
    assert np.array_equal(_bits(dl.k_roped), k)
    ref = O.decode_attention(O.bf16_to_f64(q), k, v)
    _compare_attention("tiny", _f64(out)[0], ref, atol=1e-4, bf16_out=False)


def _needle_bound_ok(got, v, p_star, w):
    """With the planted key the needle's token dominates its group's first
    head: that head's output is within 0.05 of the needle's value row."""
    vf = O.bf16_to_f64(v[p_star])
    return all(np.abs(got[w.group * g] - vf[g]).max() < 0.05 for g in range(w.hkv))


@pytest.mark.parametrize("name,units", [("native", [0]), ("long_tp2", [2])] +
                         [("long", [u]) for u in range(16)])
def test_decode_bf16_paged(Y, W, name, units):
    """Native length, one card's share of a two-way head split, and every one
    of the 16 layers of the 1,048,576-token workload (each with its needle)."""
    w = W.WORKLOADS[name]
    for u in units:
        _say(f"decode {name} layer {u}")
        dl = W.build_decode_layer(w, u, device=DEV)
        out = _decode_gpu(W, dl, w)
        gq = _bits(dl.q)[0]
        del dl
        torch.cuda.empty_cache()
        q, k, v, p_star = (_host_case_full if w.n_ctx >= (1 << 20) else _host_case)(W, w, u)
        assert np.array_equal(gq, q)
        ref = O.decode_attention(O.bf16_to_f64(q), k, v)
        got = _f64(out)[0]
        _compare_attention(f"{name}/layer{u}", got, ref)
        if p_star >= 0:
            assert _needle_bound_ok(got, v, p_star, w)


def test_decode_sessions_batched(Y, W):
    w = W.WORKLOADS["sessions"]
    _say("decode sessions")
    dl = W.build_decode_layer(w, 0, device=DEV)
    out = _f64(_decode_gpu(W, dl, w))
    del dl
    torch.cuda.empty_cache()
    for s in range(w.seqs):                      # every one of the 15 sessions
        _say(f"sessions: oracle of session {s}")
        q, k, v, _ = _host_case(W, w, s)
        ref = O.decode_attention(O.bf16_to_f64(q), k, v)
        _compare_attention(f"sessions/{s}", out[s], ref)


@pytest.mark.parametrize("u", range(16))
def test_decode_long_nvfp4_layer(Y, W, u):
    """Every layer of the 16 x 1,048,576-token NVFP4 workload.  The cache's
    K codes and scales are compared bit for bit, on every row, with the
    oracle's quantisation of the K the GPU roped (the tensor the quantiser
    received; this keeps rope rounding out of the quantiser check), the V
    codes and scales with the oracle's quantisation of V; attention against
    the oracle over its own roped and quantised cache."""
    w = W.WORKLOADS["long_fp4"]
    _say(f"decode long_fp4 layer {u}")
    dl = W.build_decode_layer(w, u, device=DEV, keep_raw=True)
    out = _f64(_decode_gpu(W, dl, w))
    out32 = torch.empty((1, 24, 256), dtype=torch.float32, device=DEV)
    _, ws = W.decode_outputs(w, dl, device=DEV)
    W.run_decode(dl, out32, ws)
    out32 = _f64(out32)
    kg = _bits(dl.k_roped)
    L = dl.layer
    kS, vS = L.k_tensor_scale.item(), L.v_tensor_scale.item()
    table = dl.block_tables[0].cpu().numpy()
    pages = L.num_blocks
    kc = O.gather_paged(L.k.cpu().numpy().reshape(-1), pages, 4, 16, 128, table, w.n_ctx)
    ks = O.gather_paged(L.k_scale.cpu().numpy().reshape(-1), pages, 4, 16, 16, table, w.n_ctx)
    vc = O.gather_paged(L.v.cpu().numpy().reshape(-1), pages, 4, 16, 128, table, w.n_ctx)
    vs = O.gather_paged(L.v_scale.cpu().numpy().reshape(-1), pages, 4, 16, 16, table, w.n_ctx)
    del dl, L
    torch.cuda.empty_cache()
    # the quantiser on the tensor it received: every row bit-exact
    assert kS == float(O.nvfp4_tensor_scale(kg))
    kq_codes, kq_scales = O.nvfp4_quantize(kg, np.float32(kS))
    assert np.array_equal(ks.reshape(kq_scales.shape), kq_scales)
    assert np.array_equal(kc.reshape(-1, 4, 128), O.nvfp4_pack(kq_codes))
    del kc, ks
    q, k, v, _ = _host_case_full(W, w, u)
    same = kg == k
    _record(f"long_fp4/layer{u}/rope_k", mismatches=int((~same).sum()))
    assert (~same).sum() <= k.size // 100000
    assert vS == float(O.nvfp4_tensor_scale(v))
    v_codes, v_scales = O.nvfp4_quantize(v, np.float32(vS))
    assert np.array_equal(vs.reshape(v_scales.shape), v_scales)
    assert np.array_equal(vc.reshape(-1, 4, 128), O.nvfp4_pack(v_codes))
    # the oracle's own cache: its rope, then its quantiser (equal to the
    # above when the two ropes agree on every element)
    if same.all():
        k_codes, k_scales, kS_o = kq_codes, kq_scales, kS
    else:
        kS_o = float(O.nvfp4_tensor_scale(k))
        k_codes, k_scales = O.nvfp4_quantize(k, np.float32(kS_o))
    del kg, kq_codes, kq_scales
    ref = O.decode_attention(O.bf16_to_f64(q), k_codes, v_codes,
                             nvfp4=(k_scales, v_scales, kS_o, vS))
    _compare_attention(f"long_fp4/layer{u}", out[0], ref)
    _compare_attention(f"long_fp4/layer{u}/f32", out32[0], ref, bf16_out=False)


def test_decode_long_int8_sampled_layer(Y, W):
    """One layer of the 16 x 1,048,576-token INT8 workload: the cache's codes
    and scales bit-exact against the oracle's quantisation of the same roped
    keys (rows where the GPU rope agrees bit for bit), then attention."""
    w = W.WORKLOADS["long_int8"]
    u = 3
    _say("decode long_int8 layer 3")
    dl = W.build_decode_layer(w, u, device=DEV, keep_raw=True)
    out32 = torch.empty((1, 24, 256), dtype=torch.float32, device=DEV)
    _, ws = W.decode_outputs(w, dl, device=DEV)
    W.run_decode(dl, out32, ws)
    torch.cuda.synchronize()
    out32 = _f64(out32)
    kg = _bits(dl.k_roped)
    L = dl.layer
    table = dl.block_tables[0].cpu().numpy()
    pages = L.num_blocks
    kc = O.gather_paged(L.k.cpu().numpy().view(np.uint8).reshape(-1), pages, 4, 16, 256, table,
                        w.n_ctx)
    ks = O.gather_paged(L.k_scale.cpu().numpy().view(np.uint8).reshape(-1), pages, 4, 16, 8,
                        table, w.n_ctx)
    vc = O.gather_paged(L.v.cpu().numpy().view(np.uint8).reshape(-1), pages, 4, 16, 256, table,
                        w.n_ctx)
    vs = O.gather_paged(L.v_scale.cpu().numpy().view(np.uint8).reshape(-1), pages, 4, 16, 8,
                        table, w.n_ctx)
    del dl, L
    torch.cuda.empty_cache()
    q, k, v, _ = _host_case_full(W, w, u)
    same = kg == k
    _record("long_int8/rope_k", mismatches=int((~same).sum()))
    assert (~same).sum() <= k.size // 100000
    del kg
    k_codes, k_scales = O.int8_quantize(k)
    v_codes, v_scales = O.int8_quantize(v)
    rows_ok = same.all(axis=-1)
    assert np.array_equal(vs.reshape(-1).view(np.uint16).reshape(v_scales.shape), v_scales)
    assert np.array_equal(vc.reshape(-1).view(np.int8).reshape(v_codes.shape), v_codes)
    assert np.array_equal(ks.reshape(-1).view(np.uint16).reshape(k_scales.shape)[rows_ok],
                          k_scales[rows_ok])
    assert np.array_equal(kc.reshape(-1).view(np.int8).reshape(k_codes.shape)[rows_ok],
                          k_codes[rows_ok])
    ref = O.decode_attention(O.bf16_to_f64(q), k_codes, v_codes, int8=(k_scales, v_scales))
    _compare_attention("long_int8/layer3/f32", out32[0], ref, bf16_out=False)


def test_decode_ragged_batch_and_empty(Y, W):
    """One batched call over sequences of lengths 0, 1, 15, 16, 17, 1000 and
    4097 (partial pages, a page-aligned end, an empty sequence)."""
    lens = [0, 1, 15, 16, 17, 1000, 4097]
    S, max_len = len(lens), 5000
    pages_per = -(-max_len // 16)
    pool = S * pages_per
    perm = synth.block_permutation(123, pool).reshape(S, pages_per)
    L = Y.KVLayer.allocate(Y.KV_BF16, 4, pool, paged=True, device=DEV)
    yp = Y.YarnParams()
    qs, refs = [], []
    for s, n in enumerate(lens):
        q_raw = synth.host_fill(124, synth.stream_id(s, synth.Q), 0, 1, 24, 256)
        k_raw = synth.host_fill(124, synth.stream_id(s, synth.K), 0, max(n, 1), 4, 256)
        v_raw = synth.host_fill(124, synth.stream_id(s, synth.V), 0, max(n, 1), 4, 256)
        qt = torch.from_numpy(q_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
        Y.yarn_rope_apply(yp, qt, torch.tensor([n], dtype=torch.int32, device=DEV))
        qs.append(qt)
        if n:
            kt = torch.from_numpy(k_raw[:n].view(np.int16)).to(DEV).view(torch.bfloat16)
            vt = torch.from_numpy(v_raw[:n].view(np.int16)).to(DEV).view(torch.bfloat16)
            pos = torch.arange(n, dtype=torch.int32, device=DEV)
            Y.yarn_rope_apply(yp, kt, pos)
            Y.kv_append_quantize(L, kt, vt, torch.from_numpy(perm[s]).to(DEV), pos)
        t = O.yarn_table()
        q = O.rope(q_raw, [n], t, bf16_out=True)[0]
        k = O.rope(k_raw[:n], np.arange(n), t, bf16_out=True)
        refs.append(O.decode_attention(O.bf16_to_f64(q), k, v_raw[:n]))
    q = torch.cat(qs)
    out = torch.empty((S, 24, 256), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(Y.decode_workspace_size(S, 24, 4, max_len), dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.decode_attention(L, q, torch.from_numpy(perm).to(DEV),
                       torch.tensor(lens, dtype=torch.int32, device=DEV), max_len, out, ws, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = _f64(out)
    assert np.all(got[0] == 0)
    for s in range(1, S):
        _compare_attention(f"ragged/len{lens[s]}", got[s], refs[s])


def test_decode_masks_and_flags_a_bad_page(Y, W):
    n, pages = 300, 19
    L = Y.KVLayer.allocate(Y.KV_BF16, 4, pages, paged=True, device=DEV)
    table = synth.block_permutation(55, pages)
    yp = Y.YarnParams()
    q_raw = synth.host_fill(56, 0, 0, 1, 24, 256)
    k_raw = synth.host_fill(56, 1, 0, n, 4, 256)
    v_raw = synth.host_fill(56, 2, 0, n, 4, 256)
    qt = torch.from_numpy(q_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    kt = torch.from_numpy(k_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    vt = torch.from_numpy(v_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    pos = torch.arange(n, dtype=torch.int32, device=DEV)
    Y.yarn_rope_apply(yp, qt, torch.tensor([n], dtype=torch.int32, device=DEV))
    Y.yarn_rope_apply(yp, kt, pos)
    bt = torch.from_numpy(table).to(DEV)
    Y.kv_append_quantize(L, kt, vt, bt, pos)
    bad = bt.clone()
    bad[5] = pages + 3
    out = torch.empty((1, 24, 256), dtype=torch.float32, device=DEV)
    ws = torch.empty(Y.decode_workspace_size(1, 24, 4, n), dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.decode_attention(L, qt, bad.view(1, -1), torch.tensor([n], dtype=torch.int32, device=DEV),
                       n, out, ws, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == Y.DEVERR_BLOCK_ID
    t = O.yarn_table()
    q = O.rope(q_raw, [n], t, bf16_out=True)[0]
    k = O.rope(k_raw, np.arange(n), t, bf16_out=True)
    keep = np.r_[0:80, 96:n]
    ref = O.decode_attention(O.bf16_to_f64(q), k[keep], v_raw[keep])
    _compare_attention("bad_page_masked", _f64(out)[0], ref, atol=1e-4, bf16_out=False)


def test_decode_paged_equals_contiguous_and_repeats_bitwise(Y, W):
    w = W.WORKLOADS["tiny"]
    dl = W.build_decode_layer(w, 0, device=DEV, keep_raw=True)
    out1, ws = W.decode_outputs(w, dl, device=DEV)
    out2 = torch.empty_like(out1)
    W.run_decode(dl, out1, ws)
    W.run_decode(dl, out2, ws)
    pages = w.pages_per_seq
    P = Y.KVLayer.allocate(Y.KV_BF16, 4, pages, paged=True, device=DEV)
    table = torch.from_numpy(synth.block_permutation(5, pages)).to(DEV)
    Y.kv_append_quantize(P, dl.k_roped, dl.v, table,
                         torch.arange(w.n_ctx, dtype=torch.int32, device=DEV))
    out3 = torch.empty_like(out1)
    Y.decode_attention(P, dl.q, table.view(1, -1), dl.seq_lens, dl.max_seq_len, out3, ws)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(out1, out3)


# -- decode: ragged batches in both cache formats and several GQA shapes -------------

_LENS = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 1000, 4097]


def _scale_bf16(bits, mul):
    """bf16 bit patterns times a power of two (exact while in range)."""
    x = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(mul)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _decode_batch(Y, kv, lens, hq, hkv, seed, paged=True, q_mul=1.0, bad_page=None, v_mul=1.0):
    """One batched decode call over sequences of the given lengths.  Keys are
    roped on the host by the oracle and appended (and, for NVFP4, quantised)
    by the library, so the cache holds exactly what the oracle quantises.
    q_mul (a power of two) scales q, and the softmax scale is divided by it:
    the same attention.  Returns (gpu fp64 [S, hq, 256], per-sequence oracle
    outputs, device error word)."""
    S = len(lens)
    max_len = max(max(lens), 1)
    pages_per = -(-max_len // 16) + 1
    pool = S * pages_per
    t = O.yarn_table()
    qs, ks, vs = [], [], []
    for s, n in enumerate(lens):
        q_raw = synth.host_fill(seed, synth.stream_id(s, synth.Q), 0, 1, hq, 256)
        k_raw = synth.host_fill(seed, synth.stream_id(s, synth.K), 0, max(n, 1), hkv, 256)[:n]
        v_raw = synth.host_fill(seed, synth.stream_id(s, synth.V), 0, max(n, 1), hkv, 256)[:n]
        if v_mul != 1.0:
            v_raw = _scale_bf16(v_raw, v_mul)
        qs.append(O.rope(q_raw, [n], t, bf16_out=True)[0])
        ks.append(O.rope(k_raw, np.arange(n), t, bf16_out=True) if n else k_raw)
        vs.append(v_raw)
    allk, allv = np.concatenate(ks), np.concatenate(vs)
    L = Y.KVLayer.allocate(kv, hkv, pool, paged=paged, device=DEV)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(
        torch.bfloat16)
    if kv == Y.KV_NVFP4:
        Y.nvfp4_tensor_scale(dev(allk), L.k_tensor_scale)
        Y.nvfp4_tensor_scale(dev(allv), L.v_tensor_scale)
        kS, vS = O.nvfp4_tensor_scale(allk), O.nvfp4_tensor_scale(allv)
        assert L.k_tensor_scale.item() == float(kS) and L.v_tensor_scale.item() == float(vS)
    if paged:
        table = synth.block_permutation(seed, pool).reshape(S, pages_per)
        bt = torch.from_numpy(table).to(DEV)
    else:
        assert S == 1
        bt = None
    for s, n in enumerate(lens):
        if n:
            Y.kv_append_quantize(L, dev(ks[s]), dev(vs[s]), bt[s] if paged else None,
                                 torch.arange(n, dtype=torch.int32, device=DEV))
    q = dev(np.stack(qs))
    if q_mul != 1.0:
        q = q * q_mul
    out = torch.empty((S, hq, 256), dtype=torch.float32, device=DEV)
    ws = torch.empty(Y.decode_workspace_size(S, hq, hkv, max_len), dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    tables = bt
    keep = [np.arange(n) for n in lens]
    if bad_page is not None:
        s_bad, page = bad_page
        tables = bt.clone()
        tables[s_bad, page] = pool + 3
        keep[s_bad] = keep[s_bad][keep[s_bad] // 16 != page]
    Y.decode_attention(L, q, tables, torch.tensor(lens, dtype=torch.int32, device=DEV), max_len,
                       out, ws, softmax_scale=1.0 / 16 / q_mul, err=err)
    torch.cuda.synchronize()
    refs = []
    for s, n in enumerate(lens):
        qf = O.bf16_to_f64(qs[s])
        kk, vv = ks[s][keep[s]], vs[s][keep[s]]
        if kv == Y.KV_NVFP4:
            kc, ksc = O.nvfp4_quantize(kk, kS)
            vc, vsc = O.nvfp4_quantize(vv, vS)
            refs.append(O.decode_attention(qf, kc, vc, nvfp4=(ksc, vsc, kS, vS)) if n else
                        np.zeros((hq, 256)))
        elif kv == Y.KV_INT8:
            kc, ksc = O.int8_quantize(kk)
            vc, vsc = O.int8_quantize(vv)
            refs.append(O.decode_attention(qf, kc, vc, int8=(ksc, vsc)) if n else
                        np.zeros((hq, 256)))
        else:
            refs.append(O.decode_attention(qf, kk, vv) if n else np.zeros((hq, 256)))
    return _f64(out), refs, int(err.item())


_FMT = {"bf16": 0, "nvfp4": 1, "int8": 2}


@pytest.mark.parametrize("hq,hkv", [(24, 4), (4, 4), (8, 4), (12, 4), (16, 4), (12, 2)])
@pytest.mark.parametrize("fmt", ["bf16", "nvfp4", "int8"])
def test_decode_ragged_shapes(Y, fmt, hq, hkv):
    """Lengths around the 16-token page and the 32-token NVFP4 step, an empty
    sequence and multi-split ones, for every supported group size and the
    12-query / 2-KV-head shape of one card's share of a two-way head split."""
    kv = _FMT[fmt]
    _say(f"decode ragged {fmt} hq={hq} hkv={hkv}")
    got, refs, err = _decode_batch(Y, kv, _LENS, hq, hkv, seed=700 + hq + 100 * hkv)
    assert err == 0
    assert np.all(got[0] == 0)
    for s in range(1, len(_LENS)):
        _compare_attention(f"ragged/{fmt}/{hq}x{hkv}/len{_LENS[s]}", got[s], refs[s],
                           bf16_out=False)


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4", "int8"])
def test_decode_max_len_zero(Y, fmt):
    """A batch whose longest sequence is empty (max_seq_len 0): zeros and no
    flag, in every cache format."""
    kv = _FMT[fmt]
    _say(f"decode max_seq_len 0 {fmt}")
    L = Y.KVLayer.allocate(kv, 4, 2, paged=True, device=DEV)
    if kv == Y.KV_NVFP4:
        L.k_tensor_scale.fill_(1.0)
        L.v_tensor_scale.fill_(1.0)
    q = torch.ones((2, 24, 256), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((2, 1), dtype=torch.int32, device=DEV)
    out = torch.full((2, 24, 256), 7.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(Y.decode_workspace_size(2, 24, 4, 0), dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.decode_attention(L, q, bt, torch.zeros(2, dtype=torch.int32, device=DEV), 0, out, ws,
                       err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.all(out == 0)


@pytest.mark.parametrize("fmt", ["nvfp4", "int8"])
def test_decode_quantised_masks_and_flags_a_bad_page(Y, fmt):
    _say(f"decode {fmt} bad page")
    got, refs, err = _decode_batch(Y, _FMT[fmt], [300, 77], 24, 4, seed=810, bad_page=(0, 5))
    assert err == Y.DEVERR_BLOCK_ID
    for s in range(2):
        _compare_attention(f"{fmt}_bad_page/{s}", got[s], refs[s], bf16_out=False)


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4", "int8"])
def test_decode_contiguous_equals_paged_bitwise(Y, fmt):
    kv = _FMT[fmt]
    _say(f"decode contiguous vs paged {fmt}")
    a, refs, _ = _decode_batch(Y, kv, [1234], 24, 4, seed=820, paged=True)
    b, _, _ = _decode_batch(Y, kv, [1234], 24, 4, seed=820, paged=False)
    assert np.array_equal(a, b)
    _compare_attention(f"contiguous/{fmt}", b[0], refs[0], bf16_out=False)


@pytest.mark.parametrize("v_mul", [2.0 ** 10, 2.0 ** -20])
@pytest.mark.parametrize("fmt", ["bf16", "nvfp4", "int8"])
def test_decode_value_magnitude(Y, fmt, v_mul):
    """Values 2^10 larger (INT8 group scales up to ~30, so p times the scale
    would leave binary16's range without the kernel's shift) and 2^20
    smaller; outputs scale with them, so the bound is relative to |v|."""
    kv = _FMT[fmt]
    _say(f"decode v x {v_mul} {fmt}")
    got, refs, err = _decode_batch(Y, kv, [500, 33, 4097], 24, 4, seed=835, v_mul=v_mul)
    assert err == 0
    for s in range(3):
        assert np.all(np.isfinite(got[s]))
        _compare_attention(f"v_mul/{fmt}/{v_mul:g}/{s}", got[s] / v_mul, refs[s] / v_mul,
                           bf16_out=False)


@pytest.mark.parametrize("q_mul", [2.0 ** 20, 2.0 ** -30])
@pytest.mark.parametrize("fmt", ["bf16", "nvfp4", "int8"])
def test_decode_query_magnitude(Y, fmt, q_mul):
    """q scaled by a power of two far outside [2^-14, 2^15] and the softmax
    scale divided by it: the same attention, which the NVFP4 and INT8 kernels
    compute with q prescaled into fp16's range."""
    kv = _FMT[fmt]
    _say(f"decode q x {q_mul} {fmt}")
    got, refs, err = _decode_batch(Y, kv, [500, 33], 24, 4, seed=830, q_mul=q_mul)
    assert err == 0
    for s in range(2):
        _compare_attention(f"q_mul/{fmt}/{q_mul:g}/{s}", got[s], refs[s], bf16_out=False)


# -- prefill ----------------------------------------------------------------------

def _prefill_small(Y, n_prior, T, paged, seed, bad_page=None, needle=None, hq=24, hkv=4):
    """needle = (t, key, mul): after rope, key position `key` of every KV head
    g is set to mul (a power of two) x the roped query of chunk token t, head
    6g (exact in bf16), so that query's score there is far above its first
    tile's maximum."""
    total = n_prior + T
    pages = -(-total // 16) + 1
    t = O.yarn_table()
    k_raw = synth.host_fill(seed, 1, 0, total, hkv, 256)
    v_raw = synth.host_fill(seed, 2, 0, total, hkv, 256)
    q_raw = synth.host_fill(seed, 0, 0, T, hq, 256)
    yp = Y.YarnParams()
    kt = torch.from_numpy(k_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    vt = torch.from_numpy(v_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    qt = torch.from_numpy(q_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    pos_all = torch.arange(total, dtype=torch.int32, device=DEV)
    Y.yarn_rope_apply(yp, kt, pos_all)
    Y.yarn_rope_apply(yp, qt, pos_all[n_prior:])
    if needle is not None:
        nt, nk, mul = needle
        for g in range(hkv):
            kt[nk, g] = qt[nt, 6 * g] * mul
    L = Y.KVLayer.allocate(Y.KV_BF16, hkv, pages, paged=paged, device=DEV)
    table = synth.block_permutation(seed, pages) if paged else None
    bt = torch.from_numpy(table).to(DEV) if paged else None
    Y.kv_append_quantize(L, kt, vt, bt, pos_all)
    if bad_page is not None:
        bt = bt.clone()
        bt[bad_page] = pages + 5
    out = torch.empty_like(qt)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = torch.full((Y.prefill_workspace_size(T, hq) // 4,), 7, dtype=torch.int32, device=DEV)
    Y.prefill_attention(L, qt, n_prior, bt, out, workspace=ws, err=err)
    torch.cuda.synchronize()
    flags = ws.cpu().numpy()
    k = O.rope(k_raw, np.arange(total), t, bf16_out=True)
    q = O.rope(q_raw, np.arange(n_prior, total), t, bf16_out=True)
    if needle is not None:
        nt, nk, mul = needle
        for g in range(hkv):    # a power-of-two multiple of a bf16 value is exact
            src = q[nt, 6 * g].astype(np.uint32) << 16
            k[nk, g] = ((src.view(np.float32) * mul).view(np.uint32) >> 16).astype(k.dtype)
    return _f64(out), O.bf16_to_f64(q), k, v_raw, int(err.item()), flags


@pytest.mark.parametrize("n_prior,T,paged,hq,hkv", [(1000, 77, True, 24, 4), (0, 200, False, 24, 4),
                                                    (4093, 130, True, 24, 4), (31, 1, True, 24, 4),
                                                    (1000, 77, True, 12, 2), (517, 300, False, 12, 2)])
def test_prefill_small_matches_oracle(Y, n_prior, T, paged, hq, hkv):
    _say(f"prefill n_prior={n_prior} T={T} paged={paged} hq={hq} hkv={hkv}")
    got, q, k, v, err, flags = _prefill_small(Y, n_prior, T, paged, seed=300 + T, hq=hq, hkv=hkv)
    assert err == 0
    assert not flags.any()       # no wave needed the rescaling second launch
    ref = O.prefill_attention(q, np.arange(n_prior, n_prior + T), k, v)
    _compare_attention(f"prefill/{hq}x{hkv}/{n_prior}+{T}", got, ref)
    if n_prior == 0:
        vf = O.bf16_to_f64(v)
        for h in range(hq):      # the first row sees only key 0
            assert np.abs(got[0, h] - vf[0, h // 6]).max() <= np.abs(vf[0]).max() * 2 ** -8


def test_prefill_flags_and_masks_a_bad_page(Y):
    n_prior, T = 500, 40
    got, q, k, v, err, _ = _prefill_small(Y, n_prior, T, True, seed=77, bad_page=3)
    assert err == Y.DEVERR_BLOCK_ID
    keep = np.r_[0:48, 64:n_prior + T]
    refs = []
    for i in range(T):
        p = n_prior + i
        kk = keep[keep <= p]
        refs.append(O.decode_attention(q[i], k[kk], v[kk]))
    _compare_attention("prefill/bad_page", got, np.stack(refs))


@pytest.mark.parametrize("paged,mul,flagged", [(True, 2, False), (False, 2, False),
                                                (True, 4, True), (False, 8, True)])
def test_prefill_score_far_above_the_first_tile(Y, paged, mul, flagged):
    """Key 500 of every KV head set to mul x the roped query of token 40,
    head 6g: that query's score there lies 39-48 (mul 2), 80-98 (mul 4) or
    162-199 (mul 8) log2 units above its first tile's maximum.  Up to 2^64
    the fixed-maximum kernel keeps the row (no flag); beyond, the row sum
    exceeds 2^64 or exp2 overflows, the wave is flagged and the rescaling
    launch recomputes its workgroup.  Either way the output matches the
    oracle."""
    n_prior, T = 1000, 77
    _say(f"prefill needle paged={paged} mul={mul}")
    got, q, k, v, err, flags = _prefill_small(Y, n_prior, T, paged, seed=411,
                                              needle=(40, 500, mul))
    assert err == 0
    assert set(np.unique(flags).tolist()) <= {0, 1}
    assert bool(flags.any()) == flagged
    ref = O.prefill_attention(q, np.arange(n_prior, n_prior + T), k, v)
    _compare_attention("prefill/needle", got, ref)
    # the needle dominates the softmax of query 40, head 6g: out ~ V[500, g]
    vf = O.bf16_to_f64(v)
    for g in range(4):
        assert np.abs(got[40, 6 * g] - vf[500, g]).max() < 0.05


def _prefill_sample(W, w):
    """workloads.prefill_sample, checked to reach every wave (48 rows) and
    row block (16 rows) of a 192-row workgroup and every query head."""
    toks, heads = W.prefill_sample(w)
    Rs = toks * w.group + heads % w.group
    assert set(((Rs % 192) // 48).tolist()) == {0, 1, 2, 3}
    assert set(((Rs % 48) // 16).tolist()) == {0, 1, 2}
    assert set(heads.tolist()) == set(range(w.hq))
    assert len(set(zip(toks.tolist(), heads.tolist()))) == len(toks)
    return toks, heads


@pytest.mark.parametrize("name", ["prefill", "prefill_tp2"])
def test_prefill_workload_sampled_rows(Y, W, name):
    """The full chunk (8,192 queries at 1,040,384..1,048,575 over a
    1,048,576-token paged cache) in the bench's launch configuration, with
    24 q / 4 KV heads and with one card's share of a two-way head split
    (12 q / 2 KV heads); 256 stratified (token, head) rows checked one by
    one against the oracle."""
    w = W.WORKLOADS[name]
    _say(f"{name} workload")
    case = W.build_prefill(w, device=DEV)
    out = torch.empty_like(case.q)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.prefill_attention(case.layer, case.q, case.q_start, case.block_table, out, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    toks, heads = _prefill_sample(W, w)
    ti = torch.from_numpy(toks).to(DEV)
    hi = torch.from_numpy(heads).to(DEV)
    got = _f64(out[ti, hi])
    qg = _bits(case.q[ti, hi])
    del case, out
    torch.cuda.empty_cache()
    N, q0 = w.n_ctx, w.n_ctx - w.prefill_chunk
    t = _oracle_table(w)
    k = O.rope(_raw_full(W, w, 0, synth.K, N), np.arange(N), t, bf16_out=True)
    v = _raw_full(W, w, 0, synth.V, N)
    q_raw = synth.host_fill(w.seed, synth.stream_id(0, synth.Q), q0, w.prefill_chunk, w.hq, 256)
    q = O.rope(q_raw[toks], q0 + toks, t, bf16_out=True)[np.arange(len(toks)), heads]
    assert np.array_equal(q, qg)
    ref = np.empty_like(got)
    for g in range(w.hkv):                     # rows of KV head g, all in one oracle call
        sel = np.nonzero(heads // w.group == g)[0]
        kg_ = np.ascontiguousarray(k[:, g:g + 1])
        vg_ = np.ascontiguousarray(v[:, g:g + 1])
        ref[sel] = O.prefill_attention(O.bf16_to_f64(q[sel])[:, None, :], q0 + toks[sel],
                                       kg_, vg_)[:, 0]
        del kg_, vg_
    _compare_attention(f"{name}/256 rows", got, ref)
