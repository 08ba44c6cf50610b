"""GPU parity of the multi-query (speculative verify) decode against the fp64
oracle: the last num_queries cached tokens of each sequence attend to the
cache causally, query i at position len - num_queries + i seeing keys
0 .. len - num_queries + i.  The oracle is the dense softmax of each query
over exactly those keys (every key the cache holds for the sequence, minus a
masked page where one is planted)."""
import numpy as np
import pytest

import oracle as O
import synth

from test_gpu_parity import (DEV, _bits, _compare_attention, _f64, _host_case,
                              _host_case_full, _say, _scale_bf16)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def Y():
    import yarn_rope_kv_amd
    return yarn_rope_kv_amd


@pytest.fixture(scope="module")
def W():
    import workloads
    return workloads


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def _verify_batch(Y, lens, nq, hq, hkv, seed, paged=True, bad_page=None, out_f32=True,
                  kv=None, v_mul=1.0):
    """One batched verify call.  Keys are roped on the host by the oracle and
    appended by the library; queries are roped by the oracle at their
    positions (clipped at 0 for the queries a too-short sequence leaves at
    negative positions, whose rows must come back zero).  Returns (gpu fp64
    [S, nq, hq, 256], per-sequence oracle outputs [nq, hq, 256], error word)."""
    S = len(lens)
    max_len = max(max(lens), 1)
    pages_per = -(-max_len // 16) + 1
    pool = S * pages_per
    t = O.yarn_table()
    qs, ks, vs = [], [], []
    for s, n in enumerate(lens):
        q_raw = synth.host_fill(seed, synth.stream_id(s, synth.Q), 0, nq, hq, 256)
        k_raw = synth.host_fill(seed, synth.stream_id(s, synth.K), 0, max(n, 1), hkv, 256)[:n]
        v_raw = synth.host_fill(seed, synth.stream_id(s, synth.V), 0, max(n, 1), hkv, 256)[:n]
        if v_mul != 1.0:
            v_raw = _scale_bf16(v_raw, v_mul)
        qs.append(O.rope(q_raw, np.maximum(np.arange(n - nq, n), 0), t, bf16_out=True))
        ks.append(O.rope(k_raw, np.arange(n), t, bf16_out=True) if n else k_raw)
        vs.append(v_raw)
    kv = Y.KV_BF16 if kv is None else kv
    L = Y.KVLayer.allocate(kv, hkv, pool, paged=paged, device=DEV)
    if paged:
        table = synth.block_permutation(seed, pool).reshape(S, pages_per)
        bt = torch.from_numpy(table).to(DEV)
    else:
        assert S == 1
        bt = None
    for s, n in enumerate(lens):
        if n:
            Y.kv_append_quantize(L, _dev(ks[s]), _dev(vs[s]), bt[s] if paged else None,
                                 torch.arange(n, dtype=torch.int32, device=DEV))
    q = _dev(np.stack(qs))
    out = torch.empty((S, nq, hq, 256), dtype=torch.float32 if out_f32 else torch.bfloat16,
                      device=DEV)
    ws = torch.empty(Y.verify_workspace_size(S, nq, hq, hkv, max_len), dtype=torch.uint8,
                     device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    tables = bt
    keep = [np.arange(n) for n in lens]
    if bad_page is not None:
        s_bad, page = bad_page
        tables = bt.clone()
        tables[s_bad, page] = pool + 3
        keep[s_bad] = keep[s_bad][keep[s_bad] // 16 != page]
    Y.verify_attention(L, q, tables, torch.tensor(lens, dtype=torch.int32, device=DEV), max_len,
                       out, ws, softmax_scale=1.0 / 16, err=err)
    torch.cuda.synchronize()
    refs = []
    for s, n in enumerate(lens):
        qf = O.bf16_to_f64(qs[s])
        r = np.zeros((nq, hq, 256))
        if kv == Y.KV_INT8 and n:
            kc, ksc = O.int8_quantize(ks[s])
            vc, vsc = O.int8_quantize(vs[s])
        for i in range(nq):
            sel = keep[s][keep[s] <= n - nq + i]
            if not len(sel):
                continue
            if kv == Y.KV_INT8:
                r[i] = O.decode_attention(qf[i], kc[sel], vc[sel], int8=(ksc[sel], vsc[sel]))
            else:
                r[i] = O.decode_attention(qf[i], ks[s][sel], vs[s][sel])
        refs.append(r)
    return _f64(out), refs, int(err.item())


_SHAPES = [(24, 4, 1), (24, 4, 2), (24, 4, 4), (24, 4, 6), (24, 4, 8), (4, 4, 6), (8, 4, 6),
           (12, 4, 5), (16, 4, 12), (12, 2, 4)]


@pytest.mark.parametrize("hq,hkv,nq", _SHAPES)
def test_verify_ragged_shapes(Y, hq, hkv, nq):
    """1 to 12 queries per sequence (query rows per KV head from 6 to the
    48-row maximum: one, two and three MFMA column blocks), every supported
    group size and the 12 q / 2 KV-head share, over lengths around the
    16-token page and several splits."""
    lens = sorted({nq, nq + 1, 15, 16, 17, 33, 100, 1000, 4097} - set(range(nq)))
    _say(f"verify ragged hq={hq} hkv={hkv} nq={nq}")
    got, refs, err = _verify_batch(Y, lens, nq, hq, hkv, seed=900 + 7 * hq + hkv + 31 * nq)
    assert err == 0
    for s, n in enumerate(lens):
        _compare_attention(f"verify/{hq}x{hkv}/q{nq}/len{n}", got[s], refs[s], bf16_out=False)


_SHAPES_I8 = [(24, 4, 1), (24, 4, 2), (24, 4, 4), (24, 4, 6), (24, 4, 8), (4, 4, 6), (8, 4, 6),
              (12, 4, 5), (16, 4, 12), (12, 2, 4)]


@pytest.mark.parametrize("hq,hkv,nq", _SHAPES_I8)
def test_verify_int8_ragged_shapes(Y, hq, hkv, nq):
    """The verify round over the INT8 group-64 cache (the pages' 1M-token
    format): every row against the oracle's dense softmax over the
    dequantised keys and values it may see."""
    lens = sorted({nq, nq + 1, 15, 16, 17, 33, 100, 1000, 4097} - set(range(nq)))
    _say(f"verify int8 ragged hq={hq} hkv={hkv} nq={nq}")
    got, refs, err = _verify_batch(Y, lens, nq, hq, hkv, seed=960 + 7 * hq + hkv + 31 * nq,
                                   kv=Y.KV_INT8)
    assert err == 0
    for s, n in enumerate(lens):
        _compare_attention(f"verify_int8/{hq}x{hkv}/q{nq}/len{n}", got[s], refs[s],
                           bf16_out=False)


@pytest.mark.parametrize("nq", [4, 6])
@pytest.mark.parametrize("v_mul", [2.0 ** 10, 2.0 ** -20])
def test_verify_int8_value_magnitude_bad_page_and_contiguous(Y, v_mul, nq):
    """Large and tiny values (the V-scale shift), a planted bad page (flagged,
    its keys masked) and the contiguous layout, at two and three column
    blocks."""
    _say(f"verify int8 v x {v_mul}, nq={nq}, bad page, contiguous")
    got, refs, err = _verify_batch(Y, [300, 77], nq, 24, 4, seed=970 + nq, bad_page=(0, 5),
                                   kv=Y.KV_INT8, v_mul=v_mul)
    assert err == Y.DEVERR_BLOCK_ID
    for s in range(2):
        assert np.all(np.isfinite(got[s]))
        _compare_attention(f"verify_int8/v_mul{v_mul:g}/q{nq}/bad_page/{s}", got[s] / v_mul,
                           refs[s] / v_mul, bf16_out=False)
    a, refs, _ = _verify_batch(Y, [1234], nq, 24, 4, seed=975, kv=Y.KV_INT8, v_mul=v_mul)
    b, _, _ = _verify_batch(Y, [1234], nq, 24, 4, seed=975, paged=False, kv=Y.KV_INT8,
                            v_mul=v_mul)
    assert np.array_equal(a, b)


def test_verify_masks_and_flags_a_bad_page(Y):
    _say("verify bad page")
    got, refs, err = _verify_batch(Y, [300, 77], 4, 24, 4, seed=910, bad_page=(0, 5))
    assert err == Y.DEVERR_BLOCK_ID
    for s in range(2):
        _compare_attention(f"verify/bad_page/{s}", got[s], refs[s], bf16_out=False)


def test_verify_contiguous_equals_paged_bitwise(Y):
    _say("verify contiguous vs paged")
    a, refs, _ = _verify_batch(Y, [1234], 6, 24, 4, seed=920, paged=True)
    b, _, _ = _verify_batch(Y, [1234], 6, 24, 4, seed=920, paged=False)
    assert np.array_equal(a, b)
    _compare_attention("verify/contiguous", b[0], refs[0], bf16_out=False)


def test_verify_bf16_output(Y):
    _say("verify bf16 output")
    got, refs, err = _verify_batch(Y, [2049, 5], 4, 24, 4, seed=925, out_f32=False)
    assert err == 0
    for s in range(2):
        _compare_attention(f"verify/bf16_out/{s}", got[s], refs[s])


def test_verify_short_sequence_flags_and_zeroes_rows(Y):
    """A sequence holding fewer tokens than queries: the queries that would sit
    at negative positions get zero rows, the others their causal attention,
    and the position bit is set."""
    _say("verify short sequence")
    got, refs, err = _verify_batch(Y, [2, 40], 4, 24, 4, seed=930)
    assert err == Y.DEVERR_POSITION
    assert np.all(got[0, :2] == 0)
    for s in range(2):
        _compare_attention(f"verify/short/{s}", got[s], refs[s], bf16_out=False)


def test_verify_nq1_matches_single_query_oracle(Y):
    """One query: the verify kernel at its smallest shape is single-query
    decode whose own key is already in the cache."""
    _say("verify one query")
    got, refs, err = _verify_batch(Y, [1, 16, 4097], 1, 24, 4, seed=940)
    assert err == 0
    for s in range(3):
        _compare_attention(f"verify/nq1/{s}", got[s], refs[s], bf16_out=False)


@pytest.mark.parametrize("name,nq", [("long", 4), ("long_int8", 4), ("long_int8", 6)])
def test_verify_long_layer(Y, W, name, nq):
    """The bench's verify step on one layer of the 1,048,576-token workload
    (bf16 cache, and the INT8 group-64 cache): nq new tokens appended at
    1,048,576 .. +nq-1 (the spare page), queries roped there, every output
    row checked against the oracle (over its own INT8 quantisation of its
    roped keys and of the values for the INT8 cache)."""
    w = W.WORKLOADS[name]
    u = 5
    _say(f"verify {name} layer {u} nq={nq}")
    N = w.n_ctx
    dl = W.build_decode_layer(w, u, device=DEV, spare_page=True)
    q, k_new, v_new = W.verify_inputs(w, u, nq, device=DEV)
    pos = torch.arange(N, N + nq, dtype=torch.int32, device=DEV)
    yp = w.yarn()
    Y.yarn_rope_apply(yp, k_new, pos)
    Y.kv_append_quantize(dl.layer, k_new, v_new, dl.block_tables[0], pos)
    qv = q.view(1, nq, w.hq, 256)
    Y.yarn_rope_apply(yp, q, pos)
    lens = torch.full((1,), N + nq, dtype=torch.int32, device=DEV)
    out = torch.empty((1, nq, w.hq, 256), dtype=torch.float32, device=DEV)
    ws = torch.empty(Y.verify_workspace_size(1, nq, w.hq, w.hkv, N + nq), dtype=torch.uint8,
                     device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.verify_attention(dl.layer, qv, dl.block_tables, lens, N + nq, out, ws, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = _f64(out)[0]
    gq = _bits(q)
    del dl, out, ws
    torch.cuda.empty_cache()
    _, k, v, _ = _host_case_full(W, w, u)
    t = O.yarn_table(original_max_position=w.orig)
    qh_raw, kh_raw, vh = W.verify_inputs_host(w, u, nq)
    qh = O.rope(qh_raw, np.arange(N, N + nq), t, bf16_out=True)
    assert np.array_equal(gq, qh)
    k = np.concatenate([k, O.rope(kh_raw, np.arange(N, N + nq), t, bf16_out=True)])
    v = np.concatenate([v, vh])
    qf = O.bf16_to_f64(qh)
    if w.int8:
        kc, ksc = O.int8_quantize(k)
        del k
        vc, vsc = O.int8_quantize(v)
        del v
    for i in range(nq):
        if w.int8:
            n = N + i + 1
            ref = O.decode_attention(qf[i], kc[:n], vc[:n], int8=(ksc[:n], vsc[:n]))
        else:
            ref = O.decode_attention(qf[i], k[: N + i + 1], v[: N + i + 1])
        _compare_attention(f"verify/{name}/q{i}", got[i], ref, bf16_out=False)
