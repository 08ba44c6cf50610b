"""GPU parity of the fused rope + append pass: the step's queries roped in
place and its keys roped on the way into the cache, against the oracle's
rope followed by its copy or quantiser (bf16, NVFP4, INT8 group-64), at
positions up to 2^20; and byte-equality with the separate rope and append
passes."""
import numpy as np
import pytest

import oracle as O
import synth

from test_gpu_parity import DEV, _bits, _say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_FMT = {"bf16": 0, "nvfp4": 1, "int8": 2}


@pytest.fixture(scope="module")
def Y():
    import yarn_rope_kv_amd
    return yarn_rope_kv_amd


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def _case(seed, T, paged, hq=24, hkv=4):
    """T tokens: raw q [T, hq, 256], k, v [T, hkv, 256] (1% x20 outliers in k
    and v), distinct positions, and for the paged layout a block table that
    gives each token's page its own block (so positions can reach 2^20 with
    a pool of T blocks)."""
    rng = np.random.default_rng(seed)
    q = synth.host_fill(seed, synth.Q, 0, T, hq, 256)
    k = synth.host_fill(seed, synth.K, 0, T, hkv, 256, outlier_stream=synth.K_OUTLIER,
                        outlier_p=0.01, outlier_mul=20.0)
    v = synth.host_fill(seed, synth.V, 0, T, hkv, 256, outlier_stream=synth.V_OUTLIER,
                        outlier_p=0.01, outlier_mul=20.0)
    if paged:
        # the first and last positions of the original window and of 2^20,
        # then distinct random pages
        special = np.array([0, 262143, 262144, (1 << 20) - 1])
        if T < len(special):               # fewer tokens: the largest positions
            special = special[len(special) - T:]
        nrest = T - len(special)
        rest = rng.choice(np.setdiff1d(np.arange(1 << 16), special // 16), size=nrest,
                          replace=False)
        pages = np.concatenate([special // 16, rest])
        pos = np.concatenate([special, rest * 16 + rng.integers(0, 16, size=nrest)])
        table = np.full(1 << 16, -1, dtype=np.int32)
        table[pages] = rng.permutation(T).astype(np.int32)
        blocks = T
    else:
        pos = rng.permutation(T)
        table = None
        blocks = -(-T // 16)
    return q, k, v, pos.astype(np.int64), table, blocks


def _pool_rows(pool_bytes, table, pos, row_bytes, blocks, hkv=4):
    """Rows [T, hkv, row_bytes] of a cache plane at the tokens' positions."""
    a = pool_bytes.reshape(-1)
    if table is None:
        return a.reshape(blocks * 16, hkv, row_bytes)[pos]
    blk = table[pos // 16]
    slot = pos % 16
    return a.reshape(blocks, hkv, 16, row_bytes)[blk, :, slot]


def _layer(Y, kv, blocks, paged, kS=None, vS=None, hkv=4):
    L = Y.KVLayer.allocate(kv, hkv, blocks, paged=paged, device=DEV)
    for t in (L.k, L.v) + ((L.k_scale, L.v_scale) if L.k_scale is not None else ()):
        t.zero_()
    if kv == Y.KV_NVFP4:
        L.k_tensor_scale.fill_(float(kS))
        L.v_tensor_scale.fill_(float(vS))
    return L


@pytest.mark.parametrize("paged,hq,hkv", [(True, 24, 4), (False, 24, 4), (True, 12, 2),
                                          (True, 6, 1)])
@pytest.mark.parametrize("fmt", ["bf16", "nvfp4", "int8"])
def test_rope_append_matches_oracle(Y, fmt, paged, hq, hkv):
    """Also one card's 12 q / 2 KV-head share and a single KV head, whose
    rows put rotary and pass-through groups in the same pass."""
    kv = _FMT[fmt]
    T = 300
    _say(f"rope_append {fmt} paged={paged} {hq}x{hkv}")
    q, k, v, pos, table, blocks = _case(1200 + kv + 10 * paged + hkv, T, paged, hq, hkv)
    t = O.yarn_table()
    q_ref = O.rope(q, pos, t, bf16_out=True)
    k_ref = O.rope(k, pos, t, bf16_out=True)
    kS = vS = None
    if kv == Y.KV_NVFP4:
        kS, vS = O.nvfp4_tensor_scale(k_ref), O.nvfp4_tensor_scale(v)
    L = _layer(Y, kv, blocks, paged, kS, vS, hkv)
    qd = _dev(q)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.rope_append(L, Y.YarnParams(), qd, _dev(k), _dev(v),
                  torch.from_numpy(table).to(DEV) if paged else None,
                  torch.from_numpy(pos.astype(np.int32)).to(DEV), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # queries: the rope kernel's bar (one bf16 step at an fp64 rounding tie at most)
    got_q = _bits(qd)
    diff = got_q != q_ref
    assert np.all(np.abs(got_q.astype(np.int32) - q_ref.astype(np.int32))[diff] <= 1)
    assert diff.sum() <= max(1, diff.size // 100000)
    if kv == Y.KV_BF16:
        gk = _pool_rows(_bits(L.k).view(np.uint8), table, pos, 512, blocks, hkv).view(np.uint16)
        gv = _pool_rows(_bits(L.v).view(np.uint8), table, pos, 512, blocks, hkv).view(np.uint16)
        assert np.array_equal(gk.reshape(k_ref.shape), k_ref)
        assert np.array_equal(gv.reshape(v.shape), v)
        return
    for raw, codes_t, scales_t, S in ((k_ref, L.k, L.k_scale, kS), (v, L.v, L.v_scale, vS)):
        cb = codes_t.cpu().numpy().view(np.uint8)
        sb = scales_t.cpu().numpy().view(np.uint8)
        if kv == Y.KV_NVFP4:
            c_ref, s_ref = O.nvfp4_quantize(raw, S)
            gc = _pool_rows(cb, table, pos, 128, blocks, hkv)
            gs = _pool_rows(sb, table, pos, 16, blocks, hkv)
            assert np.array_equal(gs.reshape(s_ref.shape), s_ref)
            assert np.array_equal(gc.reshape(-1), O.nvfp4_pack(c_ref).reshape(-1))
        else:
            c_ref, s_ref = O.int8_quantize(raw)
            gc = _pool_rows(cb, table, pos, 256, blocks, hkv)
            gs = _pool_rows(sb, table, pos, 8, blocks, hkv)
            assert np.array_equal(gs.reshape(-1).view(np.uint16).reshape(s_ref.shape), s_ref)
            assert np.array_equal(gc.reshape(-1).view(np.int8).reshape(c_ref.shape), c_ref)


@pytest.mark.parametrize("T", [1, 257, 1000])
@pytest.mark.parametrize("fmt", ["bf16", "nvfp4", "int8"])
def test_rope_append_equals_separate_passes_bitwise(Y, fmt, T):
    """The fused pass against rope (q, then k) and append on the same
    inputs: every byte of the queries, the codes and the scales.  Up to 512
    tokens a launch gives each token four waves (one token: a decode step),
    beyond that one wave per token; both are covered."""
    kv = _FMT[fmt]
    _say(f"rope_append vs separate {fmt} T={T}")
    q, k, v, pos, table, blocks = _case(1300 + kv + T, T, True)
    kS = vS = 0.0123 if kv == Y.KV_NVFP4 else None
    A = _layer(Y, kv, blocks, True, kS, vS)
    B = _layer(Y, kv, blocks, True, kS, vS)
    bt = torch.from_numpy(table).to(DEV)
    pd = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    p = Y.YarnParams()
    qa, qb, kb = _dev(q), _dev(q), _dev(k)
    Y.rope_append(A, p, qa, _dev(k), _dev(v), bt, pd)
    Y.yarn_rope_apply(p, qb, pd)
    Y.yarn_rope_apply(p, kb, pd)
    Y.kv_append_quantize(B, kb, _dev(v), bt, pd)
    torch.cuda.synchronize()
    assert torch.equal(qa.view(torch.int16), qb.view(torch.int16))
    for ta, tb in ((A.k, B.k), (A.v, B.v)) + (((A.k_scale, B.k_scale), (A.v_scale, B.v_scale))
                                             if A.k_scale is not None else ()):
        assert torch.equal(ta.view(torch.uint8), tb.view(torch.uint8))


def test_rope_append_keys_only_and_bad_position(Y):
    """Without queries; a position beyond the table is flagged and its key
    and value are skipped, the other tokens are written."""
    _say("rope_append keys only, bad position")
    q, k, v, pos, table, blocks = _case(1400, 40, True)
    pos_bad = pos.copy()
    pos_bad[7] = (1 << 20) + 3                      # beyond the 2^16-entry table
    L = _layer(Y, Y.KV_BF16, blocks, True)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.rope_append(L, Y.YarnParams(), None, _dev(k), _dev(v), torch.from_numpy(table).to(DEV),
                  torch.from_numpy(pos_bad.astype(np.int32)).to(DEV), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == Y.DEVERR_POSITION
    k_ref = O.rope(k, pos, O.yarn_table(), bf16_out=True)
    gk = _pool_rows(_bits(L.k).view(np.uint8), table, pos, 512, blocks).view(np.uint16)
    gk = gk.reshape(k_ref.shape)
    keep = np.arange(40) != 7
    assert np.array_equal(gk[keep], k_ref[keep])
    assert np.all(gk[7] == 0)                       # token 7's own block was never written


def test_rope_append_negative_position_leaves_query_and_cache(Y):
    """A negative position: that token's query is not roped, its key and
    value are not written, and the position bit is set; the other tokens'
    queries and keys are the oracle's."""
    _say("rope_append negative position")
    q, k, v, pos, table, blocks = _case(1401, 12, False)
    pos_bad = pos.copy()
    pos_bad[5] = -3
    L = _layer(Y, Y.KV_BF16, blocks, False)
    qd = _dev(q)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.rope_append(L, Y.YarnParams(), qd, _dev(k), _dev(v), None,
                  torch.from_numpy(pos_bad.astype(np.int32)).to(DEV), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == Y.DEVERR_POSITION
    keep = np.arange(12) != 5
    got_q = _bits(qd)
    assert np.array_equal(got_q[5], q[5])
    assert np.array_equal(got_q[keep], O.rope(q[keep], pos[keep], O.yarn_table(), bf16_out=True))
    gk = _pool_rows(_bits(L.k).view(np.uint8), None, pos[keep], 512, blocks).view(np.uint16)
    k_ref = O.rope(k[keep], pos[keep], O.yarn_table(), bf16_out=True)
    assert np.array_equal(gk.reshape(k_ref.shape), k_ref)
    assert np.all(_bits(L.k).reshape(blocks * 16, 4, 256)[pos[5]] == 0)   # never written
