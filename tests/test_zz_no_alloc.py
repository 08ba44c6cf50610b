"""The decode entry point that allocates nothing (yrk_decode_attention_noalloc)
against yrk_decode_attention on the same inputs, through the C ABI: the two
run the same kernels on the same split plan, so the outputs must be
byte-identical.  Two calls in a row on the library's device scratch, the
second with a smaller input (the scratch keeps the first call's partials),
in each cache format; and shapes beyond the scratch are refused on the host."""
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


def _say(msg):
    print(f"[no-alloc] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def Y():
    import yarn_rope_kv_amd
    return yarn_rope_kv_amd


@pytest.fixture(scope="module")
def W():
    import workloads
    return workloads


def _both(Y, W, w, dl):
    """(output of the workspace entry, output of the no-alloc entry, error words)."""
    out_ws, ws = W.decode_outputs(w, dl, device=DEV)
    out_na = torch.empty_like(out_ws)
    out_na.fill_(float("nan"))
    e1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    e2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y.decode_attention(dl.layer, dl.q, dl.block_tables, dl.seq_lens, dl.max_seq_len, out_ws, ws,
                       err=e1)
    Y.decode_attention_noalloc(dl.layer, dl.q, dl.block_tables, dl.seq_lens, dl.max_seq_len,
                               out_na, err=e2)
    torch.cuda.synchronize()
    return out_ws, out_na, int(e1.item()), int(e2.item())


def _same_bytes(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4", "int8"])
def test_noalloc_equals_workspace_entry_on_two_calls(Y, W, fmt):
    kw = dict(nvfp4=fmt == "nvfp4", int8=fmt == "int8",
              elem_outlier_p=0.01 if fmt != "bf16" else 0.0)
    # first call: 15 sessions x 16,384 tokens in one batched call (8 splits);
    # second: one 4,100-token sequence, fewer partial slots than the first
    big = W.Workload(f"na_big_{fmt}", 2101, 16384, seqs=15, **kw)
    small = W.Workload(f"na_small_{fmt}", 2102, 4100, **kw)
    for w in (big, small):
        _say(f"{fmt}: {w.seqs} x {w.n_ctx} tokens")
        dl = W.build_decode_layer(w, 0, device=DEV)
        need = Y.decode_workspace_size(w.seqs, w.hq, w.hkv, w.n_ctx)
        assert 0 < need <= Y.NOALLOC_SCRATCH_BYTES
        out_ws, out_na, e1, e2 = _both(Y, W, w, dl)
        assert e1 == e2 == 0
        assert bool(torch.isfinite(out_ws.float()).all())
        assert _same_bytes(out_ws, out_na), f"{fmt} {w.name}"
        del dl


def test_noalloc_ragged_batch_after_a_larger_call(Y, W):
    """Sequences of lengths 0 .. 4,097 after a call that left partials of
    other shapes in the scratch: empty sequences still give zero rows."""
    w = W.Workload("na_ragged", 2103, 4097, seqs=7)
    dl = W.build_decode_layer(w, 0, device=DEV)
    dl.seq_lens.copy_(torch.tensor([0, 1, 15, 16, 17, 1000, 4097], dtype=torch.int32))
    out_ws, out_na, e1, e2 = _both(Y, W, w, dl)
    assert e1 == e2 == 0
    assert _same_bytes(out_ws, out_na)
    assert bool((out_na[0] == 0).all())


def test_noalloc_refuses_shapes_beyond_its_scratch(Y, W):
    """Partials beyond the scratch: YRK_ENOSPC from the host, nothing
    launched, the output untouched."""
    w = W.Workload("na_tiny", 2104, 64)
    dl = W.build_decode_layer(w, 0, device=DEV)
    S = 4096                                        # 4,096 x 24 heads x 1 split x 1 KiB > 16 MiB
    assert Y.decode_workspace_size(S, 24, 4, 64) > Y.NOALLOC_SCRATCH_BYTES
    q = dl.q.expand(S, 24, 256).contiguous()
    bt = dl.block_tables.expand(S, -1).contiguous()
    lens = dl.seq_lens.expand(S).contiguous()
    out = torch.full((S, 24, 256), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(Y.YrkError) as ei:
        Y.decode_attention_noalloc(dl.layer, q, bt, lens, 64, out)
    assert ei.value.status == Y.ENOSPC
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
