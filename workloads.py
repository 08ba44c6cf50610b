"""GPU-side construction of the synthetic workloads, through the C ABI only.

Used by bench.py, the smoke check and the GPU tests.  It never imports the
oracle: the tests build the oracle's side of each case from the same seeded
generator (``synth``) on their own.

Workloads (sizes from the model the pages describe: 4 KV heads x head dim
256, 24 query heads, YaRN x4 from a 262,144-token window, rope_theta 1e7,
16-token pages):

  tiny      1 layer, 4,096 cached tokens at 0..4095, query at 4,096, YaRN x4
            from an original window of 1,024, contiguous KV, fp32 output.
  native    1 layer, 262,144 cached tokens, paged over a seeded permutation
            of 16,384 pages; K and V have 4 seeded outlier channels per head
            scaled x8.
  long      16 layers x 1,048,576 cached tokens (64 GiB of bf16 KV), one
            seeded page permutation per layer and a planted needle per layer:
            at one seeded position the key of KV head g is 2 x the roped
            query of head 6g.
  long_fp4  the same shapes over an NVFP4 cache; 1% of K and V elements are
            x20 outliers; tensor scale amax / 2688 per (layer, K or V).
  long_int8 the same shapes over an INT8 group-64 cache, with the same x20
            element outliers.
  sessions  15 sessions x 131,072 cached tokens dealt from one shared pool
            of 122,880 pages, one decode query each (one batched call).
  prefill   one 8,192-token causal chunk at positions 1,040,384..1,048,575
            over a 1,048,576-token cache (65,536 permuted pages).
  long_tp2, prefill_tp2
            one card's share when the 4 KV heads are split over two cards
            (12 query / 2 KV heads): 4 layers x 1,048,576 cached tokens with
            a needle, and the 8,192-token prefill chunk.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import synth
import yarn_rope_kv_amd as Y

HQ, HKV, D = 24, 4, 256


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    n_ctx: int
    layers: int = 1
    seqs: int = 1
    paged: bool = True
    nvfp4: bool = False
    int8: bool = False
    orig: int = 262144
    chan_outliers: int = 0        # per-head outlier channels (x8) in K and V
    elem_outlier_p: float = 0.0   # element outliers (x20) in K and V
    needle: bool = False
    f32_out: bool = False
    prefill_chunk: int = 0
    hq: int = HQ                  # query heads
    hkv: int = HKV                # KV heads

    @property
    def group(self):
        return self.hq // self.hkv

    def yarn(self) -> Y.YarnParams:
        return Y.YarnParams(rope_theta=1e7, head_dim=D, rotary_dim=64, factor=4.0,
                            original_max_position=self.orig, beta_fast=32.0, beta_slow=1.0)

    @property
    def pages_per_seq(self):
        return -(-self.n_ctx // Y.BLOCK_SIZE)


WORKLOADS = {
    "tiny": Workload("tiny", 1001, 4096, orig=1024, paged=False, f32_out=True),
    "native": Workload("native", 1002, 262144, chan_outliers=4),
    "long": Workload("long", 1003, 1048576, layers=16, needle=True),
    "long_fp4": Workload("long_fp4", 1004, 1048576, layers=16, nvfp4=True, elem_outlier_p=0.01),
    "long_int8": Workload("long_int8", 1008, 1048576, layers=16, int8=True, elem_outlier_p=0.01),
    "sessions": Workload("sessions", 1005, 131072, seqs=15),
    "prefill": Workload("prefill", 1005, 1048576, prefill_chunk=8192),
    "long_tp2": Workload("long_tp2", 1006, 1048576, layers=4, needle=True, hq=12, hkv=2),
    "prefill_tp2": Workload("prefill_tp2", 1007, 1048576, prefill_chunk=8192, hq=12, hkv=2),
}


def chan_mul(w: Workload, layer: int, tensor: int):
    if not w.chan_outliers:
        return None
    return synth.outlier_channels(w.seed, layer, tensor, w.hkv, D, w.chan_outliers, 8.0)


def gen_kv(w: Workload, unit: int, tensor: int, ntok: int, out: torch.Tensor, token0: int = 0):
    """Raw (un-roped) K or V rows [ntok, hkv, 256] of one layer / session."""
    ostream = synth.K_OUTLIER if tensor == synth.K else synth.V_OUTLIER
    synth.dev_fill(out, w.seed, synth.stream_id(unit, tensor), token0, ntok, w.hkv, D,
                   chan_mul=chan_mul(w, unit, tensor), outlier_stream=synth.stream_id(unit, ostream),
                   outlier_p=w.elem_outlier_p, outlier_mul=20.0)
    return out


def gen_q(w: Workload, unit: int, ntok: int, device, token0: int = 0):
    q = torch.empty((ntok, w.hq, D), dtype=torch.bfloat16, device=device)
    synth.dev_fill(q, w.seed, synth.stream_id(unit, synth.Q), token0, ntok, w.hq, D)
    return q


# Verify-step queries take their own slice of the query stream (decode's
# query is token 0, the bench step's new one token 1).
VERIFY_Q_TOKEN0 = 8


def verify_inputs(w: Workload, unit: int, nq: int, device):
    """Raw (un-roped) inputs of one layer's verify step: nq queries [nq, hq, 256]
    and the nq new keys and values [nq, hkv, 256] that take positions
    n_ctx .. n_ctx + nq - 1."""
    q = gen_q(w, unit, nq, device, token0=VERIFY_Q_TOKEN0)
    k = torch.empty((nq, w.hkv, D), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    gen_kv(w, unit, synth.K, nq, k, token0=w.n_ctx)
    gen_kv(w, unit, synth.V, nq, v, token0=w.n_ctx)
    return q, k, v


def verify_inputs_host(w: Workload, unit: int, nq: int):
    """The same inputs as verify_inputs, drawn by the host generator (bf16 bits)."""
    q = synth.host_fill(w.seed, synth.stream_id(unit, synth.Q), VERIFY_Q_TOKEN0, nq, w.hq, D)
    kw = dict(outlier_p=w.elem_outlier_p, outlier_mul=20.0) if w.elem_outlier_p else {}
    kv = []
    for tensor, ostream in ((synth.K, synth.K_OUTLIER), (synth.V, synth.V_OUTLIER)):
        kv.append(synth.host_fill(w.seed, synth.stream_id(unit, tensor), w.n_ctx, nq, w.hkv, D,
                                  chan_mul=chan_mul(w, unit, tensor),
                                  outlier_stream=synth.stream_id(unit, ostream), **kw))
    return q, kv[0], kv[1]


def page_table(w: Workload, unit: int):
    """Page table(s) of one layer: [seqs, pages_per_seq] int32 (numpy)."""
    if not w.paged:
        return None
    total = w.seqs * w.pages_per_seq
    perm = synth.block_permutation(w.seed + 7919 * unit, total)
    return perm.reshape(w.seqs, w.pages_per_seq)


@dataclasses.dataclass
class DecodeLayer:
    layer: Y.KVLayer
    q: torch.Tensor               # roped [S, hq, 256] bf16
    block_tables: torch.Tensor | None
    seq_lens: torch.Tensor
    max_seq_len: int
    needle_pos: int = -1


def build_decode_layer(w: Workload, unit: int, device="cuda", keep_raw=False, spare_page=False):
    """One layer of a decode workload on the GPU: roped query (position n_ctx)
    and a cache filled by rope + append (+ NVFP4 or INT8 quantisation).  spare_page
    adds one more page per sequence (table column pages_per_seq; for the
    contiguous layout one more block of capacity) so a decode step can append
    its own token at position n_ctx."""
    S, N = w.seqs, w.n_ctx
    tables = page_table(w, unit)
    num_blocks = S * w.pages_per_seq
    if spare_page and tables is not None:
        spare = np.arange(num_blocks, num_blocks + S, dtype=np.int32).reshape(S, 1)
        tables = np.ascontiguousarray(np.concatenate([tables, spare], axis=1))
        num_blocks += S
    elif spare_page:
        num_blocks += 1
    kv = Y.KV_NVFP4 if w.nvfp4 else (Y.KV_INT8 if w.int8 else Y.KV_BF16)
    layer = Y.KVLayer.allocate(kv, w.hkv, num_blocks,
                               paged=w.paged, device=device)
    yp = w.yarn()
    q = torch.empty((S, w.hq, D), dtype=torch.bfloat16, device=device)
    pos_q = torch.full((1,), N, dtype=torch.int32, device=device)
    positions = torch.arange(N, dtype=torch.int32, device=device)
    k = torch.empty((N, w.hkv, D), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    bt_dev = torch.from_numpy(tables).to(device) if tables is not None else None
    needle = -1
    for s in range(S):
        u = unit if S == 1 else s
        q[s:s + 1] = gen_q(w, u, 1, device)
        Y.yarn_rope_apply(yp, q[s:s + 1], pos_q)
        gen_kv(w, u, synth.K, N, k)
        gen_kv(w, u, synth.V, N, v)
        Y.yarn_rope_apply(yp, k, positions)
        if w.needle:
            needle = synth.needle_position(w.seed, u, N)
            for g in range(w.hkv):
                k[needle, g] = q[s, w.group * g] * 2    # exact doubling of a bf16 value
        if w.nvfp4:
            Y.nvfp4_tensor_scale(k, layer.k_tensor_scale)
            Y.nvfp4_tensor_scale(v, layer.v_tensor_scale)
        Y.kv_append_quantize(layer, k, v, bt_dev[s] if bt_dev is not None else None, positions)
    seq_lens = torch.full((S,), N, dtype=torch.int32, device=device)
    out = DecodeLayer(layer, q, bt_dev, seq_lens, N, needle)
    if keep_raw:
        out.k_roped, out.v = k, v
    else:
        del k, v
    return out


def decode_outputs(w: Workload, dl: DecodeLayer, device="cuda"):
    S = dl.q.shape[0]
    out = torch.empty((S, w.hq, D), dtype=torch.float32 if w.f32_out else torch.bfloat16,
                      device=device)
    ws = torch.empty(Y.decode_workspace_size(S, w.hq, w.hkv, dl.max_seq_len), dtype=torch.uint8,
                     device=device)
    return out, ws


def run_decode(dl: DecodeLayer, out, ws, err=None):
    return Y.decode_attention(dl.layer, dl.q, dl.block_tables, dl.seq_lens, dl.max_seq_len, out,
                              ws, err=err)


@dataclasses.dataclass
class PrefillCase:
    layer: Y.KVLayer
    q: torch.Tensor               # roped [T, hq, 256]
    block_table: torch.Tensor
    q_start: int


def build_prefill(w: Workload, device="cuda", chunk_tokens=1 << 18):
    """Cache of w.n_ctx tokens (all roped and appended, the chunk's own keys
    included) and the chunk's roped queries."""
    N, T = w.n_ctx, w.prefill_chunk
    tables = page_table(w, 0)
    layer = Y.KVLayer.allocate(Y.KV_BF16, w.hkv, w.pages_per_seq, paged=True, device=device)
    bt = torch.from_numpy(tables[0]).to(device)
    yp = w.yarn()
    k = torch.empty((chunk_tokens, w.hkv, D), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    for t0 in range(0, N, chunk_tokens):
        n = min(chunk_tokens, N - t0)
        pos = torch.arange(t0, t0 + n, dtype=torch.int32, device=device)
        gen_kv(w, 0, synth.K, n, k[:n], token0=t0)
        gen_kv(w, 0, synth.V, n, v[:n], token0=t0)
        Y.yarn_rope_apply(yp, k[:n], pos)
        Y.kv_append_quantize(layer, k[:n], v[:n], bt, pos)
    q0 = N - T
    q = gen_q(w, 0, T, device, token0=q0)
    Y.yarn_rope_apply(yp, q, torch.arange(q0, N, dtype=torch.int32, device=device))
    return PrefillCase(layer, q, bt, q0)


def prefill_sample(w: Workload, n_rows=256, seed=77):
    """A stratified sample of (token, query head) rows of a prefill chunk, the
    kernel's row order in mind: per KV head g the rows are R = 6 token +
    (head - 6 g), 192 to a workgroup, 48 to a wave, 16 to a row block.  The
    sample takes the first 64 and the last 64 R and n_rows - 128 seeded ones,
    dealt round-robin over the KV heads.  Returns (tokens, heads), int64."""
    T, G = w.prefill_chunk, w.group
    R_all = T * G
    rng = np.random.default_rng(seed)
    Rs = np.concatenate([np.arange(64), np.arange(R_all - 64, R_all),
                         rng.choice(np.arange(64, R_all - 64), n_rows - 128, replace=False)])
    gs = np.arange(n_rows) % w.hkv
    return (Rs // G).astype(np.int64), (gs * G + Rs % G).astype(np.int64)

