"""Benchmark of the decode hot path (and chunked prefill) on one MI355X.

A step is one decode step of the 16-layer, 1,048,576-token workload ("long"
in workloads.py): for every layer, rope the new query and the new key
(YaRN x4), append the new key/value to the paged bf16 cache, and run split-K
decode attention + merge over the 1,048,576 cached tokens.  All inputs are
resident in HBM before the timed region starts.

Prints one JSON line.  value = KV token-layers per second (16 x 1,048,576 per
step / step time).  roofline = the decode attention launches (split + merge),
timed with HIP events on the stream they run on, against 8 TB/s.

The "configs" object holds one entry per workload the decode path is
specified on (tiny, native, long, long_fp4, the 15-session batch and the
prefill chunk): its throughput, the median and mean of the per-launch HIP
event times, the roofline fraction of the dominant kernel, whether two runs
gave byte-identical outputs, and the oracle timed on a bounded sample of the
same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KV_BYTES_PER_TOKEN_LAYER = 4096           # 4 KV heads x 256 x 2 B x (K, V)
NVFP4_BYTES_PER_TOKEN_LAYER = 1152        # 4 x (128 code + 16 scale bytes) x (K, V)
INT8_BYTES_PER_TOKEN_LAYER = 2112         # 4 x (256 code + 4 x 2 scale bytes) x (K, V)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def profile_record(record):
    """A committed rocprofv3 record (profiles/*.json), or None when a kernel
    source it names has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", record)
    try:
        rec = json.load(open(path))
        sources = rec.get("kernel_sources") or [[rec["kernel_source"], rec["kernel_source_sha256"]]]
        for src, sha in sources:
            if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != sha:
                return None
    except (OSError, ValueError, KeyError):
        return None
    return rec


def measured_traffic(record):
    """HBM bytes per launch from a committed counter record (FETCH_SIZE and
    WRITE_SIZE scaled by the plain-copy calibration), or None."""
    rec = profile_record(record) if record else None
    if rec is None or "fetch_kib_per_call" not in rec:
        return None
    return 1024.0 * (rec["fetch_kib_per_call"] * rec["fetch_scale"] +
                     rec["write_kib_per_call"] * rec["write_scale"])


def decode_bytes_per_launch(n_ctx, per_token, hq=24, seqs=1):
    # KV stream + q and out (hq heads x 256 x 2 B each) + the page table (4 B / 16 tokens)
    return seqs * (per_token * n_ctx + 2 * hq * 256 * 2 + 4 * (n_ctx // 16))


def launch_stats(ms):
    ms = sorted(ms)
    return {"n": len(ms), "median_ms": statistics.median(ms), "mean_ms": sum(ms) / len(ms),
            "p10_ms": ms[len(ms) // 10], "p90_ms": ms[(9 * len(ms)) // 10]}


def hbm_roofline(bytes_per_launch, mean_ms, record=None, extra=None):
    achieved = bytes_per_launch / (mean_ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(record),
         "bytes_per_launch": bytes_per_launch, "avg_launch_ms": mean_ms}
    if extra:
        r.update(extra)
    return r


# -- decode steps -------------------------------------------------------------------

def build_step(W, Y, w, torch, dev, layers=None):
    """The layers of a decode workload plus a step over them: per layer (and
    per sequence) the new query and key roped at position n_ctx and the key
    and value appended (one fused pass), then one decode call for all the
    sequences over the n_ctx cached tokens."""
    if layers is None:
        layers = []
        for l in range(w.layers):
            layers.append(W.build_decode_layer(w, l, device=dev, spare_page=True))
            if l % 4 == 3:
                log(f"{w.name}: built layer {l + 1}/{w.layers}")
    N, L, S = w.n_ctx, w.layers, w.seqs
    q_in = torch.empty((L, S, w.hq, 256), dtype=torch.bfloat16, device=dev)
    k_in = torch.empty((L, S, w.hkv, 256), dtype=torch.bfloat16, device=dev)
    v_in = torch.empty((L, S, w.hkv, 256), dtype=torch.bfloat16, device=dev)
    for l in range(L):
        for s in range(S):
            u = l if S == 1 else s
            q_in[l, s:s + 1] = W.gen_q(w, u, 1, dev, token0=1)
            W.gen_kv(w, u, 1, 1, k_in[l, s:s + 1], token0=N)
            W.gen_kv(w, u, 2, 1, v_in[l, s:s + 1], token0=N)
    q_work = torch.empty_like(q_in)
    outs, wss = zip(*[W.decode_outputs(w, dl, device=dev) for dl in layers])
    pos_new = torch.full((1,), N, dtype=torch.int32, device=dev)
    yp = w.yarn()
    ev = []

    def step(timing=False):
        q_work.copy_(q_in)                               # roped in place below
        for l, dl in enumerate(layers):
            for s in range(S):
                Y.rope_append(dl.layer, yp, q_work[l, s:s + 1], k_in[l, s:s + 1],
                              v_in[l, s:s + 1],
                              dl.block_tables[s] if dl.block_tables is not None else None,
                              pos_new)
            if timing:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            Y.decode_attention(dl.layer, q_work[l], dl.block_tables, dl.seq_lens,
                               dl.max_seq_len, outs[l], wss[l])
            if timing:
                e1.record()
                ev.append((e0, e1))

    return step, ev, layers, outs


def time_steps(step, ev, steps, warmup, torch):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev.clear()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timing=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) for a, b in ev]


def repeat_identical(step, outs, torch):
    """Two more steps on the same inputs: are all outputs byte-identical?"""
    step()
    torch.cuda.synchronize()
    first = [o.clone() for o in outs]
    step()
    torch.cuda.synchronize()
    return all(torch.equal(a.view(torch.uint8), b.view(torch.uint8)) for a, b in zip(first, outs))


def bench_decode_config(W, Y, w, torch, dev, steps, warmup, per_token, desc, record=None,
                        cpu_seconds=3.0, keep_layers=False):
    log(f"{w.name}: building")
    step, ev, layers, outs = build_step(W, Y, w, torch, dev)
    log(f"{w.name}: timing {steps} steps")
    wall, ms = time_steps(step, ev, steps, warmup, torch)
    st = launch_stats(ms)
    bpl = decode_bytes_per_launch(w.n_ctx, per_token, w.hq, w.seqs)
    tokens = w.layers * w.seqs * w.n_ctx
    res = {"workload": desc, "value": tokens / (wall / steps), "unit": "KV token-layers/s",
           "ms_per_step": wall / steps * 1e3, "steps": steps, "decode_launch": st,
           "kv_gbs": tokens * per_token / (wall / steps) / 1e9,
           "roofline": hbm_roofline(bpl, st["mean_ms"], record,
                                    {"frac_at_median": bpl / (st["median_ms"] * 1e-3) / 1e9 /
                                     HBM_PEAK_GBS}),
           "repeat_byte_identical": repeat_identical(step, outs, torch)}
    kept = layers if keep_layers else None
    del step, ev, layers, outs
    torch.cuda.empty_cache()
    if cpu_seconds > 0:
        log(f"{w.name}: oracle on the host cores")
        res["cpu_baseline"] = cpu_decode_baseline(W, w, torch, dev, cpu_seconds)
    return res, kept


# -- the oracle on the host cores -----------------------------------------------------

def _raw_host(W, w, u, tensor, n, torch, dev, token0=0):
    """Raw K or V rows of one layer or session drawn by the generator's device
    twin (bit-identical to the host generator) and copied to the host."""
    import numpy as np
    t = torch.empty((n, w.hkv, 256), dtype=torch.bfloat16, device=dev)
    W.gen_kv(w, u, tensor, n, t, token0=token0)
    out = t.view(torch.int16).cpu().numpy().view(np.uint16)
    del t
    return out


def _oracle_cache(W, w, u, torch, dev, q_first=None):
    """The oracle's cache of layer (or session) u: its rope of the keys, the
    planted needle (against the decode query q_first, when given), then its
    quantiser for the workload's format.  Returns k, v and the format
    keyword of the oracle's attention calls."""
    import numpy as np
    import oracle as O
    import synth

    N = w.n_ctx
    t = O.yarn_table(original_max_position=w.orig)
    k = O.rope(_raw_host(W, w, u, synth.K, N, torch, dev), np.arange(N), t, bf16_out=True)
    v = _raw_host(W, w, u, synth.V, N, torch, dev)
    if w.needle and q_first is not None:
        p_star = synth.needle_position(w.seed, u, N)
        for g in range(w.hkv):
            k[p_star, g] = O.round_bf16(2.0 * O.bf16_to_f64(q_first[w.group * g]))
    kw = {}
    if w.nvfp4:
        kS, vS = O.nvfp4_tensor_scale(k), O.nvfp4_tensor_scale(v)
        k, ks = O.nvfp4_quantize(k, kS)
        v, vs = O.nvfp4_quantize(v, vS)
        kw = dict(nvfp4=(ks, vs, kS, vS))
    elif w.int8:
        k, ks = O.int8_quantize(k)
        v, vs = O.int8_quantize(v)
        kw = dict(int8=(ks, vs))
    return k, v, kw


def cpu_decode_baseline(W, w, torch, dev, min_seconds):
    """The oracle's decode attention on whole layers (or sessions) of the
    workload, one after another (the first again when a workload has only
    one) until at least min_seconds of oracle time; inputs (generation, the
    oracle's rope, its quantiser) are prepared outside the timed calls."""
    import oracle as O
    import synth

    N = w.n_ctx
    t = O.yarn_table(original_max_position=w.orig)
    units = w.layers if w.seqs == 1 else w.seqs

    def prepare(u):
        q = O.rope(synth.host_fill(w.seed, synth.stream_id(u, synth.Q), 0, 1, w.hq, 256), [N], t,
                   bf16_out=True)[0]
        k, v, kw = _oracle_cache(W, w, u, torch, dev, q_first=q)
        return O.bf16_to_f64(q), k, v, kw

    total, done, case, seen = 0.0, 0, None, set()
    while total < min_seconds:
        u = done % units
        if case is None or units > 1:
            case = prepare(u)
        qf, k, v, kw = case
        t0 = time.perf_counter()
        O.decode_attention(qf, k, v, **kw)
        total += time.perf_counter() - t0
        done += 1
        seen.add(u)
    what = "layers" if w.seqs == 1 else "sessions"
    return {"value": done * N / total, "unit": "KV token-layers/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"{done} calls over {len(seen)} of {units} {what} of the {w.name} "
                      f"workload: {N} cached tokens x {w.hq} q heads each, fp64, {total:.2f} s"}


def cpu_verify_baseline(W, w, torch, dev, nq=4):
    """The oracle's causal attention of nq queries (at positions N - nq ..
    N - 1, seeing keys up to their own) over layer 0's cache, once: the
    verify step's arithmetic at the workload's size."""
    import numpy as np
    import oracle as O
    import synth

    N = w.n_ctx
    t = O.yarn_table(original_max_position=w.orig)
    k, v, kw = _oracle_cache(W, w, 0, torch, dev)
    pos = np.arange(N - nq, N)
    q_raw = synth.host_fill(w.seed, synth.stream_id(0, synth.Q), 0, nq, w.hq, 256)
    qf = O.bf16_to_f64(O.rope(q_raw, pos, t, bf16_out=True))
    t0 = time.perf_counter()
    O.prefill_attention(qf, pos, k, v, **kw)
    total = time.perf_counter() - t0
    return {"value": N / total, "unit": "KV token-layers/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"one layer of the {w.name} workload: {nq} causal queries x {w.hq} q heads "
                      f"over {N} cached tokens, fp64, {total:.2f} s"}


def cpu_prefill_baseline(W, w, torch, dev):
    """The oracle on the stratified 256-row sample of the prefill chunk (the
    rows the GPU test checks), and the full chunk's time extrapolated from it
    by visible (query, key) pairs."""
    import numpy as np
    import oracle as O
    import synth

    N, T = w.n_ctx, w.prefill_chunk
    q0 = N - T
    t = O.yarn_table(original_max_position=w.orig)
    toks, heads = W.prefill_sample(w)
    k = O.rope(_raw_host(W, w, 0, synth.K, N, torch, dev), np.arange(N), t, bf16_out=True)
    v = _raw_host(W, w, 0, synth.V, N, torch, dev)
    q_raw = synth.host_fill(w.seed, synth.stream_id(0, synth.Q), q0, T, w.hq, 256)
    q = O.rope(q_raw[toks], q0 + toks, t, bf16_out=True)[np.arange(len(toks)), heads]
    qf = O.bf16_to_f64(q)
    total = 0.0
    for g in range(w.hkv):
        sel = np.nonzero(heads // w.group == g)[0]
        kg = np.ascontiguousarray(k[:, g:g + 1])
        vg = np.ascontiguousarray(v[:, g:g + 1])
        t0 = time.perf_counter()
        O.prefill_attention(qf[sel][:, None, :], q0 + toks[sel], kg, vg)
        total += time.perf_counter() - t0
    sample_pairs = float(np.sum(q0 + toks + 1))
    full_pairs = float(w.hq) * sum(q0 + i + 1 for i in range(T))
    flops = 4.0 * 256 * sample_pairs
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"256 stratified (token, head) rows of the chunk (first 64, last 64, 128 "
                      f"seeded by the kernel's row order), fp64, {total:.2f} s",
            "full_chunk_s_extrapolated": total * full_pairs / sample_pairs}


# -- verify, prefill, append ------------------------------------------------------------

def build_verify_step(W, Y, w, layers, nq, torch, dev):
    """A speculative verify step over a decode workload's layers: per layer,
    nq new tokens roped and appended at n_ctx .. n_ctx + nq - 1 (the spare
    page), then their nq queries, roped at the same positions, attend to the
    n_ctx + nq cached tokens causally."""
    N, L = w.n_ctx, w.layers
    q_in = torch.empty((L, nq, w.hq, 256), dtype=torch.bfloat16, device=dev)
    k_in = torch.empty((L, nq, w.hkv, 256), dtype=torch.bfloat16, device=dev)
    v_in = torch.empty_like(k_in)
    for l in range(L):
        q_in[l], k_in[l], v_in[l] = W.verify_inputs(w, l, nq, dev)
    q_work = torch.empty_like(q_in)
    pos_new = torch.arange(N, N + nq, dtype=torch.int32, device=dev)
    lens = torch.full((1,), N + nq, dtype=torch.int32, device=dev)
    outs = [torch.empty((1, nq, w.hq, 256), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ws = torch.empty(Y.verify_workspace_size(1, nq, w.hq, w.hkv, N + nq), dtype=torch.uint8,
                     device=dev)
    yp = w.yarn()
    ev = []

    def step(timing=False):
        q_work.copy_(q_in)                               # roped in place below
        for l, dl in enumerate(layers):
            Y.rope_append(dl.layer, yp, q_work[l], k_in[l], v_in[l], dl.block_tables[0], pos_new)
            if timing:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            Y.verify_attention(dl.layer, q_work[l:l + 1], dl.block_tables, lens, N + nq, outs[l],
                               ws)
            if timing:
                e1.record()
                ev.append((e0, e1))

    return step, ev


def bench_verify(W, Y, w, layers, torch, dev, steps, warmup, main_nq=4, sweep=(2, 4, 6),
                 per_token=KV_BYTES_PER_TOKEN_LAYER, fmt="bf16", record=None, cpu=False):
    """Verify steps at several query counts over the decode layers; the entry
    for main_nq (3 draft tokens) is the headline, the others are listed."""
    res = {}
    for nq in sweep:
        step, ev = build_verify_step(W, Y, w, layers, nq, torch, dev)
        wall, ms = time_steps(step, ev, steps, warmup, torch)
        st = launch_stats(ms)
        ctx = w.n_ctx + nq
        bpl = decode_bytes_per_launch(ctx, per_token, w.hq * nq)
        res[nq] = {"value": w.layers * ctx / (wall / steps), "launch": st,
                   "ms_per_step": wall / steps * 1e3, "bytes_per_launch": bpl,
                   "frac": bpl / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del step, ev
        torch.cuda.empty_cache()
    m = res[main_nq]
    out = {
        "workload": f"speculative verify step, {w.layers} layers x 1,048,576 + {main_nq} cached "
                    f"tokens ({fmt}), {main_nq} causal queries x 24 q / 4 KV heads",
        "value": m["value"], "unit": "KV token-layers/s", "ms_per_step": m["ms_per_step"],
        "launch": m["launch"],
        "roofline": hbm_roofline(m["bytes_per_launch"], m["launch"]["mean_ms"], record),
        "by_queries": {str(nq): {"mean_ms": r["launch"]["mean_ms"],
                                 "median_ms": r["launch"]["median_ms"], "frac": r["frac"]}
                       for nq, r in res.items()},
    }
    if cpu:
        log(f"{w.name}: verify oracle on the host cores")
        out["cpu_baseline"] = cpu_verify_baseline(W, w, torch, dev, main_nq)
    return out


def bench_prefill(W, Y, torch, dev, reps, name="prefill", cpu=False):
    w = W.WORKLOADS[name]
    case = W.build_prefill(w, device=dev)
    out = torch.empty_like(case.q)
    ws = torch.empty(Y.prefill_workspace_size(case.q.shape[0], w.hq), dtype=torch.uint8,
                     device=dev)
    T = case.q.shape[0]

    def run():
        Y.prefill_attention(case.layer, case.q, case.q_start, case.block_table, out, ws)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        ms.append((e0, e1))
    torch.cuda.synchronize()
    st = launch_stats([a.elapsed_time(b) for a, b in ms])
    first = out.clone()
    run()
    torch.cuda.synchronize()
    identical = torch.equal(first.view(torch.uint8), out.view(torch.uint8))
    pairs = sum(case.q_start + i + 1 for i in range(T))
    flops = 4.0 * 256 * pairs * w.hq
    tf = flops / (st["mean_ms"] * 1e-3) / 1e12
    record = "prefill_chunk_8192_over_1m.json" if name == "prefill" else None
    rec = profile_record(record) if record else None
    roof = {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": measured_traffic(record),
            "flop_per_launch": flops, "avg_launch_ms": st["mean_ms"]}
    if rec and "mfma_util_pct" in rec:
        roof["mfma_util_pct_counter"] = rec["mfma_util_pct"]
    res = {"workload": f"prefill: 8,192-token causal chunk at 1,040,384..1,048,575 over a "
                       f"1,048,576-token paged cache, {w.hq} q / {w.hkv} KV heads",
           "ms_per_chunk": st["mean_ms"], "launch": st, "tflops": tf, "flop_per_chunk": flops,
           "value": tf, "unit": "TFLOP/s", "roofline": roof,
           "repeat_byte_identical": identical}
    del case, out, ws
    torch.cuda.empty_cache()
    if cpu:
        log(f"{name}: oracle on the host cores (256-row sample)")
        res["cpu_baseline"] = cpu_prefill_baseline(W, w, torch, dev)
    return res


def bench_append(W, Y, torch, dev, reps=10):
    """Filling one 1,048,576-token layer (4 KV heads, paged over a seeded
    permutation): the bf16 copy, the NVFP4 and INT8 quantisers (the NVFP4
    tensor scale included), the plain rope of the keys, and the fused rope +
    append.  Algorithmic bytes: the bf16 keys and values read (4 KiB per
    token) plus what the cache format writes per token (the rope alone
    reads and writes the 64 rotary dims of each key head)."""
    w = W.WORKLOADS["long"]
    N = w.n_ctx
    k = torch.empty((N, w.hkv, 256), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    W.gen_kv(w, 0, 1, N, k)
    W.gen_kv(w, 0, 2, N, v)
    pos = torch.arange(N, dtype=torch.int32, device=dev)
    bt = torch.from_numpy(W.page_table(w, 0)[0]).to(dev)
    yp = w.yarn()

    def timed(fn):
        """Mean of reps calls, each between its own pair of HIP events (the
        median is reported beside it)."""
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        timed.median = statistics.median(ms)
        return sum(ms) / len(ms)

    out = {}
    read = 2 * w.hkv * 256 * 2 * N
    for name, kv, written in (("bf16_copy", Y.KV_BF16, 2 * w.hkv * 512),
                              ("nvfp4_quantize", Y.KV_NVFP4, 2 * w.hkv * 144),
                              ("int8_quantize", Y.KV_INT8, 2 * w.hkv * 264)):
        L = Y.KVLayer.allocate(kv, w.hkv, w.pages_per_seq, paged=True, device=dev)
        if kv == Y.KV_NVFP4:
            def fn():
                Y.nvfp4_tensor_scale(k, L.k_tensor_scale)
                Y.nvfp4_tensor_scale(v, L.v_tensor_scale)
                Y.kv_append_quantize(L, k, v, bt, pos)
            extra = read                      # the two amax passes read k and v again
        else:
            def fn():
                Y.kv_append_quantize(L, k, v, bt, pos)
            extra = 0
        ms = timed(fn)
        b = read + extra + written * N
        out[name] = {"ms": ms, "median_ms": timed.median, "bytes": b,
                     "GBs": b / (ms * 1e-3) / 1e9, "frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if kv == Y.KV_BF16:
            ms = timed(lambda: Y.rope_append(L, yp, None, k, v, bt, pos))
            b = read + written * N
            out["bf16_rope_append_fused"] = {"ms": ms, "median_ms": timed.median, "bytes": b,
                                             "GBs": b / (ms * 1e-3) / 1e9,
                                             "frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del L
        torch.cuda.empty_cache()
    kr = k.clone()
    ms = timed(lambda: Y.yarn_rope_apply(yp, kr, pos))
    b = 2 * w.hkv * 128 * N
    out["rope_keys"] = {"ms": ms, "median_ms": timed.median, "bytes": b,
                        "GBs": b / (ms * 1e-3) / 1e9, "frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    out["workload"] = ("one layer: 1,048,576 tokens x 4 KV heads x 256 (bf16 K and V in HBM), "
                       "paged over a seeded permutation of 65,536 pages")
    return out


def copy_bandwidth(torch, dev, gib=4, reps=10):
    """A plain device copy (torch) of gib GiB: read + write bytes over the
    median event time, the practical ceiling next to the 8 TB/s peak."""
    n = gib << 30
    src = torch.ones(n // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        ms.append((e0, e1))
    torch.cuda.synchronize()
    med = statistics.median(a.elapsed_time(b) for a, b in ms)
    del src, dst
    torch.cuda.empty_cache()
    gbs = 2 * n / (med * 1e-3) / 1e9
    return {"GBs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS, "bytes_read": n, "bytes_written": n,
            "median_ms": med, "kernel": "torch copy_ of a 4 GiB int32 tensor"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="only the headline workload (skip tiny, native, NVFP4, sessions)")
    ap.add_argument("--no-int8", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-append", action="store_true")
    ap.add_argument("--no-tp2", action="store_true",
                    help="skip one card's share of a two-way KV-head split (12 q / 2 KV heads)")
    ap.add_argument("--only", default="",
                    help="comma-separated sections to run for profiling (long, tiny, native, "
                         "long_fp4, sessions, prefill, int8, verify, append, tp2)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path shards by KV head or by sequence range; no multi-GPU run "
              "is built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W
    import yarn_rope_kv_amd as Y

    dev = "cuda:0"
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 3}), flush=True)
        return
    only = set(filter(None, args.only.split(",")))

    def want(section):
        return not only or section in only

    cpu = not args.no_cpu_baseline and not only
    sub_steps = max(10, args.steps // 2)
    result = {
        "metric": "decode-attn KV tokens/s + HBM GB/s at 1,048,576 ctx; prefill attn TFLOP/s",
        "value": None, "unit": "KV token-layers/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode step, 16 full-attention layers x 1,048,576 cached "
                               "tokens (bf16, 16-token pages, seeded page permutation, planted "
                               "needle), 24 q / 4 KV heads x 256, YaRN x4 from 262,144, batch 1",
                   "layers": 16, "context": 1048576, "batch": 1},
    }
    configs = {}
    w = W.WORKLOADS["long"]
    layers = None
    if want("long") or want("verify"):
        res, layers = bench_decode_config(
            W, Y, w, torch, dev, args.steps, args.warmup, KV_BYTES_PER_TOKEN_LAYER,
            result["config"]["workload"], record="decode_split_bf16_long_1m.json",
            cpu_seconds=10.0 if cpu else 0.0, keep_layers=True)
        configs["3_long_bf16"] = res
        result.update(value=res["value"], ms_per_step=res["ms_per_step"], kv_gbs=res["kv_gbs"])
        result["roofline"] = dict(res["roofline"],
                                  kernel="decode_attention (split + merge), per layer")
        if "cpu_baseline" in res:
            result["cpu_baseline"] = res["cpu_baseline"]
    if layers is not None and not args.no_verify and want("verify"):
        log("timing verify steps")
        result["verify"] = bench_verify(W, Y, w, layers, torch, dev, sub_steps, args.warmup,
                                        record="verify_split_bf16_long_q4_1m.json", cpu=cpu)
    del layers
    torch.cuda.empty_cache()
    if not args.no_configs:
        if want("tiny"):
            wt = W.WORKLOADS["tiny"]
            configs["1_tiny"], _ = bench_decode_config(
                W, Y, wt, torch, dev, 200, 20, KV_BYTES_PER_TOKEN_LAYER,
                "single decode step, 1 layer, 4,096 cached tokens (contiguous), query at 4,096, "
                "YaRN x4 from 1,024, fp32 output; latency-bound", cpu_seconds=1.0 if cpu else 0)
            c = configs["1_tiny"]
            c["latency_us"] = {"decode_median": c["decode_launch"]["median_ms"] * 1e3,
                               "step": c["ms_per_step"] * 1e3}
        if want("native"):
            configs["2_native"], _ = bench_decode_config(
                W, Y, W.WORKLOADS["native"], torch, dev, 50, 5, KV_BYTES_PER_TOKEN_LAYER,
                "one layer at native length: 262,144 cached bf16 tokens, paged over a seeded "
                "permutation, 4 outlier channels x8 per head", cpu_seconds=2.0 if cpu else 0)
        if want("long_fp4"):
            rec = profile_record("decode_split_nvfp4_long_fp4_1m.json")
            configs["4_long_nvfp4"], _ = bench_decode_config(
                W, Y, W.WORKLOADS["long_fp4"], torch, dev, sub_steps, args.warmup,
                NVFP4_BYTES_PER_TOKEN_LAYER,
                "decode step, 16 layers x 1,048,576 cached tokens, NVFP4 cache (1,152 B per "
                "token-layer), 1% x20 outliers, 24 q / 4 KV heads",
                record="decode_split_nvfp4_long_fp4_1m.json", cpu_seconds=3.0 if cpu else 0)
            if rec and "valu_busy_pct" in rec:
                configs["4_long_nvfp4"]["roofline"]["valu_busy_pct_counter"] = rec["valu_busy_pct"]
        if want("sessions"):
            configs["5_sessions_decode"], _ = bench_decode_config(
                W, Y, W.WORKLOADS["sessions"], torch, dev, 50, 5, KV_BYTES_PER_TOKEN_LAYER,
                "15 sessions x 131,072 cached bf16 tokens dealt from one shared pool of "
                "122,880 pages, one batched decode call", cpu_seconds=3.0 if cpu else 0)
    if not args.no_prefill and want("prefill"):
        log("prefill")
        configs["5_prefill"] = bench_prefill(W, Y, torch, dev, reps=10, cpu=cpu)
        result["prefill"] = configs["5_prefill"]
    result["configs"] = configs
    if not args.no_int8 and want("int8"):
        wi = W.WORKLOADS["long_int8"]
        res, li = bench_decode_config(
            W, Y, wi, torch, dev, sub_steps, args.warmup, INT8_BYTES_PER_TOKEN_LAYER,
            "decode step, 16 layers x 1,048,576 cached tokens, INT8 group-64 cache (2,112 B "
            "per token-layer), 24 q / 4 KV heads", record="decode_split_int8_long_int8_1m.json",
            cpu_seconds=3.0 if cpu else 0, keep_layers=True)
        result["int8_decode"] = res
        if not args.no_verify:
            log("timing INT8 verify steps")
            result["int8_verify"] = bench_verify(
                W, Y, wi, li, torch, dev, sub_steps, args.warmup,
                per_token=INT8_BYTES_PER_TOKEN_LAYER, fmt="INT8 group-64",
                record="verify_split_int8_long_int8_q4_1m.json", cpu=cpu)
        del li
        torch.cuda.empty_cache()
    if not args.no_append and want("append"):
        log("append and rope over one 1M-token layer")
        result["append"] = bench_append(W, Y, torch, dev)
        torch.cuda.empty_cache()
    if not args.no_tp2 and want("tp2"):
        # one card's share when the 4 KV heads are split over two cards: the
        # same kernels at 12 query / 2 KV heads (nothing is exchanged inside
        # attention, so this is the whole per-card decode and prefill work)
        wt = W.WORKLOADS["long_tp2"]
        res, _ = bench_decode_config(
            W, Y, wt, torch, dev, sub_steps, args.warmup, KV_BYTES_PER_TOKEN_LAYER * wt.hkv // 4,
            f"decode step, {wt.layers} layers x 1,048,576 cached tokens (bf16), "
            f"{wt.hq} q / {wt.hkv} KV heads", record="decode_split_bf16_tp2_share_1m.json",
            cpu_seconds=2.0 if cpu else 0)
        share = {"decode": res}
        if not args.no_prefill:
            share["prefill"] = bench_prefill(W, Y, torch, dev, reps=3, name="prefill_tp2")
        result["tp2_share"] = share
    if not only:
        log("copy bandwidth")
        result["copy_bandwidth"] = copy_bandwidth(torch, dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
