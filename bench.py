"""Benchmark of the decode hot path (and chunked prefill) on one MI355X.

A step is one decode step of the 16-layer, 1,048,576-token workload ("long"
in workloads.py): for every layer, rope the new query and the new key
(YaRN x4), append the new key/value to the paged bf16 cache, and run split-K
decode attention + merge over the 1,048,576 cached tokens.  All inputs are
resident in HBM before the timed region starts.

Prints one JSON line.  value = KV token-layers per second (16 x 1,048,576 per
step / step time).  roofline = the decode attention launches (split + merge),
timed with HIP events on the stream they run on, against 8 TB/s.
"""
from __future__ import annotations

import argparse
import json
import os
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


def measured_traffic(record):
    """HBM bytes per launch from a committed rocprofv3 counter record, or None
    when the kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", record)
    try:
        rec = json.load(open(path))
        sources = rec.get("kernel_sources") or [[rec["kernel_source"], rec["kernel_source_sha256"]]]
        for src, sha in sources:
            if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != sha:
                return None
    except (OSError, ValueError, KeyError):
        return None
    return 1024.0 * (rec["fetch_kib_per_call"] * rec["fetch_scale"] +
                     rec["write_kib_per_call"] * rec["write_scale"])


def decode_bytes_per_launch(n_ctx, per_token, hq=24):
    # KV stream + q and out (hq heads x 256 x 2 B each) + the page table (4 B / 16 tokens)
    return per_token * n_ctx + 2 * hq * 256 * 2 + 4 * (n_ctx // 16)


def build_step(W, Y, w, torch, dev):
    """The layers of a decode workload plus the per-step inputs."""
    layers = []
    for l in range(w.layers):
        layers.append(W.build_decode_layer(w, l, device=dev, spare_page=True))
        if l % 4 == 3:
            log(f"{w.name}: built layer {l + 1}/{w.layers}")
    N = w.n_ctx
    L = w.layers
    q_in = torch.empty((L, w.hq, 256), dtype=torch.bfloat16, device=dev)
    k_in = torch.empty((L, w.hkv, 256), dtype=torch.bfloat16, device=dev)
    v_in = torch.empty((L, w.hkv, 256), dtype=torch.bfloat16, device=dev)
    for l in range(L):
        q_in[l:l + 1] = W.gen_q(w, l, 1, dev, token0=1)
        W.gen_kv(w, l, 1, 1, k_in[l:l + 1], token0=N)
        W.gen_kv(w, l, 2, 1, v_in[l:l + 1], token0=N)
    q_work = torch.empty_like(q_in)
    outs, wss = zip(*[W.decode_outputs(w, dl, device=dev) for dl in layers])
    pos_new = torch.full((1,), N, dtype=torch.int32, device=dev)
    yp = w.yarn()
    ev = []

    def step(timing=False):
        q_work.copy_(q_in)                               # roped in place below
        for l, dl in enumerate(layers):
            # the new query and key roped at position N, key and value appended
            Y.rope_append(dl.layer, yp, q_work[l:l + 1], k_in[l:l + 1], v_in[l:l + 1],
                          dl.block_tables[0], pos_new)
            if timing:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            Y.decode_attention(dl.layer, q_work[l:l + 1], dl.block_tables, dl.seq_lens,
                               dl.max_seq_len, outs[l], wss[l])
            if timing:
                e1.record()
                ev.append((e0, e1))

    return step, ev, layers


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
                 per_token=KV_BYTES_PER_TOKEN_LAYER, fmt="bf16", record=None):
    """Verify steps at several query counts over the decode layers; the entry
    for main_nq (3 draft tokens) is the headline, the others are listed."""
    res = {}
    for nq in sweep:
        step, ev = build_verify_step(W, Y, w, layers, nq, torch, dev)
        wall, kms = time_steps(step, ev, steps, warmup, torch)
        ctx = w.n_ctx + nq
        bpl = decode_bytes_per_launch(ctx, per_token, w.hq * nq)
        res[nq] = {"value": w.layers * ctx / (wall / steps), "avg_launch_ms": kms,
                   "ms_per_step": wall / steps * 1e3, "bytes_per_launch": bpl,
                   "frac": bpl / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del step, ev
        torch.cuda.empty_cache()
    m = res[main_nq]
    return {
        "workload": f"speculative verify step, {w.layers} layers x 1,048,576 + {main_nq} cached "
                    f"tokens ({fmt}), {main_nq} causal queries x 24 q / 4 KV heads",
        "value": m["value"], "unit": "KV token-layers/s", "ms_per_step": m["ms_per_step"],
        "avg_launch_ms": m["avg_launch_ms"],
        "roofline": {"bound": "hbm", "achieved": m["bytes_per_launch"] / (m["avg_launch_ms"] * 1e-3)
                     / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": m["frac"],
                     "traffic": measured_traffic(record) if record else None,
                     "bytes_per_launch": m["bytes_per_launch"]},
        "by_queries": {str(nq): {"avg_launch_ms": r["avg_launch_ms"], "frac": r["frac"]}
                       for nq, r in res.items()},
    }


def time_steps(step, ev, steps, warmup, torch):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev.clear()
    t0 = time.perf_counter()
    for i in range(steps):
        step(timing=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    return wall, sum(kern_ms) / len(kern_ms)


def cpu_baseline(W, w, min_seconds=10.0):
    """The oracle timed on whole layers of the decode workload (all 1,048,576
    tokens, 24 query heads, the planted needle), one layer after another
    until at least min_seconds of oracle time; inputs are prepared outside
    the timed calls."""
    import numpy as np
    import oracle as O
    import synth

    N = w.n_ctx
    t = O.yarn_table(original_max_position=w.orig)
    total, done = 0.0, 0
    for u in range(w.layers):
        q = O.rope(synth.host_fill(w.seed, synth.stream_id(u, synth.Q), 0, 1, w.hq, 256), [N], t,
                   bf16_out=True)[0]
        k = O.rope(synth.host_fill(w.seed, synth.stream_id(u, synth.K), 0, N, w.hkv, 256),
                   np.arange(N), t, bf16_out=True)
        v = synth.host_fill(w.seed, synth.stream_id(u, synth.V), 0, N, w.hkv, 256)
        if w.needle:
            p_star = synth.needle_position(w.seed, u, N)
            for g in range(w.hkv):
                k[p_star, g] = O.round_bf16(2.0 * O.bf16_to_f64(q[w.group * g]))
        qf = O.bf16_to_f64(q)
        t0 = time.perf_counter()
        O.decode_attention(qf, k, v)
        total += time.perf_counter() - t0
        done += 1
        del k, v
        if total >= min_seconds:
            break
    cores = O.num_threads()
    return {"value": done * N / total, "unit": "KV token-layers/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{done} of {w.layers} layers of the long workload: {N} cached tokens x "
                      f"{w.hq} q heads each, fp64, {total:.2f} s"}


def bench_prefill(W, Y, torch, dev, reps, name="prefill"):
    w = W.WORKLOADS[name]
    case = W.build_prefill(w, device=dev)
    out = torch.empty_like(case.q)
    T = case.q.shape[0]
    for _ in range(2):
        Y.prefill_attention(case.layer, case.q, case.q_start, case.block_table, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        Y.prefill_attention(case.layer, case.q, case.q_start, case.block_table, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    pairs = sum(case.q_start + i + 1 for i in range(T))
    flops = 4.0 * 256 * pairs * w.hq
    tf = flops / (ms * 1e-3) / 1e12
    record = "prefill_chunk_8192_over_1m.json" if name == "prefill" else None
    return {"workload": f"prefill: 8,192-token causal chunk at 1,040,384..1,048,575 over a "
                        f"1,048,576-token paged cache, {w.hq} q / {w.hkv} KV heads",
            "ms_per_chunk": ms, "tflops": tf, "flop_per_chunk": flops,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS,
                         "traffic": measured_traffic(record) if record else None}}


def bench_append(W, Y, torch, dev, reps=3):
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
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

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
        out[name] = {"ms": ms, "bytes": b, "GBs": b / (ms * 1e-3) / 1e9,
                     "frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if kv == Y.KV_BF16:
            ms = timed(lambda: Y.rope_append(L, yp, None, k, v, bt, pos))
            b = read + written * N
            out["bf16_rope_append_fused"] = {"ms": ms, "bytes": b, "GBs": b / (ms * 1e-3) / 1e9,
                                             "frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del L
        torch.cuda.empty_cache()
    kr = k.clone()
    ms = timed(lambda: Y.yarn_rope_apply(yp, kr, pos))
    b = 2 * w.hkv * 128 * N
    out["rope_keys"] = {"ms": ms, "bytes": b, "GBs": b / (ms * 1e-3) / 1e9,
                        "frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    out["workload"] = ("one layer: 1,048,576 tokens x 4 KV heads x 256 (bf16 K and V in HBM), "
                       "paged over a seeded permutation of 65,536 pages")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-nvfp4", action="store_true")
    ap.add_argument("--no-int8", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-append", action="store_true")
    ap.add_argument("--no-tp2", action="store_true",
                    help="skip one card's share of a two-way KV-head split (12 q / 2 KV heads)")
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
    w = W.WORKLOADS["long"]
    log("building the 16-layer 1,048,576-token bf16 cache")
    step, ev, layers = build_step(W, Y, w, torch, dev)
    log("timing decode steps")
    wall, kern_ms = time_steps(step, ev, args.steps, args.warmup, torch)
    ms_step = wall / args.steps * 1e3
    tokens = w.layers * w.n_ctx
    value = tokens / (wall / args.steps)
    bpl = decode_bytes_per_launch(w.n_ctx, KV_BYTES_PER_TOKEN_LAYER)
    achieved = bpl / (kern_ms * 1e-3) / 1e9
    result = {
        "metric": "decode-attn KV tokens/s + HBM GB/s at 1,048,576 ctx; prefill attn TFLOP/s",
        "value": value, "unit": "KV token-layers/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode step, 16 full-attention layers x 1,048,576 cached "
                               "tokens (bf16, 16-token pages, seeded page permutation, planted "
                               "needle), 24 q / 4 KV heads x 256, YaRN x4 from 262,144, batch 1",
                   "layers": w.layers, "context": w.n_ctx, "batch": 1},
        "kv_gbs": tokens * KV_BYTES_PER_TOKEN_LAYER / (wall / args.steps) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("decode_split_bf16_long_1m.json"),
                     "kernel": "decode_attention (split + merge), per layer",
                     "bytes_per_launch": bpl, "avg_launch_ms": kern_ms},
    }
    del step, ev
    if not args.no_verify:
        log("timing verify steps")
        result["verify"] = bench_verify(W, Y, w, layers, torch, dev, max(3, args.steps // 2),
                                        args.warmup,
                                        record="verify_split_bf16_long_q4_1m.json")
    del layers
    torch.cuda.empty_cache()
    if not args.no_nvfp4:
        wf = W.WORKLOADS["long_fp4"]
        log("building the NVFP4 16-layer cache")
        stepf, evf, lf = build_step(W, Y, wf, torch, dev)
        wallf, kf = time_steps(stepf, evf, max(3, args.steps // 2), args.warmup, torch)
        bplf = decode_bytes_per_launch(wf.n_ctx, NVFP4_BYTES_PER_TOKEN_LAYER)
        result["nvfp4_decode"] = {
            "value": wf.layers * wf.n_ctx / (wallf / max(3, args.steps // 2)),
            "unit": "KV token-layers/s", "avg_launch_ms": kf,
            "roofline": {"bound": "hbm", "achieved": bplf / (kf * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bplf / (kf * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_split_nvfp4_long_fp4_1m.json"),
                         "bytes_per_launch": bplf}}
        del lf, stepf, evf
        torch.cuda.empty_cache()
    if not args.no_int8:
        wi = W.WORKLOADS["long_int8"]
        log("building the INT8 16-layer cache")
        stepi, evi, li = build_step(W, Y, wi, torch, dev)
        si = max(3, args.steps // 2)
        walli, ki = time_steps(stepi, evi, si, args.warmup, torch)
        bpli = decode_bytes_per_launch(wi.n_ctx, INT8_BYTES_PER_TOKEN_LAYER)
        result["int8_decode"] = {
            "workload": "decode step, 16 layers x 1,048,576 cached tokens, INT8 group-64 cache "
                        "(2,112 B per token-layer), 24 q / 4 KV heads",
            "value": wi.layers * wi.n_ctx / (walli / si),
            "unit": "KV token-layers/s", "avg_launch_ms": ki,
            "roofline": {"bound": "hbm", "achieved": bpli / (ki * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bpli / (ki * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_split_int8_long_int8_1m.json"),
                         "bytes_per_launch": bpli}}
        del stepi, evi
        if not args.no_verify:
            log("timing INT8 verify steps")
            result["int8_verify"] = bench_verify(
                W, Y, wi, li, torch, dev, si, args.warmup, per_token=INT8_BYTES_PER_TOKEN_LAYER,
                fmt="INT8 group-64", record="verify_split_int8_long_int8_q4_1m.json")
        del li
        torch.cuda.empty_cache()
    if not args.no_append:
        log("append and rope over one 1M-token layer")
        result["append"] = bench_append(W, Y, torch, dev)
        torch.cuda.empty_cache()
    if not args.no_prefill:
        log("prefill")
        try:
            result["prefill"] = bench_prefill(W, Y, torch, dev, reps=3)
        except Y.YrkError as e:
            result["prefill"] = {"error": str(e)}
        torch.cuda.empty_cache()
    if not args.no_tp2:
        # one card's share when the 4 KV heads are split over two cards: the
        # same kernels at 12 query / 2 KV heads (nothing is exchanged inside
        # attention, so this is the whole per-card decode and prefill work)
        wt = W.WORKLOADS["long_tp2"]
        log("building the 12 q / 2 KV-head share")
        stept, evt, lt = build_step(W, Y, wt, torch, dev)
        st = max(3, args.steps // 2)
        wallt, kt = time_steps(stept, evt, st, args.warmup, torch)
        bplt = decode_bytes_per_launch(wt.n_ctx, KV_BYTES_PER_TOKEN_LAYER * wt.hkv // 4, wt.hq)
        share = {"decode": {
            "workload": f"decode step, {wt.layers} layers x 1,048,576 cached tokens (bf16), "
                        f"{wt.hq} q / {wt.hkv} KV heads",
            "value": wt.layers * wt.n_ctx / (wallt / st), "unit": "KV token-layers/s",
            "avg_launch_ms": kt,
            "roofline": {"bound": "hbm", "achieved": bplt / (kt * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bplt / (kt * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_split_bf16_tp2_share_1m.json"),
                         "bytes_per_launch": bplt}}}
        del lt, stept, evt
        torch.cuda.empty_cache()
        if not args.no_prefill:
            share["prefill"] = bench_prefill(W, Y, torch, dev, reps=3, name="prefill_tp2")
            torch.cuda.empty_cache()
        result["tp2_share"] = share
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(W, w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
