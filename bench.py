#!/usr/bin/env python3
"""Benchmark of the CSA2 decode hot path on one MI355X.

One step = one pass of every layer of the workload's CSA2 group (quantize-on-
write, indexer scoring, Top-K, sparse attention; static Full / Reindex /
Reuse modes) for every sequence of the batch, through csa2_layer_step.  The
default workload is the four-layer group at 256K context (batch 4, Full ->
Reindex -> Reuse -> Reuse, Top-K 2048, 128-token FP8 window).  Inputs are
seeded synthetic tensors, resident in HBM before the timed region.  The
timed loop rotates over `--copies` identical cache sets so that successive
steps do not find their 75 MB index cache in the 256 MB last-level cache.

Prints one JSON line: decode queries/s (value), KV GB/s, the roofline of the
dominant kernel (indexer scoring; HIP events around each launch on its
stream, in a second, instrumented pass of the same steps) and the CPU oracle
timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix, published

METRIC = "CSA2 decode queries/s + FP4 KV GB/s vs HBM peak at 256K ctx"


def kv_bytes_per_query(w) -> dict:
    """Algorithmic KV bytes one query moves per layer: FP4 index rows
    streamed (72 B), FP4 main rows gathered (324 B), FP8 window rows (576 B)."""
    from sparse_attention_decode_e2m1_amd import inputs as I
    irow = w.DI // 2 + w.DI // 16
    mrow = w.D // 2 + w.D // 16
    per_layer = []
    scan = 0
    first_full_pool = False
    for m in w.modes:
        b = (0 if m == I.SWA else w.K * mrow) + w.W * w.D
        if m == I.FULL:
            b += w.N * irow
            scan += w.N * irow
            first_full_pool = w.P > 0
        elif m == I.REINDEX:
            n = w.P if first_full_pool else w.N
            b += n * irow
            scan += n * irow
        per_layer.append(b)
    # index-key bytes the scoring kernel streams per step (all queries)
    return {"per_layer": per_layer, "total": sum(per_layer), "index_scan_per_step": scan * w.B * w.T}


def cpu_baseline(w, budget_s: float) -> dict:
    """The oracle (as it stands) on one sequence of the workload, repeated
    for about `budget_s` seconds on all of this host's cores, then for about
    `budget_s` / 2 seconds on one core."""
    import oracle
    from oracle.group import SeqGroup
    oracle.lib()
    t_set = time.perf_counter()
    g = SeqGroup(w, 0)
    setup = time.perf_counter() - t_set

    def run(budget):
        n = 0
        t0 = time.perf_counter()
        while True:
            g.step()
            n += 1
            el = time.perf_counter() - t0
            if el >= budget or n >= 50:
                return n, el

    cores = oracle.num_threads()
    n, el = run(budget_s)
    oracle.set_num_threads(1)
    n1, el1 = run(budget_s / 2)
    oracle.set_num_threads(cores)
    return {"value": n / el, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "single_thread": {"value": n1 / el1, "unit": "queries/s", "cores": 1},
            "sample": f"sequence 0 of {w.B}, {n} full group steps ({len(w.modes)} layers) in "
                      f"{el:.1f} s on {cores} threads, {n1} in {el1:.1f} s on 1 thread "
                      f"(set-up {setup:.1f} s untimed)"}


def stream_read_peak(nbytes: int = 1 << 30, reps: int = 5) -> dict:
    """The library's plain streaming-read kernel over `nbytes` (beyond the
    256 MB last-level cache), HIP events around `reps` launches, for a few
    grid sizes; the best rate is the measured HBM read reference."""
    import torch
    from sparse_attention_decode_e2m1_amd import api
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    best, per = 0.0, {}
    for blocks in (1024, 2048, 4096, 8192):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        api.stream_read(src, sink, blocks)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            api.stream_read(src, sink, blocks)
        e1.record()
        torch.cuda.synchronize()
        gbps = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        per[str(blocks)] = round(gbps, 1)
        best = max(best, gbps)
    del src
    return {"GBps": round(best, 1), "bytes": nbytes, "by_blocks": per,
            "kernel": "stream_read_kernel (csa2_stream_read)"}


def stream_read_same_size(nbytes: int, reps: int = 40) -> dict:
    """The streaming-read kernel over `nbytes` per launch (the roofline
    kernel's bytes), launched back to back over buffers rotated through more
    than the 256 MB last-level cache, as the scan's launches run: the rate a
    read of that size reaches with its own start-up and tail included."""
    import torch
    from sparse_attention_decode_e2m1_amd import api
    words = max(4, (nbytes // 16) * 4)  # whole 16-byte words
    copies = max(2, -(-(768 << 20) // (words * 4)))
    bufs = [torch.ones(words, dtype=torch.int32, device="cuda") for _ in range(copies)]
    best_us, per = None, {}
    for blocks in (512, 1024, 2048, 4096):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        for i in range(copies):
            api.stream_read(bufs[i], sink, blocks)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            api.stream_read(bufs[i % copies], sink, blocks)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        per[str(blocks)] = round(us, 2)
        best_us = us if best_us is None else min(best_us, us)
    del bufs
    return {"us": round(best_us, 2), "GBps": round(words * 4 / best_us / 1e3, 1), "bytes": words * 4,
            "us_by_blocks": per}


def hierarchical_recall(w, dw) -> list:
    """For a workload whose Full layer keeps a pool: recall of each later
    indexing layer's Top-K (searched inside the pool) against the same layer
    searching the whole context (the workload with no pool), per layer, mean
    over query rows."""
    import dataclasses

    import torch
    from sparse_attention_decode_e2m1_amd import harness
    from sparse_attention_decode_e2m1_amd import inputs as I
    flat = harness.DeviceWorkload(dataclasses.replace(w, P=0), copies=1)
    flat.step()
    dw.step(copy=0)
    torch.cuda.synchronize()
    out = []
    for li, m in enumerate(w.modes):
        if m != I.REINDEX:
            continue
        h = dw.layers[li].idx_out.cpu().numpy()
        f = flat.layers[li].idx_out.cpu().numpy()
        rec = [len(set(h[r][h[r] >= 0]) & set(f[r][f[r] >= 0])) / max(1, int((f[r] >= 0).sum()))
               for r in range(h.shape[0])]
        out.append({"layer": li, "recall": round(float(sum(rec) / len(rec)), 4)})
    del flat
    return out


def time_rope_quantize(rows: int, reps: int = 50) -> dict:
    """Fused rotary + quantize-on-write of `rows` bf16 rows of 576 channels
    (last 64 rotary) against the plain quantize-on-write, HIP events around
    `reps` launches of each; rows scattered into a 4x larger cache."""
    import torch
    from sparse_attention_decode_e2m1_amd import api
    from sparse_attention_decode_e2m1_amd import inputs as I
    g = torch.Generator().manual_seed(7)
    x = torch.randn(rows, 576, generator=g).to(torch.bfloat16).cuda()
    cs = I.rope_cos_sin(torch.randint(0, 1 << 20, (rows,), generator=g), 64).cuda()
    dst = torch.randperm(4 * rows, generator=g)[:rows].cuda()
    codes = torch.zeros((4 * rows, 288), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((4 * rows, 36), dtype=torch.uint8, device="cuda")
    res = {}
    for name, fn in (("rope_quantize", lambda: api.rope_quantize_kv(x, 64, cs, codes, scales, dst)),
                     ("quantize", lambda: api.quantize_kv(x, codes, scales, dst))):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = rows * (576 * 2 + 324 + 8) + (rows * 32 * 8 if name == "rope_quantize" else 0)
        res[name] = {"us_per_launch": round(us, 2), "GBps": round(nbytes / us / 1e3, 1)}
    return {"rope_quantize_rows": rows, "channels": 576, "rotary_channels": 64, "input": "bf16",
            **res}


def time_attn_fp4_vs_fp8(B: int, N: int, K: int, W: int, copies: int, reps: int = 64) -> dict:
    """Sparse attention of B decode queries (16 heads, 576 channels, Top-K K
    plus a W-token FP8 window) over an FP4 main cache (E2M1 + E4M3 per 16
    channels, 324 B a row) and over an FP8 one (E4M3 + fp32 per row, 580 B a
    row) holding the same quantized rows' source values.  HIP events around
    `reps` launches of each; every launch takes the next of `copies` cache
    sets and its own random Top-K rows, so that rows are gathered from HBM
    rather than found in the last-level cache."""
    import torch
    from sparse_attention_decode_e2m1_amd import api
    from sparse_attention_decode_e2m1_amd import inputs as I
    g = torch.Generator().manual_seed(11)
    gd = torch.Generator(device="cuda").manual_seed(11)
    D, S = 576, 128
    c4 = torch.empty((B, N, D // 2), dtype=torch.uint8, device="cuda")
    s4 = torch.empty((B, N, D // 16), dtype=torch.uint8, device="cuda")
    c8 = torch.empty((B, N, D), dtype=torch.uint8, device="cuda")
    s8 = torch.empty((B, N), dtype=torch.float32, device="cuda")
    for b in range(B):
        x = torch.randn((N, D), generator=gd, device="cuda").to(torch.bfloat16)
        api.quantize_kv(x, c4[b], s4[b])
        api.quantize_kv_fp8(x, c8[b], s8[b])
        del x
    sets4 = [(c4, s4)] + [(c4.clone(), s4.clone()) for _ in range(copies - 1)]
    sets8 = [(c8, s8)] + [(c8.clone(), s8.clone()) for _ in range(copies - 1)]
    swa_b, swa_s = I.fp8_rows(torch.randn((B * S, D), generator=g))
    swa = swa_b.reshape(B, S, D).cuda()
    swa_scale = torch.full((B,), float(swa_s), dtype=torch.float32, device="cuda")
    pos0 = torch.full((B,), N - S, dtype=torch.int32, device="cuda")
    q_pos = torch.full((B,), N - 1, dtype=torch.int32, device="cuda")
    q = torch.randn((B, 16, D), generator=g).to(torch.bfloat16).cuda()
    idx = [torch.stack([torch.sort(torch.randperm(N, generator=g)[:K])[0] for _ in range(B)])
           .to(torch.int32).cuda() for _ in range(copies)]
    out = torch.empty((B, 16, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, 16), dtype=torch.float32, device="cuda")
    ws = api.workspace(api.sparse_attn_workspace_bytes(B, K, W, 512))
    sm = 1.0 / D ** 0.5
    cache4 = [api.cache(c, s, D, N) for c, s in sets4]
    cache8 = [api.fp8_cache(c, s, D, N) for c, s in sets8]
    run = {
        "fp4": lambda i: api.sparse_attn(q, B, 1, cache4[i % copies], idx[i % copies], K, swa,
                                         swa_scale, pos0, S, W, q_pos, sm, 512, out, lse, ws),
        "fp8": lambda i: api.sparse_attn_fp8(q, B, 1, cache8[i % copies], idx[i % copies], K, swa,
                                             swa_scale, pos0, S, W, q_pos, sm, 512, out, lse, ws),
    }
    row_bytes = {"fp4": D // 2 + D // 16, "fp8": D + 4}
    res = {}
    for name, fn in run.items():
        for i in range(8):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        per_q = K * row_bytes[name] + W * D
        res[name] = {"us_per_launch": round(us, 2), "kv_bytes_per_query": per_q,
                     "GBps": round(B * per_q / us / 1e3, 1)}
    res["fp8_over_fp4_time"] = round(res["fp8"]["us_per_launch"] / res["fp4"]["us_per_launch"], 3)
    return {"attn_kv_compare": {"B": B, "N": N, "K": K, "W": W, "heads": 16, "channels": D,
                                "copies": copies, "launches": reps}, **res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C3_group_b4_256k")
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true",
                    help="skip the instrumented passes (roofline, per-layer, warm, stream peak)")
    ap.add_argument("--rope-quantize-rows", type=int, default=0,
                    help="only time the fused rotary + quantize-on-write of this many bf16 rows "
                         "(576 channels, 64 rotary) against the plain quantize-on-write, and exit")
    ap.add_argument("--reuse-one-launch", action="store_true",
                    help="run the Reuse (and window-only) layers through the one-launch "
                         "attention (split and merge in one kernel) instead of split + merge")
    ap.add_argument("--attn-kv-compare", action="store_true",
                    help="only time the sparse attention of the workload's decode queries over "
                         "an FP4 and an FP8 main cache (same Top-K, window), and exit")
    ap.add_argument("--attn-batch", type=int, default=0,
                    help="with --attn-kv-compare: decode queries per launch (default: the "
                         "workload's batch)")
    ap.add_argument("--copy-kernel-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes 5 times (the "
                         "reference kernel that calibrates the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; the path shards by sequence or by "
              "context across GPUs only in design (no multi-GPU run)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_decode_e2m1_amd import api, harness, profiling
    from sparse_attention_decode_e2m1_amd import inputs as I

    if args.copy_kernel_bytes:
        n = args.copy_kernel_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)  # one elementwise pass: reads n*4, writes n*4 bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "passes": 5}), flush=True)
        return

    if args.rope_quantize_rows:
        print(json.dumps(time_rope_quantize(args.rope_quantize_rows)), flush=True)
        return

    w = I.WORKLOADS[args.workload]
    if args.attn_kv_compare:
        api.lib()
        print(json.dumps(time_attn_fp4_vs_fp8(args.attn_batch or w.B, w.N, w.K, w.W,
                                              max(args.copies, 8))),
              flush=True)
        return
    api.lib()  # fails loudly if the HIP library is missing
    print(f"[bench] workload {w.name}: B={w.B} N={w.N} T={w.T} K={w.K} modes={w.modes}; "
          f"set-up with {args.copies} cache copies", file=sys.stderr, flush=True)
    t_set = time.perf_counter()
    dw = harness.DeviceWorkload(w, copies=args.copies, reuse_one_launch=args.reuse_one_launch)
    print(f"[bench] set-up {time.perf_counter() - t_set:.1f} s", file=sys.stderr, flush=True)

    for i in range(args.warmup):
        dw.step(copy=i % args.copies)
    torch.cuda.synchronize()
    print("[bench] warm-up done", file=sys.stderr, flush=True)

    # ---- timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        dw.step(copy=k % args.copies)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = t1 - t0
    ms_per_step = sec * 1e3 / args.steps
    queries = w.B * w.T * args.steps
    value = queries / sec
    kvb = kv_bytes_per_query(w)
    kv_gbps = kvb["total"] * w.B * w.T * args.steps / sec / 1e9
    print(f"[bench] {ms_per_step * 1e3:.1f} us/step, {value:.0f} queries/s, {kv_gbps:.0f} GB/s",
          file=sys.stderr, flush=True)

    # ---- warm steps (one cache copy, so the index cache stays in the
    # last-level cache between steps), and per-layer time (events on the
    # launch stream between the layers of each step)
    warm_ms = None
    layer_us = None
    if not args.no_profile:
        for _ in range(3):
            dw.step(copy=0)
        torch.cuda.synchronize()
        t4 = time.perf_counter()
        for _ in range(args.steps):
            dw.step(copy=0)
        torch.cuda.synchronize()
        warm_ms = (time.perf_counter() - t4) * 1e3 / args.steps
        nl = len(dw.layers)
        acc = [0.0] * nl
        for k in range(args.steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)]
            ev[0].record()
            for li in range(nl):
                dw.run_layer(li, copy=k % args.copies)
                ev[li + 1].record()
            torch.cuda.synchronize()
            for li in range(nl):
                acc[li] += ev[li].elapsed_time(ev[li + 1])
        layer_us = [{"layer": li, "mode": I.MODE_NAMES[w.modes[li]],
                     "us": round(acc[li] * 1e3 / args.steps, 2)} for li in range(nl)]

    # ---- instrumented pass: HIP events around every launch, same steps
    roofline = None
    prof = None
    if not args.no_profile:
        api.profile_begin()
        t2 = time.perf_counter()
        for k in range(args.steps):
            dw.step(copy=k % args.copies)
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        prof = api.profile_end()
        n_sc, ms_sc = prof["index_score"]
        if w.T == 1 and n_sc:
            # algorithmic index-key bytes of every profiled scoring launch over
            # their summed duration
            scan_bytes = kvb["index_scan_per_step"] * args.steps
            achieved = scan_bytes / (ms_sc * 1e-3) / 1e9
            traffic = profiling.read_traffic(
                os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                             f"index_score_kernel.{w.name}.traffic.txt"), "index_score_kernel")
            roofline = {"bound": "hbm", "kernel": "index_score_kernel", "achieved": round(achieved, 1),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBPS, 4),
                        "traffic": None if traffic is None else round(traffic),
                        "avg_launch_us": round(ms_sc * 1e3 / n_sc, 2), "launches": n_sc,
                        "bytes_per_launch": scan_bytes // n_sc}
        prof = {k: {"launches": c, "avg_us": round(t * 1e3 / c, 2) if c else 0.0}
                for k, (c, t) in prof.items()}
        prof["instrumented_ms_per_step"] = round((t3 - t2) * 1e3 / args.steps, 4)

    stream = None
    recall = None
    if not args.no_profile:
        stream = stream_read_peak()
        if roofline is not None:
            roofline["measured_read_peak_GBps"] = stream["GBps"]
            roofline["frac_of_measured_peak"] = round(roofline["achieved"] / stream["GBps"], 4)
            same = stream_read_same_size(roofline["bytes_per_launch"])
            roofline["same_size_read"] = same
            roofline["frac_of_same_size_read"] = round(roofline["achieved"] / same["GBps"], 4)
        if w.P > 0 and w.T == 1:
            recall = hierarchical_recall(w, dw)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_budget)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "context": w.N, "query_tokens": w.T,
                   "layers": [I.MODE_NAMES[m] for m in w.modes], "top_k": w.K,
                   "pool": w.P, "window": w.W, "heads": w.H, "latent": w.D, "index_heads": w.HI,
                   "index_dim": w.DI, "kv_bytes_per_query": kvb["total"],
                   "kv_GBps": round(kv_gbps, 1), "kv_frac_of_hbm_peak": round(kv_gbps / HBM_PEAK_GBPS, 4),
                   "cache_copies": args.copies,
                   "reuse_attention": "one launch" if args.reuse_one_launch else "split + merge",
                   "storage": "fp4 e2m1 + e4m3/16 (kv, index), fp8 e4m3 window",
                   "compute": "fp16 MFMA operands, fp32 accumulation"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": prof,
        "per_layer_us": layer_us,
        "warm_ms_per_step": None if warm_ms is None else round(warm_ms, 4),
        "stream_read_peak": stream,
        "hierarchical_recall_vs_flat": recall,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
