"""Benchmark of the INT8-KV hot path on one MI355X.

Default workload (decode_8b): one step = for every layer of the 8B-shaped
decode workload (batch 16, 32 query / 8 KV heads, head_dim 128, per-token fp32
scales, 4 outlier channels x10 per KV head, 32 layers each with its own cache):
quantize-append the new token at position 4095 and run decode attention over
4096 tokens (kvq_append_decode, one launch per layer).  The 32 caches (4.44 GB)
are visited in order, as a model does, so no K/V byte is re-read from the
256 MB Infinity Cache within a step.

``--workload chunked_prefill``: one step = quantize-append 512 new tokens
after 8192 cached ones (batch 4, 32/8 heads, head_dim 128) and run causal
chunked-prefill attention for the 512 queries (kvq_attention_chunk); the
figure is TFLOP/s over the visible keys only.

The other workloads (recent_window, sliding_decode, sliding_chunk,
bf16_scales, fp8_e4m3, fp8_chunk, chunk_group32, recent_chunk, q8_group32,
paged_decode, tiny_decode, recent_block_head, recent_block_channel,
chunk_d256, decode_d256) are the same steps on the cache variants their names give;
stream_read times a plain read of the decode step's bytes; ``--help`` lists
them.

Inputs are seeded synthetic data, already resident in HBM when timing starts.
Prints one JSON line (see --help).  ``--gpus N`` with N > 1 is refused: this
path is measured on one GPU.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, AMD published peak


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    summarised in profiles/ (one record per workload), or None when none was
    taken for this kernel on this workload or its sources have changed since."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))[workload]
        if rec["kernel"] != kernel:
            return None
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def step_bytes(w: wl.Workload, L: int) -> dict:
    """Algorithmic bytes of one layer-step (each byte the step must move once)."""
    B, H, KVH, D = w.batch, w.num_heads, w.num_kv_heads, w.head_dim
    # scales per row (per-channel block scales: D per 16 rows)
    G = D // 16 if w.extra.get("block") == "channel" else (1 if w.group == 0 else D // 32)
    in_bytes = 4 if w.kv_dtype == "f32" else 2
    sb = 2 if w.extra.get("scale_bf16") else (0 if w.extra.get("fp8") else 4)   # bytes per scale (FP8: none)
    W = w.extra.get("window", 0)
    if W:
        # recent window: INT8 rows below L - W (the row leaving the window is
        # written once, as codes and scale), W + 1 bf16 ring rows (the W - 1
        # attended ones, the one read for eviction, the new one written), the
        # new input row, queries and outputs
        int8 = 2 * B * KVH * (L - W) * (D + 4 * G)
        ring = 2 * B * KVH * (W + 1) * D * 2
        qo = 2 * B * H * D * 2
        app_in = 2 * B * KVH * D * in_bytes
        return {"decode": int8 + ring + qo, "append": app_in, "step": int8 + ring + qo + app_in}
    codes = 2 * B * KVH * L * D
    scales = 2 * B * KVH * L * G * sb
    q = B * H * D * 2
    out = B * H * D * 2
    app_in = 2 * B * KVH * D * in_bytes
    app_codes = 2 * B * KVH * D
    app_scales = 2 * B * KVH * G * sb
    decode = codes + scales + q + out
    return {"decode": decode, "append": app_in + app_codes + app_scales,
            "step": decode + app_in + app_codes + app_scales}


def chunk_counts(w: wl.Workload) -> dict:
    """Chunked-prefill step: MFMA flops over visible keys (QK and PV, 2 flops
    per multiply-add each) and algorithmic bytes."""
    B, H, KVH, D, n, L0 = w.batch, w.num_heads, w.num_kv_heads, w.head_dim, w.n_new, w.ctx
    win = w.extra.get("sliding", 0)
    if win:   # query i sees min(window, L0 + i + 1) keys
        visible = sum(min(win, L0 + i + 1) for i in range(n))
    else:
        visible = n * (L0 + 1) + n * (n - 1) // 2      # sum over i < n of L0 + i + 1
    flops = 4 * B * H * D * visible
    L = L0 + n
    rows = L - max(0, L0 - win + 1) if win else L    # keys some query of the chunk sees
    G = D // 32 if w.group == 32 else 1
    scale_b = 0 if w.extra.get("fp8") else 4 * G
    qo = 2 * B * H * n * D * 2
    rw = w.extra.get("window", 0)
    if rw:
        # hybrid cache: INT8 rows below L - W, bf16 ring rows above
        kv = 2 * B * KVH * ((L - rw) * (D + scale_b) + rw * D * 2)
        # append: the input rows; the n rows leaving the window quantized
        # (ring rows read, codes and scales written); the last W stored in the ring
        append = 2 * B * KVH * (n * D * 2 + min(n, rw) * D * 2 + n * (D + scale_b) + rw * D * 2)
        return {"flops": flops, "chunk_bytes": kv + qo, "step_bytes": kv + qo + append}
    kv = 2 * B * KVH * rows * (D + scale_b)
    append = 2 * B * KVH * n * (D * 2 + D + scale_b)
    return {"flops": flops, "chunk_bytes": kv + qo, "step_bytes": kv + qo + append}


# ----------------------------------------------------------------------------
# GPU setup
# ----------------------------------------------------------------------------

def build_layers(w: wl.Workload, kvq, torch, stream, threads: int):
    """Allocate and prefill every layer's cache through kvq_append."""
    T = w.ctx + w.n_new
    dev = torch.device("cuda")
    layers = []

    def gen(layer):
        return wl.layer_inputs(w, layer)

    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = {ex.submit(gen, l): l for l in range(min(w.layers, threads))}
        nxt = len(futs)
        done_layers = {}
        while futs:
            fut = next(cf.as_completed(futs))
            l = futs.pop(fut)
            done_layers[l] = fut.result()
            if nxt < w.layers:
                futs[ex.submit(gen, nxt)] = nxt
                nxt += 1
            while len(layers) in done_layers:
                li = len(layers)
                x = done_layers.pop(li)
                cache = kvq.Int8KVCache(w.batch, w.num_heads, w.num_kv_heads, w.head_dim, max_len=w.max_len,
                                        group32=(w.group == 32), recent_window=w.extra.get("window", 0),
                                        scale_bf16=w.extra.get("scale_bf16", False), fp8=w.extra.get("fp8"),
                                        block_scales=w.extra.get("block"))
                k_raw, v_raw = x["k_raw"], x["v_raw"]
                tdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32

                def up(a):
                    t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a))
                    return t.to(dev, non_blocking=False).view(tdt)

                with torch.cuda.stream(stream):
                    chunk = 1024
                    for p0 in range(0, w.ctx, chunk):
                        n = min(chunk, w.ctx - p0)
                        cache.append(up(k_raw[:, :, p0:p0 + n]), up(v_raw[:, :, p0:p0 + n]),
                                     torch.full((w.batch,), p0, dtype=torch.int32, device=dev), stream=stream)
                    k_new = up(k_raw[:, :, w.ctx:T])
                    v_new = up(v_raw[:, :, w.ctx:T])
                    q = torch.from_numpy(x["q_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
                stream.synchronize()
                layers.append({"cache": cache, "k_new": k_new, "v_new": v_new, "q": q,
                               "out": torch.empty_like(q)})
                if len(layers) % 8 == 0 or len(layers) == w.layers:
                    log(f"prefilled {len(layers)}/{w.layers} layers ({time.time() - t0:.1f}s)")
    return layers


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ----------------------------------------------------------------------------

def blas_thread_count() -> int:
    """Threads numpy's BLAS may use (the oracle's matrix products); its
    elementwise work is single-threaded."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return 1


def cpu_baseline_recent(w: wl.Workload, target_s: float = 12.0):
    """The oracle's hybrid cache on whole sequences of layer 0: append the new
    token (the row leaving the window is quantized) and attend over the
    get_kv view, per sequence."""
    import copy
    import oracle as orc
    blas_threads = blas_thread_count()
    T = w.ctx + w.n_new
    W = w.extra["window"]
    x = wl.layer_inputs(w, 0)
    base = []
    for b in range(w.batch):
        if w.extra.get("block"):
            c = orc.BlockRecentCache(w.num_kv_heads, w.head_dim, W, w.extra["block"])
        else:
            c = orc.RecentWindowCache(w.num_kv_heads, w.head_dim, W, w.group)
        c.append(x["k"][b, :, :w.ctx], x["v"][b, :, :w.ctx])
        base.append(c)

    def one_seq(b):
        c = copy.deepcopy(base[b])
        c.append(x["k"][b, :, w.ctx:T], x["v"][b, :, w.ctx:T])
        return orc.attention_decode_recent(x["q"][b:b + 1], [c], w.attn_scale)

    per_seq_bytes = step_bytes(w, T)["step"] / w.batch
    done = 0
    t0 = time.perf_counter()
    while True:
        one_seq(done % w.batch)
        done += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    rate = per_seq_bytes * done / el / 1e12
    return {"value": rate, "unit": "TB/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{done} sequences of layer 0 ({done / w.batch:.2f} layer-steps: append 1 token to the "
                      f"hybrid cache (window {W}) + fp64 attention over {T} tokens, {w.num_heads} heads), {el:.1f}s wall; "
                      f"BLAS threads {blas_threads}; host {platform.processor() or 'x86_64'} nproc {os.cpu_count()}",
            "seconds": el}


def cpu_baseline(w: wl.Workload, target_s: float = 12.0):
    import oracle as orc
    blas_threads = blas_thread_count()
    T = w.ctx + w.n_new
    # one sequence's worth of the step per call: quantize the new K/V rows,
    # then fp64 attention over the dequantized cache for all its heads
    x = wl.layer_inputs(w, 0)
    nb = w.batch

    fp8 = w.extra.get("fp8")

    def quant(a):  # per-token / group-32, per-token with the scale kept as bf16, or FP8 codes
        if fp8:
            return orc.fp8_encode(a, fp8), np.zeros(a.shape[:-1] + (1,), np.float32)
        if w.extra.get("scale_bf16"):
            c, sb = orc.quantize_bf16_scale(a)
            return c, orc.bf16_bits_to_f32(sb)
        return orc.quantize(a, w.group)

    def deq(c, s):
        return orc.fp8_decode(c, fp8) if fp8 else orc.dequantize_exact(c, s)

    caches = []
    for b in range(nb):
        kc, ks = quant(x["k"][b:b + 1, :, :w.ctx])
        vc, vs = quant(x["v"][b:b + 1, :, :w.ctx])
        caches.append((kc, ks, vc, vs))

    def one_seq(b):
        kc, ks, vc, vs = caches[b]
        nk, nks = quant(x["k"][b:b + 1, :, w.ctx:T])
        nv, nvs = quant(x["v"][b:b + 1, :, w.ctx:T])
        kcat = np.concatenate([kc, nk], axis=2)
        kscat = np.concatenate([ks, nks], axis=2)
        vcat = np.concatenate([vc, nv], axis=2)
        vscat = np.concatenate([vs, nvs], axis=2)
        return orc.attention_decode(x["q"][b:b + 1], deq(kcat, kscat), deq(vcat, vscat), [T], w.attn_scale)

    per_seq_bytes = step_bytes(w, T)["step"] / w.batch
    done = 0
    t0 = time.perf_counter()
    while True:
        one_seq(done % nb)
        done += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    rate = per_seq_bytes * done / el / 1e12
    return {"value": rate, "unit": "TB/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{done} sequences of layer 0 ({done / w.batch:.2f} layer-steps: quantize 1 new token "
                      f"+ fp64 attention over {T} tokens, {w.num_heads} heads), {el:.1f}s wall; numpy elementwise "
                      f"single-threaded, BLAS threads {blas_threads}; host {platform.processor() or 'x86_64'} "
                      f"nproc {os.cpu_count()}",
            "seconds": el}


def cpu_baseline_chunk(w: wl.Workload, x: dict, target_s: float = 12.0):
    """The oracle on whole query rows of the chunk step: quantize the cache of
    one (sequence, KV head), then fp64 attention for sampled query rows."""
    import oracle as orc
    blas_threads = blas_thread_count()
    hpg = w.num_heads // w.num_kv_heads
    rng = np.random.default_rng(7)
    flops = 0
    rows = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < target_s:
        b = int(rng.integers(w.batch))
        g = int(rng.integers(w.num_kv_heads))
        fp8 = w.extra.get("fp8")
        if fp8:
            kh = orc.fp8_decode(orc.fp8_encode(x["k"][b, g], fp8), fp8)
            vh = orc.fp8_decode(orc.fp8_encode(x["v"][b, g], fp8), fp8)
        elif w.extra.get("window"):  # the hybrid cache's get_kv view
            rc = orc.RecentWindowCache(1, w.head_dim, w.extra["window"], w.group)
            rc.append(x["k"][b, g:g + 1], x["v"][b, g:g + 1])
            kh, vh = (a[0] for a in rc.kv())
        else:
            kc, ks = orc.quantize(x["k"][b, g], w.group)
            vc, vs = orc.quantize(x["v"][b, g], w.group)
            kh, vh = orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs)
        for _ in range(64):
            h = g * hpg + int(rng.integers(hpg))
            i = int(rng.integers(w.n_new))
            total = w.ctx + i + 1
            first = max(0, total - w.extra.get("sliding", 0)) if w.extra.get("sliding") else 0
            orc.softmax_attend(x["q"][b, h, i].astype(np.float64), kh[first:total], vh[first:total],
                               w.attn_scale, None)
            flops += 4 * w.head_dim * (total - first)
            rows += 1
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{rows} query rows (random sequence, head, position) of the chunk step, each fp64 "
                      f"attention over its visible keys, plus the oracle quantization of the K/V of their "
                      f"(sequence, KV head); {el:.1f}s wall; numpy, BLAS threads {blas_threads}; host "
                      f"{platform.processor() or 'x86_64'} nproc {os.cpu_count()}"}


def with_one_thread(baseline, *args, target_s: float = 6.0):
    """The same oracle sample with numpy's BLAS held to one thread: the
    single-thread figure beside the all-cores one."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        r = baseline(*args, target_s=target_s)
    return {"value": r["value"], "unit": r["unit"], "cores": 1, "seconds": round(r.get("seconds", target_s), 1)}


def time_calls(fn, reps: int, stream, torch) -> float:
    """Average milliseconds of fn() over reps calls, HIP events on `stream`."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    stream.synchronize()
    return e0.elapsed_time(e1) / reps


def run_chunk(args, w: wl.Workload, kvq, torch, stream):
    win = w.extra.get("sliding", 0)
    x = wl.layer_inputs(w, 0)
    B, KVH, T, D = x["k"].shape
    dev = torch.device("cuda")
    fp8 = w.extra.get("fp8")
    rw = w.extra.get("window", 0)
    cache = kvq.Int8KVCache(B, w.num_heads, KVH, D, max_len=w.max_len, fp8=fp8, group32=(w.group == 32),
                            recent_window=rw)

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a))
        return t.to(dev).view(torch.bfloat16 if a.dtype == np.uint16 else torch.float32)

    with torch.cuda.stream(stream):
        for p0 in range(0, w.ctx, 1024):
            n = min(1024, w.ctx - p0)
            cache.append(up(x["k_raw"][:, :, p0:p0 + n]), up(x["v_raw"][:, :, p0:p0 + n]),
                         torch.full((B,), p0, dtype=torch.int32, device=dev), stream=stream)
        k_new = up(x["k_raw"][:, :, w.ctx:])
        v_new = up(x["v_raw"][:, :, w.ctx:])
        q = up(x["q_bits"])
        out = torch.empty_like(q)
        ctx = torch.full((B,), w.ctx, dtype=torch.int32, device=dev)
        ws = cache.workspace(T, w.n_new)
    stream.synchronize()
    log(f"prefilled {w.ctx} tokens")

    def step():  # quantize-append the chunk's rows, then attention for its queries
        cache.append(k_new, v_new, ctx, stream=stream)
        cache.chunk(q, ctx, True, w.attn_scale, w.ctx, out=out, workspace=ws, stream=stream, window=win)

    def kernel_pass():
        cache.chunk(q, ctx, True, w.attn_scale, w.ctx, out=out, workspace=ws, stream=stream, window=win)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        stream.synchronize()
        torch.cuda.synchronize()
        log(f"warmup {args.warmup} steps done; timing {args.steps} steps")
        t0 = time.perf_counter()
        step_ms = time_calls(step, args.steps, stream, torch)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        k_ms = time_calls(kernel_pass, args.kernel_reps, stream, torch)
    cnt = chunk_counts(w)
    kname = "kvq_attention_chunk_window" if win else ("kvq_attention_chunk_recent" if rw else "kvq_attention_chunk")
    tflops = cnt["flops"] / (step_ms * 1e-3) / 1e12
    k_tflops = cnt["flops"] / (k_ms * 1e-3) / 1e12
    log(f"step {step_ms * 1e3:.1f} us ({tflops:.1f} TFLOP/s), wall {wall * 1e3 / args.steps:.3f} ms/step; "
        f"{kname} {k_ms * 1e3:.1f} us = {k_tflops:.1f} TFLOP/s "
        f"({k_tflops / MFMA_F16_PEAK_TFLOPS * 100:.1f}% of {MFMA_F16_PEAK_TFLOPS:.0f})")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline_chunk(w, x)
        cpu["single_thread"] = with_one_thread(cpu_baseline_chunk, w, x)
    codes_what = (f"FP8 {fp8.upper()} codes" if fp8 else
                  "group-32 fp32 scales" if w.group == 32 else "per-token fp32 scales")
    if rw:
        codes_what += f", last {rw} tokens bf16 (recent window)"
    result = {
        "metric": ("FP8" if fp8 else "INT8") + "-KV chunked-prefill attention: MFMA TFLOP/s over visible keys"
                  + (" (sliding window)" if win else "") + (" (recent window)" if rw else ""),
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: batch {B}, {w.num_heads} q / {KVH} kv heads, head_dim {D}, "
                               f"{w.ctx} cached + {w.n_new} new tokens, causal"
                               + (f", sliding window {win}" if win else "") + f", {codes_what}; "
                               f"append the {w.n_new} rows + chunk attention",
                   "batch": B, "seq_len": T, "flops_per_step": cnt["flops"], "bytes_per_step": cnt["step_bytes"]},
        "roofline": {"bound": "mfma", "kernel": kname,
                     "achieved": round(k_tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(k_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(kname, w.name),
                     "flops_per_launch": cnt["flops"], "bytes_per_launch": cnt["chunk_bytes"],
                     "us_per_launch": round(k_ms * 1e3, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def paged_bytes(w: wl.Workload, lens) -> dict:
    """Algorithmic bytes of one paged step: every cached code and scale once,
    queries, outputs, and the appended rows (input, codes, scales)."""
    H, KVH, D = w.num_heads, w.num_kv_heads, w.head_dim
    total = int(np.sum(lens))
    B = len(lens)
    decode = 2 * total * KVH * (D + 4) + 2 * B * H * D * 2 + w.max_blocks_read * 4
    append = 2 * B * KVH * (D * 2 + D + 4)
    return {"decode": decode, "step": decode + append}


def run_paged(args, w: wl.Workload, kvq, torch, stream):
    """Paged decode: 64 sequences with lengths U[512, 32768] over a shared
    arena of 16-token pages dealt out in random order; one step appends one
    token per sequence and runs decode attention (kvq_append_decode)."""
    lens, table, num_pages = wl.paged_layout(w)
    B, H, KVH, D = w.batch, w.num_heads, w.num_kv_heads, w.head_dim
    Lmax = int(lens.max())
    w.max_blocks_read = int(((lens + 15) // 16).sum())  # block-table entries the step reads
    dev = torch.device("cuda")
    cache = kvq.Int8KVCache(B, H, KVH, D, num_pages=num_pages,
                            block_table=torch.from_numpy(table).to(dev))
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    t0 = time.time()
    with torch.cuda.stream(stream):
        zero = torch.zeros(B, dtype=torch.int32, device=dev)
        step = 1024
        for p0 in range(0, Lmax - 1, step):
            n = min(step, Lmax - 1 - p0)
            k = torch.randn((B, KVH, n, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            v = torch.randn((B, KVH, n, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            cache.append(k, v, zero + p0, stream=stream)
        k_new = torch.randn((B, KVH, 1, D), generator=gen, device=dev).to(torch.bfloat16)
        v_new = torch.randn((B, KVH, 1, D), generator=gen, device=dev).to(torch.bfloat16)
        q_bits, _ = wl.paged_q(w)
        q = torch.from_numpy(q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        out = torch.empty_like(q)
        seq_lens = torch.from_numpy(lens).to(dev)
        ws = cache.workspace(Lmax, 1)
    stream.synchronize()
    log(f"paged arena: {num_pages} pages, {int(lens.sum())} tokens, lengths {int(lens.min())}..{Lmax}; "
        f"prefilled in {time.time() - t0:.1f}s")

    if args.separate:
        last = seq_lens - 1

        def step_fn():  # two launches: append at seq_lens[b] - 1, then decode
            cache.append(k_new, v_new, last, stream=stream)
            cache.decode(q, seq_lens, w.attn_scale, Lmax, out=out, workspace=ws, stream=stream)
    else:
        def step_fn():  # rows at position seq_lens[b] - 1, then attention over seq_lens[b] tokens
            cache.append_decode(k_new, v_new, q, seq_lens, w.attn_scale, Lmax, out=out, workspace=ws,
                                stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step_fn()
        stream.synchronize()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        step_ms = time_calls(step_fn, args.steps, stream, torch)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t1
    nb = paged_bytes(w, lens)
    tbps = nb["step"] / (step_ms * 1e-3) / 1e12
    k_gbs = nb["step"] / (step_ms * 1e-3) / 1e9
    ceil, _ = stream_ceiling(kvq, torch, stream, nb["step"], 1, reps=5, shapes=STREAM_QUICK)
    log(f"step {step_ms * 1e3:.1f} us, {tbps:.3f} TB/s ({tbps * 1e3 / HBM_PEAK_GBS * 100:.1f}% of 8 TB/s), "
        f"wall {wall * 1e3 / args.steps:.3f} ms/step")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline_paged(w, lens)
        cpu["single_thread"] = with_one_thread(cpu_baseline_paged, w, lens)
    result = {
        "metric": "INT8-KV paged decode attention: achieved HBM TB/s (% of peak)",
        "value": round(tbps, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "pct_of_hbm_peak": round(tbps * 1e3 / HBM_PEAK_GBS * 100, 2),
        "pct_of_stream": round(k_gbs / ceil["gbs"] * 100, 2),
        "stream": {"kernel": "kvq_stream_read", "gbs": ceil["gbs"], "us_per_launch": ceil["us_per_launch"]},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: batch {B}, {H} q / {KVH} kv heads, head_dim {D}, page size 16, "
                               f"lengths U[512, 32768] (seed {w.seed}: {int(lens.sum())} tokens), pages dealt "
                               f"from a shared arena in random order, per-token fp32 scales; append 1 token + "
                               f"decode ({'two launches' if args.separate else 'one fused launch'})",
                   "batch": B, "seq_len": Lmax, "bytes_per_step": nb["step"]},
        "roofline": {"bound": "hbm", "kernel": "kvq_append + kvq_attention_decode" if args.separate
                     else "kvq_append_decode",
                     "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if args.separate else recorded_traffic("kvq_append_decode", w.name),
                     "bytes_per_launch": nb["step"], "us_per_launch": round(step_ms * 1e3, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def sliding_bytes(w: wl.Workload) -> dict:
    """Algorithmic bytes of one sliding-window layer-step: codes and scales of
    the min(L, window) visible rows, queries, outputs, the appended row."""
    B, H, KVH, D = w.batch, w.num_heads, w.num_kv_heads, w.head_dim
    vis = min(w.ctx + w.n_new, w.extra["sliding"])
    decode = 2 * B * KVH * vis * (D + 4) + 2 * B * H * D * 2
    append = 2 * B * KVH * (D * 2 + D + 4)
    return {"decode": decode, "step": decode + append}


def run_sliding(args, w: wl.Workload, kvq, torch, stream):
    """Sliding-window decode: every layer's cache holds 8192 tokens (drawn on
    the device from a seeded generator); one step appends one token per
    sequence and attends over the last `window` tokens (one fused launch per
    layer)."""
    B, H, KVH, D = w.batch, w.num_heads, w.num_kv_heads, w.head_dim
    T = w.ctx + w.n_new
    win = w.extra["sliding"]
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    t0 = time.time()
    layers = []
    with torch.cuda.stream(stream):
        zero = torch.zeros(B, dtype=torch.int32, device=dev)
        for _ in range(w.layers):
            cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T)
            for p0 in range(0, w.ctx, 2048):
                n = min(2048, w.ctx - p0)
                k = torch.randn((B, KVH, n, D), generator=gen, device=dev).to(torch.bfloat16)
                v = torch.randn((B, KVH, n, D), generator=gen, device=dev).to(torch.bfloat16)
                cache.append(k, v, zero + p0, stream=stream)
            layers.append({"cache": cache,
                           "k_new": torch.randn((B, KVH, 1, D), generator=gen, device=dev).to(torch.bfloat16),
                           "v_new": torch.randn((B, KVH, 1, D), generator=gen, device=dev).to(torch.bfloat16),
                           "q": torch.randn((B, H, D), generator=gen, device=dev).to(torch.bfloat16)})
            layers[-1]["out"] = torch.empty_like(layers[-1]["q"])
        seq_lens = torch.full((B,), T, dtype=torch.int32, device=dev)
        ws = layers[0]["cache"].workspace(T, 1, win)
    stream.synchronize()
    log(f"prefilled {w.layers} layers of {T} tokens in {time.time() - t0:.1f}s")

    def step():
        for ly in layers:
            ly["cache"].append_decode(ly["k_new"], ly["v_new"], ly["q"], seq_lens, w.attn_scale, T, out=ly["out"],
                                      workspace=ws, stream=stream, window=win)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        stream.synchronize()
        step_ms = time_calls(step, args.steps, stream, torch)
        k_ms = time_calls(step, args.kernel_reps, stream, torch)
    nb = sliding_bytes(w)
    tbps = nb["step"] * w.layers / (step_ms * 1e-3) / 1e12
    us_launch = k_ms * 1e3 / w.layers
    k_gbs = nb["step"] / (us_launch * 1e-6) / 1e9
    ceil, _ = stream_ceiling(kvq, torch, stream, nb["step"], w.layers, reps=5, shapes=STREAM_QUICK)
    log(f"{step_ms * 1e3 / w.layers:.2f} us/layer-step, {tbps:.3f} TB/s; kvq_append_decode_window "
        f"{us_launch:.2f} us/launch = {k_gbs:.0f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline_sliding(w)
        cpu["single_thread"] = with_one_thread(cpu_baseline_sliding, w)
    result = {
        "metric": "INT8-KV sliding-window decode attention: us/layer-step and achieved HBM TB/s (% of peak)",
        "value": round(tbps, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "us_per_layer_step": round(step_ms * 1e3 / w.layers, 3),
        "pct_of_hbm_peak": round(tbps * 1e3 / HBM_PEAK_GBS * 100, 2),
        "pct_of_stream": round(k_gbs / ceil["gbs"] * 100, 2),
        "stream": {"kernel": "kvq_stream_read", "gbs": ceil["gbs"], "us_per_launch": ceil["us_per_launch"]},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: batch {B}, {H} q / {KVH} kv heads, head_dim {D}, context {T}, "
                               f"sliding window {win}, per-token fp32 scales, {w.layers} layers, append 1 token "
                               f"+ decode per layer (one fused launch)",
                   "batch": B, "seq_len": T, "layers": w.layers, "bytes_per_step": nb["step"] * w.layers},
        "roofline": {"bound": "hbm", "kernel": "kvq_append_decode_window",
                     "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("kvq_append_decode_window", w.name),
                     "bytes_per_launch": nb["step"], "us_per_launch": round(us_launch, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def cpu_baseline_sliding(w: wl.Workload, target_s: float = 12.0):
    """The oracle on whole sequences of the same shapes (drawn on the host):
    quantize the sequence's K/V, fp64 attention of its heads with the window
    mask applied to all of its keys."""
    import oracle as orc
    blas_threads = blas_thread_count()
    T = w.ctx + w.n_new
    win = w.extra["sliding"]
    per_seq = sliding_bytes(w)["step"] / w.batch
    rng = np.random.default_rng([w.seed, 7])
    q = wl.bits_to_f32(wl.bf16_bits(wl.normal(rng, (1, w.num_heads, w.head_dim))))
    seqs = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < target_s:
        x = wl.sequence_kv(w, seqs % w.batch, T)
        kc, ks = orc.quantize(x["k"], 0)
        vc, vs = orc.quantize(x["v"], 0)
        orc.attention_decode(q, orc.dequantize_exact(kc, ks)[None], orc.dequantize_exact(vc, vs)[None], [T],
                             w.attn_scale, window=win)
        seqs += 1
    el = time.perf_counter() - t0
    return {"value": per_seq * seqs / el / 1e12, "unit": "TB/s", "cores": blas_threads, "kind": "oracle",
            "sample": f"{seqs} sequences of {T} tokens drawn on the host with the workload's shapes (quantize the "
                      f"sequence's K/V, fp64 attention of {w.num_heads} heads under a {win}-token window), {el:.1f}s wall; "
                      f"bytes counted as the step's per-sequence algorithmic bytes; BLAS threads {blas_threads}; "
                      f"host {platform.processor() or 'x86_64'} nproc {os.cpu_count()}"}


def cpu_baseline_paged(w: wl.Workload, lens, target_s: float = 12.0):
    """The oracle on whole sequences of the paged step (quantize the sequence's
    K/V, fp64 attention for its heads), on a bounded sample of sequences."""
    import oracle as orc
    blas_threads = blas_thread_count()
    q_bits, q = wl.paged_q(w)
    done_bytes = 0
    seqs = 0
    t0 = time.perf_counter()
    b = 0
    while time.perf_counter() - t0 < target_s:
        L = int(lens[b])
        x = wl.sequence_kv(w, b, L)
        kc, ks = orc.quantize(x["k"], 0)
        vc, vs = orc.quantize(x["v"], 0)
        orc.attention_decode(q[b:b + 1], orc.dequantize_exact(kc, ks)[None], orc.dequantize_exact(vc, vs)[None],
                             [L], w.attn_scale)
        done_bytes += 2 * L * w.num_kv_heads * (w.head_dim + 4)
        seqs += 1
        b = (b + 1) % len(lens)
    el = time.perf_counter() - t0
    return {"value": done_bytes / el / 1e12, "unit": "TB/s", "cores": blas_threads, "kind": "oracle",
            "sample": f"{seqs} sequences of the paged step in order (quantize the sequence's K/V, fp64 attention "
                      f"for its {w.num_heads} heads), {el:.1f}s wall; bytes counted as the cache codes and scales those "
                      f"sequences occupy; numpy elementwise single-threaded, BLAS threads {blas_threads}; host "
                      f"{platform.processor() or 'x86_64'} nproc {os.cpu_count()}"}


# ----------------------------------------------------------------------------
# Read-bandwidth ceiling: a plain read stream of the same bytes per launch
# ----------------------------------------------------------------------------

STREAM_SHAPES = [  # (workgroups, waves per workgroup, KB in flight per wave (x1..x2), interleaved[, non-temporal])
    (256, 8, 2, True), (256, 8, 4, True), (512, 8, 2, True), (512, 8, 4, True),
    (1024, 8, 2, True), (1024, 4, 4, True), (2048, 4, 2, True), (256, 16, 2, True),
    (512, 8, 4, False), (1024, 8, 2, False),
    (256, 8, 2, True, True), (512, 8, 8, True, True), (1024, 8, 2, True, True), (256, 8, 4, False, True),
]


# the best shapes of the sweep above (bench.py --workload stream_read), timed
# beside every decode line for its percent-of-stream figure
STREAM_QUICK = [(256, 8, 2, True), (512, 8, 8, True), (1024, 8, 2, True), (256, 8, 4, False),
                (256, 8, 2, True, True), (1024, 8, 2, True, True)]


def stream_ceiling(kvq, torch, stream, nbytes: int, launches: int, reps: int = 5, shapes=STREAM_SHAPES):
    """Best rate of the read-only stream kernel over `launches` buffers of
    `nbytes` each (one launch per buffer, visited in turn as the decode step
    visits its layers, so nothing is re-read from the Infinity Cache), over a
    sweep of launch shapes.  Returns (best record, every record)."""
    nbytes = nbytes // 16 * 16
    buf = torch.empty(launches * nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    recs = []
    with torch.cuda.stream(stream):
        for shape in shapes:
            wg, wv, dep, il = shape[:4]
            nt = len(shape) > 4 and shape[4]

            def one():
                for i in range(launches):
                    kvq.kvq.kvq_stream_read(buf.data_ptr() + i * nbytes, nbytes, sink, wg, wv, dep, il, stream=stream,
                                            nontemporal=nt)
            one()
            ms = time_calls(one, reps, stream, torch)
            us = ms * 1e3 / launches
            recs.append({"workgroups": wg, "waves": wv, "kb_in_flight_per_wave": dep, "interleaved": il,
                         "nontemporal": nt, "us_per_launch": round(us, 3), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)})
    del buf
    best = max(recs, key=lambda r: r["gbs"])
    return best, recs


def run_ctx_sweep(args, kvq, torch, stream):
    """The fused decode step of the 8B-shaped workload's shape (B16, 32/8
    heads, D128, per-token scales) at contexts 1024..16384 on a fixed grid
    (two splits per head group: one round of 256 workgroups at every
    context), eight layers of synthetic codes, beside the read stream of the
    same bytes.  A straight-line fit of time against bytes separates the
    per-launch fixed cost from the streaming rate."""
    import numpy as np
    os.environ["KVQ_NUM_SPLITS"] = "2"
    B, H, KVH, D, NL = 16, 32, 8, 128, 8
    pts = []
    for ctx in (1024, 2048, 4096, 8192, 16384):
        g = torch.Generator(device="cuda").manual_seed(ctx)
        caches = []
        for _ in range(NL):
            c = kvq.Int8KVCache(B, H, KVH, D, max_len=ctx)
            c.k_codes.random_(0, 256, generator=g)
            c.v_codes.random_(0, 256, generator=g)
            c.k_scales.uniform_(0.001, 0.01, generator=g)
            c.v_scales.uniform_(0.001, 0.01, generator=g)
            caches.append(c)
        q = torch.randn(B, H, D, device="cuda", generator=g).to(torch.bfloat16)
        kn = torch.randn(B, KVH, D, device="cuda", generator=g).to(torch.bfloat16)
        vn = torch.randn(B, KVH, D, device="cuda", generator=g).to(torch.bfloat16)
        sl = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
        ws = caches[0].workspace(ctx, 1)
        out = torch.empty_like(q)
        torch.cuda.synchronize()  # the fills above ran on the default stream

        def one():
            for c in caches:
                c.append_decode(kn, vn, q, sl, 0.088, ctx, out=out, workspace=ws, stream=stream)
        with torch.cuda.stream(stream):
            for _ in range(max(args.warmup, 1)):
                one()
            us = time_calls(one, args.steps, stream, torch) * 1e3 / NL
        nbytes = 2 * B * KVH * ctx * (D + 4) + 2 * B * H * D * 2 + 2 * B * KVH * D * 2
        best, _ = stream_ceiling(kvq, torch, stream, nbytes, NL, reps=5, shapes=STREAM_QUICK)
        pts.append({"ctx": ctx, "bytes": nbytes, "us": round(us, 3), "stream_us": best["us_per_launch"]})
        log(f"ctx {ctx}: {us:.2f} us per launch, read stream {best['us_per_launch']:.2f} us")
        del caches
        torch.cuda.empty_cache()
    x = np.array([p["bytes"] for p in pts], dtype=np.float64)
    fit = {}
    for key in ("us", "stream_us"):
        y = np.array([p[key] for p in pts])
        slope, icpt = np.polyfit(x, y, 1)
        fit[key] = {"fixed_us": round(float(icpt), 2), "rate_gbs": round(float(1e-3 / slope), 1)}
    log(f"fit: decode {fit['us']}, read stream {fit['stream_us']}")
    print(json.dumps({"metric": "fused decode time vs context (fixed grid)", "unit": "us", "points": pts, "fit": fit,
                      "data": "synthetic", "config": {"workload": "decode_ctx_sweep: batch 16, 32 q / 8 kv heads, "
                                                      "head_dim 128, per-token fp32 scales, 8 layers, 2 splits"}}),
          flush=True)


def run_stream(args, kvq, torch, stream):
    """The read-only stream kernel alone: the 8B-shaped decode's bytes per
    layer-step (one launch per layer, 32 layers), and one 4 GiB launch."""
    w = wl.ALL["decode_8b"]
    per_layer = step_bytes(w, w.ctx + w.n_new)["step"]
    best, recs = stream_ceiling(kvq, torch, stream, per_layer, w.layers, reps=args.steps)
    for r in recs:
        log(f"stream {r}")
    big, big_recs = stream_ceiling(kvq, torch, stream, 1 << 32, 1, reps=3,
                                   shapes=[(1024, 8, 4, True), (2048, 8, 4, False), (4096, 4, 4, True)])
    for r in big_recs:
        log(f"stream 4 GiB {r}")
    result = {
        "metric": "read-only stream kernel: achieved HBM GB/s (ceiling for the decode kernels)",
        "value": best["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": 1,
        "ms_per_step": round(best["us_per_launch"] * w.layers * 1e-3, 4),
        "pct_of_hbm_peak": round(best["gbs"] / HBM_PEAK_GBS * 100, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"stream_read: {per_layer} B per launch (the 8B-shaped decode's bytes per "
                               f"layer-step), {w.layers} buffers read in turn; best of {len(recs)} launch shapes",
                   "best_shape": best, "asymptote_4gib": big},
        "roofline": {"bound": "hbm", "kernel": "kvq_stream_read", "achieved": best["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(best["gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": per_layer, "us_per_launch": best["us_per_launch"]},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


# ----------------------------------------------------------------------------
# main
# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_8b", choices=["decode_8b", "q8_group32", "chunked_prefill", "paged_decode",
                                                            "recent_window", "sliding_decode", "sliding_chunk",
                                                            "bf16_scales", "fp8_e4m3", "fp8_chunk", "chunk_group32",
                                                            "recent_chunk", "tiny_decode", "stream_read",
                                                            "recent_block_head", "recent_block_channel", "chunk_d256",
                                                            "decode_d256", "decode_ctx_sweep"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate", action="store_true",
                    help="time kvq_append + kvq_attention_decode as two launches instead of kvq_append_decode")
    ap.add_argument("--kernel-reps", type=int, default=10,
                    help="passes over all layers when timing the decode kernel alone")
    ap.add_argument("--threads", type=int, default=min(16, os.cpu_count() or 8))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures the INT8-KV decode path on one GPU; --gpus {args.gpus} is not supported "
              "(sequences and KV heads shard with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import int8_quantized_kv_amd as kvq

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        with torch.cuda.stream(stream):
            for _ in range(5):
                b.copy_(a)
        stream.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return

    if args.workload == "stream_read":
        run_stream(args, kvq, torch, stream)
        return
    if args.workload == "decode_ctx_sweep":
        run_ctx_sweep(args, kvq, torch, stream)
        return
    w = wl.ALL[args.workload]
    if w.name == "sliding_decode":
        run_sliding(args, w, kvq, torch, stream)
        return
    if w.name in ("chunked_prefill", "sliding_chunk", "fp8_chunk", "chunk_group32", "recent_chunk", "chunk_d256"):
        run_chunk(args, w, kvq, torch, stream)
        return
    if w.name == "paged_decode":
        run_paged(args, w, kvq, torch, stream)
        return
    T = w.ctx + w.n_new
    log(f"workload {w.name}: B={w.batch} H={w.num_heads} KVH={w.num_kv_heads} D={w.head_dim} "
        f"L={T} layers={w.layers} group={w.group}")
    layers = build_layers(w, kvq, torch, stream, args.threads)
    dev = torch.device("cuda")
    start_pos = torch.full((w.batch,), w.ctx, dtype=torch.int32, device=dev)
    seq_lens = torch.full((w.batch,), T, dtype=torch.int32, device=dev)
    ws = layers[0]["cache"].workspace(T, 1)

    if args.separate:
        def step():
            for ly in layers:
                c = ly["cache"]
                c.append(ly["k_new"], ly["v_new"], start_pos, stream=stream)
                c.decode(ly["q"], seq_lens, w.attn_scale, T, out=ly["out"], workspace=ws, stream=stream)

        def kernel_pass():  # the dominant kernel alone: decode attention
            for ly in layers:
                ly["cache"].decode(ly["q"], seq_lens, w.attn_scale, T, out=ly["out"], workspace=ws, stream=stream)
        kernel_name, kernel_bytes = "kvq_attention_decode", "decode"
    else:
        def step():  # one launch per layer: quantize-append at position 4095, then decode over 4096
            for ly in layers:
                ly["cache"].append_decode(ly["k_new"], ly["v_new"], ly["q"], seq_lens, w.attn_scale, T,
                                          out=ly["out"], workspace=ws, stream=stream)
        kernel_pass = step
        kernel_name = "kvq_append_decode_recent" if w.extra.get("window") else "kvq_append_decode"
        kernel_bytes = "step"

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        stream.synchronize()
        torch.cuda.synchronize()
        log(f"warmup {args.warmup} steps done; timing {args.steps} steps")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = e0.elapsed_time(e1) / args.steps
        log(f"timed {args.steps} steps: {step_ms:.3f} ms/step (events), wall {wall * 1e3 / args.steps:.3f} ms/step")

        # the dominant kernel alone, same launch configuration
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(args.kernel_reps):
            kernel_pass()
        d1.record(stream)
        stream.synchronize()
        dec_us = d0.elapsed_time(d1) * 1e3 / (args.kernel_reps * w.layers)

    nbytes = step_bytes(w, T)
    total_bytes = nbytes["step"] * w.layers
    ceil, _ = stream_ceiling(kvq, torch, stream, nbytes[kernel_bytes], w.layers, reps=5, shapes=STREAM_QUICK)
    tbps = total_bytes / (step_ms * 1e-3) / 1e12
    us_layer = step_ms * 1e3 / w.layers
    dec_gbs = nbytes[kernel_bytes] / (dec_us * 1e-6) / 1e9
    log(f"{us_layer:.2f} us/layer-step, {tbps:.3f} TB/s ({tbps * 1e3 / HBM_PEAK_GBS * 100:.1f}% of 8 TB/s); "
        f"{kernel_name} {dec_us:.2f} us/launch = {dec_gbs:.0f} GB/s; read stream of the same bytes "
        f"{ceil['us_per_launch']:.2f} us = {ceil['gbs']:.0f} GB/s ({dec_gbs / ceil['gbs'] * 100:.1f}% of it)")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        base = cpu_baseline_recent if w.extra.get("window") else cpu_baseline
        cpu = base(w)
        cpu.pop("seconds", None)
        cpu["single_thread"] = with_one_thread(base, w)

    fp8 = w.extra.get("fp8")
    codes_what = (f"FP8 {fp8.upper()} codes (no scales)" if fp8 else
                  f"{'per-token' if w.group == 0 else 'group-32'} "
                  f"{'bf16' if w.extra.get('scale_bf16') else 'fp32'} scales")
    result = {
        "metric": ("FP8" if fp8 else "INT8") + "-KV decode attention: us/layer-step and achieved HBM TB/s (% of peak)",
        "value": round(tbps, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "us_per_layer_step": round(us_layer, 3),
        "pct_of_hbm_peak": round(tbps * 1e3 / HBM_PEAK_GBS * 100, 2),
        "pct_of_stream": round(dec_gbs / ceil["gbs"] * 100, 2),
        "stream": {"kernel": "kvq_stream_read", "gbs": ceil["gbs"], "us_per_launch": ceil["us_per_launch"],
                   "shape": {k: ceil[k] for k in ("workgroups", "waves", "kb_in_flight_per_wave", "interleaved", "nontemporal")},
                   "what": f"read-only stream of the same {nbytes[kernel_bytes]} B per launch, {w.layers} buffers "
                           f"in turn; pct_of_stream compares the kernel's algorithmic GB/s with it"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"fp8{fp8}" if fp8 else "u8",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: batch {w.batch}, {w.num_heads} q / {w.num_kv_heads} kv heads, "
                               f"head_dim {w.head_dim}, context {T}, {codes_what}, {w.layers} layers, "
                               + (f"last {w.extra['window']} tokens bf16 (recent window), " if w.extra.get("window")
                                  else "") +
                               f"append 1 token + decode per layer "
                               f"({'two launches' if args.separate else 'one fused launch'})",
                   "batch": w.batch, "seq_len": T, "layers": w.layers, "bytes_per_step": total_bytes},
        "roofline": {"bound": "hbm", "kernel": kernel_name,
                     "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(kernel_name, w.name),
                     "bytes_per_launch": nbytes[kernel_bytes], "us_per_launch": round(dec_us, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
