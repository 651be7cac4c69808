"""Benchmark of the paged int8 KV-cache decode step on one MI355X.

A step is one pass of the hot path over one batch: store the batch's new K/V tokens into the paged
cache (quantized), then grouped-query decode attention of the new queries over the cache.  The
default workload is the Qwen3-8B-shaped decode batch (batch 32, 32/8 heads, head_dim 128,
block_size 16, context lengths ~ U[1024, 4096], int8 per-token scales); ``--config`` selects
another one.  Inputs are seeded and synthetic and are resident in HBM before timing starts.

To keep the 256 MB Infinity Cache from serving the working set, the step cycles over R replicas of
the cache (R chosen so the replicas hold >= 768 MB of touched bytes).

Prints ONE JSON line (rank 0):
  value       decode-attention HBM GB/s of the whole step (algorithmic bytes / step time)
  roofline    the dominant kernel (split-KV decode, partial + merge) against 8 TB/s
  cpu_baseline the CPU oracle on the same workload (store + fp64 attention), timed on this host
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_F16_TFLOPS = 2500.0  # dense fp16 / bf16 matrix-core peak of MI355X
MALL_BYTES = 256 * 2 ** 20
MAX_REPLICAS = 64  # tiny workloads are latency-bound: a few replicas suffice


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1,
                    help="workload index (0..4; 5 = paged prefill, measured in TFLOP/s); 1 = Qwen3-8B decode")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--prompt-len", type=int, default=0,
                    help="paged prefill (--config 5): prompts of this many tokens, 8192 // N of them (0: 4 x 2048)")
    ap.add_argument("--quant-mode", type=int, default=None,
                    help="run the workload's shapes with another cache mode (3 = static per-channel scales)")
    ap.add_argument("--partition", type=int, default=0,
                    help="int8-score kernel key partition: 0 planned, 1 fixed, 2 balanced")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: each query attends to its last W positions (0: all)")
    ap.add_argument("--kernel", type=int, default=0, help="0 = library choice, 1 = VALU, 2 = MFMA fp16 scores, 3 = MFMA int8 scores, 4 = tile (many rows per KV head)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-baseline sample")
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas (0 = auto)")
    ap.add_argument("--mla", type=int, default=-1,
                    help="paged MLA (latent cache) workload index instead of the GQA ones (1 = DeepSeek-V3-shaped)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (for scaling HBM byte counters)")
    ap.add_argument("--separate-store", action="store_true",
                    help="a decode batch's store as its own call before the decode (default: one call)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="the default run measures the long-context decode too and reports it as 'secondary'")
    ap.add_argument("--op", default="decode", choices=["decode", "store-fill", "dequant", "walk"],
                    help="decode: the decode step (default); store-fill: the prompt-style store of every "
                         "prior token of the workload; dequant: the gather of the whole cache to bf16 rows; "
                         "walk: only the cache reads of the int8 decode (its read ceiling, pkv_cache_walk)")
    ap.add_argument("--walk-depth", type=int, default=1, help="walk: 64-key blocks in flight per wave (1..3)")
    return ap.parse_args()


def calibrate_copy(steps):
    """A plain 1 GiB device-to-device copy, repeated: the reference against which rocprofv3's
    FETCH_SIZE / WRITE_SIZE readings of the decode kernel are scaled to bytes."""
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "ms_per_launch": round(ms, 4), "gbs_read_plus_write": round(2 * n / ms / 1e6, 1)}))


def step_bytes(w, window=0):
    """Algorithmic HBM bytes of one step: every cache byte the attention must read once, plus the
    queries, outputs, block-table entries and context lengths it reads, plus the store's input and
    output.  Split-KV partials are overhead and excluded.  With a sliding window of W keys a
    sequence's attention reads only the keys its queries see: from the first query's window start
    to its last key."""
    ctx = w.context_lengths.astype(np.int64)
    if window > 0:
        first = np.maximum(w.prior_lengths.astype(np.int64) - window + 1, 0)
        ctx = ctx - np.minimum(first, ctx)
    hkv, d, bs = w.num_kv_heads, w.head_dim, w.block_size
    if w.quant_mode == 0:
        per_tok = hkv * (2 * d + 8)
        kv = int(ctx.sum()) * per_tok
    elif w.quant_mode == 3:  # static per-channel scales: read once per KV head
        kv = int(ctx.sum()) * hkv * 2 * d + hkv * d * 4 * 2
    elif w.quant_mode == 1:
        kv = int(ctx.sum()) * hkv * 2 * d + int(np.ceil(ctx / bs).sum()) * hkv * 8
    else:
        kv = int(ctx.sum()) * hkv * 4 * d
    tq = w.num_new_tokens if not w.decode_only else w.batch
    qo = 2 * tq * w.num_q_heads * d * 2
    meta = int(np.ceil(ctx / bs).sum()) * 4 + w.batch * 4
    decode = kv + qo + meta
    t = w.num_new_tokens
    if w.quant_mode == 2:
        store = t * hkv * d * 2 * 2 * 2
    elif w.quant_mode == 0:
        store = t * hkv * d * 2 * 2 + t * hkv * (d + 4) * 2
    elif w.quant_mode == 3:
        store = t * hkv * d * 2 * 2 + t * hkv * d * 2 + hkv * d * 4 * 2
    else:  # per block: new tokens in and out, plus the touched old codes read and rewritten
        store = t * hkv * d * 2 * 2 + t * hkv * d * 2
    return decode, store


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


def traffic_record(kernel_key):
    """HBM traffic of the dominant kernel measured with rocprofv3 counters (committed under
    profiles/), valid only while the kernel sources hash to the recorded value."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_key)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec.get("sources", []):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(max(args.steps, 1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.mla >= 0:
        if args.op == "walk":
            main_mla_walk(args)
        else:
            main_mla(args)
        return
    if args.op == "walk":
        main_walk(args)
        return
    if args.op != "decode":
        main_codec(args)
        return
    res = run_decode(args, args.config, args.quant_mode, not args.no_cpu_baseline)
    default_flags = (args.kernel == 0 and args.split_tokens == 0 and args.window == 0 and args.partition == 0
                     and args.quant_mode is None and not args.separate_store)
    if args.config == 1 and default_flags and not args.no_secondary:
        # the other target workload, measured the same way (no CPU leg), reported beside the first
        sec = run_decode(args, 2, None, False)
        res["secondary"] = {k: sec[k] for k in ("value", "unit", "ms_per_step", "ms_per_step_median", "pct_of_peak",
                                                "tokens_per_s", "kv_tokens_per_s", "bytes_per_step", "roofline")}
        res["secondary"]["workload"] = sec["config"]["workload"]
    print(json.dumps(res), flush=True)


def run_decode(args, config_index, quant_mode, with_cpu):
    """One workload's decode step, timed; returns the result record."""

    import torch

    import gen
    import paged_kv_cache_c8_amd as pkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = gen.make_config(config_index, quant_mode=quant_mode, prompt_len=args.prompt_len)
    t = gen.gen_tensors(w, device=dev)
    k_prior, k_new = gen.split_prior_new(w, t["k_all"])
    v_prior, v_new = gen.split_prior_new(w, t["v_all"])
    i32 = lambda x: torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device=dev)
    bt, ctx, prior, cu_prior = i32(w.block_table), i32(w.context_lengths), i32(w.prior_lengths), i32(w.cu_prior)
    cu_q = None if w.decode_only else i32(w.cu_q_lens)
    q = t["q"]
    decode_bytes, store_bytes = step_bytes(w, args.window)
    touched = decode_bytes + store_bytes
    reps = args.replicas or min(MAX_REPLICAS, max(1, int(np.ceil(3 * MALL_BYTES / touched))))

    caches = []
    for _ in range(reps):
        c = pkv.Cache(w.quant_mode, w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, device=dev)
        if w.quant_mode == gen.QUANT_PER_CHANNEL:
            c.k_scale.copy_(t["k_scale"])
            c.v_scale.copy_(t["v_scale"])
        if int(w.prior_lengths.sum()):
            pkv.store_c8(c, k_prior, v_prior, cu_q_lens=cu_prior, context_lengths=prior, block_table=bt,
                         max_q_len=int(w.prior_lengths.max()))
        caches.append(c)
    scale = 1.0 / float(np.sqrt(w.head_dim))
    mql = w.max_q_len if cu_q is not None else 1
    ws_bytes = pkv.decode_workspace_size(w.batch, w.num_q_heads, caches[0], w.max_blocks_per_seq, mql,
                                         split_tokens=args.split_tokens, kernel=args.kernel, window=args.window,
                                         partition=args.partition)
    workspace = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)  # zero-filled once
    out = torch.empty_like(q)
    plan = pkv.decode_plan(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_blocks_per_seq,
                           w.block_size, mql, w.quant_mode, split_tokens=args.split_tokens, kernel=args.kernel, window=args.window,
                                         partition=args.partition)

    def store(c):
        if w.decode_only:
            pkv.store_c8(c, k_new, v_new, context_lengths=ctx, block_table=bt)
        else:
            pkv.store_c8(c, k_new, v_new, cu_q_lens=cu_q, context_lengths=ctx, block_table=bt,
                         max_q_len=w.max_q_len)

    def decode(c):
        pkv.decode_gqa(q, c, bt, ctx, scale, cu_q_lens=cu_q, max_q_len=mql, out=out, workspace=workspace,
                       split_tokens=args.split_tokens, kernel=args.kernel, window=args.window,
                                         partition=args.partition)

    # a decode batch (one new token per sequence) runs its store and attention as one call
    fused = w.decode_only and not args.separate_store

    def store_decode(c):
        pkv.store_decode_gqa(q, k_new, v_new, c, bt, ctx, scale, out=out, workspace=workspace,
                             split_tokens=args.split_tokens, kernel=args.kernel, window=args.window,
                             partition=args.partition)

    def step(i):
        c = caches[i % reps]
        if fused:
            store_decode(c)
        else:
            store(c)
            decode(c)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- whole-step timing
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # ---- dominant call: the store + decode call (a decode batch) or the decode call, bracketed by
    #      events on the launch stream (the current stream)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        c = caches[i % reps]
        if not fused:
            store(c)
        evs[i][0].record(stream)
        if fused:
            store_decode(c)
        else:
            decode(c)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in evs]
    dec_ms = float(np.mean(call_ms))
    call_bytes = decode_bytes + (store_bytes if fused else 0)

    step_s = ms_per_step * 1e-3
    value = touched / step_s / 1e9
    new_tokens = w.num_new_tokens if not w.decode_only else int((w.context_lengths > 0).sum())
    achieved = call_bytes / (dec_ms * 1e-3) / 1e9
    # the counters were taken with the library's own choice of kernel and split
    default_plan = (args.kernel == 0 and args.split_tokens == 0 and args.window == 0 and args.partition == 0
                    and not args.separate_store)
    mode_key = "" if quant_mode is None else f".mode{quant_mode}"
    plen_key = f".p{args.prompt_len}" if args.prompt_len > 0 else ""
    traffic = traffic_record(f"decode.config{config_index}{mode_key}{plen_key}") if default_plan else None

    cpu = None
    if with_cpu:
        cpu = cpu_baseline(w, t, args.cpu_seconds, touched, new_tokens, args.window)

    dtype = {0: "int8", 1: "int8", 2: "bf16", 3: "int8"}[w.quant_mode]
    roofline = {
        "bound": "hbm",
        "kernel": ("pkv_store_decode_gqa (new-token store + split-KV partial, log-sum-exp merge)" if fused
                   else "pkv_decode_gqa (tile kernel, 128 query rows per workgroup"
                   + (", key splits + log-sum-exp merge)" if plan["num_splits"] > 1 else ")")
                   if plan["kernel"] == 4 else "pkv_decode_gqa (split-KV partial + log-sum-exp merge)"),
        "achieved": round(achieved, 2),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": call_bytes,
        "avg_launch_ms": round(dec_ms, 5),
        "median_launch_ms": round(float(np.median(call_ms)), 5),
    }
    if w.name.startswith("paged-prefill"):
        # a prompt's attention is a dense contraction: 2 * 2 * D algorithmic flops per visible
        # (query head, key) pair (Q.K and P.V), against the 2.5 PFLOP/s of the dense fp16 / bf16
        # matrix cores (the tile kernel runs Q.K and P.V in fp16 on the matrix cores; only the
        # algorithmic flops count)
        pairs = sum(int(w.q_lens[b]) * (2 * int(w.prior_lengths[b]) + int(w.q_lens[b]) + 1) // 2
                    for b in range(w.batch))
        flops = 4.0 * pairs * w.num_q_heads * w.head_dim
        tflops = flops / (dec_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": roofline["kernel"], "achieved": round(tflops, 2),
                    "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_F16_TFLOPS, 4),
                    "traffic": traffic, "flops_per_launch": flops, "avg_launch_ms": round(dec_ms, 5)}
    res = {
        "metric": "decode-attn HBM GB/s (% of peak) + tokens/s, int8 paged-KV GQA",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_median": round(float(np.median(call_ms)), 5) if fused else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, random block tables)",
        "config": {
            "workload": w.name,
            "batch": w.batch, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "quant_mode": w.quant_mode,
            "sum_context": int(w.context_lengths.sum()), "new_tokens": new_tokens,
            "cache_replicas": reps, "split_tokens": plan["split_tokens"], "num_splits": plan["num_splits"],
            "window": args.window,
            "kernel": {1: "valu", 2: "mfma-f16", 3: "mfma-i8", 4: "tile"}[plan["kernel"]],
            "store": "in the decode call" if fused else "separate call",
            "parallelism": "single-gpu",
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(new_tokens / step_s, 1),
        "kv_tokens_per_s": round(float(w.context_lengths.sum()) / step_s, 1),
        "bytes_per_step": touched,
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    return res


def codec_bytes(w, op):
    """Algorithmic HBM bytes of one launch of the store (every prior token of the workload, stored
    in one prompt-style call) or of the dequant (every position of every sequence gathered to bf16
    rows): each input byte read once, each output byte written once."""
    hkv, d, bs = w.num_kv_heads, w.head_dim, w.block_size
    if op == "store-fill":
        t = int(w.prior_lengths.sum())
        if w.quant_mode == 2:
            out = t * hkv * d * 2 * 2
        elif w.quant_mode == 0:
            out = t * hkv * (2 * d + 8)
        elif w.quant_mode == 3:
            out = t * hkv * 2 * d + hkv * d * 4 * 2
        else:
            out = t * hkv * 2 * d + int(np.ceil(w.prior_lengths / bs).sum()) * hkv * 8
        meta = w.batch * 4 * 2 + int(np.ceil(w.prior_lengths / bs).sum()) * 4
        return t * hkv * d * 2 * 2, out + meta, t
    n = int(w.context_lengths.sum())
    if w.quant_mode == 2:
        rd = n * hkv * d * 2 * 2
    elif w.quant_mode == 0:
        rd = n * hkv * (2 * d + 8)
    elif w.quant_mode == 3:
        rd = n * hkv * 2 * d + hkv * d * 4 * 2
    else:
        rd = n * hkv * 2 * d + int(np.ceil(w.context_lengths / bs).sum()) * hkv * 8
    rd += w.batch * 4 + int(np.ceil(w.context_lengths / bs).sum()) * 4
    return rd, n * hkv * d * 2 * 2, n


def walk_bytes(w, split):
    """Bytes pkv_cache_walk reads: every K row of every position, the whole 16-slot V tiles that
    hold them, the per-token scales (per-block: each page once per wave that touches it), and the
    block-table entries each wave stages."""
    hkv, d, bs = w.num_kv_heads, w.head_dim, w.block_size
    total = 0
    for c in w.context_lengths.astype(np.int64):
        for t0 in range(0, int(c), split):
            t1 = min(t0 + split, int(c))
            pages = (t1 - 1) // bs - t0 // bs + 1
            total += (t1 - t0) * d + ((t1 - t0 + 15) // 16) * 16 * d + pages * 4
            if w.quant_mode == 0:
                total += (t1 - t0) * 8
            elif w.quant_mode == 1:
                total += pages * 8
    return total * hkv


def main_walk(args):
    """The int8 decode's cache reads alone (pkv_cache_walk): same pages, same layout, same wave
    order and keys per wave as the decode's fixed partition, nothing computed.  Its rate is the
    read ceiling of the access pattern, the number the decode's own HBM fraction is judged by."""
    import torch

    import gen
    import paged_kv_cache_c8_amd as pkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = gen.make_config(args.config, quant_mode=args.quant_mode, prompt_len=args.prompt_len)
    if w.quant_mode == gen.QUANT_NONE_BF16:
        raise SystemExit("--op walk: int8 caches only")
    t = gen.gen_tensors(w, device=dev)
    k_prior, _ = gen.split_prior_new(w, t["k_all"])
    v_prior, _ = gen.split_prior_new(w, t["v_all"])
    del t["k_all"], t["v_all"]
    i32 = lambda x: torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device=dev)
    bt, ctx, prior, cu_prior = i32(w.block_table), i32(w.context_lengths), i32(w.prior_lengths), i32(w.cu_prior)
    split = args.split_tokens
    if split <= 0:
        mq = 1 if w.decode_only else int(np.diff(w.cu_q_lens).max())
        split = pkv.decode_plan(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_blocks_per_seq,
                                w.block_size, mq, w.quant_mode)["split_tokens"] or 256
    read_b = walk_bytes(w, split)
    reps = args.replicas or min(MAX_REPLICAS, max(1, int(np.ceil(3 * MALL_BYTES / read_b))))
    caches = []
    mql = int(w.prior_lengths.max())
    for _ in range(reps):
        c = pkv.Cache(w.quant_mode, w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, device=dev)
        if w.quant_mode == gen.QUANT_PER_CHANNEL:
            c.k_scale.copy_(t["k_scale"])
            c.v_scale.copy_(t["v_scale"])
        if mql > 0:  # positions past the prior tokens hold whatever the pool held (timing only)
            pkv.store_c8(c, k_prior, v_prior, cu_q_lens=cu_prior, context_lengths=prior, block_table=bt,
                         max_q_len=mql)
        caches.append(c)
    del k_prior, v_prior
    nsplit = -(-w.max_blocks_per_seq * w.block_size // split)
    outs = [torch.empty((w.batch, w.num_kv_heads, nsplit), dtype=torch.int32, device=dev) for _ in range(reps)]

    def launch(i):
        pkv.cache_walk(caches[i % reps], bt, ctx, split, depth=args.walk_depth, out=outs[i % reps])
    for i in range(max(args.warmup, 2)):
        launch(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    steps = max(args.steps, 5)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        launch(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    ms = float(np.median(times))
    achieved = read_b / (ms * 1e-3) / 1e9
    res = {
        "op": "walk", "workload": w.name, "quant_mode": w.quant_mode, "split_tokens": split,
        "depth": args.walk_depth, "waves": int(w.batch * w.num_kv_heads * nsplit), "cache_replicas": reps,
        "bytes_read": read_b, "ms_median": round(ms, 5), "ms_mean": round(float(np.mean(times)), 5),
        "launches": steps,
        "roofline": {"bound": "hbm", "kernel": "pkv_cache_walk (the decode's cache reads only)",
                     "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_launch": read_b,
                     "avg_launch_ms": round(ms, 5)},
    }
    print(json.dumps(res), flush=True)


def main_codec(args):
    """The store of a whole prompt (the workload's prior tokens, one call) or the dequant of the
    whole cache, timed alone with HIP events on the launch stream; inputs and outputs resident in
    HBM.  Two input copies and two caches alternate so the 256 MB Infinity Cache cannot serve a
    launch from the previous one."""
    import torch

    import gen
    import paged_kv_cache_c8_amd as pkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = gen.make_config(args.config, quant_mode=args.quant_mode, prompt_len=args.prompt_len)
    t = gen.gen_tensors(w, device=dev)
    k_prior, _ = gen.split_prior_new(w, t["k_all"])
    v_prior, _ = gen.split_prior_new(w, t["v_all"])
    del t["k_all"], t["v_all"]
    i32 = lambda x: torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device=dev)
    bt, ctx, prior, cu_prior = i32(w.block_table), i32(w.context_lengths), i32(w.prior_lengths), i32(w.cu_prior)
    read_b, write_b, units = codec_bytes(w, args.op)
    caches = []
    for _ in range(2):
        c = pkv.Cache(w.quant_mode, w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, device=dev)
        if w.quant_mode == gen.QUANT_PER_CHANNEL:
            c.k_scale.copy_(t["k_scale"])
            c.v_scale.copy_(t["v_scale"])
        caches.append(c)
    mql = int(w.prior_lengths.max())
    if args.op == "store-fill":
        ins = [(k_prior, v_prior), (k_prior.clone(), v_prior.clone())]

        def launch(i):
            k, v = ins[i % 2]
            pkv.store_c8(caches[i % 2], k, v, cu_q_lens=cu_prior, context_lengths=prior, block_table=bt,
                         max_q_len=mql)
        kernel = "pkv_store_c8 (prompt-style store of every prior token)"
    else:
        for c in caches:
            pkv.store_c8(c, k_prior, v_prior, cu_q_lens=cu_prior, context_lengths=prior, block_table=bt,
                         max_q_len=mql)
        del k_prior, v_prior
        rows = int(w.context_lengths.sum())
        outs = [(torch.empty((rows, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16, device=dev),
                 torch.empty((rows, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16, device=dev))
                for _ in range(2)]
        # the dequant reads every position < context length: the prior tokens plus the new ones,
        # which hold whatever the pool held (timing only)

        def launch(i):
            ko, vo = outs[i % 2]
            pkv.dequant(caches[i % 2], bt, ctx, k_out=ko, v_out=vo)
        kernel = "pkv_dequant (gather of every position to bf16 rows)"
    steps = max(args.steps // 10, 5)
    for i in range(max(args.warmup // 5, 2)):
        launch(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        launch(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    ms = float(np.median(times))
    achieved = (read_b + write_b) / (ms * 1e-3) / 1e9
    res = {
        "op": args.op, "workload": w.name, "quant_mode": w.quant_mode,
        "tokens": units, "bytes_read": read_b, "bytes_written": write_b,
        "ms_median": round(ms, 5), "ms_mean": round(float(np.mean(times)), 5), "launches": steps,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_record(f"{args.op}.config{args.config}.mode{w.quant_mode}"),
                     "algorithmic_bytes_per_launch": read_b + write_b, "avg_launch_ms": round(ms, 5)},
    }
    print(json.dumps(res), flush=True)


def mla_step_bytes(w):
    """Algorithmic HBM bytes of one MLA decode step: each key's int8 latent and rotary rows and their
    two fp32 scales read once (shared by all heads), the queries and outputs, the block-table entries
    and context lengths; the store reads each new token's bf16 rows and writes its codes and scales."""
    ctx = w.context_lengths.astype(np.int64)
    per_key = w.latent_dim + w.rope_dim + 8
    qo = w.batch * w.num_heads * ((w.latent_dim + w.rope_dim) * 2 + w.latent_dim * 2)
    meta = int(np.ceil(ctx / w.block_size).sum()) * 4 + w.batch * 4
    decode = int(ctx.sum()) * per_key + qo + meta
    t = int((ctx > 0).sum())
    store = t * ((w.latent_dim + w.rope_dim) * 2 + per_key)
    return decode, store


def main_mla(args):
    """The paged MLA decode step: store one new latent/rotary token per sequence, then latent
    attention of every head over the int8 cache (split partials + log-sum-exp merge), as one call
    (pkv_mla_store_decode; --separate-store: the store and the decode as two calls)."""
    import torch

    import gen
    import paged_kv_cache_c8_amd as pkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = gen.make_mla_config(args.mla)
    t = gen.gen_mla_tensors(w, device=dev)
    bt = torch.as_tensor(w.block_table, device=dev)
    ctx = torch.as_tensor(w.context_lengths, device=dev)
    prior = w.prior_lengths
    cu_ctx = w.cu_context
    pri = torch.as_tensor(np.concatenate([np.arange(cu_ctx[b], cu_ctx[b] + prior[b]) for b in range(w.batch)]),
                          device=dev)
    rows = torch.as_tensor(np.array([cu_ctx[b + 1] - 1 for b in range(w.batch)], np.int64), device=dev)
    cu_p = np.zeros(w.batch + 1, np.int32)
    cu_p[1:] = np.cumsum(prior)
    lat_new = t["latent_all"].index_select(0, rows).contiguous()
    rot_new = t["rope_all"].index_select(0, rows).contiguous()
    decode_bytes, store_bytes = mla_step_bytes(w)
    touched = decode_bytes + store_bytes
    reps = args.replicas or min(MAX_REPLICAS, max(1, int(np.ceil(3 * MALL_BYTES / touched))))
    caches = []
    for _ in range(reps):
        c = pkv.MLACache(w.num_blocks, w.block_size, device=dev)
        pkv.mla_store_c8(c, t["latent_all"].index_select(0, pri), t["rope_all"].index_select(0, pri),
                         cu_q_lens=torch.as_tensor(cu_p, device=dev), context_lengths=torch.as_tensor(prior, device=dev),
                         block_table=bt)
        caches.append(c)
    del pri
    ws_bytes = pkv.mla_decode_workspace_size(w.batch, w.num_heads, w.max_blocks_per_seq, w.block_size,
                                             args.split_tokens)
    workspace = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(t["q_latent"])
    plan = pkv.mla_decode_plan(w.batch, w.num_heads, w.max_blocks_per_seq, w.block_size, args.split_tokens)

    def store(c):
        pkv.mla_store_c8(c, lat_new, rot_new, context_lengths=ctx, block_table=bt)

    def decode(c):
        pkv.mla_decode(t["q_latent"], t["q_rope"], c, bt, ctx, w.softmax_scale, out=out, workspace=workspace,
                       split_tokens=args.split_tokens)

    fused = not args.separate_store

    def store_decode(c):
        pkv.mla_store_decode(t["q_latent"], t["q_rope"], lat_new, rot_new, c, bt, ctx, w.softmax_scale, out=out,
                             workspace=workspace, split_tokens=args.split_tokens)

    def step(c):
        if fused:
            store_decode(c)
        else:
            store(c)
            decode(c)

    for i in range(args.warmup):
        step(caches[i % reps])
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(args.steps):
        step(caches[i % reps])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        if not fused:
            store(caches[i % reps])
        evs[i][0].record()
        if fused:
            store_decode(caches[i % reps])
        else:
            decode(caches[i % reps])
        evs[i][1].record()
    torch.cuda.synchronize()
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    step_s = ms_per_step * 1e-3
    value = touched / step_s / 1e9
    call_bytes = decode_bytes + (store_bytes if fused else 0)
    achieved = call_bytes / (dec_ms * 1e-3) / 1e9
    default_plan = args.split_tokens == 0
    traffic = traffic_record(f"mla_decode.config{args.mla}") if default_plan and fused else None
    cpu = None if args.no_cpu_baseline else mla_cpu_baseline(w, t, args.cpu_seconds, touched)
    res = {
        "metric": "decode-attn HBM GB/s (% of peak) + tokens/s, int8 paged-KV GQA",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,1) bf16 latent/rotary rows and queries, random block tables)",
        "config": {
            "workload": w.name, "batch": w.batch, "num_heads": w.num_heads, "latent_dim": w.latent_dim,
            "rope_dim": w.rope_dim, "block_size": w.block_size, "sum_context": int(w.context_lengths.sum()),
            "new_tokens": w.batch, "cache_replicas": reps, "split_tokens": plan["split_tokens"],
            "num_splits": plan["num_splits"], "store": "in the decode call" if fused else "separate call",
            "parallelism": "single-gpu",
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(w.batch / step_s, 1),
        "kv_tokens_per_s": round(float(w.context_lengths.sum()) / step_s, 1),
        "bytes_per_step": touched,
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": ("pkv_mla_store_decode (new-token store + split partial, log-sum-exp merge)" if fused
                       else "pkv_mla_decode (split partial + log-sum-exp merge)"),
            "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": call_bytes, "avg_launch_ms": round(dec_ms, 5),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def main_mla_walk(args):
    """The MLA decode's cache reads alone (pkv_mla_cache_walk): the latent and rotary rows and scales
    of every key, with the decode's lane layout and two blocks in flight per wave, nothing computed;
    one workgroup per split of --split-tokens keys (default: the decode's keys per workgroup, about
    the number of workgroups its balanced partition runs).  Its rate is the read ceiling of the MLA
    decode's access pattern."""
    import torch

    import gen
    import paged_kv_cache_c8_amd as pkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = gen.make_mla_config(args.mla)
    t = gen.gen_mla_tensors(w, device=dev)
    bt = torch.as_tensor(w.block_table, device=dev)
    ctx = torch.as_tensor(w.context_lengths, device=dev)
    cu = torch.as_tensor(np.asarray(w.cu_context, np.int32), device=dev)
    read_b = int(w.context_lengths.sum()) * (w.latent_dim + w.rope_dim + 8)
    reps = args.replicas or min(MAX_REPLICAS, max(1, int(np.ceil(3 * MALL_BYTES / read_b))))
    caches = []
    for _ in range(reps):
        c = pkv.MLACache(w.num_blocks, w.block_size, device=dev)
        pkv.mla_store_c8(c, t["latent_all"], t["rope_all"], cu_q_lens=cu, context_lengths=ctx, block_table=bt)
        caches.append(c)
    del t
    split = args.split_tokens
    if split <= 0:
        plan = pkv.mla_decode_plan(w.batch, w.num_heads, w.max_blocks_per_seq, w.block_size)
        blocks = int(sum(-(-int(c) // 64) for c in w.context_lengths))
        wgs = plan["num_splits"] if plan["split_tokens"] == 0 else 512
        split = min(4096, 64 * -(-blocks // max(wgs, 1)))
    nsplit = -(-w.max_blocks_per_seq * w.block_size // split)
    outs = [torch.empty((w.batch, nsplit), dtype=torch.int32, device=dev) for _ in range(reps)]

    def launch(i):
        pkv.mla_cache_walk(caches[i % reps], bt, ctx, split, out=outs[i % reps])
    for i in range(max(args.warmup, 2)):
        launch(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    steps = max(args.steps, 5)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        launch(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    ms = float(np.median(times))
    achieved = read_b / (ms * 1e-3) / 1e9
    workgroups = int(sum(-(-int(c) // split) for c in w.context_lengths))
    res = {
        "op": "walk", "workload": w.name, "split_tokens": split, "workgroups": workgroups,
        "cache_replicas": reps, "bytes_read": read_b, "ms_median": round(ms, 5),
        "ms_mean": round(float(np.mean(times)), 5), "launches": steps,
        "roofline": {"bound": "hbm", "kernel": "pkv_mla_cache_walk (the MLA decode's cache reads only)",
                     "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_launch": read_b,
                     "avg_launch_ms": round(ms, 5)},
    }
    print(json.dumps(res), flush=True)


def mla_cpu_baseline(w, t, budget_s, touched):
    """The oracle's MLA store + fp64 latent attention on a bounded sample of the sequences, scaled to
    the whole batch by context share."""
    import torch

    import oracle

    model, ncores = cpu_info()
    nthreads = max(1, min(ncores, 16))
    bits = lambda x: x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    macs = w.context_lengths.astype(np.float64) * w.num_heads * (2 * w.latent_dim + w.rope_dim)
    est_rate = 2.0e8 * nthreads
    sel, acc = [], 0.0
    for b in range(w.batch):
        if acc + macs[b] > est_rate * budget_s / 3 and sel:
            break
        sel.append(b)
        acc += macs[b]
    cu_ctx = w.cu_context
    ctx_s = w.context_lengths[sel].astype(np.int32)
    prior_s = np.maximum(ctx_s - 1, 0).astype(np.int32)
    bt_s = np.ascontiguousarray(w.block_table[sel])
    dev = t["latent_all"].device
    pri = torch.as_tensor(np.concatenate([np.arange(cu_ctx[b], cu_ctx[b + 1] - 1) for b in sel]), device=dev)
    new = torch.as_tensor(np.array([cu_ctx[b + 1] - 1 for b in sel], np.int64), device=dev)
    hc = oracle.MLAHostCache(w.num_blocks, w.block_size, w.latent_dim, w.rope_dim)
    cu_p = np.zeros(len(sel) + 1, np.int32)
    cu_p[1:] = np.cumsum(prior_s)
    oracle.mla_store(hc, bits(t["latent_all"].index_select(0, pri)), bits(t["rope_all"].index_select(0, pri)),
                     cu_q_lens=cu_p, context_lengths=prior_s, block_table=bt_s)
    ln, rn = bits(t["latent_all"].index_select(0, new)), bits(t["rope_all"].index_select(0, new))
    sel_t = torch.as_tensor(np.array(sel, np.int64), device=dev)
    ql, qr = bits(t["q_latent"].index_select(0, sel_t)), bits(t["q_rope"].index_select(0, sel_t))
    times = []
    t_start = time.perf_counter()
    while True:
        s0 = time.perf_counter()
        oracle.mla_store(hc, ln, rn, context_lengths=ctx_s, block_table=bt_s)
        oracle.mla_decode(hc, ql, qr, bt_s, ctx_s, w.softmax_scale, nthreads=nthreads, want_f64=False)
        times.append(time.perf_counter() - s0)
        if time.perf_counter() - t_start > budget_s * 0.5 or len(times) >= 2000:
            break
    sec = float(np.median(times))
    frac = float(ctx_s.sum()) / float(w.context_lengths.sum())
    full_step = sec / frac
    return {
        "value": round(touched / full_step / 1e9, 4),
        "unit": "GB/s",
        "cores": nthreads,
        "kind": "oracle",
        "cpu_model": model,
        "host_cores_visible": ncores,
        "sample": f"{len(sel)} of {w.batch} sequences ({int(ctx_s.sum())} of {int(w.context_lengths.sum())} "
                  f"context tokens), {len(times)} timed steps of store + fp64 latent attention; scaled to the "
                  f"full batch by context share",
        "sample_step_s": round(sec, 4),
        "tokens_per_s": round(w.batch / full_step, 2),
    }


def cpu_baseline(w, t, budget_s, touched, new_tokens, window=0):
    """The oracle as it stands (plain C, fp64 attention), timed on this host's cores on a bounded
    sample of the same workload: whole steps (store of the new tokens + attention of every query)
    over as many sequences as fit in the time budget, with every core the process may use, and on
    one thread over a smaller sample."""
    import dataclasses

    import torch

    import oracle

    model, ncores = cpu_info()
    nthreads = max(1, min(ncores, 16))
    bits = lambda x: x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    g = w.num_q_heads // w.num_kv_heads
    qlen = np.maximum(w.q_lens, 1)
    macs = w.context_lengths.astype(np.float64) * w.num_kv_heads * g * qlen * 2 * w.head_dim
    seen = lambda x: x.context_lengths.astype(np.int64) - (
        np.minimum(np.maximum(x.prior_lengths.astype(np.int64) - window + 1, 0), x.context_lengths) if window > 0 else 0)
    dev = t["q"].device
    idx = lambda a: torch.as_tensor(a, device=dev)
    scale = 1.0 / np.sqrt(w.head_dim)

    def timed(threads, seconds):
        # a sample of sequences small enough for the budget (conservative multiply-add rate)
        est_rate = 2.0e8 * threads
        sel, acc = [], 0.0
        for b in range(w.batch):
            if acc + macs[b] > est_rate * seconds / 3 and sel:
                break
            sel.append(b)
            acc += macs[b]
        sel = np.array(sel)
        ws = dataclasses.replace(w, batch=len(sel), context_lengths=w.context_lengths[sel].copy(),
                                 q_lens=w.q_lens[sel].copy(), block_table=w.block_table[sel].copy())
        cu_ctx = w.cu_context
        kv_idx = np.concatenate([np.arange(cu_ctx[b], cu_ctx[b + 1]) for b in sel])
        k_all = bits(t["k_all"].index_select(0, idx(kv_idx)))
        v_all = bits(t["v_all"].index_select(0, idx(kv_idx)))
        if w.decode_only:
            qh = bits(t["q"].index_select(0, idx(sel)))
        else:
            cu_q = w.cu_q_lens
            qh = bits(t["q"].index_select(0, idx(np.concatenate([np.arange(cu_q[b], cu_q[b + 1]) for b in sel]))))
        hc = oracle.HostCache(w.quant_mode, w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        if w.quant_mode == 3:
            hc.k_scale[...] = t["k_scale"].cpu().numpy()
            hc.v_scale[...] = t["v_scale"].cpu().numpy()
        cu_s = ws.cu_context
        prior = ws.prior_lengths
        pri = np.concatenate([np.arange(cu_s[b], cu_s[b] + prior[b]) for b in range(ws.batch)]).astype(np.int64)
        new = np.concatenate([np.arange(cu_s[b] + prior[b], cu_s[b + 1]) for b in range(ws.batch)]).astype(np.int64)
        if len(pri):
            oracle.store(hc, k_all[pri], v_all[pri], cu_q_lens=ws.cu_prior.astype(np.int32), context_lengths=prior,
                         block_table=ws.block_table)
        cu = None if ws.decode_only else ws.cu_q_lens
        kn, vn = np.ascontiguousarray(k_all[new]), np.ascontiguousarray(v_all[new])
        times = []
        t_start = time.perf_counter()
        while True:
            s0 = time.perf_counter()
            oracle.store(hc, kn, vn, cu_q_lens=cu, context_lengths=ws.context_lengths, block_table=ws.block_table)
            oracle.decode(hc, qh, ws.num_q_heads, ws.block_table, ws.context_lengths, scale, cu_q_lens=cu,
                          nthreads=threads, want_f64=False, window=window)
            times.append(time.perf_counter() - s0)
            if time.perf_counter() - t_start > seconds * 0.5 or len(times) >= 2000:
                break
        sec = float(np.median(times))
        # the sample's step time scaled to the whole batch (attention work is linear in the keys seen)
        frac = float(seen(ws).sum()) / float(seen(w).sum())
        return sec, sec / frac, ws, len(times)

    sec, full_step, ws, n = timed(nthreads, budget_s * 0.75)
    sec1, full1, ws1, n1 = timed(1, budget_s * 0.25)
    return {
        "value": round(touched / full_step / 1e9, 4),
        "unit": "GB/s",
        "cores": nthreads,
        "kind": "oracle",
        "cpu_model": model,
        "host_cores_visible": ncores,
        "sample": f"{ws.batch} of {w.batch} sequences ({int(ws.context_lengths.sum())} of "
                  f"{int(w.context_lengths.sum())} context tokens), {n} timed steps of store + "
                  f"fp64 attention; scaled to the full batch by the keys the queries see",
        "sample_step_s": round(sec, 4),
        "tokens_per_s": round(new_tokens / full_step, 2),
        "value_1thread": round(touched / full1 / 1e9, 4),
        "sample_1thread": f"{ws1.batch} sequences ({int(ws1.context_lengths.sum())} context tokens), {n1} timed "
                          f"steps on one thread, scaled the same way",
        "sample_step_s_1thread": round(sec1, 4),
    }


if __name__ == "__main__":
    main()
