#!/usr/bin/env python3
"""Benchmark: MLA decode step on one MI355X (236B-shaped layer, batch 64 x 8192 cached tokens).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one mla_decode call: compress and append each new token, the query path with the
k_nope absorption, split-K attention over the paged bf16 latent cache, the log-sum-exp merge
and the v projection.  Inputs are seeded synthetic data already resident in HBM.  Prints one
JSON line with whole-step throughput, the roofline of the dominant kernel (the attention,
timed with HIP events recorded around it on the library's stream in a second pass over the
same K steps, since an event record drains the stream and would inflate the throughput pass)
and the fp64 CPU oracle timed on a bounded sample of the same workload.  Unless --no-prefill,
detail.prefill also reports the chunked prefill of the mixed 236B workload (4 x 4096 prompt
tokens, fp8 cache, chunks of 1024): prompt tokens/s and algorithmic MFMA TFLOP/s against the
dense bf16 peak.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode tokens/s + achieved HBM GB/s & MFMA TFLOP/s (% roofline), 1 GPU"
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
ATTN_SOURCE = os.path.join(ROOT, "mla_latent_kv_compress_amd", "csrc", "k_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_{}_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="dsv2_bf16")
    p.add_argument("--splits", type=int, default=None, help="override the number of K splits")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for the CPU sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain 1 GiB device copy (reference for hardware byte counters)")
    p.add_argument("--graph", action="store_true",
                   help="time the step as HIP-graph replays (the attention pass stays eager)")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the chunked-prefill measurement reported under detail.prefill")
    return p.parse_args()


def prefill_measure(passes=3):
    """Chunked prefill of the mixed workload (236B shape, fp8 cache: 4 prompts x 4096 tokens in
    chunks of 1024, every chunk one mla_prefill call), timed as whole passes over the chunks."""
    import numpy as np
    import torch
    from mla_latent_kv_compress_amd import configs
    from mla_latent_kv_compress_amd.workload import Layer, PrefillBatch

    wl = configs.WORKLOADS["dsv2_mixed_fp8"]
    s = wl.shape
    layer = Layer(s, wl.act_dtype, wl.cache_dtype, out_dtype="bf16")
    pb = PrefillBatch(layer, wl.prefill_seqs, wl.prefill_len, wl.prefill_chunk)
    ws = torch.empty(pb.workspace_size(), dtype=torch.uint8, device="cuda")
    out = None

    def one_pass():
        nonlocal out
        for k in range(pb.num_chunks):
            out = pb.run_chunk(k, workspace=ws, out=out)

    one_pass()                                   # warm-up (also fills the cache once)
    times = []
    for _ in range(passes):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        one_pass()
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    T, H = wl.prefill_seqs * wl.prefill_len, s.num_heads
    pairs = wl.prefill_seqs * wl.prefill_len * (wl.prefill_len + 1) / 2      # causal (query, key) pairs
    flops = {
        "q_path": 2.0 * T * (s.hidden_size * s.q_lora_rank + s.q_lora_rank * H * s.qk_head_dim),
        "kv_a": 2.0 * T * s.hidden_size * s.row_width,
        "kv_b": 2.0 * T * s.kv_lora_rank * H * (s.qk_nope_head_dim + s.v_head_dim),
        "attention": 2.0 * pairs * H * (s.qk_head_dim + s.v_head_dim),
    }
    total = sum(flops.values())
    return {
        "workload": f"dsv2_mixed_fp8 prefill: {wl.prefill_seqs} x {wl.prefill_len} tokens in chunks of "
                    f"{wl.prefill_chunk}, fp8 cache",
        "ms": t * 1e3, "tokens_per_s": T / t, "passes": passes, "timing": "median of whole passes, synchronized",
        "alg_tflop": total / 1e12, "alg_tflop_by_part": {k: v / 1e12 for k, v in flops.items()},
        "mfma_tflops": total / t / 1e12, "mfma_frac": total / t / 1e12 / BF16_PEAK_TFLOPS,
        "bound": "mfma (bf16)",
    }


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        path = "libamdhip64.so"
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]          # the runtime torch (and libmla) already use
                break
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_baseline(layer, batch, target_s):
    """The fp64 oracle's decode on whole sequences of the same workload, one at a time.

    Each sampled sequence's stored history rows are computed first (they are the cache, already
    resident for the GPU, so untimed); the timed part is the oracle's decode of that sequence's
    new token: compress + append, query path, per-head decompression and softmax attention.
    """
    import numpy as np
    import oracle
    from mla_latent_kv_compress_amd import inputs
    s = layer.shape
    d = oracle.Dims(s.hidden_size, s.num_heads, s.q_lora_rank, s.kv_lora_rank, s.qk_nope_head_dim,
                    s.qk_rope_head_dim, s.v_head_dim, s.rope_theta, s.rms_eps, s.softmax_scale)
    W = {k: v.astype(np.float64) for k, v in layer.w_host.items()}
    timed, n = 0.0, 0
    for b in range(len(batch.hist)):
        L = int(batch.hist[b])
        rows = np.empty((L, d.row_width))
        for c0 in range(0, L, 8192):
            c1 = min(L, c0 + 8192)
            x = inputs.history_hidden(s, b, c0, c1 - c0, layer.act).astype(np.float64)
            rows[c0:c1] = oracle.cache_rows(d, W, x, np.arange(c0, c1), layer.cache_dtype)[0]
        t0 = time.perf_counter()
        oracle.decode_one(d, W, batch.x_host[b].astype(np.float64), rows, layer.cache_dtype)
        timed += time.perf_counter() - t0
        n += 1
        if timed >= target_s:
            break
    return {"value": n / timed, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{n} of {len(batch.hist)} decode sequences (context {int(batch.ctx[0])}, all "
                      f"{s.num_heads} heads), fp64 numpy explicit form, {timed:.1f} s timed"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each MI355X holds whole "
              "sequences; see the design notes on sharding). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from mla_latent_kv_compress_amd import api, configs
    from mla_latent_kv_compress_amd.workload import DecodeBatch, Layer

    api.lib()
    torch.cuda.set_device(0)
    wl = configs.WORKLOADS[args.workload]
    if wl.decode_batch <= 0:
        raise SystemExit(f"workload {args.workload} has no decode batch")
    t_setup = time.perf_counter()
    layer = Layer(wl.shape, wl.act_dtype, wl.cache_dtype, out_dtype="f32")
    batch = DecodeBatch(layer, wl)
    B = len(batch.hist)
    max_blocks = batch.table.shape[1]
    splits = args.splits if args.splits is not None else (wl.num_splits or api.decode_num_splits(layer.cfg, B, max_blocks))
    ws = torch.empty(api.decode_workspace_size(layer.cfg, B, max_blocks, splits), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, wl.shape.num_heads, wl.shape.v_head_dim), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    print(f"setup {setup_s:.1f} s: {args.workload} B={B} splits={splits}", file=sys.stderr, flush=True)

    ev = HipEvents()

    def attn_pass(steps):
        """The same decode steps with HIP events recorded around the attention kernel."""
        pairs = [(ev.create(), ev.create()) for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            batch.run(num_splits=splits, out=out, workspace=ws, attn_events=pairs[i])
        torch.cuda.synchronize()
        ms = [ev.elapsed_ms(a, b) for a, b in pairs]
        for e in [x for p in pairs for x in p]:
            ev.destroy(e)
        return ms

    # Throughput pass: K plain steps (no event records: each record drains the stream for a few
    # microseconds, which would inflate the step time).
    if not args.graph:
        for _ in range(args.warmup):
            batch.run(num_splits=splits, out=out, workspace=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            batch.run(num_splits=splits, out=out, workspace=ws)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    else:
        # One decode step captured as a HIP graph.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            batch.run(num_splits=splits, out=out, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            batch.run(num_splits=splits, out=out, workspace=ws)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        del graph
    # Attention pass: the same K steps again, eager, with the kernel bracketed by HIP events on
    # the library's stream (the stream it is launched on).
    attn_ms = attn_pass(args.steps)

    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = B / (ms_per_step * 1e-3)
    s = wl.shape
    ctx = batch.ctx.astype(np.int64)
    row_bytes = s.row_width * (2 if wl.cache_dtype == "bf16" else 1) + (4 if wl.cache_dtype == "fp8" else 0)
    if wl.cache_dtype == "f32":
        row_bytes = s.row_width * 4
    attn_bytes = float(ctx.sum()) * row_bytes                      # algorithmic: each cached row once
    attn_flops = float(ctx.sum()) * 2 * s.num_heads * (2 * s.kv_lora_rank + s.qk_rope_head_dim)
    attn_avg_ms = float(np.mean(attn_ms))
    achieved = attn_bytes / (attn_avg_ms * 1e-3) / 1e9

    traffic = None
    tf = TRAFFIC_FILE.format(args.workload)
    if os.path.exists(tf):
        rec = json.load(open(tf))
        src = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") == src and rec.get("splits") == splits:
            traffic = rec.get("bytes_per_launch")

    # whole-step algorithmic bytes: cache rows + every weight matrix once (+ activations, small)
    asz = 2 if wl.act_dtype == "bf16" else 4
    H, D = s.num_heads, s.hidden_size
    w_elems = (s.row_width * D + H * (s.qk_nope_head_dim + s.v_head_dim) * s.kv_lora_rank
               + (s.q_lora_rank * D + H * s.qk_head_dim * s.q_lora_rank if s.q_lora_rank else H * s.qk_head_dim * D))
    step_bytes = attn_bytes + w_elems * asz
    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.act_dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {wl.description}", "global_batch": B,
                   "seq_len": int(ctx.max()), "cache_dtype": wl.cache_dtype, "num_splits": splits,
                   "parallelism": "single GPU", "launch": "hip_graph" if args.graph else "eager"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic},
        "detail": {
            "dominant_kernel": "decode_attn_latent_kernel (split-K attention over the latent cache)",
            "attn_avg_ms": attn_avg_ms,
            "attn_timing": "HIP events around the kernel on the library stream, second pass of the same steps",
            "attn_alg_bytes": attn_bytes,
            "attn_mfma_tflops": attn_flops / (attn_avg_ms * 1e-3) / 1e12,
            "attn_mfma_frac": attn_flops / (attn_avg_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "step_alg_bytes": step_bytes,
            "step_hbm_gbps": step_bytes / (ms_per_step * 1e-3) / 1e9,
            "step_hbm_frac": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "setup_s": setup_s,
        },
    }
    if not args.no_prefill:
        line["detail"]["prefill"] = prefill_measure()
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["detail"]["copy_calibration_bytes"] = 1 << 30
        del src, dst
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(layer, batch, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
