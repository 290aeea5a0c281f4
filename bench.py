#!/usr/bin/env python3
"""Benchmark: MLA decode step on one MI355X (236B-shaped layer, batch 64 x 8192 cached tokens).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-detail]

A step is one mla_decode call: compress and append each new token, the query path with the
k_nope absorption, split-K attention over the paged latent cache, the log-sum-exp merge, the
v projection and the output projection o_proj (the layer's whole attention step).  Inputs are
seeded synthetic data already resident in HBM.

Timing protocol: W untimed warm-up steps; then K steps, each preceded (outside its timed region)
by a read of a 1 GiB buffer through the library's stream-read reference kernel, which evicts the
caches (the 256 MB Infinity Cache would otherwise hold the weights, and all of a small
workload's cache, between steps) and leaves only clean lines behind: a write-based flush leaves
up to 256 MB of dirty lines whose write-back then runs inside the next timed step (measured: a
plain 604 MB read took 172 us after a 512 MiB fill, 119 us after the read sweep).  Each step is
bracketed by HIP events on the library's stream, and the line reports the median with p10 / p90.
A second pass over the same K flushed steps records HIP events around the attention kernel
alone (an event recorded inside the step costs a few microseconds of its own, so the two are
separate passes); the dominant kernel's roofline uses that kernel's mean duration.  A third pass
times K steps back to back between two synchronisations (caches warm), reported beside it; a
fourth captures the step once in a HIP graph and replays it K times under the same flush (the
gaps between the step's kernel launches are what it removes).

One JSON line: `value` is decode tokens/s of the whole step (B / median step time); `roofline`
is the attention kernel's; `detail` holds the whole-step fractions, the other decode workloads
(Lite 32 x 4096, 128K x 64 splits, the mixed fp8 ragged batch), the chunked prefill of the mixed
workload, a stream bandwidth measured in the same run, the GPU, ROCm version, clocks and power;
`cpu_baseline` is the fp64 oracle on a bounded sample of the headline workload.
"""
import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode tokens/s + achieved HBM GB/s & MFMA TFLOP/s (% roofline), 1 GPU"
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
FLUSH_BYTES = 1 << 30
ATTN_SOURCE = os.path.join(ROOT, "mla_latent_kv_compress_amd", "csrc", "k_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_{}_traffic.json")
DETAIL_WORKLOADS = ("lite_bf16", "dsv2_128k", "dsv2_mixed_fp8")


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
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the chunked-prefill measurement reported under detail.prefill")
    p.add_argument("--no-detail", action="store_true",
                   help="skip the other decode workloads reported under detail.decode")
    p.add_argument("--no-flush", action="store_true", help="do not evict the caches between timed steps")
    return p.parse_args()


def stats(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "mean": float(a.mean()), "n": int(a.size)}


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


def smi_snapshot():
    """Current shader / memory clock and socket power as rocm-smi reports them (None if absent).

    Skipped under a profiler: its preloaded library would initialise the GPU in the child
    process before that child starts rocm-smi."""
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True, text=True,
                           timeout=30)
        data = json.loads(r.stdout)
    except Exception:
        return None
    out = {}
    for card, vals in data.items():
        if not isinstance(vals, dict):
            continue
        for k, v in vals.items():
            kl = k.lower()
            if "sclk" in kl or "mclk" in kl or "power" in kl or "fclk" in kl:
                out[k] = v
        break
    return out or None


def gpu_info(torch):
    props = torch.cuda.get_device_properties(0)
    return {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hbm_gib": round(props.total_memory / 2 ** 30, 1),
            "rocm_hip": torch.version.hip, "torch": torch.__version__}


def stream_bandwidth(torch, nbytes=4 << 30, reps=5):
    """Read bandwidth over `nbytes` (more than the caches hold, read after a sweep of another
    buffer) of the library's fastest read (non-temporal direct loads into LDS, the reference), of
    its plain read into registers, and of a torch device copy (read + write)."""
    from mla_latent_kv_compress_amd import api
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    flush = Flusher(torch)
    dst.copy_(src)
    api.stream_read(src, sink, 1)
    api.stream_read(src, sink, 0)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    cp, rd, rd0 = [], [], []
    for _ in range(reps):
        flush()
        e[0].record()
        api.stream_read(src, sink, 1)
        e[1].record()
        flush()
        e[2].record()
        api.stream_read(src, sink, 0)
        e[3].record()
        flush()
        e[4].record()
        dst.copy_(src)
        e[5].record()
        torch.cuda.synchronize()
        rd.append(e[0].elapsed_time(e[1]))
        rd0.append(e[2].elapsed_time(e[3]))
        cp.append(e[4].elapsed_time(e[5]))
    del src, dst, sink, flush
    torch.cuda.empty_cache()
    med = lambda v: sorted(v)[len(v) // 2]
    return {"read_gbps": nbytes / (med(rd) * 1e-3) / 1e9, "plain_read_gbps": nbytes / (med(rd0) * 1e-3) / 1e9,
            "copy_gbps": 2 * nbytes / (med(cp) * 1e-3) / 1e9, "bytes": nbytes,
            "method": "mla_stream_read mode 1 (non-temporal direct loads into LDS: read_gbps, the reference) and "
                      "mode 0 (plain loads into registers: plain_read_gbps), torch device copy (read + write); "
                      "median of 5, each after a 1 GiB read sweep"}


class Flusher:
    """Evicts the caches by reading FLUSH_BYTES through the stream-read kernel (clean lines only)."""

    def __init__(self, torch):
        from mla_latent_kv_compress_amd import api
        self.api = api
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def __call__(self):
        self.api.stream_read(self.buf, self.sink, 0)


def workload_work(wl, ctx):
    """Algorithmic bytes and flops of one decode step: the attention core and the whole step."""
    s = wl.shape
    B = len(ctx)
    H, D = s.num_heads, s.hidden_size
    row_bytes = {"bf16": s.row_width * 2, "fp8": s.row_width + 4, "f32": s.row_width * 4}[wl.cache_dtype]
    asz = 2 if wl.act_dtype == "bf16" else 4
    n_ctx = float(sum(int(c) for c in ctx))
    attn_bytes = n_ctx * row_bytes
    attn_flops = n_ctx * 2 * H * (2 * s.kv_lora_rank + s.qk_rope_head_dim)
    uk_uv = H * (s.qk_nope_head_dim + s.v_head_dim) * s.kv_lora_rank
    qpath = (s.q_lora_rank * D + H * s.qk_head_dim * s.q_lora_rank) if s.q_lora_rank else H * s.qk_head_dim * D
    kv_a = s.row_width * D
    o_proj = D * H * s.v_head_dim
    core_bytes = attn_bytes + uk_uv * asz
    core_flops = attn_flops + B * 2.0 * uk_uv
    step_bytes = core_bytes + (qpath + kv_a + o_proj) * asz
    step_flops = core_flops + B * 2.0 * (qpath + kv_a + o_proj)
    return dict(attn_bytes=attn_bytes, attn_flops=attn_flops, core_bytes=core_bytes, core_flops=core_flops,
                step_bytes=step_bytes, step_flops=step_flops)


def measure_decode(name, steps, warmup, flush, splits=None, keep=False):
    """Time one decode workload under the flushed per-step protocol (and back to back)."""
    import numpy as np
    import torch
    from mla_latent_kv_compress_amd import api, configs
    from mla_latent_kv_compress_amd.workload import DecodeBatch, Layer

    wl = configs.WORKLOADS[name]
    t_setup = time.perf_counter()
    layer = Layer(wl.shape, wl.act_dtype, wl.cache_dtype, out_dtype="f32", o_proj=True)
    batch = DecodeBatch(layer, wl)
    B = len(batch.hist)
    max_blocks = batch.table.shape[1]
    if splits is None:
        splits = wl.num_splits or api.decode_num_splits(layer.cfg, B, max_blocks)
    ws = torch.empty(api.decode_workspace_size(layer.cfg, B, max_blocks, splits), dtype=torch.uint8, device="cuda")
    out = torch.empty(api.out_shape(layer.cfg, layer.w, B), dtype=torch.float32, device="cuda")
    scratch = Flusher(torch) if flush else None
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    print(f"setup {setup_s:.1f} s: {name} B={B} splits={splits}", file=sys.stderr, flush=True)

    def step(events=None):
        batch.run(num_splits=splits, out=out, workspace=ws, attn_events=events)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents()
    # pass 1: whole steps, caches evicted before each (outside the events)
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        if flush:
            scratch()
        marks[i][0].record()
        step()
        marks[i][1].record()
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in marks]
    # pass 2: the attention kernel alone, HIP events on the library's stream
    pairs = [(ev.create(), ev.create()) for _ in range(steps)]
    for i in range(steps):
        if flush:
            scratch()
        step(events=pairs[i])
    torch.cuda.synchronize()
    attn_ms = [ev.elapsed_ms(a, b) for a, b in pairs]
    for e in [x for p in pairs for x in p]:
        ev.destroy(e)
    # pass 3: back to back, synchronised on both sides (caches warm between steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    b2b_ms = (time.perf_counter() - t0) * 1e3 / steps
    # pass 4: the same step captured once in a HIP graph and replayed, flushed as in pass 1
    # (the graph holds the step's kernels only; the flush runs eagerly between replays)
    graph_ms = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        gmarks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            if flush:
                scratch()
            gmarks[i][0].record()
            g.replay()
            gmarks[i][1].record()
        torch.cuda.synchronize()
        graph_ms = stats([a.elapsed_time(b) for a, b in gmarks])
        del g
    except Exception as e:                         # reported, not fatal: the eager step is the headline
        graph_ms = {"error": str(e)}

    ctx = batch.ctx.astype(np.int64)
    work = workload_work(wl, ctx)
    st, at = stats(step_ms), stats(attn_ms)
    med_s, attn_mean_s = st["median"] * 1e-3, at["mean"] * 1e-3
    bound_attn = "mfma (bf16)" if wl.cache_dtype == "fp8" else "hbm"
    res = {
        "workload": f"{name}: {wl.description}",
        "batch": B, "max_ctx": int(ctx.max()), "sum_ctx": int(ctx.sum()), "num_splits": splits,
        "cache_dtype": wl.cache_dtype, "setup_s": setup_s, "caches_evicted_between_steps": bool(flush),
        "step_ms": st, "decode_tokens_per_s": B / med_s,
        "back_to_back_ms_per_step": b2b_ms, "back_to_back_tokens_per_s": B / (b2b_ms * 1e-3),
        "graph_step_ms": graph_ms,
        "graph_tokens_per_s": (B / (graph_ms["median"] * 1e-3)) if graph_ms and "median" in graph_ms else None,
        "attn_ms": at,
        "attn_alg_bytes": work["attn_bytes"], "attn_alg_flops": work["attn_flops"],
        "attn_hbm_gbps": work["attn_bytes"] / attn_mean_s / 1e9,
        "attn_hbm_frac": work["attn_bytes"] / attn_mean_s / 1e9 / HBM_PEAK_GBPS,
        "attn_mfma_tflops": work["attn_flops"] / attn_mean_s / 1e12,
        "attn_mfma_frac": work["attn_flops"] / attn_mean_s / 1e12 / BF16_PEAK_TFLOPS,
        "attn_bound": bound_attn,
        "step_alg_bytes": work["step_bytes"], "step_alg_flops": work["step_flops"],
        "step_hbm_gbps": work["step_bytes"] / med_s / 1e9,
        "step_hbm_frac": work["step_bytes"] / med_s / 1e9 / HBM_PEAK_GBPS,
        "step_mfma_tflops": work["step_flops"] / med_s / 1e12,
        "step_mfma_frac": work["step_flops"] / med_s / 1e12 / BF16_PEAK_TFLOPS,
    }
    if keep:
        return res, (layer, batch)
    del layer, batch, ws, out, scratch
    torch.cuda.empty_cache()
    return res, None


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
    del layer, pb, ws, out
    torch.cuda.empty_cache()
    return {
        "workload": f"dsv2_mixed_fp8 prefill: {wl.prefill_seqs} x {wl.prefill_len} tokens in chunks of "
                    f"{wl.prefill_chunk}, fp8 cache",
        "ms": t * 1e3, "tokens_per_s": T / t, "passes": passes, "timing": "median of whole passes, synchronized",
        "alg_tflop": total / 1e12, "alg_tflop_by_part": {k: v / 1e12 for k, v in flops.items()},
        "mfma_tflops": total / t / 1e12, "mfma_frac": total / t / 1e12 / BF16_PEAK_TFLOPS,
        "bound": "mfma (bf16)",
    }


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


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
            "host_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"{n} of {len(batch.hist)} decode sequences (context {int(batch.ctx[0])}, all "
                      f"{s.num_heads} heads), fp64 numpy explicit form, {timed:.1f} s timed"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each MI355X holds whole "
              "sequences; see the design notes on sharding). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_latent_kv_compress_amd import api, configs

    api.lib()
    torch.cuda.set_device(0)
    wl = configs.WORKLOADS[args.workload]
    if wl.decode_batch <= 0:
        raise SystemExit(f"workload {args.workload} has no decode batch")
    flush = not args.no_flush
    smi_before = smi_snapshot()
    head, keep = measure_decode(args.workload, args.steps, args.warmup, flush, splits=args.splits,
                                keep=not args.no_cpu_baseline)
    smi_after_headline = smi_snapshot()
    B = head["batch"]

    traffic = None
    tf = TRAFFIC_FILE.format(args.workload)
    if os.path.exists(tf):
        rec = json.load(open(tf))
        src = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") == src and rec.get("splits") == head["num_splits"]:
            traffic = rec.get("bytes_per_launch")

    detail = {
        "dominant_kernel": "decode_attn_latent_kernel (split-K attention over the latent cache)",
        "headline": head,
        "gpu": gpu_info(torch),
        "clocks_power_before": smi_before,
        "clocks_power_after_headline": smi_after_headline,
    }
    try:
        detail["stream"] = stream_bandwidth(torch)
    except Exception as e:                        # measurement aid only
        detail["stream"] = {"error": str(e)}
    if not args.no_detail:
        detail["decode"] = {}
        for name in DETAIL_WORKLOADS:
            if name == args.workload:
                continue
            res, _ = measure_decode(name, min(args.steps, 20), min(args.warmup, 3), flush)
            detail["decode"][name] = res
    if not args.no_prefill:
        detail["prefill"] = prefill_measure()
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        detail["copy_calibration_bytes"] = 1 << 30
        del src, dst
    detail["clocks_power_after"] = smi_snapshot()

    achieved = head["attn_hbm_gbps"]
    stream_read = detail["stream"].get("read_gbps") if isinstance(detail.get("stream"), dict) else None
    line = {
        "metric": METRIC,
        "value": head["decode_tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["step_ms"]["median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.act_dtype,
        "data": "synthetic",
        "config": {"workload": head["workload"], "global_batch": B, "seq_len": head["max_ctx"],
                   "cache_dtype": wl.cache_dtype, "num_splits": head["num_splits"], "parallelism": "single GPU",
                   "launch": "eager", "timing": "median of per-step HIP events, caches evicted between steps"},
        "roofline": {"kernel": "decode_attn_latent_kernel", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "frac_of_measured_stream_read": (achieved / stream_read) if stream_read else None,
                     "step_frac": head["step_hbm_frac"]},
        "detail": detail,
    }
    if not args.no_cpu_baseline:
        layer, batch = keep
        line["cpu_baseline"] = cpu_baseline(layer, batch, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
