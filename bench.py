"""Benchmark of one PagedAttention decode step on one MI355X.

A step is the whole hot path over one batch: slot mapping, cache write of every
sequence's new token and the attention work plan (one fused launch), the attention
partition kernel, the log-sum-exp reduce.
Inputs are seeded synthetic batches already resident in HBM.  The headline is the
KV bytes the step must read (sum of context lengths x kv heads x head_dim x 2 x
element size) per second, the same figure as a fraction of the 8 TB/s HBM peak, and
sequences (tokens) per second.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--config llama3_8b]
                    [--partition-size 512] [--no-cpu-baseline]

A config named *_fp8 runs the same workload over E4M3 (8-bit float) caches: the
prologue quantises the new rows, attention decodes the codes (balanced split only).
The configs spec_verify and chunked_prefill run steps with several new tokens per
sequence (slot mapping, cache write, causal multi-token attention).

Prints one JSON line.  The fp64 CPU oracle is timed on the same batch (all of it
unless --cpu-sample-seqs says otherwise), on one host thread, repeated for about
10 s of CPU work, and its outputs are compared with the GPU's.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
# Sources the partition kernel is built from: stored traffic counters are used only
# while these are unchanged.
KERNEL_SOURCES = ("paged_attention.hip", "paged_attention_stream.hip", "pkv_device.hpp",
                  "pkv_launch.hpp", "pkv_plan.hpp", "pkv_tile.hpp", "pkv_stream.hpp")
PROFILES = os.path.join(ROOT, "profiles")


def traffic_file(kernel: str, workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_441_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel: str, workload: str, partition_size: int):
    """HBM bytes per partition-kernel launch from the committed rocprofv3 counter runs,
    or None when they were taken on other kernel sources or another workload."""
    try:
        with open(traffic_file(kernel, workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("source_sha256") != kernel_source_hash() or t.get("workload") != workload
            or t.get("partition_size") != partition_size):
        return None
    return t.get("traffic_bytes_per_launch")


METRIC = "paged-attn decode KV HBM GB/s (% of peak) and tokens/s at batch×ctx, 1 GPU"

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hip_runtime_api.h


class HipTimer:
    """HIP events created with hipEventDisableSystemFence and recorded on the launch
    stream: a timestamp only.  An event with the default flags makes the GPU write
    back and invalidate its caches when it is reached; between two kernels of a
    decode step that costs about 2.5 us per event on MI355X and counts as step time.
    The events come from the HIP runtime torch has already loaded (the one the
    library's launches use)."""

    def __init__(self, stream):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self._ct = ctypes
        self._hip = ctypes.CDLL(path)
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_uint]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._stream = ctypes.c_void_p(stream.cuda_stream)
        self._events = []

    def event(self):
        ev = self._ct.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(self._ct.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self._events.append(ev)
        return ev

    def record(self, ev):
        rc = self._hip.hipEventRecord(ev, self._stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, a, b) -> float:
        out = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def close(self):
        for ev in self._events:
            self._hip.hipEventDestroy(ev)
        self._events = []


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama3_8b")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="tokens per context partition; 0 selects the balanced split "
                         "(equal shares of the tile list per workgroup); default: the "
                         "workload's own")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=0,
                    help="sequences the CPU oracle runs on (0: the whole batch)")
    ap.add_argument("--component", default="decode",
                    choices=["decode", "copy_blocks", "prefix_cache"],
                    help="decode: the decode step (default); copy_blocks: the copy-on-write "
                         "block copy kernel alone; prefix_cache: the host pool's prefix "
                         "caching (lookup, allocation, registration, release)")
    ap.add_argument("--copy-pairs", type=int, default=4096,
                    help="block pairs per copy_blocks launch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the "
                         "known-size reference for HBM traffic counters)")
    return ap.parse_args(argv)


def copy_calibration() -> int:
    """A plain copy of known size, for scaling FETCH_SIZE / WRITE_SIZE readings."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": 3}), flush=True)
    return 0


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main(argv=None) -> int:
    args = parse(argv)
    if args.copy_calibration:
        return copy_calibration()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the decode path "
                                   "has no multi-GPU mode (use --gpus 1)"}))
        return 2
    if args.component == "copy_blocks":
        return bench_copy_blocks(args)
    if args.component == "prefix_cache":
        return bench_prefix_cache(args)
    from workloads import MULTI_CONFIGS
    if args.config in MULTI_CONFIGS:
        return bench_multi(args)

    import torch
    import paged_kv_cache_441_amd as pkv
    from workloads import FP8_CONFIGS, make_config, make_fp8_config

    fp8 = args.config in FP8_CONFIGS
    if fp8 and args.partition_size not in (None, 0):
        print(json.dumps({"error": "E4M3 caches run the balanced split only (partition size 0)"}))
        return 2
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    pkv.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t_gen = time.perf_counter()
    b = make_fp8_config(args.config, device=dev) if fp8 else make_config(args.config, device=dev)
    spec = b.spec
    P = spec.partition_size if args.partition_size is None else args.partition_size
    ks, vs = b.extra.get("k_scale"), b.extra.get("v_scale")
    B, H, Hkv, D, BS, NB = (b.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim,
                            spec.block_size, spec.num_blocks)
    MB = b.max_blocks_per_seq
    bt = torch.as_tensor(b.block_tables, device=dev)
    cl = torch.as_tensor(b.context_lens, device=dev)
    kc, vc = b.key_cache, b.value_cache
    out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    slots = torch.empty(B, dtype=torch.int32, device=dev)
    ws = pkv.alloc_workspace(b.query, bt, BS, P)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen

    # The step's arguments are checked once; each stage is then one C call, so the
    # host stays ahead of the GPU and the events time the kernels, not the host.
    ds = pkv.DecodeStep(b.query, b.key, b.value, kc, vc, bt, cl, b.scale, P, out=out,
                        workspace=ws, slot_mapping=slots, k_scale=ks, v_scale=vs)

    # Fence-free HIP events (see HipTimer).  Each still costs about 1.7 us of GPU time
    # on MI355X, so the timed steps carry only the two around the attention kernel
    # (the roofline's duration); the per-stage breakdown, with events between every
    # stage, runs in a pass of its own after the timed one.
    timer = HipTimer(torch.cuda.current_stream(dev))

    def step(ev=None):
        ds.prologue()
        if ev is not None:
            timer.record(ev[0])
        ds.partition()
        if ev is not None:
            timer.record(ev[1])
        ds.reduce()

    def step_staged(ev):
        timer.record(ev[0])
        ds.prologue()
        timer.record(ev[1])
        ds.partition()
        timer.record(ev[2])
        ds.reduce()
        timer.record(ev[3])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    events = [[timer.event() for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    t_part = np.array([timer.ms(e[0], e[1]) for e in events])

    staged = [[timer.event() for _ in range(4)] for _ in range(K)]
    for k in range(K):
        step_staged(staged[k])
    torch.cuda.synchronize()
    t_write = np.array([timer.ms(e[0], e[1]) for e in staged])
    t_red = np.array([timer.ms(e[2], e[3]) for e in staged])
    t_gpu = np.array([timer.ms(e[0], e[3]) for e in staged])
    timer.close()

    kv_bytes = b.kv_bytes()
    # fixed partitions run in the same streaming kernel (one workgroup per partition);
    # stored traffic counters exist for the balanced split only
    kernel = "paged_attention_stream"
    tokens = int(b.context_lens.astype(np.int64).sum())
    step_s = ms_step / 1e3
    kv_gbs_step = kv_bytes / step_s / 1e9
    part_ms = float(t_part.mean())
    part_gbs = kv_bytes / (part_ms / 1e3) / 1e9
    attn_ms = float(t_part.mean()) + float(t_red.mean())

    result = {
        "metric": METRIC,
        "value": round(kv_gbs_step, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "fp8": "fp8_e4m3"}[spec.kv_dtype],
        "data": "synthetic",
        "config": {
            "workload": spec.name,
            "num_seqs": B, "num_heads": H, "num_kv_heads": Hkv, "head_dim": D,
            "block_size": BS, "num_blocks": NB, "max_blocks_per_seq": MB,
            "partition_size": P, "kv_dtype": spec.kv_dtype, "accumulate": "f32",
            "out_dtype": "f32", "context": str(spec.ctx),
            **({"query_dtype": "bf16", "k_scale": ks, "v_scale": vs} if fp8 else {}),
            "context_sum": tokens, "context_mean": round(tokens / B, 1),
            "context_max": int(b.context_lens.max()), "seed": spec.seed,
        },
        "pct_of_peak": round(100.0 * kv_gbs_step / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(B / step_s, 1),
        "tokens_per_s_32_layers": round(B / (32 * step_s), 1),
        "kv_bytes_per_step": kv_bytes,
        "attention_kv_gbs": round(kv_bytes / (attn_ms / 1e3) / 1e9, 1),
        "kernel_ms": {
            "decode_prologue (slot mapping, cache write, plan)": round(float(t_write.mean()), 5),
            "attention_partition": round(part_ms, 5),
            "attention_reduce": round(float(t_red.mean()), 5),
            "step_events (stage pass, four events per step)": round(float(t_gpu.mean()), 5),
            "attention_partition_p10_p50_p90": [round(float(x), 5) for x in
                                                np.percentile(t_part, [10, 50, 90])],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"{kernel}_kernel" + (f" (fixed {P}-token partitions)" if P else ""),
            "achieved": round(part_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(part_gbs / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(kernel, spec.name, P),
            "traffic_unit": "bytes per launch (FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000, "
                            "factors from a plain 1 GiB copy)",
        },
        "device": torch.cuda.get_device_name(dev),
        "cu_count": torch.cuda.get_device_properties(dev).multi_processor_count,
        "input_generation_s": round(gen_s, 2),
    }

    # ---- CPU oracle on a bounded sample, and a parity spot check -----------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(b, out, args.cpu_sample_seqs)

    print(json.dumps(result), flush=True)
    return 0


def _prefix_requests(n, seed=11):
    """Synthetic arrivals: 64 system prompts of 512 tokens (popularity falling as 1/k)
    plus unique suffixes of 16..512 tokens, vocabulary 32000."""
    rng = np.random.default_rng(seed)
    systems = rng.integers(0, 32000, (64, 512)).astype(np.int32)
    w = 1.0 / np.arange(1, 65)
    pick = rng.choice(64, size=n, p=w / w.sum())
    lens = rng.integers(16, 513, n)
    return [np.concatenate([systems[k], rng.integers(0, 32000, m).astype(np.int32)])
            for k, m in zip(pick, lens)]


def bench_prefix_cache(args) -> int:
    """The host pool with prefix caching, on the Llama-3-8B-shaped pool (200,000 blocks of
    16 tokens): each request looks up its prompt, allocates the rest, registers its
    full blocks; 256 requests are live at a time (the oldest leaves).  No GPU work."""
    import paged_kv_cache_441_amd as pkv
    from collections import deque

    BS, NB, LIVE = 16, 200_000, 256
    reqs = _prefix_requests(max(args.steps, 1) * 100)
    pool = pkv.BlockPool(NB)
    live = deque()
    hits = blocks = 0

    def run(rs):
        nonlocal hits, blocks
        for toks in rs:
            h = pool.match_prefix(toks, BS)
            need = -(-len(toks) // BS) - len(h)
            table = h + [pool.allocate() for _ in range(need)]
            pool.register_prefix(toks, table, BS)
            hits += len(h)
            blocks += len(table)
            live.append(table)
            if len(live) > LIVE:
                pool.release(live.popleft())

    w = min(len(reqs) // 10, 500)
    run(reqs[:w])
    hits = blocks = 0
    t0 = time.perf_counter()
    run(reqs[w:])
    dt = time.perf_counter() - t0
    n = len(reqs) - w
    tokens = int(sum(len(t) for t in reqs[w:]))
    # the oracle, untuned, on the first requests of the same stream (about 10 s)
    from oracle import prefix_cache as opc
    ora = opc.PrefixCachingPool(NB)
    olive = deque()
    t1, m = time.perf_counter(), 0
    for toks in reqs:
        if time.perf_counter() - t1 > 10.0:
            break
        tl = toks.tolist()
        h = ora.match_prefix(tl, BS)
        table = h + [ora.allocate() for _ in range(-(-len(tl) // BS) - len(h))]
        ora.register(tl, table, BS)
        olive.append(table)
        if len(olive) > LIVE:
            ora.release_table(olive.popleft())
        m += 1
    odt = time.perf_counter() - t1
    print(json.dumps({
        "metric": "prefix-cache requests/s on the host pool (lookup, allocate, register, "
                  "release)",
        "value": round(n / dt, 1), "unit": "requests/s", "n_gpus": 0, "steps": n,
        "warmup": w, "ms_per_step": round(dt * 1e3 / n, 5), "higher_is_better": True,
        "dtype": "int32 tokens, uint64 hashes", "data": "synthetic",
        "config": {"workload": "prefix_cache", "block_size": BS, "num_blocks": NB,
                   "live_requests": LIVE, "system_prompts": 64, "system_prompt_tokens": 512,
                   "suffix_tokens": [16, 512]},
        "tokens_per_s": round(tokens / dt, 1), "hit_blocks_fraction": round(hits / blocks, 4),
        "roofline": None,
        "roofline_note": "host C++ called per request through the ctypes binding; no GPU kernel",
        "cpu_baseline": {"value": round(m / odt, 1), "unit": "requests/s", "cores": 1,
                         "kind": "oracle",
                         "sample": f"the first {m} requests of the same stream, one thread"},
    }), flush=True)
    return 0


def bench_copy_blocks(args) -> int:
    """The copy-on-write block copy on the workload's pool: --copy-pairs disjoint
    (src, dst) pairs of random blocks per launch; bytes = pairs x block bytes x 2
    caches, read and written."""
    import torch
    import paged_kv_cache_441_amd as pkv
    from workloads import CONFIGS

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    pkv.load_library()
    spec = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if spec.kv_dtype == "bf16" else torch.float32
    shape = (spec.num_blocks, spec.block_size, spec.num_kv_heads, spec.head_dim)
    kc = torch.zeros(shape, dtype=dt, device=dev)
    vc = torch.zeros(shape, dtype=dt, device=dev)
    n = min(args.copy_pairs, spec.num_blocks // 2)
    perm = np.random.default_rng(spec.seed).permutation(spec.num_blocks)
    pairs = torch.as_tensor(np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int32), device=dev)
    for _ in range(args.warmup):
        pkv.copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    timer = HipTimer(torch.cuda.current_stream(dev))
    ev = [timer.event() for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        timer.record(ev[k])
        pkv.copy_blocks(kc, vc, pairs)
    timer.record(ev[-1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t = np.array([timer.ms(ev[k], ev[k + 1]) for k in range(args.steps)])
    timer.close()
    block_bytes = kc[0].numel() * kc.element_size()
    moved = n * block_bytes * 2 * 2
    gbs = moved / (float(t.mean()) / 1e3) / 1e9
    print(json.dumps({
        "metric": "copy_blocks HBM GB/s (bytes read + written)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "dtype": spec.kv_dtype, "data": "synthetic",
        "config": {"workload": spec.name, "pairs": n, "block_bytes": block_bytes},
        "kernel_ms": round(float(t.mean()), 5),
        "roofline": {"bound": "hbm", "kernel": "copy_blocks_kernel", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
    }), flush=True)
    return 0


FP32_MATRIX_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix peak
BF16_MATRIX_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def bench_multi(args) -> int:
    """Steps with several new tokens per sequence: slot mapping, cache write, causal
    multi-token attention (plan, attention kernel and merge in one library call)."""
    import torch
    import paged_kv_cache_441_amd as pkv
    from workloads import make_multi_config

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    pkv.load_library()
    dev = torch.device("cuda:0")
    b = make_multi_config(args.config, device=dev)
    spec = b.spec
    B, H, Hkv, D, BS, NB = (b.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim,
                            spec.block_size, spec.num_blocks)
    qsl_np = b.extra["query_start_loc"]
    T = int(qsl_np[-1])
    bt = torch.as_tensor(b.block_tables, device=dev)
    cl = torch.as_tensor(b.context_lens, device=dev)
    qsl = torch.as_tensor(qsl_np, device=dev)
    kc, vc = b.key_cache, b.value_cache
    out = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    slots = torch.empty(T, dtype=torch.int32, device=dev)
    ws = torch.empty(pkv.multi_query_workspace_bytes(B, T, H, Hkv, D, BS, bt.shape[1]),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    timer = HipTimer(torch.cuda.current_stream(dev))

    def step(ev=None):
        if ev is not None:
            timer.record(ev[0])
        pkv.slot_mapping_multi_query(bt, cl, qsl, T, BS, NB, out=slots)
        pkv.kv_cache_write(b.key, b.value, kc, vc, slots)
        if ev is not None:
            timer.record(ev[1])
        pkv.paged_attention_multi_query(b.query, kc, vc, bt, cl, qsl, b.scale, out=out,
                                        workspace=ws)
        if ev is not None:
            timer.record(ev[2])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    events = [[timer.event() for _ in range(3)] for _ in range(K)]
    t0 = time.perf_counter()
    for k in range(K):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    t_write = np.array([timer.ms(e[0], e[1]) for e in events])
    t_attn = np.array([timer.ms(e[1], e[2]) for e in events])
    timer.close()
    attn_s = float(t_attn.mean()) / 1e3
    elem = {"bf16": 2, "f32": 4}[spec.kv_dtype]
    ctx = b.context_lens.astype(np.int64)
    ql = b.extra["query_lens"].astype(np.int64)
    kv_bytes = int(ctx.sum()) * Hkv * D * 2 * elem
    # causal: new token j of sequence i sees ctx - q_len + j + 1 positions
    seen = sum(int((c - q) * q + q * (q + 1) // 2) for c, q in zip(ctx, ql))
    flops = 4 * H * D * seen               # Q.K^T and P.V, 2 flops per product each
    pv_flops = flops // 2
    gbs = kv_bytes / attn_s / 1e9
    tflops = flops / attn_s / 1e12
    pv_tflops = pv_flops / attn_s / 1e12
    hbm_bound = args.config != "chunked_prefill"
    # The matrix-bound case is priced on the algorithmic causal flops (Q.K^T and P.V)
    # against the dense peak of the operand type: bf16 caches run both products on bf16
    # matrix instructions (P.V as two products, P split into bf16 hi + lo parts, not
    # counted twice), fp32 caches on fp32 ones.
    mpeak = BF16_MATRIX_PEAK_TFLOPS if spec.kv_dtype == "bf16" else FP32_MATRIX_PEAK_TFLOPS
    roof = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4)} if hbm_bound else
            {"bound": "mfma", "achieved": round(tflops, 2), "peak": mpeak,
             "unit": "TFLOP/s", "frac": round(tflops / mpeak, 4),
             "contraction": f"Q.K^T and P.V, {spec.kv_dtype} operands, fp32 accumulation"})
    roof.update({"kernel": "paged_attention_multi_query (plan + attention + merge)",
                 "traffic": None})
    result = {
        "metric": "multi-token step: KV GB/s, TFLOP/s and new tokens/s, 1 GPU",
        "value": round(gbs, 1) if hbm_bound else round(tflops, 2),
        "unit": "GB/s" if hbm_bound else "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec.kv_dtype, "data": "synthetic",
        "config": {"workload": args.config, "num_seqs": B, "num_new_tokens": T,
                   "num_heads": H, "num_kv_heads": Hkv, "head_dim": D, "block_size": BS,
                   "context_sum": int(ctx.sum()), "query_lens": sorted(set(ql.tolist())),
                   "kv_dtype": spec.kv_dtype, "accumulate": "f32"},
        "kv_bytes_per_step": kv_bytes, "causal_flops_per_step": flops,
        "kv_gbs": round(gbs, 1), "tflops": round(tflops, 2), "pv_tflops": round(pv_tflops, 2),
        "new_tokens_per_s": round(T / (ms_step / 1e3), 1),
        "kernel_ms": {"slot mapping + cache write": round(float(t_write.mean()), 5),
                      "attention (plan + kernel + merge)": round(float(t_attn.mean()), 5)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline_multi(b, out)
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline_multi(b, gpu_out, min_seconds=10.0):
    """The oracle, untuned, on one host thread, over whole sequences of the batch taken
    in order until about ``min_seconds`` of CPU work; rate in new tokens per second."""
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import multi_query as omq

    qsl = b.extra["query_start_loc"]
    done, secs, tokens, err = [], 0.0, 0, 0.0
    with threadpool_limits(limits=1):
        for i in range(b.num_seqs):
            if secs >= min_seconds:
                break
            bt = b.block_tables[[i]]
            ids = np.unique(bt[bt >= 0])
            idx = torch.as_tensor(ids.astype(np.int64), device=b.key_cache.device)
            kc = b.numpy_storage(b.key_cache.index_select(0, idx))
            vc = b.numpy_storage(b.value_cache.index_select(0, idx))
            cbt = np.where(bt >= 0, np.searchsorted(ids, np.maximum(bt, 0)), -1).astype(np.int32)
            q0, q1 = int(qsl[i]), int(qsl[i + 1])
            t0 = time.perf_counter()
            _, _, _, ref = omq.multi_query_step(
                b.numpy_storage(b.query)[q0:q1], b.numpy_storage(b.key)[q0:q1],
                b.numpy_storage(b.value)[q0:q1], kc, vc, cbt, b.context_lens[[i]],
                np.array([0, q1 - q0]), b.scale, b.kv_dtype)
            secs += time.perf_counter() - t0
            tokens += q1 - q0
            done.append(i)
            g = gpu_out[q0:q1].float().cpu().numpy().astype(np.float64)
            err = max(err, float(np.abs(g - ref).max()))
    base = {"value": round(tokens / secs, 2), "unit": "new tokens/s", "cores": 1,
            "kind": "oracle", "cpu_model": cpu_model(), "seconds": round(secs, 2),
            "sample": f"the first {len(done)} of {b.num_seqs} sequences ({tokens} new tokens): "
                      "slot mapping, cache write and fp64 causal attention for all heads, one "
                      "host thread"}
    parity = {"tokens": tokens, "max_abs_err_vs_oracle": err, "tolerance": 2e-3,
              "ok": bool(err <= 2e-3)}
    return base, parity


def cpu_baseline(b, gpu_out, n_sample, min_seconds=10.0, max_reps=20):
    """The oracle, untuned, on one host thread: slot mapping, cache write and fp64
    attention over the first ``n_sample`` sequences of the batch (all of them by
    default), repeated until about ``min_seconds`` of CPU work have run.  The rate
    is the median repetition's."""
    import torch
    from threadpoolctl import threadpool_limits

    import oracle

    B = b.num_seqs
    n = min(B, n_sample) if n_sample else B
    bt = b.block_tables[:n]
    ids = np.unique(bt[bt >= 0])
    idx = torch.as_tensor(ids.astype(np.int64), device=b.key_cache.device)
    kc = b.numpy_storage(b.key_cache.index_select(0, idx))
    vc = b.numpy_storage(b.value_cache.index_select(0, idx))
    tables = np.where(bt >= 0, np.searchsorted(ids, np.maximum(bt, 0)), -1).astype(np.int32)
    q = b.numpy_storage(b.query)[:n]
    k = b.numpy_storage(b.key)[:n]
    v = b.numpy_storage(b.value)[:n]
    ctx = b.context_lens[:n]
    fp8 = b.kv_dtype == "fp8"

    def run():
        if not fp8:
            return oracle.decode_step(q, k, v, kc, vc, tables, ctx, b.scale, b.kv_dtype)[3]
        from oracle import fp8 as of8
        ks, vs = b.extra["k_scale"], b.extra["v_scale"]
        slots = oracle.slot_mapping(tables, ctx, b.spec.block_size)
        kc2, vc2 = of8.cache_write_fp8(kc, vc, oracle.bf16_bits_to_f64(k),
                                       oracle.bf16_bits_to_f64(v), slots, b.spec.block_size,
                                       ks, vs)
        return of8.paged_attention_decode_fp8(oracle.bf16_bits_to_f64(q), kc2, vc2, tables, ctx,
                                              b.scale, ks, vs)

    times = []
    with threadpool_limits(limits=1):
        while len(times) < max_reps and sum(times) < min_seconds:
            t0 = time.perf_counter()
            ref = run()
            times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    sample_kv = int(ctx.astype(np.int64).sum()) * b.spec.num_kv_heads * b.spec.head_dim * 2 * \
        {"bf16": 2, "f32": 4, "fp8": 1}[b.kv_dtype]
    g = gpu_out[:n].float().cpu().numpy().astype(np.float64)
    err = float(np.abs(g - ref).max())
    what = "the whole batch" if n == B else f"the first {n} of {B} sequences"
    base = {
        "value": round(sample_kv / dt / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(n / dt, 2),
        "seconds_per_rep": round(dt, 3),
        "reps": len(times),
        "cpu_seconds_total": round(sum(times), 2),
        "cores": 1,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "host_cpus_visible": len(os.sched_getaffinity(0)),
        "sample": f"{what} ({n} sequences, {int(ctx.sum())} context tokens): slot mapping, "
                  f"cache write and fp64 attention for all {b.spec.num_heads} heads, "
                  f"{len(times)} repetitions on one host thread; median repetition",
    }
    parity = {"sequences": n, "max_abs_err_vs_oracle": err, "tolerance": 2e-3,
              "ok": bool(err <= 2e-3)}
    return base, parity


if __name__ == "__main__":
    sys.exit(main())
