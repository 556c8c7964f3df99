"""Benchmark of one decode step (kv_append + paged decode attention) on one GPU.

The step is one kv_decode_step call: on bf16 pools, and on INT4 pools with one
new token per sequence, the append runs inside the attention kernel (then the
merge kernel); fp32 pools launch the append kernel first.

Prints one JSON line. A step appends one token to every sequence and runs
paged decode attention over the cache (the decode-step listing of "KV Cache는
왜 LLM 서빙의 핵심인가", section "KV Cache: O(T²)를 O(T)로"), on seeded
synthetic inputs already resident in HBM.

  value     KV-tokens/s: tokens attended per step (summed over sequences)
            divided by the measured step time
  roofline  the split attention kernel's algorithmic bytes per launch divided
            by its average launch time (HIP events on the launch stream,
            recorded around the kernel on every --event-every-th timed step:
            a record costs the stream a few microseconds), against 8 TB/s
  cpu_baseline  the oracle (fp64 C, OpenMP) on the host, on the same inputs

Consecutive steps rotate over pool replicas whose total size exceeds twice the
256 MB last-level (Infinity) cache, so a step never finds its KV there.

The default workload is the 70B-shaped decode layer (256 sequences of 2048
tokens, 64 query and 8 kv heads), the largest configuration that fits one GPU;
--workload selects the others (llama3_8b, kvquant_int4, long_shared, tiny).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PARITY_TOL = 2e-3  # max |error| of the fp32 attention output vs the fp64 oracle
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """sha256 over the source files the attention kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    for f in ("attention.hip", "device.h", "internal.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_169_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(workload: str, kernel: str = "attn_mfma_balanced"):
    """HBM bytes per dispatch of the decode kernel from the committed counter
    summary (profiles/<kernel>_<workload>_counters.md), or None when there is
    none or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    if "```json" not in text:
        return None
    block = text.split("```json", 1)[1].split("```", 1)[0]
    d = json.loads(block)
    if d.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return int(d["hbm_bytes_per_dispatch"])


def shared_prefix_groups(tables, ctx):
    """(group_start, prefix_blocks) for prefix_groups(): runs of consecutive
    sequences whose tables start with the same physical blocks as the run's
    first sequence; prefix_blocks is the shortest such common start (whole
    attended blocks only). A sequence that shares nothing is a group of one
    with no prefix."""
    B = tables.shape[0]
    full = [int(ctx[b]) // 16 for b in range(B)]
    group_start, prefix = [0], []
    b = 0
    while b < B:
        e, common = b + 1, full[b]
        while e < B:
            n = min(full[b], full[e])
            same = int((tables[b, :n] == tables[e, :n]).long().cumprod(0).sum()) if n > 0 else 0
            if same == 0:
                break
            common = min(common, same)
            e += 1
        prefix.append(common if e - b > 1 else 0)
        group_start.append(e)
        b = e
    return group_start, prefix


def unique_attended_tokens(tables, ctx) -> int:
    """Attended (physical block, slot) positions counted once: every sequence
    attends slots [0, min(16, n - 16 j)) of its logical block j, so a physical
    block contributes the largest such count over the entries that name it."""
    import torch
    best = {}
    for b in range(tables.shape[0]):
        n = int(ctx[b])
        nb = (n + 15) // 16
        ids = tables[b, :nb].tolist()
        for j, pid in enumerate(ids):
            cnt = min(16, n - 16 * j)
            if cnt > best.get(pid, 0):
                best[pid] = cnt
    return sum(best.values())


class HipEvents:
    """hipEvent_t handles through the HIP runtime (ctypes). The events only
    time work: they are created without the system-scope fence a recorded
    event otherwise performs (a cache writeback and invalidate that would add
    to every step they sit in)."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama2_70b",
                    choices=["tiny", "llama3_8b", "llama2_70b", "kvquant_int4", "long_shared"])
    ap.add_argument("--kernel", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA")
    ap.add_argument("--split", type=int, default=0, help="blocks per split, 0 = library's choice")
    ap.add_argument("--schedule", type=int, default=0, help="0 auto, 1 fixed splits, 2 balanced")
    ap.add_argument("--event-every", type=int, default=0,
                    help="record the kernel-boundary events on every E-th timed step (each record costs the "
                         "stream about a microsecond: 3-4 us per step, 1 %% of the 70B-shaped step); 1 = every "
                         "step; 0 (default): every 4th step, every 2nd when fewer than 40 steps are timed")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time budget on all host threads, and again on one thread; 0 skips it")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence: 1 is decode; k > 1 appends k tokens and runs the "
                         "multi-token (verification) attention over them")
    ap.add_argument("--shared", type=int, default=-1,
                    help="1: the shared-prefix entry point (each shared block read once per group), 0: the plain "
                         "call; -1 (default): shared for the long shared-prefix workload, plain otherwise")
    ap.add_argument("--op", default="decode", choices=["decode", "append", "quantize", "rope", "copy", "offload", "select"],
                    help="decode: the decode step (default); the others time one secondary kernel")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path has no "
              "multi-GPU mode. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import __graft_entry__
    __graft_entry__.ensure_built()
    import paged_kv_cache_169_amd as kv
    import workloads as wl

    dev = torch.device("cuda:0")
    if args.op != "decode":
        return bench_op(args, torch, kv, wl, dev)
    name = args.workload
    t_setup = time.time()
    k = args.q_len
    c = wl.workload(name, device=dev, poison=False, n_new=k if k > 1 else None)
    int4 = c.int4
    B, n_h, n_kv, D = c.batch, c.n_h, c.n_kv, c.d
    es = 4 if c.dtype == "f32" else 2
    ctx = c.ctx_lens.cpu()
    tokens_per_step = int(ctx.sum().item())

    # replicas: consecutive steps never share KV addresses in the 256 MB MALL
    probe = kv.make_desc(c.num_blocks, n_kv, D, "int4" if int4 else c.dtype, B if int4 else 0)
    pool_bytes = kv.kv_pool_required_bytes(probe)
    reps = max(2, math.ceil(2 * MALL_BYTES / pool_bytes) + 1)
    pools = []
    src = None
    if int4:
        src = kv.KVPool(c.num_blocks, n_kv, D, "bf16", device=dev)
        src.K.copy_(c.K)
        src.V.copy_(c.V)
    for r in range(reps):
        if int4:
            p = kv.KVPool(c.num_blocks, n_kv, D, "int4", max_seqs=B, device=dev)
            kv.kv_quantize_int4(p, src, c.tables, c.seq_lens)
        else:
            p = kv.KVPool(c.num_blocks, n_kv, D, c.dtype, device=dev)
            p.K.copy_(c.K)
            p.V.copy_(c.V)
        pools.append(p)
    del src
    if name == "long_shared":
        for p in pools:
            kv.rope_rerotate(p, c.chunk_blocks, 0, c.chunk_tokens, c.delta, c.rope_base, 0)
    max_ctx = int(ctx.max().item())
    opts = kv.attn_opts(split_blocks=args.split, kernel=args.kernel, schedule=args.schedule)
    shared = args.shared == 1 or (args.shared < 0 and name == "long_shared")
    groups = None
    if shared:
        # sequences that name the same physical blocks from the start of their tables
        starts, prefix = shared_prefix_groups(c.tables.cpu(), ctx)
        groups = kv.prefix_groups(starts, prefix)
        ws_bytes = kv.paged_decode_attention_shared_workspace_bytes(pools[0], B, n_h, max_ctx, groups, opts)
    else:
        ws_bytes = kv.paged_multi_token_attention_workspace_bytes(pools[0], B, n_h, k, max_ctx, opts)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((B, n_h, D) if k == 1 else (B, k, n_h, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {name}: B={B} n_h={n_h} n_kv={n_kv} d={D} dtype={'int4' if int4 else c.dtype} "
        f"tokens/step={tokens_per_step} pool={pool_bytes/1e6:.1f} MB x {reps} replicas, "
        f"workspace={ws_bytes/1e6:.2f} MB, setup {time.time()-t_setup:.1f}s")

    hip = HipEvents()
    stream = torch.cuda.current_stream()

    def step(i, events=None):
        p = pools[i % reps]
        o = opts
        if events is not None:
            o = kv.attn_opts(split_blocks=args.split, kernel=args.kernel, schedule=args.schedule, events=events)
        if shared:
            o = kv.attn_opts(split_blocks=args.split, kernel=args.kernel, schedule=args.schedule,
                             events=events) if events is not None else opts
            kv.paged_decode_attention_shared(p, c.q, out, c.tables, c.ctx_lens, c.scale, max_ctx, groups, ws, opts=o,
                                             stream=stream)
        elif c.append:
            # append + attention in one call (fused into the attention kernel on bf16 pools)
            kv.kv_decode_step(p, c.k_new, c.v_new, c.q, out, c.tables, c.seq_lens, c.scale, max_ctx, ws, opts=o,
                              stream=stream)
        else:
            kv.paged_decode_attention(p, c.q, out, c.tables, c.ctx_lens, c.scale, max_ctx, ws, opts=o, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronized on both sides
    every = args.event_every if args.event_every > 0 else (4 if args.steps >= 40 else 2)
    ev = [[hip.create() for _ in range(3)] if i % every == 0 else None for i in range(args.steps)]
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        step(i, ev[i])
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e_start.elapsed_time(e_end)
    ms_per_step = ms_total / args.steps
    ev = [e for e in ev if e is not None]
    split_ms = [hip.elapsed_ms(e[0], e[1]) for e in ev]
    merge_ms = [hip.elapsed_ms(e[1], e[2]) for e in ev]
    for e in ev:
        for x in e:
            hip.destroy(x)
    split_avg = sum(split_ms) / len(split_ms)
    merge_avg = sum(merge_ms) / len(merge_ms)
    split_sorted = sorted(split_ms)
    pct = lambda f: split_sorted[min(len(split_sorted) - 1, int(f * len(split_sorted)))] * 1e3
    copy_rate = streaming_copy_rate(torch, stream)
    read_rate, read_wg = read_ceiling(torch, kv, stream)

    # algorithmic bytes of one split-kernel launch: K and V of every attended
    # (token, kv head) once, q, the output, the block-table entries and lengths.
    # Where tables share physical blocks (the long shared-prefix workload) a
    # shared token's K and V count once: the unique bytes are what HBM must
    # deliver; the logical bytes (every sequence's tokens) are reported beside.
    nblk = ((ctx + 15) // 16)
    per_token = n_kv * (164 if int4 else 2 * D * es)
    logical_tokens = int(ctx.sum().item())
    unique_tokens = unique_attended_tokens(c.tables.cpu(), ctx.cpu())
    kv_bytes = unique_tokens * per_token
    alg_bytes = kv_bytes + k * (B * n_h * D * es + B * n_h * D * 4) + int(nblk.sum().item()) * 4 + B * 4
    logical_bytes = alg_bytes + (logical_tokens - unique_tokens) * per_token
    fused = c.append and not shared and args.kernel in (0, 2) and c.dtype == "bf16" and (not int4 or k == 1)
    if fused and not int4:  # the kernel also writes the step's new K and V rows into the pool
        alg_bytes += B * k * n_kv * 2 * D * es
        logical_bytes += B * k * n_kv * 2 * D * es
    elif fused:
        # INT4: per (sequence, kv head) the new K and V rows are read (2 x 2 d_h B)
        # and the V code row, its scale/min and the K tail row written; a token
        # that fills its block also reads the 15 other tail rows and writes the
        # block's K codes and per-channel scale/min
        fills = int(((c.seq_lens.cpu() % 16) == 15).sum().item())
        extra = B * n_kv * (2 * 2 * D + D // 2 + 4 + 2 * D) + fills * n_kv * (15 * 2 * D + 16 * D // 2 + 2 * 2 * D)
        alg_bytes += extra
        logical_bytes += extra
    achieved = alg_bytes / (split_avg * 1e-3) / 1e9
    value = tokens_per_step / (ms_per_step * 1e-3)
    traffic_bytes = None
    if args.kernel == 0 and args.split == 0 and args.schedule == 0 and k == 1:  # the counters' configuration
        traffic_bytes = profiled_traffic(name, "attn_mfma_shared_balanced" if shared else "attn_mfma_balanced")
    traffic = traffic_bytes / (split_avg * 1e-3) / 1e9 if traffic_bytes else None
    log(f"[bench] step {ms_per_step*1e3:.1f} us (wall {wall/args.steps*1e6:.1f} us), split kernel "
        f"{split_avg*1e3:.1f} us, merge {merge_avg*1e3:.1f} us, {achieved:.0f} GB/s "
        f"({100*achieved/PEAK_HBM_GBS:.1f}% of 8 TB/s), {value/1e9:.3f} G KV-tokens/s")
    log(f"[bench] achievable on this device: streaming read {read_rate:.0f} GB/s (kernel at "
        f"{100*achieved/read_rate:.1f}% of it), streaming copy {copy_rate:.0f} GB/s; kernel p10/p50/p90 "
        f"{pct(0.1):.1f}/{pct(0.5):.1f}/{pct(0.9):.1f} us")

    cpu = None
    if args.cpu_seconds > 0 and k == 1:
        import numpy as np
        import oracle
        p0 = pools[0]
        tab = c.tables.cpu().numpy()
        ctx_np = c.ctx_lens.cpu().numpy()
        qh = wl.to_host_bits(c.q)
        if int4:
            img = oracle.Q4Image(c.num_blocks, n_kv, D, B)
            for a, t in zip(img.arrays(), [p0.KQ, p0.KS, p0.KM, p0.VQ, p0.VS, p0.VM, p0.KTAIL]):
                h = t.detach().cpu().contiguous()
                a[...] = h.view(torch.int16).numpy().view(np.uint16) if h.element_size() == 2 else h.numpy()
            Kh, Vh = oracle.q4_dequant(img, tab, ctx_np)
        else:
            Kh, Vh = wl.to_host_bits(p0.K), wl.to_host_bits(p0.V)
        threads = oracle.max_threads()
        done_tokens, t_cpu, runs = 0, 0.0, 0
        ref = None
        # whole-batch oracle passes until the time budget is spent (at least one)
        while t_cpu < args.cpu_seconds or runs == 0:
            t1 = time.perf_counter()
            ref = oracle.attention(Kh, Vh, qh, tab, ctx_np, c.scale)
            t_cpu += time.perf_counter() - t1
            done_tokens += tokens_per_step
            runs += 1
        # the timed steps' output against the oracle on the same inputs, every row
        err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref))) if ref.size else 0.0
        # one thread: passes over the first sequences (a bounded sample of the
        # same workload, about a tenth of the budget per pass) until the budget
        # is spent
        per_seq = t_cpu / runs * threads / max(1, B)  # estimated one-thread seconds per sequence
        n1 = int(max(1, min(B, args.cpu_seconds / 10 / max(per_seq, 1e-9))))
        sub = slice(0, n1)
        tok1 = int(ctx_np[sub].sum())
        oracle.set_threads(1)
        done1, t1_cpu, runs1 = 0, 0.0, 0
        try:
            while t1_cpu < args.cpu_seconds or runs1 == 0:
                t1 = time.perf_counter()
                oracle.attention(Kh, Vh, qh[sub], tab[sub], ctx_np[sub], c.scale)
                t1_cpu += time.perf_counter() - t1
                done1 += tok1
                runs1 += 1
        finally:
            oracle.set_threads(threads)
        cpu = {"value": done_tokens / t_cpu, "unit": "KV-tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{runs} full pass(es) of the {name} attention ({tokens_per_step} tokens x {n_h} heads, "
                         f"fp64, OpenMP over (sequence, head)), {t_cpu:.1f} s",
               "single_thread_value": done1 / t1_cpu,
               "single_thread_sample": f"{runs1} pass(es) over the first {n1} of {B} sequences ({tok1} tokens x "
                                       f"{n_h} heads), one thread, {t1_cpu:.1f} s",
               "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
               "gpu_max_abs_err": err, "gpu_rows_checked": int(B * k * n_h), "tolerance": PARITY_TOL}
        log(f"[bench] oracle: {cpu['value']/1e6:.3f} M KV-tokens/s on {threads} threads ({runs} runs, {t_cpu:.1f}s), "
            f"{cpu['single_thread_value']/1e6:.4f} M on one thread ({runs1} runs over {n1} sequences); "
            f"GPU output vs oracle: max |err| {err:.2e} over all {B * n_h} rows")
        if not err <= PARITY_TOL:
            raise SystemExit(f"bench: GPU output differs from the oracle by {err:.3e} (> {PARITY_TOL})")

    line = {
        "metric": "paged GQA decode attention: KV-tokens/s and achieved HBM GB/s (% of peak)",
        "value": value,
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4" if int4 else c.dtype,
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "ctx": "U[512,4096]+1" if "uniform" in str(wl.WORKLOADS[name]["lens"])
                   else int(ctx.max().item()), "tokens_per_step": tokens_per_step, "n_h": n_h, "n_kv": n_kv,
                   "head_dim": D, "block_size": 16, "kernel": args.kernel, "split_blocks": args.split,
                   "schedule": args.schedule,
                   "accumulate": "f32", "pool_replicas": reps, "q_len": k, "shared_prefix_call": shared,
                   "query_tokens_per_s": B * k / (ms_per_step * 1e-3)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "traffic_bytes_per_launch": traffic_bytes,
                     "kernel": ("shared-prefix decode attention kernel (before the merge)" if shared else
                                "decode attention kernel (before the merge)" + (", append fused" if fused else "")),
                     "avg_launch_us": split_avg * 1e3,
                     "launch_us_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
                     "timed_launches": len(split_ms),
                     "merge_avg_us": merge_avg * 1e3, "alg_bytes_per_launch": alg_bytes,
                     "logical_bytes_per_launch": logical_bytes,
                     "achievable": {"read_GBps": read_rate, "frac_of_read": achieved / read_rate,
                                    "read_how": f"kv_read_probe over a 2 GiB buffer (the attention kernels' tile "
                                                f"loads, nothing written), best grid {read_wg} workgroups, "
                                                "bytes read per second",
                                    "copy_GBps": copy_rate, "frac_of_copy": achieved / copy_rate,
                                    "copy_how": "torch copy_ of a 1 GiB buffer on the same device, "
                                                "bytes read + written per second"}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def streaming_copy_rate(torch, stream, nbytes: int = 1 << 30, iters: int = 10) -> float:
    """Achievable HBM rate on this device: torch's copy between two buffers far
    larger than the caches, as bytes read + written per second."""
    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.copy_(a)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    rate = 2 * nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return rate


def read_ceiling(torch, kv, stream, nbytes: int = 2 << 30, iters: int = 10):
    """Achievable read rate on this device for the attention kernels' access
    pattern: kv_read_probe over a buffer far larger than the caches, the best
    of a few grid sizes. Returns (GB/s, workgroups)."""
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best, best_wg = 0.0, 0
    for wg in (1024, 2048, 4096, 8192):
        kv.kv_read_probe(buf, sink, wg, stream=stream)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(iters):
            kv.kv_read_probe(buf, sink, wg, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        rate = nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if rate > best:
            best, best_wg = rate, wg
    del buf
    torch.cuda.empty_cache()
    return best, best_wg


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def hold_queue(torch, launches: int) -> None:
    """Keep the GPU busy while the host enqueues the timed launches, so that
    host-side call overhead never shows up between a kernel's two events
    (a spin kernel of about 300 us per launch to come)."""
    torch.cuda._sleep(int(launches * 300e-6 * 2.4e9))


def bench_op(args, torch, kv, wl, dev):
    """Time one secondary kernel on its natural workload; one JSON line.

    append    kv_append of one token per sequence, 8B-shaped decode layer
    quantize  kv_quantize_int4 of the INT4 workload's bf16 cache
    rope      rope_rerotate of the long workload's 4096-token chunk
    copy      kv_copy_blocks of 4096 blocks of the 8B-shaped pool
    offload   kv_gather_blocks of 2048 blocks into pinned host memory, then
              kv_scatter_blocks back (host link bandwidth)
    select    kv_token_deviation over every reused token of the selection
              workload (16 requests x 8192 tokens, 8B-shaped KV); the top-k
              of each request at the 15 % floor is timed beside it
    All rates are algorithmic bytes (every byte read or written once) per
    second of the kernel's average duration (HIP events, launch stream)."""
    hip = HipEvents()
    stream = torch.cuda.current_stream()
    name = {"append": "llama3_8b", "quantize": "kvquant_int4", "rope": "long_shared", "copy": "llama3_8b",
            "offload": "llama3_8b", "select": "blend_select"}[args.op]
    c = wl.blend_workload(name, dev) if args.op == "select" else wl.workload(name, device=dev, poison=False)
    D, n_kv, B = c.d, c.n_kv, c.batch
    pool = kv.KVPool(c.num_blocks, n_kv, D, c.dtype, device=dev)
    pool.K.copy_(c.K)
    pool.V.copy_(c.V)
    extra = {}
    if args.op == "select":
        dev_out = torch.empty(c.n_rows, dtype=torch.float64, device=dev)
        fn = lambda: kv.kv_token_deviation(pool, c.tables, c.row_seq, c.row_pos, c.k_re, c.v_re, dev_out,
                                           stream=stream)
        es = 2 if c.dtype == "bf16" else 4
        # per row: recomputed K and V rows, cached K and V rows, (seq, pos), the fp64 result
        nbytes = c.n_rows * (4 * n_kv * D * es + 8 + 8)
        ratio = wl.BLEND_WORKLOADS[name]["ratio"]
        lens = (c.seg_offsets[1:] - c.seg_offsets[:-1]).tolist()
        ks = torch.tensor([kv.kv_recompute_count(ratio, n) for n in lens], dtype=torch.int32, device=dev)
        sel = torch.empty(c.n_rows, dtype=torch.int32, device=dev)
        back = lambda: kv.kv_topk_select(dev_out, c.seg_offsets, ks, sel, stream=stream)
    elif args.op == "append":
        fn = lambda: kv.kv_append(pool, c.k_new, c.v_new, c.tables, c.seq_lens, stream=stream)
        nbytes = 2 * (B * n_kv * 2 * D * 2)
    elif args.op == "quantize":
        dst = kv.KVPool(c.num_blocks, n_kv, D, "int4", max_seqs=B, device=dev)
        fn = lambda: kv.kv_quantize_int4(dst, pool, c.tables, c.seq_lens, stream=stream)
        toks = int(c.seq_lens.sum().item())
        nbytes = toks * n_kv * (2 * D * 2) + toks * n_kv * 164
    elif args.op == "rope":
        fn = lambda: kv.rope_rerotate(pool, c.chunk_blocks, 0, c.chunk_tokens, c.delta, c.rope_base, 0, stream=stream)
        nbytes = 2 * c.chunk_tokens * n_kv * D * 2
    elif args.op == "copy":
        g = torch.Generator(device="cpu").manual_seed(5)
        perm = torch.randperm(c.num_blocks, generator=g)[:8192].to(torch.int32).to(dev)
        src, dst = perm[:4096].contiguous(), perm[4096:].contiguous()
        fn = lambda: kv.kv_copy_blocks(pool, src, dst, stream=stream)
        nbytes = 2 * 4096 * kv.kv_block_bytes(pool)
    else:
        g = torch.Generator(device="cpu").manual_seed(6)
        blocks = torch.randperm(c.num_blocks, generator=g)[:2048].to(torch.int32).to(dev)
        host = torch.empty(2048 * kv.kv_block_bytes(pool), dtype=torch.uint8).pin_memory()
        fn = lambda: kv.kv_gather_blocks(pool, blocks, host, stream=stream)
        back = lambda: kv.kv_scatter_blocks(pool, blocks, host, stream=stream)
        nbytes = 2048 * kv.kv_block_bytes(pool)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(hip.create(), hip.create()) for _ in range(args.steps)]
    hold_queue(torch, args.steps)
    for a, b in evs:
        hip.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hip.hipEventRecord(a, ctypes.c_void_p(stream.cuda_stream))
        fn()
        hip.hip.hipEventRecord(b, ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    ms = sum(hip.elapsed_ms(a, b) for a, b in evs) / len(evs)
    if args.op in ("offload", "select"):
        evs2 = [(hip.create(), hip.create()) for _ in range(args.steps)]
        hold_queue(torch, args.steps)
        for a, b in evs2:
            hip.hip.hipEventRecord(a, ctypes.c_void_p(stream.cuda_stream))
            back()
            hip.hip.hipEventRecord(b, ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        ms_back = sum(hip.elapsed_ms(a, b) for a, b in evs2) / len(evs2)
        if args.op == "offload":
            extra = {"restore_avg_us": ms_back * 1e3, "restore_GBps": nbytes / (ms_back * 1e-3) / 1e9,
                     "direction_of_value": "device -> pinned host"}
        else:
            extra = {"topk_avg_us": ms_back * 1e3, "topk_segments": len(lens), "topk_k": int(ks[0].item()),
                     "rows": c.n_rows}
    rate = nbytes / (ms * 1e-3) / 1e9
    line = {"metric": f"{args.op}: algorithmic bytes per second", "value": rate, "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "avg_us": ms * 1e3, "bytes_per_launch": nbytes,
            "higher_is_better": True, "data": "synthetic", "config": {"workload": name, "op": args.op},
            "roofline": {"bound": "hbm", "achieved": rate, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": rate / PEAK_HBM_GBS}}
    line.update(extra)
    log(f"[bench] {args.op}: {ms*1e3:.1f} us per launch, {rate:.0f} GB/s" +
        (f", restore {extra['restore_avg_us']:.1f} us ({extra['restore_GBps']:.0f} GB/s)" if "restore_avg_us" in extra
         else "") + (f", top-k {extra['topk_avg_us']:.1f} us" if "topk_avg_us" in extra else ""))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
