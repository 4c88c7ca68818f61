"""Decode-attention benchmark over JoLT-compressed KV caches on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--ratio 3x]

A step is one decode step of the workload: every layer of every sequence
(one jolt_decode_attention call per layer, all sequences batched) with the
compressed caches already resident in HBM.  The default workload is the
largest single-GPU one: the MHA shape (Llama-2-7B-like: 32 layers in 8 groups
of 4, 32 KV = 32 query heads, d=128, T=8192) with 16 sequences per decode
step and its fixed rank/bit schedule (key ranks 64..512, value ranks 512..64,
residuals of 0/2/4/8 bits; ~17 GiB compressed, 64 GiB dense per step).
Small caches are rotated over enough device copies (> 512 MiB) that a step
reads HBM, not the 256 MiB Infinity Cache.  The timed steps run twice: eagerly, with HIP events recorded by the
library around each split-kernel launch on its stream (the kernel time of the
roofline figure), and captured once into a HIP graph that is replayed (the
step time reported as `value`; --no-graph reports the eager time instead).
Prints one JSON line: compressed-context tokens/s, the dominant kernel's
roofline position, the dense decode comparator on the same shape (timed the
same way) and the CPU oracle baseline.
"""
import argparse
import ctypes as C
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_MFMA_BF16 = 2.5e15    # FLOP/s, dense bf16/fp16 MFMA
MALL_BYTES = 256 << 20


_SPIN_CYCLES_PER_MS = None


def hold_stream(ms):
    """Occupy the current stream for about ``ms`` milliseconds with torch's
    spin kernel (its cycle rate is measured once), so that launches queued
    behind it start back to back."""
    import torch
    global _SPIN_CYCLES_PER_MS
    if _SPIN_CYCLES_PER_MS is None:
        n = 1 << 20
        torch.cuda._sleep(n)  # first launch loads the kernel
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(n)
        b.record()
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS = n / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(min(ms, 5000.0) * _SPIN_CYCLES_PER_MS))


def achievable_peak(bound, dev):
    """A measured ceiling on this GPU for the roofline's bound, beside the
    published peak: a bf16 matrix product through torch.matmul (8192^3,
    hipBLASLt) for "mfma", a 1 GiB device-to-device copy (read + write
    bytes) for "hbm".  Calibration only; nothing of the decode path runs
    through it."""
    import torch
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if bound == "mfma":
        n, reps = 8192, 10
        x = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
        y = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            z = x @ y
        torch.cuda.synchronize()
        a_.record()
        for _ in range(reps):
            z = x @ y
        b_.record()
        torch.cuda.synchronize()
        del x, y, z
        return 2.0 * n ** 3 * reps / (a_.elapsed_time(b_) * 1e-3) / 1e12, \
            "torch.matmul bf16 8192x8192x8192"
    n, reps = 1 << 30, 10
    src = torch.ones(n // 2, device=dev, dtype=torch.bfloat16)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a_.record()
    for _ in range(reps):
        dst.copy_(src)
    b_.record()
    torch.cuda.synchronize()
    del src, dst
    return 2.0 * n * reps / (a_.elapsed_time(b_) * 1e-3) / 1e9, "device copy of 1 GiB (read + write)"


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its stream)."""

    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = C.c_void_p()
            assert self.hip.hipEventCreate(C.byref(e)) == 0
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        f = C.c_float()
        assert self.hip.hipEventSynchronize(C.c_void_p(b)) == 0
        assert self.hip.hipEventElapsedTime(C.byref(f), C.c_void_p(a), C.c_void_p(b)) == 0
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(C.c_void_p(e))


def load_alloc(cfg, ratio, seq=0):
    """(budget key, per-group allocation) of one sequence: the oracle
    allocator's table for this workload and budget (per sequence where the
    workload allocates each sequence on its own)."""
    path = os.path.join(ROOT, "tests", "golden", "allocations.json")
    tables = json.load(open(path))[str(cfg.idx)]["tables"]
    if "fixed" in tables:
        key = "fixed"
    elif f"{ratio}/seq{seq}" in tables:
        key = f"{ratio}/seq{seq}"
    elif ratio in tables:
        key = ratio
    else:
        raise SystemExit(f"no allocation for {cfg.name} at {ratio}: have {sorted(tables)}")
    return key.split("/")[0], [tuple(map(tuple, g)) for g in tables[key]["groups"]]


def algorithmic(cfg, alloc, layer):
    """Bytes and MFMA FLOPs of one layer call for one sequence (unpadded ranks)."""
    g = layer // cfg.group_size
    (rTk, rFk, bk), (rTv, rFv, bv) = alloc[g]
    T, H, Hq, d, sf = cfg.T, cfg.H, cfg.H_q, cfg.d, cfg.factor_bytes
    sq = 4 if cfg.q_dtype == "f32" else 2
    nbytes = (T * sf * (rTk + rTv) + H * T * (d * (bk + bv) // 8 + 4 * ((bk > 0) + (bv > 0)))
              + sf * (H * (rTk * rFk + rTv * rFv) + d * (rFk + rFv)) + sf * d * d
              + Hq * d * (sq + 4))
    flops = (T * H * (2 * rTk * rFk + 2 * (rFk + d * (bk > 0)) * d) + T * Hq * 2 * d
             + T * Hq * 2 * (rTv + d * (bv > 0)))
    return nbytes, flops


def measured_traffic(workload, kernel_name):
    """HBM bytes per launch from the committed rocprofv3 counter runs, only if
    the kernel sources are unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{workload}/{kernel_name}")
    from compressed_cache_decode_jolt_amd.profiling import kernel_hash
    if not rec or rec.get("kernel_hash") != kernel_hash():
        return None
    return rec["bytes_per_launch"]


def blas_info():
    """(threads, vendor) of the BLAS numpy uses on this host."""
    threads, vendor = len(os.sched_getaffinity(0)), "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            threads = max(i.get("num_threads", 1) for i in info)
            vendor = ",".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info}))
    except Exception:
        pass
    return int(threads), vendor


def cpu_baseline(cfg, cache, seconds):
    """The oracle decode (numpy float64) on the host cores, on a bounded
    sample of the workload: one layer call (one sequence) per layer group,
    timed separately and repeated while the time budget lasts; a group's
    time is the median of its repeats, and the step estimate sums the groups
    times their layers and the batch.  Workloads of one layer also get a
    single-core run."""
    from oracle import attention as att
    from oracle.rotation import rotation
    from workloads import gen
    threads, vendor = blas_info()
    inv = gen.rope_inv_freq_input(cfg.rope_base, cfg.d)
    Pi = rotation(cache["rotation_seed"], cfg.d)
    gstart = cache["group_start"]
    layers = [gstart[g] for g in range(len(gstart) - 1)]

    def sample(budget, min_rounds):
        times = {l: [] for l in layers}
        t0 = time.perf_counter()
        rounds = 0
        while True:
            for l in layers:
                q = gen.cfg_queries(cfg, 0, l).astype(np.float64)
                a = time.perf_counter()
                att.decode_layer(cache, l, q, cfg.T, inv, 1 / math.sqrt(cfg.d), Pi)
                times[l].append(time.perf_counter() - a)
            rounds += 1
            el = time.perf_counter() - t0
            if rounds >= min_rounds and (el >= budget or el * (rounds + 1) / rounds > 2 * budget):
                break
            if rounds >= 10:
                break
        per_group = [float(np.median(times[l])) for l in layers]
        step = sum(t * (gstart[g + 1] - gstart[g]) for g, t in enumerate(per_group)) * cfg.batch
        return step, rounds, el

    step, rounds, el = sample(seconds, 1)
    out = {"value": cfg.batch * cfg.T / step, "unit": "tokens/s", "cores": threads,
           "kind": "oracle", "blas": vendor,
           "sample": f"{rounds} round(s) of one layer call per layer group ({len(layers)} "
                     f"groups, one sequence; {el:.1f} s), median per group, scaled to a full "
                     f"step of {cfg.n_layers} layers x {cfg.batch} sequences"}
    if cfg.n_layers == 1:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                s1, r1, _ = sample(min(seconds, 10.0), 3)
            out["single_core_value"] = cfg.batch * cfg.T / s1
        except Exception:
            pass
    return out


def log(msg):
    """Progress line on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--ratio", default=None, help="byte budget, e.g. 3x (default: the "
                    "workload's first budget)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "generic", "mfma"])
    ap.add_argument("--split-tokens", type=int, default=0, help="tokens per split (0 = auto)")
    ap.add_argument("--dense-split-tokens", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0,
                    help="device copies of the caches rotated over the steps (default: enough "
                         "that a step reads HBM, not the Infinity Cache)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--deterministic", action="store_true",
                    help="fixed token-block schedule (bitwise repeatable outputs)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (default: the timed steps are also captured "
                         "in one HIP graph and replayed; value comes from the replay)")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the measured-ceiling probe reported beside the published peak")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build measures the single-GPU decode path "
              "(the multi-GPU sharding is described, not run)", file=sys.stderr)
        sys.exit(2)

    import torch
    import compressed_cache_decode_jolt_amd as J
    from workloads import gen, get_config

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}))
        return

    cfg = get_config(args.config)
    ratio = args.ratio or (f"{cfg.budgets[0]:g}x" if cfg.budgets else "fixed")
    allocs = [load_alloc(cfg, ratio, s) for s in range(cfg.batch)]
    ratio_key, alloc = allocs[0]
    kernel = {"auto": None, "generic": J.KERNEL_GENERIC, "mfma": J.KERNEL_MFMA}[args.kernel]
    B, L, H, Hq, d, T = cfg.batch, cfg.n_layers, cfg.H, cfg.H_q, cfg.d, cfg.T
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # caches: one synthetic cache per sequence, loaded `copies` times
    host = []
    for s in range(B):
        host.append(gen.synthetic_cache(cfg, allocs[s][1], seq=s))
        log(f"{cfg.name}: synthetic cache {s + 1}/{B} built")
    step_bytes = sum(algorithmic(cfg, allocs[s][1], l)[0] for s in range(B) for l in range(L))
    copies = args.copies or max(1, math.ceil(2 * MALL_BYTES / step_bytes))
    caches = []
    for c in range(copies):
        caches.append([])
        for s in range(B):
            caches[-1].append(J.jolt_load_cache(host[s]))
            if copies * B <= 64 or s == B - 1:
                log(f"cache copy {c + 1}/{copies}, sequence {s + 1}/{B} loaded")
    inv = gen.rope_inv_freq_input(cfg.rope_base, d)
    scale = 1.0 / math.sqrt(d)
    qdt = torch.bfloat16 if cfg.q_dtype == "bf16" else torch.float32
    qs = [torch.from_numpy(np.stack([gen.cfg_queries(cfg, s, l) for s in range(B)])).to(qdt).to(dev)
          for l in range(L)]
    q_pos = [T] * B
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    split = args.split_tokens
    ws_bytes = max(J.jolt_decode_workspace_size(caches[0], l, kernel=kernel, split_tokens=split)
                   for l in range(L))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    ev = HipEvents()
    n_ev = args.steps * L
    evb, eve = ev.create(n_ev), ev.create(n_ev)
    stream = torch.cuda.current_stream()

    def step(i, timed):
        cs = caches[i % copies]
        st = torch.cuda.current_stream()
        for l in range(L):
            e = (evb[(i * L + l) % n_ev], eve[(i * L + l) % n_ev]) if timed else None
            J.jolt_decode_attention(cs, l, qs[l], q_pos, inv, scale, out, ws, kernel=kernel,
                                    split_tokens=split, stream=st, events=e,
                                    deterministic=args.deterministic)

    def timed_steps(run):
        """Warm-up steps, then exactly args.steps steps between two events."""
        for i in range(args.warmup):
            run(i, False)
        torch.cuda.synchronize()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        run(None, True)
        b_.record()
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) / args.steps

    # eager: one library call per layer from Python
    def eager(i, timed):
        if i is not None:
            step(i, False)
        else:
            for k in range(args.steps):
                step(k, False)
    eager_ms = timed_steps(eager)

    # split-kernel time: the library sets each pair of HIP events to the split
    # kernel's own start and end.  The steps are queued behind a spin kernel,
    # so they run back to back as in the graph-replayed step rather than
    # after idle gaps of the Python loop.
    torch.cuda.synchronize()
    hold_stream(3.0 * eager_ms * args.steps + 1.0)
    for k in range(args.steps):
        step(k, True)
    torch.cuda.synchronize()
    split_ms = [ev.elapsed_ms(a, b) for a, b in zip(evb, eve)]
    ev.destroy(evb + eve)
    kern_ms = float(np.mean(split_ms))
    log(f"split kernel: {kern_ms * 1e3:.2f} us per launch")

    def graphed(run_step, n):
        """One HIP graph holding n steps (copies rotate as in eager mode)."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run_step(0, False)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for k in range(n):
                run_step(k, False)
        torch.cuda.synchronize()
        return g

    log(f"eager: {eager_ms:.4f} ms per step")
    ms_per_step = eager_ms
    graph_ms = None
    if not args.no_graph:
        g = graphed(step, args.steps)
        graph_ms = timed_steps(lambda i, t: g.replay() if i is None else step(i, False))
        ms_per_step = graph_ms
        del g
        log(f"graph: {graph_ms:.4f} ms per step")

    per_launch = [[algorithmic(cfg, allocs[s][1], l) for s in range(B)] for l in range(L)]
    bytes_launch = float(np.mean([sum(p[0] for p in pl) for pl in per_launch]))
    flops_launch = float(np.mean([sum(p[1] for p in pl) for pl in per_launch]))
    mfma_bound = flops_launch / PEAK_MFMA_BF16 > bytes_launch / PEAK_HBM
    kname = ("decode_mfma" if args.kernel != "generic" and cfg.factor_dtype == "bf16" and d == 128
             else "decode_generic")
    if mfma_bound:
        achieved = flops_launch / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_BF16 / 1e12,
                "unit": "TFLOP/s", "frac": achieved / (PEAK_MFMA_BF16 / 1e12)}
    else:
        achieved = bytes_launch / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": achieved / (PEAK_HBM / 1e9)}
    roof["traffic"] = measured_traffic(f"{cfg.name}@{ratio_key}", kname)
    roof["kernel_ms"] = kern_ms
    roof["alg_bytes_per_launch"] = bytes_launch
    roof["alg_flops_per_launch"] = flops_launch
    if not args.no_achievable:
        ceil, probe = achievable_peak(roof["bound"], dev)
        roof["achievable"] = {"peak": ceil, "unit": roof["unit"], "frac": achieved / ceil,
                              "probe": probe}
        log(f"achievable {roof['bound']} ceiling: {ceil:.1f} {roof['unit']} ({probe})")

    # dense comparator on the same shape (random bf16 post-RoPE K and V)
    dense = None
    if not args.no_dense:
        dense_step = 2 * B * L * H * T * d * 2
        dcopies = max(1, math.ceil(2 * MALL_BYTES / dense_step))
        g = torch.Generator(device=dev).manual_seed(0)
        kv = [[(torch.randn((B, H, T, d), generator=g, device=dev).to(torch.bfloat16),
                torch.randn((B, H, T, d), generator=g, device=dev).to(torch.bfloat16))
               for _ in range(L)] for _ in range(dcopies)]
        dsplit = args.dense_split_tokens
        dws = torch.zeros(J.jolt_dense_workspace_size(B, H, Hq, d, T, split_tokens=dsplit),
                          dtype=torch.uint8, device=dev)

        def dstep(i, timed=False):
            st = torch.cuda.current_stream()
            for l in range(L):
                k, v = kv[i % dcopies][l]
                J.jolt_dense_attention(k, v, qs[l], q_pos, inv, scale, out, dws,
                                       split_tokens=dsplit, stream=st)

        d_eager = timed_steps(lambda i, t: [dstep(k) for k in range(args.steps)]
                              if i is None else dstep(i))
        dms = d_eager
        d_graph = None
        if not args.no_graph:
            dg = graphed(dstep, args.steps)
            d_graph = timed_steps(lambda i, t: dg.replay() if i is None else dstep(i))
            dms = d_graph
            del dg
        log(f"dense: {dms:.4f} ms per step")
        dense = {"ms_per_step": dms, "eager_ms_per_step": d_eager, "graph_ms_per_step": d_graph,
                 "hbm_GBps": dense_step / (dms * 1e-3) / 1e9, "jolt_speedup": dms / ms_per_step}
        del kv

    cpu = None if args.no_cpu else cpu_baseline(cfg, host[0], args.cpu_seconds)
    value = B * T / (ms_per_step * 1e-3)
    rec = {
        "metric": "compressed-context tokens/s per decode step",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "layers": L, "kv_heads": H, "q_heads": Hq,
                   "head_dim": d, "T": T, "budget": ratio_key,
                   "allocation": [list(map(list, a)) for a in alloc[:1]] if L == 1 else ratio_key,
                   "kernel": args.kernel, "split_tokens": split, "cache_copies": copies,
                   "schedule": "fixed" if args.deterministic else "on-demand",
                   "step_alg_bytes": step_bytes},
        "timing": {"eager_ms_per_step": eager_ms, "graph_ms_per_step": graph_ms,
                   "reported": "graph" if graph_ms is not None else "eager"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "dense": dense,
        "step_hbm_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
