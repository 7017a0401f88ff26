"""Benchmark of the verify-attention hot path on one MI355X.

A step is one layer of speculative-verify attention (attn_run + attn_combine through the C ABI)
over the whole batch, cycling through independent per-layer KV caches so that no layer's cache
is still in L2/MALL when it is read again (the pages time 16 per-layer working sets under graph
replay: "DFlash2 concurrent long-context attention", section "Attention-only measurements").

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Order of a run: inputs built in HBM; the split kernel event-timed until its launch time is steady
(the GPU's clocks ramp up over the first few tens of launches after an idle moment; the first
launches' time is reported under "cold_start"), then K more event-timed launches for the roofline;
W warmup steps; exactly K timed steps (the reported value); the graph-replay protocol; streaming
probes; the other synthetic configurations (default workload only); the CPU oracle baseline.

Prints one JSON line: KV read GB/s (whole job), ms per layer, the roofline of the split kernel
(HBM bytes it must read / its event-timed duration vs 8 TB/s), ms per layer and KV GB/s of the
other synthetic configurations ("configs"), and the FP64 CPU oracle timed on a bounded sample of
the same workload. With a long-prefill workload (--workload
prefill_q8192_kv262144_hkv{1,2,4}) a step is one attn_prefill call and the line reports logical
causal TFLOP/s against the FP16 MFMA peak instead.
"""
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
DEFAULT_WORKLOAD = "verify_b8_ctx128k_gqa6_16layers"
METRIC = "KV read GB/s (% of 8 TB/s HBM) + attention ms/layer, B8 q8 D256 GQA6 128K ctx"


def counters_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"split_kernel_{workload}_counters.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("attn_kernels.hip", "attn_internal.h"):
        with open(os.path.join(ROOT, "verify_attention_e4m3_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, units_per_launch: int):
    """HBM bytes per split-kernel launch from committed rocprofv3 counters, if they were taken on
    the current kernel source; otherwise None."""
    path = counters_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return int(rec["hbm_bytes_per_dispatch"])


PROBE_GRIDS = {False: (2048, 4096, 8192), True: (512, 1024, 2048)}


def stream_read_probe(torch, dev, nbytes: int, lds: bool, reps: int = 10) -> float:
    """GB/s of a streaming-read probe (libattn_probe.so) over about nbytes of device memory: the
    register-load form (256-thread workgroups), or the LDS-DMA form the split kernel uses
    (lds=True, one wave per workgroup). The best of a few grid sizes: the probe stands for the
    read rate the part can sustain, and which grid reaches it differs between the two forms."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "verify_attention_e4m3_amd", "libattn_probe.so"))
    fn = lib.attn_probe_stream_read_lds if lds else lib.attn_probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    grids = PROBE_GRIDS[lds]
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(max(grids) * 4, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    best = None
    for grid in grids:
        n = nbytes - nbytes % (grid * 16384) if lds else nbytes     # whole 16 KB stages per wave
        if lds and n < grid * 2 * 16384:                             # at least two stages per wave
            continue
        if fn(src.data_ptr(), n, sink.data_ptr(), grid, stream) != 0:
            raise RuntimeError("stream probe launch failed")
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn(src.data_ptr(), n, sink.data_ptr(), grid, stream)
        e.record()
        torch.cuda.synchronize()
        gbs = n * reps / (s.elapsed_time(e) * 1e-3) / 1e9
        best = gbs if best is None else max(best, gbs)
    return best


def run_context(torch, dev) -> dict:
    """What the numbers were measured with: the library's SHA-256 and the device's name and CUs."""
    from verify_attention_e4m3_amd import attention as A
    h = hashlib.sha256()
    with open(A.LIB_PATH, "rb") as f:
        h.update(f.read())
    props = torch.cuda.get_device_properties(dev)
    return {"library_sha256": h.hexdigest(), "device": props.name,
            "arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count}


def host_cpu() -> dict:
    """CPU model and logical CPU count of the host the oracle baseline runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count()}


def cpu_baseline(w, case, budget_s: float = 15.0):
    """The FP64 oracle on (slot, KV head) pairs of layer 0 until about budget_s of CPU work."""
    import numpy as np
    import oracle
    from verify_attention_e4m3_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    pairs_all = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    done, t_total, bytes_total = [], 0.0, 0
    lens = case["seq_lens"].cpu().tolist()
    for pair in pairs_all:
        c = wl.host_subset(case, [pair])
        t0 = time.perf_counter()
        oracle.verify_attention(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"],
                                float(c["k_scale"][0]), float(c["v_scale"][0]), page_size=c["page_size"],
                                kv_format=c["kv_format"], pairs=[pair])
        t_total += time.perf_counter() - t0
        bytes_total += wl.kv_bytes([lens[pair[0]]], 1, w.head_dim, wl.ELEMENT_BYTES[w.kv_format])
        done.append(pair)
        if t_total >= budget_s:
            break
    return {"value": round(bytes_total / t_total / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(done)} of {len(pairs_all)} (slot, KV head) pairs of layer 0 "
                      f"({bytes_total / 1e9:.3f} GB of KV), FP64 NumPy, {t_total:.1f} s",
            "ms_per_layer_extrapolated": round(t_total / len(done) * len(pairs_all) * 1e3, 1), **host_cpu()}


FP16_MFMA_PEAK_TFLOPS = 2500.0
PREFILL_METRIC = "prefill logical causal TFLOP/s, Q8192 x KV262144 D256 GQA6, FP16 in, FP32 accumulation"


def prefill_cpu_baseline(w, c, budget_s: float = 15.0):
    """The FP64 oracle on single query tokens of the prefill (each against the keys it sees)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    qn, kn, vn = c["q"].cpu().numpy(), c["k"].cpu().numpy()[None], c["v"].cpu().numpy()[None]
    table = np.zeros((1, 1), dtype=np.int32)
    flops, t_total, done = 0, 0.0, 0
    for t in range(w.q_len - 1, -1, -997):
        L = w.kv_len - (w.q_len - 1 - t)
        t1 = time.perf_counter()
        oracle.verify_attention(qn[t][None, None], kn, vn, table, np.array([L], np.int32), 1.0, 1.0,
                                page_size=w.kv_len, kv_format="fp16")
        t_total += time.perf_counter() - t1
        flops += 4 * w.head_dim * w.num_q_heads * L
        done += 1
        if t_total > budget_s:
            break
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} query tokens x {w.num_q_heads} heads, each against its visible keys, FP64 NumPy, "
                      f"{t_total:.1f} s", **host_cpu()}


def bench_prefill(args, torch, A, wl):
    """K timed attn_prefill calls on one Q8192 x KV262144 shape (a step = one call)."""
    w = wl.PREFILL_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    c = wl.prefill_case(q_len=w.q_len, kv_len=w.kv_len, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                        head_dim=w.head_dim, seed=w.seed, device=dev)
    out = torch.empty_like(c["q"])
    flops = wl.prefill_flops(w.q_len, w.kv_len, w.num_q_heads, w.head_dim)
    steps = args.steps if args.steps_given else 10
    warmup = args.warmup if args.warmup_given else 3
    for _ in range(warmup):
        A.prefill(c["q"], c["k"], c["v"], out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        A.prefill(c["q"], c["k"], c["v"], out=out)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s_, e_ in ev:
        s_.record(stream)
        A.prefill(c["q"], c["k"], c["v"], out=out)
        e_.record(stream)
    torch.cuda.synchronize()
    kms = statistics.fmean(s_.elapsed_time(e_) for s_, e_ in ev)
    achieved = flops / (kms * 1e-3) / 1e12
    res = {
        "metric": PREFILL_METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": w.name, "q_len": w.q_len, "kv_len": w.kv_len, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "causal": True,
                   "logical_flops_per_call": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_kernel", "kernel_ms_mean": round(kms, 4)},
    }
    res["run"] = run_context(torch, c["q"].device)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = prefill_cpu_baseline(w, c)
    print(json.dumps(res))


def verify_setup(torch, A, wl, w, dev, layers=None):
    """Inputs, plan, workspace and argument blocks of one verify workload (all resident in HBM)."""
    n_layers = layers or w.layers
    cases = [wl.workload_case(w, device=dev, layer=i) for i in range(n_layers)]
    c0 = cases[0]
    plan = A.Plan(q_len=w.q_len, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                  page_size=w.page_size, max_seq_len=w.max_seq_len, max_pages_per_seq=c0["max_pages_per_seq"],
                  batch_capacity=w.batch, kv_dtype=w.kv_format, device=dev)
    ws = torch.empty(plan.workspace_bytes(w.batch) // 4, dtype=torch.float32, device=dev)
    outs = [torch.empty_like(c["q"]) for c in cases]
    arglist = [plan.make_args(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["k_scale"],
                              c["v_scale"], o, ws) for c, o in zip(cases, outs)]
    lens = [int(x) for x in c0["seq_lens"].cpu().tolist()]
    elem = wl.ELEMENT_BYTES[w.kv_format]
    return dict(w=w, cases=cases, plan=plan, ws=ws, outs=outs, args=arglist, lens=lens, elem=elem,
                kv_bytes=wl.kv_bytes(lens, w.num_kv_heads, w.head_dim, elem),
                token_heads=sum(lens) * w.num_kv_heads, stream=torch.cuda.current_stream(dev))


def step(env, i):
    """One pass of the hot path over the batch: attn_run (split kernel) then attn_combine."""
    a = env["args"][i % len(env["args"])]
    env["plan"].split(a)
    env["plan"].combine(a)


def event_split_ms(torch, env, n, first=0):
    """n steps with HIP events around every split-kernel launch, on the stream it is launched on;
    returns the split kernel's durations in ms."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        a = env["args"][(first + i) % len(env["args"])]
        ev[i][0].record(env["stream"])
        env["plan"].split(a)
        ev[i][1].record(env["stream"])
        env["plan"].combine(a)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def settled_split_ms(torch, env, k, window=16, min_windows=3, max_windows=20, tol=0.015):
    """The split kernel's per-launch duration once it is steady. After the GPU has idled (0.2 s is
    enough) its clocks ramp up over the first few tens of launches of this load, and early launches
    run up to a quarter slower; windows of event-timed launches run until two consecutive window
    means agree within tol, then k more launches are timed. Returns (k durations, cold-start record)."""
    step(env, 0)                 # the first launch also loads the kernels' code object
    torch.cuda.synchronize()
    means = []
    done = 1
    for wdx in range(max_windows):
        ms = event_split_ms(torch, env, window, first=done)
        done += window
        means.append(statistics.fmean(ms))
        if wdx + 1 >= min_windows and abs(means[-1] - means[-2]) <= tol * means[-1]:
            break
    timed = event_split_ms(torch, env, k, first=done)
    cold = {"first_window_split_ms": round(means[0], 5), "settled_split_ms": round(statistics.fmean(timed), 5),
            "launches_to_settle": done, "window": window}
    return timed, cold


def timed_region(torch, env, steps, warmup):
    """W untimed warmup steps, then exactly K steps bracketed by device synchronisation; ms per step."""
    for i in range(warmup):
        step(env, i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(env, warmup + i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def graph_protocol(torch, env, layers=None, replays=8, samples=5):
    """The pages' protocol: one graph over the per-layer working sets, `replays` replays per sample,
    median of `samples` samples; ms per layer."""
    n = layers or len(env["args"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            step(env, i)
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(samples):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(replays):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e) / (replays * n))
    del g
    return out


# The other synthetic configurations of the benchmark recipe, timed in the same process as the
# headline: (workload, label). Each cycles its own per-layer caches.
OTHER_CONFIGS = [
    ("verify_b1_ctx3297_hq6_hkv1", "B1 x 3297, q8, Hq6/Hkv1, E4M3 D256, page 1648 (latency-bound)"),
    ("verify_b4_ctx32k_gqa6", "B4 x 32768, q8, Hq24/Hkv4, E4M3 D256 (0.5 N(0,1), scales 2.0), page 1648"),
    ("verify_b16_mixed_ctx256k_page3296", "B16 mixed lengths <= 262144 (2 zero rows, 3 padded slots), q8, "
                                          "Hq24/Hkv4, E4M3 D256, page 3296"),
    ("decode_b8_ctx32k_d128_fp16_gqa4", "B8 x 32768, q1, Hq32/Hkv8 (GQA4), FP16 KV D128, page 1648"),
]


def other_configs(torch, A, wl, dev, steps=64, warmup=16):
    """ms per layer, KV GB/s and the fraction of 8 TB/s of every other synthetic configuration."""
    res = {}
    for name, label in OTHER_CONFIGS:
        w = wl.WORKLOADS[name]
        env = verify_setup(torch, A, wl, w, dev)
        split_ms, cold = settled_split_ms(torch, env, 32)
        ms = timed_region(torch, env, steps, warmup)
        graph = graph_protocol(torch, env)
        kvb = env["kv_bytes"]
        res[name] = {"label": label, "kv_bytes_per_layer": kvb, "ms_per_layer": round(ms, 5),
                     "kv_gbs": round(kvb / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(kvb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "split_ms_mean": round(statistics.fmean(split_ms), 5),
                     "graph_ms_per_layer_median": round(statistics.median(graph), 5),
                     "graph_kv_gbs": round(kvb / (statistics.median(graph) * 1e-3) / 1e9, 1),
                     "steps": steps, "warmup": warmup, "layers": len(env["args"])}
        del env
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip timing the other synthetic configurations")
    args = ap.parse_args()
    args.steps_given = any(a.startswith("--steps") for a in sys.argv[1:])
    args.warmup_given = any(a.startswith("--warmup") for a in sys.argv[1:])
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no cross-GPU step (each GPU runs its own share "
              "of requests / KV heads); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from verify_attention_e4m3_amd import attention as A
    from verify_attention_e4m3_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # All work goes to a stream of its own, as in a serving loop: torch's default stream is
    # HIP's null stream, whose implicit synchronisation with other streams costs several µs
    # per launch.
    torch.cuda.set_stream(torch.cuda.Stream(dev))
    if args.workload in wl.PREFILL_WORKLOADS:
        return bench_prefill(args, torch, A, wl)
    w = wl.WORKLOADS[args.workload]
    env = verify_setup(torch, A, wl, w, dev)
    plan, lens, kv_bytes, token_heads, elem = env["plan"], env["lens"], env["kv_bytes"], env["token_heads"], env["elem"]
    c0 = env["cases"][0]
    # split_kernel<format, row tiles per wave, KV heads per workgroup, row groups>: format 0 = E4M3
    # D256, 1 = FP16 D128, 2 = E5M2 D256, 3 = FP16 D256, 4 = E4M3 D128; 16 packed rows per tile; a
    # workgroup holds the largest group of KV heads (up to 4 for E4M3 D128, 2 otherwise) that
    # divides Hkv while the grid still covers every CU, and two row groups of half the row tiles
    # each when a grid of one-head workgroups gives each CU at most one (formats other than E4M3
    # D128, two or three row tiles; three groups of one row tile for the one-byte D256 formats at
    # three row tiles) - the library's rules.
    fmt = {"e4m3": 0 if w.head_dim == 256 else 4, "fp16": 1 if w.head_dim == 128 else 3, "e5m2": 2}[w.kv_format]
    gs = plan.info["grid_splits"]
    row_tiles = -(-plan.info["rows"] // 16)
    hp = 1
    for cand in ((4, 2) if fmt == 4 else (2,)):
        if w.num_kv_heads % cand == 0 and w.batch * (w.num_kv_heads // cand) * gs >= plan.info["num_cus"]:
            hp = cand
            break
    rg = 2 if fmt != 4 and row_tiles >= 2 and hp == 1 and w.batch * w.num_kv_heads * gs <= plan.info["num_cus"] else 1
    kernel_name = f"split_kernel<{fmt}, {-(-row_tiles // rg)}, {hp}, {rg}>"
    if rg == 2 and row_tiles == 3 and fmt in (0, 2):
        kernel_name = f"split_kernel_rg3<{fmt}>"           # three row groups, one row tile per wave

    # The split kernel's own duration for the roofline: HIP events around every split launch on its
    # stream, taken once the launch time is steady (events add dispatch gaps, so they stay out of the
    # timed region). This pass also brings the GPU's clocks to their loaded state before the timed
    # region; how slow the first launches were is reported under "cold_start".
    split_ms, cold = settled_split_ms(torch, env, args.steps)
    split_ms_mean = statistics.fmean(split_ms)
    achieved = kv_bytes / (split_ms_mean * 1e-3) / 1e9

    # Timed region: W warmup steps, then exactly K steps (split + combine per step), eager on the
    # work stream, bracketed by device synchronisation. Nothing else is enqueued in between.
    ms_per_step = timed_region(torch, env, args.steps, args.warmup)
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9

    graph = None
    if not args.no_graph:
        samples = graph_protocol(torch, env)
        graph = {"ms_per_layer_median": round(statistics.median(samples), 5),
                 "ms_per_layer_min": round(min(samples), 5), "ms_per_layer_max": round(max(samples), 5),
                 "kv_gbs_median": round(kv_bytes / (statistics.median(samples) * 1e-3) / 1e9, 1)}

        # The bounded-graph set: host selector on the CPU length hints, copies of the live batch
        # into its static buffers, one replay of its graph over all layers. Every layer uses
        # layer 0's block table and lengths here (the per-layer caches hold the same page pool),
        # as the layers of one model share their requests.
        from verify_attention_e4m3_amd.graphs import LayerCache, VerifyGraphs
        gset = VerifyGraphs(plan, [LayerCache(c["k_cache"], c["v_cache"], c["k_scale"], c["v_scale"])
                                   for c in env["cases"]], batch_sizes=(w.batch,), bank=A.WorkspaceBank())
        gset.capture()
        qs = [c["q"] for c in env["cases"]]
        _, route = gset.run(qs, c0["block_table"], c0["seq_lens"], lens)
        torch.cuda.synchronize()
        samples = []
        for _ in range(5):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(8):
                gset.run(qs, c0["block_table"], c0["seq_lens"], lens)
            e.record()
            torch.cuda.synchronize()
            samples.append(s.elapsed_time(e) / (8 * w.layers))
        graph["graph_set"] = {"route": route, "ms_per_layer_median": round(statistics.median(samples), 5),
                              "kv_gbs_median": round(kv_bytes / (statistics.median(samples) * 1e-3) / 1e9, 1)}
        del gset

    # Plain copy probe (read + write of the same byte count as one layer's KV); its rocprofv3
    # FETCH_SIZE / WRITE_SIZE readings calibrate those counters against a known byte count.
    probe_src = torch.empty(kv_bytes // 2, dtype=torch.uint8, device=dev)
    probe_dst = torch.empty_like(probe_src)
    probe_dst.copy_(probe_src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(10):
        probe_dst.copy_(probe_src)
    e.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * probe_src.numel() * 10 / (s.elapsed_time(e) * 1e-3) / 1e9
    del probe_src, probe_dst
    read_gbs = stream_read_probe(torch, dev, kv_bytes, lds=False)
    dma_gbs = stream_read_probe(torch, dev, kv_bytes, lds=True)
    traffic = measured_traffic(w.name, token_heads)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "q_len": w.q_len,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "page_size": w.page_size, "kv_format": w.kv_format, "layers": w.layers,
                   "kv_bytes_per_layer": kv_bytes, "splits_per_row": plan.splits(lens[0])[0]},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": kernel_name, "split_ms_mean": round(split_ms_mean, 5),
                     "algorithmic_bytes_per_launch": kv_bytes, "units_per_launch": token_heads,
                     "bytes_per_unit": 2 * w.head_dim * elem},
        "cold_start": cold,
        "graph_replay": graph,
        "copy_probe_gbs": round(copy_gbs, 1),
        "read_probe_gbs": round(read_gbs, 1),
        "lds_dma_read_probe_gbs": round(dma_gbs, 1) if dma_gbs else None,
        "split_frac_of_lds_dma_probe": round(achieved / dma_gbs, 4) if dma_gbs else None,
        "split_ms_p10_p50_p90": [round(x, 5) for x in statistics.quantiles(split_ms, n=10)[0::4]],
    }
    res["run"] = run_context(torch, dev)
    if not args.no_configs and w.name == DEFAULT_WORKLOAD:
        del env
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        res["configs"] = other_configs(torch, A, wl, dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, c0)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
