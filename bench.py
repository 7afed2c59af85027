"""Benchmark: fused chunked top-K KL loss, forward + backward, on one MI355X.

A step is one pass of the whole path over one batch:
  - the fused forward: loss, lse, the per-row KL and the gathered top-K logits;
  - the fused backward: recompute, gradient tile, dH and dW.
The workload is the gpt-oss-120b LM head: N = 32768 rows (B = 1, S = 32768), d = 2880,
V = 201,088, K = 100 cached teacher entries per row, chunk 2048, T = 1. Inputs are seeded
synthetic bf16, resident in HBM before timing starts.

Prints one JSON line. Along with the throughput it carries:
  - roofline: for the kernel with the largest share of the step, measured with the library's
    per-launch HIP events on its stream, and its HBM bytes from the committed counter summary;
  - cpu_baseline: the fp64 oracle timed on the host on a bounded slice of rows;
  - formulations: time and peak device memory of the same step through the other three
    formulations (single pass, forward-chunked, dense), the frozen-head and memory-lean fused
    backward, and the autograd term with an fp32 dW accumulator, on the same inputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config gptoss] [--chunk C]
       [--no-cpu-baseline] [--no-dense] [--no-formulations] [--low-memory]
       python bench.py --sweep   (per-config timings and the peak-memory sweep over S; not the
                                  headline line)
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused chunked KL fwd+bwd tokens/s at V=201088,d=2880; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="gptoss")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--rows", type=int, default=0, help="override N (default: the config's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-formulations", action="store_true",
                    help="skip timing the single-pass and forward-chunked formulations")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="rows of the workload the oracle is timed on, three times (about 20 s on 16 host threads)")
    ap.add_argument("--sweep", action="store_true",
                    help="time the fused path at every timed config (small, the Qwen-like head over its "
                         "chunk sweep, gpt-oss, the pages' full shape) and sweep S for peak memory")
    ap.add_argument("--low-memory", action="store_true",
                    help="time the fused step with the memory-lean backward (KD_LOW_MEMORY) as the step "
                         "(for its kernel trace; the default step is the headline)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 1 GiB device-to-device once (reference for the HBM byte counters)")
    ap.add_argument("--producer", action="store_true",
                    help="only time the top-K cache producer on the config's logits shape")
    return ap.parse_args()


def producer(dev, stream, N: int, V: int, K: int, seed: int, reps: int = 5) -> dict:
    """The offline top-K cache producer on teacher logits of the workload's shape: seeded
    synthetic bf16 rows N(0, 4), K = the cache width. HBM-bound; reported against one read of
    the logits, as the median of `reps` timed calls after one untimed call."""
    import statistics

    import torch

    import lm_head_kl_amd as kd

    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    tl = torch.empty((N, V), dtype=torch.bfloat16, device=dev)
    for r0 in range(0, N, 4096):
        tl[r0:r0 + 4096] = (torch.randn((min(4096, N - r0), V), generator=gen, device=dev) * 2.0).to(torch.bfloat16)
    kd.topk_cache(tl, K)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        kd.topk_cache(tl, K)
        e[1].record(stream)
        torch.cuda.synchronize()
        times.append(e[0].elapsed_time(e[1]))
    del tl
    ms = statistics.median(times)
    read_gb = N * V * 2 / 1e9
    return {"rows": N, "V": V, "K": K, "dtype": "bf16", "ms": ms, "ms_calls": [round(t, 4) for t in times],
            "rows_per_s": N / (ms / 1e3), "logits_read_once_gb_s": read_gb / (ms / 1e3),
            "frac_of_hbm_peak": read_gb / (ms / 1e3) / PEAK_HBM_GBS}


def kernel_sources_sha(csrc: str | None = None) -> str:
    """Hash of the kernel sources' code, with comments and layout whitespace dropped: a traffic
    figure measured on other code is stale."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "lm_head_kl_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(name.encode() + b"\0" + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(config: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary for this workload,
    or None when there is none or it was taken on other kernel sources. Lines look like
    'traffic <kernel> fetch_bytes <F> write_bytes <W> sources <sha>'."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{config}.txt")
    if not os.path.exists(path):
        return None
    sha = kernel_sources_sha()
    for line in open(path):
        f = line.split()
        if len(f) == 8 and f[0] == "traffic" and f[1] == kernel and f[7] == sha:
            return float(f[3]) + float(f[5])
    return None


def cpu_baseline(p, n_rows, reps=3):
    """The oracle as it stands (fp64 numpy, forward-chunked formulation, forward + backward)
    on the first n_rows rows at the config's full V and d, timed `reps` times (the median is
    reported); rows/s is tokens/s since the cost is linear in rows."""
    import numpy as np

    import datagen
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    sub = datagen.make(p.name, N=n_rows)
    Hs, Ws, ts = sub.f64("H"), sub.f64("W"), sub.f64("tlog")
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.kl_chunked(Hs, Ws, sub.idx, ts, sub.T, chunk=min(1024, n_rows), n_norm=p.N)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    return {
        "value": n_rows / dt,
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{n_rows} rows of the same workload at full V={p.V}, d={p.d}, K={p.K}: fp64 numpy "
                  f"oracle (forward-chunked formulation, forward and backward), median of {reps} runs "
                  f"({', '.join(f'{x:.1f}' for x in times)} s) on the host",
    }


def sweep(dev, steps: int):
    """Fused forward + backward at every timed config, and peak device memory over S.

    Timings: one warm-up step, then `steps` steps between HIP events on the current stream.
    Peak memory: torch's allocator peak over one fused forward + backward, counted from the
    inputs (H, W, idx, t) up, so it holds the workspace, lse, row_kl, dH and dW. The S sweep
    runs the gpt-oss head at N in {4096, 8192, 16384, 32768}; what grows with N is dH (2d
    bytes a row) and the O(N*K) cache-side buffers (plan entries, p_t, zk), nothing of size
    N x V."""
    import torch

    import datagen
    import lm_head_kl_amd as kd

    stream = torch.cuda.current_stream(dev)

    def to_dev(a):
        import numpy as np
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    def run(cfg, chunk=None, N=None, n_steps=steps):
        p = datagen.make(cfg, N=N)
        c = chunk or p.chunk
        H, W, idx, t = to_dev(p.H), to_dev(p.W), to_dev(p.idx), to_dev(p.tlog)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        dW = torch.empty(W.shape, dtype=torch.float32, device=dev)

        def step():
            f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=c, want_row_kl=True)
            return kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=c, dW=dW)

        step()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev) - base
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(n_steps):
            step()
        e[1].record(stream)
        torch.cuda.synchronize()
        ms = e[0].elapsed_time(e[1]) / n_steps
        fl = 8.0 * p.N * p.d * p.V
        r = {"config": cfg, "N": p.N, "d": p.d, "V": p.V, "K": p.K, "T": p.T, "chunk": c, "ms": ms,
             "tokens_per_s": p.N / (ms / 1e3), "pct_bf16_peak": 100.0 * fl / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12),
             "peak_beyond_inputs_gb": peak / 1e9, "dH_gb": H.numel() * H.element_size() / 1e9}
        del H, W, idx, t, dW
        torch.cuda.empty_cache()
        print(json.dumps(r), flush=True)
        return r

    rows = [run("small")]
    rows += [run("qwen", chunk=c) for c in (512, 1024, 2048, 4096)]
    rows.append(run("gptoss"))
    rows.append(run("full", n_steps=max(1, steps // 2)))
    srows = [run("gptoss", N=n, n_steps=1) for n in (4096, 8192, 16384, 32768)]
    print("| config | N | d | V | K | T | chunk | ms per step | tokens/s | % bf16 peak | peak beyond inputs GB |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['config']} | {r['N']} | {r['d']} | {r['V']} | {r['K']} | {r['T']} | {r['chunk']} | "
              f"{r['ms']:.2f} | {r['tokens_per_s']:,.0f} | {r['pct_bf16_peak']:.1f} | {r['peak_beyond_inputs_gb']:.3f} |")
    print()
    print("| N (gpt-oss head, chunk 2048) | peak beyond inputs GB | minus dH GB | growth per added row, bytes |")
    print("|---|---|---|---|")
    prev = None
    for r in srows:
        grow = "" if prev is None else f"{(r['peak_beyond_inputs_gb'] - prev['peak_beyond_inputs_gb']) * 1e9 / (r['N'] - prev['N']):.0f}"
        print(f"| {r['N']} | {r['peak_beyond_inputs_gb']:.3f} | {r['peak_beyond_inputs_gb'] - r['dH_gb']:.3f} | {grow} |")
        prev = r
    # The oracle as it stands on each config: the whole tiny and small batches, and the first
    # 1024 rows at full V and d for the larger heads (cost is linear in rows).
    gpu_rate = {}
    for r in rows:
        if r["config"] not in gpu_rate or r["chunk"] == datagen.CONFIGS[r["config"]]["chunk"]:
            gpu_rate[r["config"]] = r["tokens_per_s"]
    print()
    print("| config | oracle rows | oracle s | oracle tokens/s | threads | GPU fused step tokens/s | GPU / oracle |")
    print("|---|---|---|---|---|---|---|")
    for name, n in (("tiny", 256), ("small", 4096), ("qwen", 1024), ("gptoss", 1024), ("full", 1024)):
        cb = cpu_baseline(datagen.make(name, N=n), n, reps=1)
        g = gpu_rate.get(name)
        print(f"| {name} | {n} | {n / cb['value']:.2f} | {cb['value']:,.0f} | {cb['cores']} | "
              + (f"{g:,.0f} | {g / cb['value']:,.0f} |" if g else "— | — |"), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported: the path is "
              f"measured on one GPU's share of a token-parallel job", file=sys.stderr)
        sys.exit(2)

    import torch

    import datagen
    import lm_head_kl_amd as kd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_probe:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 1 << 30}))
        return
    if args.sweep:
        sweep(dev, args.steps)
        return
    if args.producer:
        p = datagen.make(args.config, N=args.rows or None)
        res = producer(dev, torch.cuda.current_stream(), p.N, p.V, p.K, p.extra.get("seed", 0) + 9, reps=args.steps)
        print(json.dumps({"topk_producer": res, "config": {"workload": p.name}}))
        return
    t_gen = time.perf_counter()
    p = datagen.make(args.config, N=args.rows or None)
    chunk = args.chunk or p.chunk

    def dt(a):
        import numpy as np
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    H, W, idx, t = dt(p.H), dt(p.W), dt(p.idx), dt(p.tlog)
    torch.cuda.synchronize()
    print(f"[bench] inputs {args.config} N={p.N} d={p.d} V={p.V} K={p.K} chunk={chunk} ready in "
          f"{time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    step_flags = kd.KD_LOW_MEMORY if args.low_memory else 0
    prob = kd.make_problem(H, W, idx, t, p.T, chunk, flags=step_flags)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    inputs_mem = torch.cuda.memory_allocated(dev)
    ws = torch.empty(kd.fused_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    dW = torch.empty(W.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=chunk, want_row_kl=True, flags=step_flags, workspace=ws)
        if ev:
            ev[1].record(stream)
        kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=chunk, flags=step_flags, dW=dW, workspace=ws)
        if ev:
            ev[2].record(stream)
        return f

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    kd.timing_reset()
    kd.timing_enable(True)  # the library brackets each of its launches with HIP events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kd.timing_enable(False)
    kernels = kd.timing_read()
    peak_fused = torch.cuda.max_memory_allocated(dev) - inputs_mem
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    ms_step = wall * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.2f} ms/step (fwd {fwd_ms:.2f}, bwd {bwd_ms:.2f})",
          file=sys.stderr, flush=True)

    N, d, V = p.N, p.d, p.V
    flops_step = 8.0 * N * d * V
    tokens_s = N / (ms_step / 1e3)
    # Each GEMM-shaped kernel does 2*N*d*V counted FLOPs per step: the forward in one launch,
    # the recompute (bwd_grad), dH and dW in one launch per chunk.
    gemm_kinds = ("fwd", "bwd_grad", "dh", "dw")
    per_kernel = {}
    for name, (n, ms) in kernels.items():
        e = {"launches": n, "avg_ms": ms / n, "ms_per_step": ms / args.steps}
        if name in gemm_kinds:
            e["tflops"] = 2.0 * N * d * V * args.steps / (ms / 1e3) / 1e12
        per_kernel[name] = e
    dom = max((k for k in per_kernel if k in gemm_kinds), key=lambda k: per_kernel[k]["ms_per_step"])
    dom_flops_launch = 2.0 * N * d * V * args.steps / per_kernel[dom]["launches"]
    achieved = dom_flops_launch / (per_kernel[dom]["avg_ms"] / 1e3) / 1e12

    out = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; bf16 H ~ N(0,1), W ~ N(0,1/d), top-K cache peaked/flat mix)",
        "config": {
            "workload": f"{args.config}: LM-head fused chunked top-K KL, N={N}, d={d}, V={V}, K={p.K}, "
                        f"chunk={chunk}, T={p.T}" + (", memory-lean backward" if args.low_memory else ""),
            "N": N, "d": d, "V": V, "K": p.K, "chunk": chunk, "T": p.T,
        },
        "pct_bf16_peak": 100.0 * flops_step / (ms_step / 1e3) / (PEAK_BF16_TFLOPS * 1e12),
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "counted_flops_per_step": flops_step,
        "peak_hbm_fused_gb": peak_fused / 1e9,
        "kernels": per_kernel,
        "roofline": {
            "kernel": f"{dom} (largest share of the step; {per_kernel[dom]['launches'] // args.steps} "
                      f"launch(es) per step, {dom_flops_launch:.4g} counted FLOP per launch)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            # the committed counters are for the default step's kernels
            "traffic": None if args.low_memory else measured_traffic(args.config, dom),
        },
    }

    # The same step replayed from a HIP graph (torch.cuda.CUDAGraph): every launch of the
    # forward and backward captured once with the step's buffers, then replayed. Shows what
    # launch overhead the eager step carries; the headline figure stays the eager one.
    if not args.no_formulations:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                step()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            graph.replay()
            torch.cuda.synchronize()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            for _ in range(args.steps):
                graph.replay()
            e[1].record(stream)
            torch.cuda.synchronize()
            out["graph_replay_ms_per_step"] = e[0].elapsed_time(e[1]) / args.steps
            del graph
            torch.cuda.empty_cache()
            print("[bench] graph replay done", file=sys.stderr, flush=True)
        except (RuntimeError, torch.OutOfMemoryError) as ex:
            out["graph_replay_ms_per_step"] = None
            out["graph_replay_error"] = str(ex)[:200]

    # The other formulations on the same inputs: one call each does forward and backward.
    # Each is warmed up once and timed over a few calls; peak memory is measured from the
    # inputs up, like the fused path's.
    del ws, dW
    forms = {"fused_recompute": {"ms": ms_step, "peak_hbm_gb": peak_fused / 1e9, "counted_flops": flops_step}}
    def frozen_head():
        f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=chunk, want_row_kl=True)
        return kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=chunk, flags=kd.KD_SKIP_DW)

    def low_memory():
        f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=chunk, want_row_kl=True, flags=kd.KD_LOW_MEMORY)
        return kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=chunk, flags=kd.KD_LOW_MEMORY)

    # The autograd term of a training step on a bf16 head: H and W as leaves, dW accumulated in a
    # caller-owned fp32 buffer (allocated once, like an optimizer's main gradient; its 4 V d bytes
    # count in the peak), dH returned to H.grad.
    acc_box = []

    def autograd_step():
        if not acc_box:
            acc_box.append(torch.zeros(W.shape, dtype=torch.float32, device=dev))
        Hl = H.detach().requires_grad_(True)
        loss = kd.fused_kl(Hl, W, idx, t, T=p.T, chunk=chunk, dw_accumulator=acc_box[0])
        loss.backward()
        return Hl.grad

    # counted FLOPs of each: single pass and forward-chunked compute the logits once (6 N d V);
    # the frozen head (KD_SKIP_DW) recomputes them but skips dW (6 N d V); the memory-lean and
    # autograd steps do the whole fused step (8 N d V)
    others = [("single_pass", lambda: kd.fused_kl_fwdbwd(H, W, idx, t, T=p.T, chunk=chunk), 6.0),
              ("forward_chunked", lambda: kd.chunked_kl(H, W, idx, t, T=p.T, chunk=chunk), 6.0),
              ("fused_frozen_head", frozen_head, 6.0),
              ("fused_low_memory", low_memory, 8.0),
              ("fused_autograd_fp32_dw", autograd_step, 8.0)]
    if not args.no_dense:
        others.append(("dense", lambda: kd.dense_kl(H, W, idx, t, T=p.T), 8.0))
    for name, call, fl in others:
        if args.no_formulations and name != "dense":
            continue
        torch.cuda.empty_cache()
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        try:
            call()
            torch.cuda.synchronize()
            peak = (torch.cuda.max_memory_allocated(dev) - base) / 1e9
            reps = 1 if name == "dense" else 3
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            for _ in range(reps):
                call()
            e[1].record(stream)
            torch.cuda.synchronize()
            forms[name] = {"ms": e[0].elapsed_time(e[1]) / reps, "peak_hbm_gb": peak,
                           "counted_flops": fl * N * d * V}
        except (RuntimeError, torch.OutOfMemoryError) as ex:
            forms[name] = {"error": str(ex)[:200]}
        acc_box.clear()
        torch.cuda.empty_cache()
        print(f"[bench] {name} path done", file=sys.stderr, flush=True)
    for f in forms.values():
        if "ms" in f:
            f["tokens_per_s"] = N / (f["ms"] / 1e3)
            f["pct_bf16_peak_of_counted"] = 100.0 * f["counted_flops"] / (f["ms"] / 1e3) / (PEAK_BF16_TFLOPS * 1e12)
    out["formulations"] = forms
    if "dense" in forms and "ms" in forms["dense"]:
        out["dense_ms"] = forms["dense"]["ms"]
        out["peak_hbm_dense_gb"] = forms["dense"]["peak_hbm_gb"]

    if not args.no_formulations:
        try:
            torch.cuda.empty_cache()
            out["topk_producer"] = producer(dev, stream, N, V, p.K, p.extra.get("seed", 0) + 9)
            torch.cuda.empty_cache()
            print("[bench] top-K producer done", file=sys.stderr, flush=True)
        except (RuntimeError, torch.OutOfMemoryError) as ex:
            out["topk_producer"] = {"error": str(ex)[:200]}

    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        try:
            out["cpu_baseline"] = cpu_baseline(p, args.cpu_rows)
        except Exception as ex:  # the headline line is printed whatever happens here
            out["cpu_baseline"] = {"value": None, "error": str(ex)[:200]}

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
