"""Benchmark of the NF4 / QLoRA linear path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-train]

Prints ONE JSON line.  Workload (the decode-shaped 8B q_proj): a 4096 x 4096
NF4 weight (blocks of 64, absmax double-quantized in groups of 256, weights
N(0, 0.02)), LoRA r = 16, alpha = 32, forward at 1 and at 16 tokens of
N(0, 1) bf16 activations.  A step is one forward at T = 1 plus one at T = 16,
each on a different weight of a pool of 64 quantized copies (554 MB, more
than the 256 MB Infinity Cache), so every step streams its weights from HBM.

value = NF4 weight-stream throughput of the step, in GB/s of algorithmic
bytes (packed codes + 8-bit absmax + group scales + X + Y + A + B per call).

Also reported ("extra"): nf4_quantize of the 4096 x 4096 fp32 weight and
of the flat 2^30-element tensor; fwd+bwd TFLOP/s of every projection of the
8B MLP (T = 4096, r = 64), the 8B attention projections (T = 8192, r = 16)
and the 70B MLP (T = 4096, r = 64) -- the large-token half of the metric --
each with the oracle timed on the host beside it (skipped with --no-train);
the host's CPU model and thread counts and the GPU shader clock sampled
during the large-token legs.

The roofline entry is for the dominant kernel, the fused small-token forward
(one launch per call); its average duration comes from HIP events on the
stream the library launches on (torch's current stream).
"""

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s and NF4 weight-stream GB/s (% of roofline)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk, dense
DROPOUT_P = 0.05  # the lora_dropout value the pages configure
NF4_BYTES_PER_WEIGHT = 0.515869140625
# untimed calls before a standalone timing: short kernels run on clocks that
# are still ramping for the first tens of milliseconds of sustained load
WARM_CALLS = 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pool", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the small-token legs (the headline, q|k|v and the MLP-sized weights)")
    ap.add_argument("--counters-probe", action="store_true",
                    help="only run the T=16 small-token forward over the weight pool and a "
                         "256 MiB copy (for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes)")
    ap.add_argument("--mlp-probe", action="store_true",
                    help="only run the fwd + bwd step of one large-token workload (--probe-workload: "
                         "3 = 8B MLP, 4 = 8B attention, 5 = 70B MLP) and print its figures (for "
                         "rocprofv3 --pmc passes over the large-token GEMMs)")
    ap.add_argument("--probe-workload", type=int, default=3, choices=(3, 4, 5))
    ap.add_argument("--bwd-min", action="store_true",
                    help="with --mlp-probe: every backward in its smallest workspace (the dX GEMM "
                         "dequantizes the weight tiles while staging them)")
    ap.add_argument("--only-leg", choices=("quantize", "merge", "bwd_small"),
                    help="only run one standalone leg (the 2^30 flat quantize, or the 8B and 70B gate "
                         "merges) and then the 256 MiB copy, and print its figures (for rocprofv3 "
                         "kernel-trace and --pmc FETCH_SIZE / WRITE_SIZE passes)")
    return ap.parse_args()


# Sources that define the small-token forward kernel, and the compile flags
# (bit_nf4_quantized_20_amd/build.py: flags()); the HBM traffic recorded from
# hardware counters is reported only while they are unchanged.
DECODE_SOURCES = ("bit_nf4_quantized_20_amd/csrc/k_decode.hip",
                  "bit_nf4_quantized_20_amd/csrc/nf4_format.hpp",
                  "bit_nf4_quantized_20_amd/csrc/common.hpp")
TRAFFIC_RECORD = "profiles/k_decode_fwd_split_qproj4096x4096_T16_traffic.md"
COPY_BYTES = 256 << 20


def compile_flags():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "qlora_build", os.path.join(ROOT, "bit_nf4_quantized_20_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return " ".join(mod.flags())


def decode_fingerprint():
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(compile_flags().encode())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the T=16 small-token forward, from the counter
    record in profiles/ (FETCH_SIZE + WRITE_SIZE, each scaled by what the same
    counter reads for a copy of known size), or None when the record is
    missing or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, TRAFFIC_RECORD)
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("sources_sha256") != decode_fingerprint():
        return None
    return int(rec["hbm_bytes_per_launch"])


def decode_call_bytes(n_out, n_in, T, r):
    """Algorithmic HBM bytes of one small-token forward call."""
    weight = n_out * n_in * NF4_BYTES_PER_WEIGHT
    return int(weight + 2 * T * (n_in + n_out) + 2 * r * (n_in + n_out))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_nf4_quantized_20_amd as q
    import synth

    dev = torch.device("cuda:0")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    if args.only_leg:
        if args.only_leg == "quantize":
            res = {"quantize_flat_2pow30": flat_quantize_leg(q, synth, dev, False)}
        elif args.only_leg == "merge":
            res = {"merge_8b_gate": merge_leg(q, synth, dev, bf, 3),
                   "merge_70b_gate": merge_leg(q, synth, dev, bf, 5)}
        else:
            res = {"bwd_small": bwd_small_leg(q, synth, dev, bf)}
        copy_calibration(dev)
        print(json.dumps(res), flush=True)
        return

    wl = synth.WORKLOADS[2]
    proj = wl.projections[0]
    n_out, n_in, r, alpha = proj.out_features, proj.in_features, wl.r, wl.alpha

    # ---------------------------------------------------------------- inputs
    w_host = synth.weight(2, 0, n_out, n_in)
    w_dev = torch.from_numpy(w_host).to(dev)
    pool = [q.nf4_quantize_weight(w_dev) for _ in range(args.pool)]
    A = bf(synth.lora_A(2, 0, r, n_in))
    B = bf(synth.lora_B(2, 0, n_out, r))
    X1 = bf(synth.activations(2, 0, 1, n_in))
    X16 = bf(synth.activations(2, 0, 16, n_in))
    Y1 = torch.empty(1, n_out, dtype=torch.bfloat16, device=dev)
    Y16 = torch.empty(16, n_out, dtype=torch.bfloat16, device=dev)
    ws = q.make_workspace(q.qlora_workspace_bytes(16, n_in, n_out, r, False), dev)
    torch.cuda.synchronize()

    if args.counters_probe:
        counters_probe(q, pool, X16, Y16, A, B, r, alpha, ws, dev)
        return
    if args.mlp_probe:
        del pool
        wid = args.probe_workload
        if args.bwd_min:
            wl = synth.WORKLOADS[wid]
            flop = sum(step_flop(wl.tokens[0], p.in_features, p.out_features, wl.r) for p in wl.projections)
            res = grouped_step_leg(q, synth, dev, bf, wid, [[i] for i in range(len(wl.projections))], 5, flop,
                                   bwd_min=True)
        else:
            res = large_step_leg(q, synth, dev, bf, wid, steps=5)
        print(json.dumps(res), flush=True)
        return

    b1 = decode_call_bytes(n_out, n_in, 1, r)
    b16 = decode_call_bytes(n_out, n_in, 16, r)
    P = len(pool)

    def step(i):
        q.qlora_linear_fwd(pool[(2 * i) % P], X1, A, B, r, alpha, Y=Y1, ws=ws)
        q.qlora_linear_fwd(pool[(2 * i + 1) % P], X16, A, B, r, alpha, Y=Y16, ws=ws)

    # The timed step is captured once as a HIP graph (the way a decode loop
    # drives it: one launch per call, no host launch cost in the loop) and
    # replayed; steps cycle through the weight pool inside the graph.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    value = (b1 + b16) * args.steps / (ms_total * 1e-3) / 1e9

    # ------------------------------------------------ dominant kernel alone
    # the small-token forward is one kernel launch per call; its average
    # launch duration from events around a graph of n back-to-back launches
    def per_launch_us(X, Y, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                q.qlora_linear_fwd(pool[i % P], X, A, B, r, alpha, Y=Y, ws=ws)
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def eager_us(X, Y, n):
        for i in range(10):
            q.qlora_linear_fwd(pool[i % P], X, A, B, r, alpha, Y=Y, ws=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            q.qlora_linear_fwd(pool[i % P], X, A, B, r, alpha, Y=Y, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    us16 = per_launch_us(X16, Y16, 400)
    us1 = per_launch_us(X1, Y1, 400)
    ach16 = b16 / (us16 * 1e-6) / 1e9
    ceiling = read_ceiling_leg(pool, 400)

    extra = {
        "fwd_T1": {"us_per_call": round(us1, 3), "GB_per_s": round(b1 / (us1 * 1e-6) / 1e9, 1),
                   "algorithmic_bytes": b1},
        "fwd_T16": {"us_per_call": round(us16, 3), "GB_per_s": round(ach16, 1),
                    "algorithmic_bytes": b16},
        "eager_us_per_call": {"T1": round(eager_us(X1, Y1, 200), 2),
                              "T16": round(eager_us(X16, Y16, 200), 2)},
        "read_ceiling": dict(ceiling, fwd_T1_frac_of_ceiling=round(b1 / (us1 * 1e-6) / 1e9 / ceiling["GB_per_s"], 3),
                             fwd_T16_frac_of_ceiling=round(ach16 / ceiling["GB_per_s"], 3)),
        "timing": "HIP graph replay of back-to-back calls (events on the library's stream)",
        "weight_pool_bytes": int(P * n_out * n_in * NF4_BYTES_PER_WEIGHT),
    }

    if args.decode_only:
        extra["qkv8b_decode"] = qkv_decode_leg(q, synth, dev, bf)
        extra["mlp_weights_decode"] = mlp_decode_leg(q, synth, dev, bf)
        print(json.dumps({"value": round(value, 2), "ms_per_step": round(ms_per_step, 5), "extra": extra}),
              flush=True)
        return

    # ------------------------------------------------------------ quantize
    codes, aq, sc = pool[0].codes, pool[0].absmax_q, pool[0].absmax_scale
    for _ in range(WARM_CALLS):
        q.nf4_quantize(w_dev, codes, aq, sc)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    nq = 50
    for _ in range(nq):
        q.nf4_quantize(w_dev, codes, aq, sc)
    e1.record()
    torch.cuda.synchronize()
    us_q = e0.elapsed_time(e1) * 1e3 / nq
    qbytes = int(n_out * n_in * (4 + NF4_BYTES_PER_WEIGHT))
    extra["quantize_4096x4096"] = {"us_per_call": round(us_q, 2),
                                   "GB_per_s": round(qbytes / (us_q * 1e-6) / 1e9, 1)}

    # standalone dequantize (D1) and the format without double quantization
    def per_call_us(fn, n=50):
        for _ in range(WARM_CALLS):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    nw = n_out * n_in
    wout = torch.empty(nw, dtype=torch.bfloat16, device=dev)
    us_d = per_call_us(lambda: q.nf4_dequantize(codes, aq, sc, nw, out=wout))
    dbytes = int(nw * (NF4_BYTES_PER_WEIGHT + 2))
    extra["dequantize_4096x4096"] = {"us_per_call": round(us_d, 2),
                                     "GB_per_s": round(dbytes / (us_d * 1e-6) / 1e9, 1)}
    c2, a2 = q.nf4_quantize_nodq(w_dev)
    us_qn = per_call_us(lambda: q.nf4_quantize_nodq(w_dev, codes=c2, absmax=a2))
    us_dn = per_call_us(lambda: q.nf4_dequantize_nodq(c2, a2, nw, out=wout))
    extra["nodq_4096x4096"] = {"quantize_us": round(us_qn, 2),
                               "quantize_GB_per_s": round(nw * 4.5625 / (us_qn * 1e-6) / 1e9, 1),
                               "dequantize_us": round(us_dn, 2),
                               "dequantize_GB_per_s": round(nw * 2.5625 / (us_dn * 1e-6) / 1e9, 1)}

    # ------------------------------------------------------ adapter merge
    extra["merge_8b_gate"] = merge_leg(q, synth, dev, bf, 3)
    extra["merge_70b_gate"] = merge_leg(q, synth, dev, bf, 5)
    extra["bwd_small"] = bwd_small_leg(q, synth, dev, bf)

    # ------------------------------------------- q|k|v at decode sizes
    extra["qkv8b_decode"] = qkv_decode_leg(q, synth, dev, bf)

    # ------------------------------ MLP-sized weights at decode sizes
    extra["mlp_weights_decode"] = mlp_decode_leg(q, synth, dev, bf)

    # ---------------------------------------- flat 2^30-element quantize
    del pool
    torch.cuda.empty_cache()
    extra["quantize_flat_2pow30"] = flat_quantize_leg(q, synth, dev, not args.no_cpu_baseline)

    # ------------------------------------------- large-token fwd + bwd
    if not args.no_train:
        sampler = SclkSampler()
        sampler.start()
        for wid, key in ((3, "mlp8b_fwd_bwd"), (4, "attn8b_fwd_bwd"), (5, "mlp70b_fwd_bwd")):
            extra[key] = large_step_leg(q, synth, dev, bf, wid, steps=10 if wid < 5 else 5)
        extra["mlp8b_variants"] = train_leg(q, synth, dev, bf, extra["mlp8b_fwd_bwd"])
        # the projections that share X as one multi-projection call (q|k|v, gate|up)
        extra["attn8b_qkv_fused"] = grouped_step_leg(q, synth, dev, bf, 4, [[0, 1, 2], [3]], 10,
                                                     extra["attn8b_fwd_bwd"]["step_flop"])
        extra["mlp70b_gate_up_fused"] = grouped_step_leg(q, synth, dev, bf, 5, [[0, 1], [2]], 5,
                                                         extra["mlp70b_fwd_bwd"]["step_flop"])
        extra["mid_tokens"] = mid_tokens_leg(q, synth, dev, bf)
        # the backward in its smallest workspace: dX without the expanded W_hat^T
        extra["mlp8b_bwd_min_workspace"] = grouped_step_leg(q, synth, dev, bf, 3, [[0], [1], [2]], 10,
                                                            extra["mlp8b_fwd_bwd"]["step_flop"], bwd_min=True)
        extra["mlp70b_bwd_min_workspace"] = grouped_step_leg(q, synth, dev, bf, 5, [[0], [1], [2]], 5,
                                                             extra["mlp70b_fwd_bwd"]["step_flop"], bwd_min=True)
        extra["gpu_sclk_mhz"] = sampler.stop()
        if not args.no_cpu_baseline:
            for wid, key in ((3, "mlp8b_fwd_bwd"), (4, "attn8b_fwd_bwd"), (5, "mlp70b_fwd_bwd")):
                extra[key]["oracle"] = oracle_step_timing(synth, wid)
    extra["host"] = host_info()

    # --------------------------------------------------------- cpu baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(n_out, n_in, r, alpha, X1, X16, A, B, b1 + b16)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations)",
        "config": {"workload": "decode-shaped 8B q_proj: NF4 W 4096x4096 (block 64, double-quant "
                               "256), fwd at T=1 and T=16, LoRA r=16 alpha=32, 64-weight pool",
                   "out_features": n_out, "in_features": n_in, "tokens": [1, 16], "r": r,
                   "alpha": alpha, "weight_pool": P},
        "roofline": {"bound": "hbm", "kernel": "k_decode_fwd_split (T=16)", "achieved": round(ach16, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach16 / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic()},
        "cpu_baseline": cpu,
        "extra": extra,
        "wall_s_timed_region": round(wall, 6),
    }
    print(json.dumps(out), flush=True)


def read_ceiling_leg(pool, n):
    """The fastest plain read of one pool weight's packed codes (8 MiB) in a
    single launch: a graph of n back-to-back launches over the pool, as the
    small-token forward is timed, for each (threads, loads per thread) of a
    small sweep; the best is the practical ceiling of a one-launch weight
    stream of this size (launch overhead and memory latency included)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "bit_nf4_quantized_20_amd", "libqlora_bench.so"))
    fn = lib.qlora_bench_read_ceiling
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    nbytes = pool[0].codes.numel()
    P = len(pool)
    sink = torch.empty(nbytes // 16 + 1024, dtype=torch.int32, device=pool[0].codes.device)
    best = None
    for threads in (256, 512):
        for per in (1, 2, 4, 8):
            def launch(i):
                st = fn(pool[i % P].codes.data_ptr(), nbytes, threads, per, sink.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
                if st != 0:
                    raise RuntimeError(f"qlora_bench_read_ceiling returned {st}")
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    launch(i)
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / n
            if best is None or us < best[0]:
                best = (us, threads, per)
    us, threads, per = best
    return {"bytes": int(nbytes), "us_per_call": round(us, 3), "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "threads": threads, "loads_per_thread": per}


def qkv_decode_leg(q, synth, dev, bf, P=24, n=192):
    """The 8B attention q|k|v projections (4096 -> 4096, 1024, 1024; r = 16,
    alpha = 32) at T = 1 and T = 16: one multi-projection call (a single
    small-token launch over all three weights) against three single-projection
    calls.  Each is captured as a graph of n back-to-back calls cycling
    through P copies of the weights (P x 13 MB, past the 256 MB last-level
    cache) and replayed; microseconds per q|k|v forward."""
    import torch
    wl = synth.WORKLOADS[4]
    r, alpha = wl.r, wl.alpha
    projs = wl.projections[:3]
    n_in = projs[0].in_features
    outs = [p.out_features for p in projs]
    base = [q.nf4_quantize_weight(torch.from_numpy(synth.weight(4, i, p.out_features, n_in)).to(dev))
            for i, p in enumerate(projs)]
    pool = [[q.NF4Weight(W.codes.clone(), W.absmax_q.clone(), W.absmax_scale.clone(), W.rows, W.cols)
             for W in base] for _ in range(P)]
    As = [bf(synth.lora_A(4, i, r, n_in)) for i in range(3)]
    Bs = [bf(synth.lora_B(4, i, p.out_features, r)) for i, p in enumerate(projs)]
    res = {"outs": outs, "in": n_in, "r": r}
    for T in (1, 16):
        X = bf(synth.activations(4, 0, T, n_in))
        Y = torch.empty(T, sum(outs), dtype=torch.bfloat16, device=dev)
        Ys = [torch.empty(T, o, dtype=torch.bfloat16, device=dev) for o in outs]

        def multi(i):
            q.qlora_linear_fwd_multi(pool[i % P], X, As, Bs, r, alpha, Y=Y)

        def single(i):
            for W, A, B, Yi in zip(pool[i % P], As, Bs, Ys):
                q.qlora_linear_fwd(W, X, A, B, r, alpha, Y=Yi)

        def graph_us(fn):
            for i in range(4):
                fn(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    fn(i)
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / n

        us_m, us_s = graph_us(multi), graph_us(single)
        # X counted once: the three projections share it
        nbytes = sum(decode_call_bytes(o, n_in, T, r) for o in outs) - 2 * 2 * T * n_in
        res[f"T{T}"] = {"multi_us": round(us_m, 2), "three_calls_us": round(us_s, 2),
                        "multi_GB_per_s": round(nbytes / (us_m * 1e-6) / 1e9, 1),
                        "algorithmic_bytes": nbytes}
    return res


def mlp_decode_leg(q, synth, dev, bf, n=96):
    """The small-token forward on the MLP weights of the 8B and 70B shapes
    (8B gate 14336 x 4096 and down 4096 x 14336, 70B gate 28672 x 8192; their
    r = 64 and alpha) at T = 1 and T = 16: how close the weight stream comes
    to the HBM peak once the weight, not the launch, dominates.  Graph replay
    of n back-to-back calls cycling through copies of the weight that together
    exceed the 256 MB last-level cache; microseconds per call."""
    import torch
    cases = [(3, 0, "8b_gate"), (3, 2, "8b_down"), (5, 0, "70b_gate")]
    res = {}
    for wid, pi, name in cases:
        wl = synth.WORKLOADS[wid]
        p = wl.projections[pi]
        n_out, n_in, r, alpha = p.out_features, p.in_features, wl.r, wl.alpha
        w = torch.from_numpy(synth.weight(wid, pi, n_out, n_in)).to(dev)
        W0 = q.nf4_quantize_weight(w)
        del w
        copies = max(2, -(-320 * 2**20 // int(n_out * n_in * NF4_BYTES_PER_WEIGHT)))
        pool = [W0] + [q.NF4Weight(W0.codes.clone(), W0.absmax_q.clone(), W0.absmax_scale.clone(),
                                   W0.rows, W0.cols) for _ in range(copies - 1)]
        A = bf(synth.lora_A(wid, pi, r, n_in))
        B = bf(synth.lora_B(wid, pi, n_out, r))
        entry = {"out": n_out, "in": n_in, "r": r, "copies": copies}
        for T in (1, 16):
            X = bf(synth.activations(wid, pi, T, n_in))
            Y = torch.empty(T, n_out, dtype=torch.bfloat16, device=dev)
            for i in range(copies):
                q.qlora_linear_fwd(pool[i], X, A, B, r, alpha, Y=Y)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    q.qlora_linear_fwd(pool[i % copies], X, A, B, r, alpha, Y=Y)
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / n
            nbytes = decode_call_bytes(n_out, n_in, T, r)
            gbs = nbytes / (us * 1e-6) / 1e9
            entry[f"T{T}"] = {"us_per_call": round(us, 2), "GB_per_s": round(gbs, 1),
                              "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 3)}
            del g
        res[name] = entry
        del pool, W0
        torch.cuda.empty_cache()
    return res


def bwd_small_leg(q, synth, dev, bf):
    """Small-token backward (T = 1 and 16): qlora_linear_bwd, whose dX
    streams the codes once, against the expanded-weight route of the same
    call (qlora_linear_bwd_dropout with every element kept and p = 0: W_hat^T
    expanded into the workspace, then the GEMM), on the 8B q_proj (r = 16)
    and gate (r = 64) weights.  30 untimed and 50 timed calls each."""
    import numpy as np
    import torch
    res = {}
    for name, wid, proj in (("q_proj", 2, 0), ("8b_gate", 3, 0)):
        wl = synth.WORKLOADS[wid]
        pr = wl.projections[proj]
        r, alpha = wl.r, wl.alpha
        n_out, n_in = pr.out_features, pr.in_features
        W = q.nf4_quantize_weight(torch.from_numpy(synth.weight(wid, proj, n_out, n_in)).to(dev))
        A, B = bf(synth.lora_A(wid, proj, r, n_in)), bf(synth.lora_B(wid, proj, n_out, r))
        entry = {"out": n_out, "in": n_in, "r": r}
        for T in (1, 16):
            X = bf(synth.activations(wid, proj, T, n_in))
            dY = bf(synth.activations(wid, proj, T, n_out, "dY"))
            keep = torch.full((T, n_in // 8), 0xFF, dtype=torch.uint8, device=dev)
            dX = torch.empty(T, n_in, dtype=torch.bfloat16, device=dev)
            dA = torch.empty(r, n_in, dtype=torch.float32, device=dev)
            dB = torch.empty(n_out, r, dtype=torch.float32, device=dev)
            ws_small = q.qlora_workspace_bytes(T, n_in, n_out, r, True)
            ws_exp = q.qlora_workspace_bytes_dropout(T, n_in, n_out, r, True)
            ws = q.make_workspace(max(ws_small, ws_exp), dev)

            def timed(fn, n=50):
                for _ in range(WARM_CALLS):
                    fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(n):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / n
            us_new = timed(lambda: q.qlora_linear_bwd(W, X, dY, A, B, r, alpha, dX, dA, dB, ws))
            us_old = timed(lambda: q.qlora_linear_bwd_dropout(W, X, dY, keep, 0.0, A, B, r, alpha, dX, dA, dB,
                                                              ws))
            entry[f"T{T}"] = {"streamed_us": round(us_new, 2), "expanded_us": round(us_old, 2),
                              "workspace_bytes": {"streamed": ws_small, "expanded": ws_exp}}
        res[name] = entry
    return res


def merge_leg(q, synth, dev, bf, wid):
    """qlora_merge of an MLP gate projection (8B: 14336 x 4096, 70B:
    28672 x 8192, NF4, r = 64): W_merged = bf16(W_hat + (alpha/r) B A),
    HBM-bound (codes + absmax read, 2 B per weight written)."""
    import torch
    wl = synth.WORKLOADS[wid]
    p = wl.projections[0]
    r, alpha = wl.r, wl.alpha
    n_out, n_in = p.out_features, p.in_features
    W = q.nf4_quantize_weight(torch.from_numpy(synth.weight(wid, 0, n_out, n_in)).to(dev))
    A = bf(synth.lora_A(wid, 0, r, n_in))
    B = bf(synth.lora_B(wid, 0, n_out, r))
    out = torch.empty(n_out, n_in, dtype=torch.bfloat16, device=dev)
    ws = q.make_workspace(q.qlora_merge_workspace_bytes(n_in, n_out, r), dev)
    for _ in range(WARM_CALLS):
        q.qlora_merge(W, A, B, r, alpha, out=out, ws=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    n = 40
    for _ in range(n):
        q.qlora_merge(W, A, B, r, alpha, out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    nbytes = int(n_out * n_in * (NF4_BYTES_PER_WEIGHT + 2) + 2 * r * (n_in + n_out))
    return {"out": n_out, "in": n_in, "r": r, "us_per_call": round(us, 2), "algorithmic_bytes": nbytes,
            "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def counters_probe(q, pool, X, Y, A, B, r, alpha, ws, dev):
    """Workload of the counter passes: one T=16 forward on each pool weight
    (64 launches, every one streaming its weight from HBM), then a plain
    256 MiB fp32 copy (torch.neg into a second buffer: COPY_BYTES read and
    COPY_BYTES written), whose counter readings calibrate the scale."""
    import torch
    for W in pool:
        q.qlora_linear_fwd(W, X, A, B, r, alpha, Y=Y, ws=ws)
    copy_calibration(dev)
    print(json.dumps({"probe": "decode T=16 x %d, copy %d B x 4" % (len(pool), COPY_BYTES),
                      "sources_sha256": decode_fingerprint()}), flush=True)


def copy_calibration(dev):
    """Four plain 256 MiB fp32 copies (torch.neg into a second buffer:
    COPY_BYTES read and COPY_BYTES written each), whose FETCH_SIZE /
    WRITE_SIZE readings calibrate the counters' scale."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def train_leg(q, synth, dev, bf, plain):
    """Variants of the 8B-MLP step (gate and up 4096 -> 14336, down
    14336 -> 4096; T = 4096, r = 64, alpha = 128), next to its plain figures
    `plain` (large_step_leg): every projection with LoRA dropout p = 0.05;
    gate and up as one multi-projection call each way; and the forward of
    gate|up at T = 1792 through both routes (dequantization inside the GEMM's
    LDS staging with the smallest workspace, the weight expanded first with
    the full one).  Each call is warmed up, then timed over 20 calls."""
    import torch
    wl = synth.WORKLOADS[3]
    T, r, alpha = wl.tokens[0], wl.r, wl.alpha
    res = {}

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    tot_dms = 0.0
    for pi, p in enumerate(wl.projections):
        n_out, n_in = p.out_features, p.in_features
        w = torch.from_numpy(synth.weight(3, pi, n_out, n_in)).to(dev)
        W = q.nf4_quantize_weight(w)
        del w
        X = bf(synth.activations(3, pi, T, n_in))
        dY = bf(synth.activations(3, pi, T, n_out, "dY"))
        A = bf(synth.lora_A(3, pi, r, n_in))
        B = bf(synth.lora_B(3, pi, n_out, r))
        Y = torch.empty(T, n_out, dtype=torch.bfloat16, device=dev)
        dX = torch.empty(T, n_in, dtype=torch.bfloat16, device=dev)
        dA = torch.empty(r, n_in, dtype=torch.float32, device=dev)
        dB = torch.empty(n_out, r, dtype=torch.float32, device=dev)
        keep = torch.from_numpy(synth.keep_mask(synth.seed_for(3, pi, "keep"), T, n_in, DROPOUT_P)).to(dev)
        wdf = q.make_workspace(q.qlora_workspace_bytes_dropout(T, n_in, n_out, r, False), dev)
        wsb = q.make_workspace(q.qlora_workspace_bytes_dropout(T, n_in, n_out, r, True), dev)

        def dfwd():
            q.qlora_linear_fwd_dropout(W, X, keep, DROPOUT_P, A, B, r, alpha, Y=Y, ws=wdf)

        def dbwd():
            q.qlora_linear_bwd_dropout(W, X, dY, keep, DROPOUT_P, A, B, r, alpha, dX=dX, dA=dA, dB=dB,
                                       ws=wsb)

        for _ in range(4):
            dfwd()
            dbwd()
        dms_f = timed(dfwd, 20)
        dms_b = timed(dbwd, 20)
        res[f"dropout_{p.name}"] = {"fwd_ms": round(dms_f, 3), "bwd_ms": round(dms_b, 3)}
        tot_dms += dms_f + dms_b
        del W, X, dY, Y, dX, wdf, wsb, keep
    tot_flop = plain["step_flop"]
    res["mlp_dropout"] = {"p": DROPOUT_P, "fwd_bwd_ms": round(tot_dms, 3),
                          "fwd_bwd_TFLOPs": round(tot_flop / (tot_dms * 1e-3) / 1e12, 1)}

    # gate and up share X: one multi-projection call each way (one LoRA
    # down-projection pass, one GEMM launch over both, one dX GEMM)
    gu = wl.projections[:2]
    n_in = gu[0].in_features
    Ws, As, Bs = [], [], []
    for pi, p in enumerate(gu):
        w = torch.from_numpy(synth.weight(3, pi, p.out_features, n_in)).to(dev)
        Ws.append(q.nf4_quantize_weight(w))
        del w
        As.append(bf(synth.lora_A(3, pi, r, n_in)))
        Bs.append(bf(synth.lora_B(3, pi, p.out_features, r)))
    N = sum(p.out_features for p in gu)
    X = bf(synth.activations(3, 0, T, n_in))
    dY = bf(synth.activations(3, 0, T, N, "dY"))
    Y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(T, n_in, dtype=torch.bfloat16, device=dev)
    dAs = [torch.empty(r, n_in, dtype=torch.float32, device=dev) for _ in gu]
    dBs = [torch.empty(p.out_features, r, dtype=torch.float32, device=dev) for p in gu]
    outs = [p.out_features for p in gu]
    wsf = q.make_workspace(q.qlora_workspace_bytes_multi(T, n_in, outs, r, False), dev)
    wsb = q.make_workspace(q.qlora_workspace_bytes_multi(T, n_in, outs, r, True), dev)

    def fwd2():
        q.qlora_linear_fwd_multi(Ws, X, As, Bs, r, alpha, Y=Y, ws=wsf)

    def bwd2():
        q.qlora_linear_bwd_multi(Ws, X, dY, As, Bs, r, alpha, dX=dX, dAs=dAs, dBs=dBs, ws=wsb)

    for _ in range(4):
        fwd2()
        bwd2()
    ms_f = timed(fwd2, 20)
    ms_b = timed(bwd2, 20)
    flop_f = 2 * T * n_in * N + 2 * T * r * (2 * n_in + N)
    flop_b = 2 * T * n_in * N + 4 * T * r * (2 * n_in + N)
    res["gate_up_fused"] = {"fwd_ms": round(ms_f, 3), "bwd_ms": round(ms_b, 3),
                            "fwd_TFLOPs": round(flop_f / (ms_f * 1e-3) / 1e12, 1),
                            "bwd_TFLOPs": round(flop_b / (ms_b * 1e-3) / 1e12, 1)}
    d = plain["down"]
    fused_ms = ms_f + ms_b + d["fwd_ms"] + d["bwd_ms"]
    tf2 = tot_flop / (fused_ms * 1e-3) / 1e12
    res["mlp_fused_fwd_bwd_ms"] = round(fused_ms, 3)
    res["mlp_fused_fwd_bwd_TFLOPs"] = round(tf2, 1)
    res["mlp_fused_frac_of_bf16_peak"] = round(tf2 / BF16_PEAK_TFLOPS, 4)

    # gate and up at T = 1792 (7 x 112 tiles): with the smallest forward
    # workspace the GEMM dequantizes the weight inside its LDS staging (W_hat
    # never written); with the full one (the default) it expands W_hat first
    Tf = 1792
    Xf = X[:Tf].contiguous()
    Yf = torch.empty(Tf, N, dtype=torch.bfloat16, device=dev)
    flop_ff = 2 * Tf * n_in * N + 2 * Tf * r * (2 * n_in + N)
    for key, need in (("gate_up_fused_nf4_fwd_T1792", q.qlora_workspace_bytes_fwd_min(Tf, n_in, outs, r)),
                      ("gate_up_expanded_fwd_T1792", q.qlora_workspace_bytes_multi(Tf, n_in, outs, r, False))):
        wsff = q.make_workspace(need, dev)

        def fwdf():
            q.qlora_linear_fwd_multi(Ws, Xf, As, Bs, r, alpha, Y=Yf, ws=wsff)

        for _ in range(4):
            fwdf()
        ms_ff = timed(fwdf, 20)
        tff = flop_ff / (ms_ff * 1e-3) / 1e12
        res[key] = {"fwd_ms": round(ms_ff, 3), "fwd_TFLOPs": round(tff, 1),
                    "frac_of_bf16_peak": round(tff / BF16_PEAK_TFLOPS, 4), "workspace_bytes": int(need)}
        del wsff
    del Ws, X, dY, Y, dX, wsf, wsb
    torch.cuda.empty_cache()
    return res


def blas_threads():
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"])
    except Exception:
        pass
    return None


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cores_in_affinity": host_cores(), "blas_threads": blas_threads(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


class SclkSampler:
    """Samples the GPU shader clock (the active level of pp_dpm_sclk of the
    device torch uses) every few milliseconds on a host thread while the
    large-token legs run; reports min / median / max in MHz, or why it could
    not read them."""

    def __init__(self, period_s=0.005):
        import threading
        self.period = period_s
        self.samples = []
        self.stop_flag = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)
        self.path = self._find()

    @staticmethod
    def _find():
        import glob
        try:
            import torch
            pr = torch.cuda.get_device_properties(0)
            bdf = "%04x:%02x:%02x.0" % (getattr(pr, "pci_domain_id", 0), pr.pci_bus_id, pr.pci_device_id)
            cand = f"/sys/bus/pci/devices/{bdf}/pp_dpm_sclk"
            if os.path.exists(cand):
                return cand
        except Exception:
            pass
        found = glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")
        return found[0] if len(found) == 1 else None

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if line.strip().endswith("*"):
                    m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                    if m:
                        return int(m.group(1))
        return None

    def _run(self):
        while not self.stop_flag.is_set():
            try:
                v = self._read()
                if v is not None:
                    self.samples.append(v)
            except OSError:
                return
            self.stop_flag.wait(self.period)

    def start(self):
        if self.path:
            self.thread.start()

    def stop(self):
        if not self.path:
            return {"unavailable": "no readable pp_dpm_sclk for the device"}
        self.stop_flag.set()
        self.thread.join()
        v = sorted(self.samples)
        if not v:
            return {"unavailable": f"{self.path} gave no active level"}
        return {"min": v[0], "median": v[len(v) // 2], "max": v[-1], "samples": len(v),
                "source": self.path}


def cpu_baseline(n_out, n_in, r, alpha, X1, X16, A, B, step_bytes):
    """The oracle (NumPy, fp64 BLAS) doing the same step on the same workload:
    dequantize an NF4 weight it quantized itself from the same seeded fp32
    weight, then the T=1 and T=16 forwards; repeated for ~10 s."""
    import numpy as np
    import torch
    import synth
    from oracle import dense, native, nf4

    def bits(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    codes, aq, sc = nf4.quantize(synth.weight(2, 0, n_out, n_in), nearest=native.nearest_level)
    hx1, hx16, ha, hb = bits(X1), bits(X16), bits(A), bits(B)
    n = 0
    t0 = time.perf_counter()
    while True:
        w_hat = nf4.dequantize(codes, aq, sc).reshape(n_out, n_in)
        dense.linear_fwd(w_hat, hx1, ha, hb, alpha, r)
        w_hat = nf4.dequantize(codes, aq, sc).reshape(n_out, n_in)
        dense.linear_fwd(w_hat, hx16, ha, hb, alpha, r)
        n += 1
        if time.perf_counter() - t0 > 10.0 or n >= 50:
            break
    dt = time.perf_counter() - t0
    threads = blas_threads() or host_cores()
    return {"value": round(step_bytes * n / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} steps (dequantize + T=1 and T=16 forward, fp64 BLAS on {threads} threads) "
                      f"of the same workload on one weight, {dt:.1f} s"}


def step_flop(T, n_in, n_out, r):
    """fwd + bwd algorithmic flop of one projection: 4 T in out + 6 T r (in + out)
    (no weight-gradient GEMM: the NF4 weight is frozen)."""
    return 4 * T * n_in * n_out + 6 * T * r * (n_in + n_out)


def oracle_step_timing(synth, wid, t_rows=256, out_rows=2048):
    """The oracle's fwd + bwd of every projection of workload `wid`, timed on
    the host on a bounded sub-problem and scaled to the whole step by
    operation counts: per projection the oracle quantizes (untimed) the first
    `out_rows` rows of the seeded fp32 weight, then dequantizes them and runs
    Y, dX, dA, dB in fp64 for the first `t_rows` tokens (timed).  The GEMM
    part scales with T * out * in, the dequantization with out * in."""
    import numpy as np
    from oracle import dense, native, nf4
    wl = synth.WORKLOADS[wid]
    T, r, alpha = wl.tokens[0], wl.r, wl.alpha
    total_s, total_flop = 0.0, 0
    for pi, p in enumerate(wl.projections):
        n_out, n_in = p.out_features, p.in_features
        ro = min(out_rows, n_out)
        w = synth.weight(wid, pi, n_out, n_in)[:ro]
        X = synth.activations(wid, pi, t_rows, n_in)
        dY = synth.activations(wid, pi, t_rows, ro, "dY")
        A = synth.lora_A(wid, pi, r, n_in)
        B = synth.lora_B(wid, pi, n_out, r)[:ro]
        codes, aq, sc = nf4.quantize(w, nearest=native.nearest_level)
        t0 = time.perf_counter()
        w_hat = nf4.dequantize(codes, aq, sc).reshape(ro, n_in)
        t1 = time.perf_counter()
        dense.linear_fwd(w_hat, X, A, B, alpha, r)
        dense.linear_bwd(w_hat, X, dY, A, B, alpha, r)
        t2 = time.perf_counter()
        total_s += (t1 - t0) * (n_out / ro) + (t2 - t1) * (T / t_rows) * (n_out / ro)
        total_flop += step_flop(T, n_in, n_out, r)
    threads = blas_threads() or host_cores()
    return {"value": round(total_flop / total_s / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "step_s_estimated": round(total_s, 2),
            "sample": f"per projection: dequantize of {out_rows} weight rows and fp64 fwd+bwd of "
                      f"{t_rows} tokens x those rows, scaled to the full step by operation counts"}


def flat_quantize_leg(q, synth, dev, with_oracle):
    """nf4_quantize of a 2^30-element fp32 tensor (N(0, 0.02)): the seeded
    recipe's first 2^26 draws (seed 5000) repeated 16 times on the device
    (the quantize cost depends only on the value distribution).  4 B read and
    0.515869 B written per weight.  Timed over 10 calls after 20 untimed
    ones (the clocks settle under sustained load);
    the oracle (NumPy + the plain-C nearest-level search) quantizes a 2^24
    sample of the same draws on the host, scaled to 2^30 elements."""
    import numpy as np
    import torch
    n = synth.FLAT_QUANTIZE_NUMEL
    part = synth.normal_f32(synth.FLAT_QUANTIZE_SEED, (1 << 26,), synth.W_STD)
    w = torch.from_numpy(part).to(dev).repeat(n // part.size)
    codes, aq, sc = q.nf4_quantize(w)
    for _ in range(20):
        q.nf4_quantize(w, codes, aq, sc)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    k = 10
    for _ in range(k):
        q.nf4_quantize(w, codes, aq, sc)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / k
    nbytes = int(n * (4 + NF4_BYTES_PER_WEIGHT))
    gbs = nbytes / (us * 1e-6) / 1e9
    res = {"numel": n, "us_per_call": round(us, 1), "algorithmic_bytes": nbytes, "GB_per_s": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del w, codes, aq, sc
    torch.cuda.empty_cache()
    if with_oracle:
        from oracle import native, nf4
        m = 1 << 24
        t0 = time.perf_counter()
        nf4.quantize(part[:m], nearest=native.nearest_level)
        dt = (time.perf_counter() - t0) * (n / m)
        res["oracle"] = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "kind": "oracle",
                         "cores": int(os.environ.get("OMP_NUM_THREADS", host_cores())),
                         "sample": "quantize of 2^24 elements (NumPy fp32 + plain-C nearest level, "
                                   "OpenMP), scaled to 2^30", "call_s_estimated": round(dt, 1)}
    return res


def large_step_leg(q, synth, dev, bf, wid, steps):
    """fwd + bwd of every projection of workload `wid` (the 8B attention
    projections q, k, v, o at T = 8192, r = 16; the 70B MLP gate, up, down at
    T = 4096, r = 64): a step is each projection's forward then backward, in
    order, each projection on its own weight, activations and gradients (the
    step's working set is several times the 256 MB last-level cache).  2
    untimed steps, then `steps` timed steps with events around every call."""
    import torch
    wl = synth.WORKLOADS[wid]
    T, r, alpha = wl.tokens[0], wl.r, wl.alpha
    items = []
    ws_f = ws_b = 0
    for pi, p in enumerate(wl.projections):
        n_out, n_in = p.out_features, p.in_features
        w = torch.from_numpy(synth.weight(wid, pi, n_out, n_in)).to(dev)
        it = {"name": p.name, "out": n_out, "in": n_in, "W": q.nf4_quantize_weight(w),
              "X": bf(synth.activations(wid, pi, T, n_in)), "dY": bf(synth.activations(wid, pi, T, n_out, "dY")),
              "A": bf(synth.lora_A(wid, pi, r, n_in)), "B": bf(synth.lora_B(wid, pi, n_out, r)),
              "Y": torch.empty(T, n_out, dtype=torch.bfloat16, device=dev),
              "dX": torch.empty(T, n_in, dtype=torch.bfloat16, device=dev),
              "dA": torch.empty(r, n_in, dtype=torch.float32, device=dev),
              "dB": torch.empty(n_out, r, dtype=torch.float32, device=dev)}
        del w
        items.append(it)
        ws_f = max(ws_f, q.qlora_workspace_bytes(T, n_in, n_out, r, False))
        ws_b = max(ws_b, q.qlora_workspace_bytes(T, n_in, n_out, r, True))
    wsf, wsb = q.make_workspace(ws_f, dev), q.make_workspace(ws_b, dev)

    def run(evs=None):
        for j, it in enumerate(items):
            if evs is not None:
                evs[j][0].record()
            q.qlora_linear_fwd(it["W"], it["X"], it["A"], it["B"], r, alpha, Y=it["Y"], ws=wsf)
            if evs is not None:
                evs[j][1].record()
            q.qlora_linear_bwd(it["W"], it["X"], it["dY"], it["A"], it["B"], r, alpha, dX=it["dX"], dA=it["dA"],
                               dB=it["dB"], ws=wsb)
            if evs is not None:
                evs[j][2].record()

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    all_evs = [[(mk(), mk(), mk()) for _ in items] for _ in range(steps)]
    for k in range(steps):
        run(all_evs[k])
    torch.cuda.synchronize()
    res = {"T": T, "r": r, "alpha": alpha, "steps": steps}
    tot_flop, tot_ms = 0, 0.0
    for j, it in enumerate(items):
        f_ms = sum(all_evs[k][j][0].elapsed_time(all_evs[k][j][1]) for k in range(steps)) / steps
        b_ms = sum(all_evs[k][j][1].elapsed_time(all_evs[k][j][2]) for k in range(steps)) / steps
        n_in, n_out = it["in"], it["out"]
        flop_f = 2 * T * n_in * n_out + 2 * T * r * (n_in + n_out)
        flop_b = 2 * T * n_in * n_out + 4 * T * r * (n_in + n_out)
        res[it["name"]] = {"out": n_out, "in": n_in, "fwd_ms": round(f_ms, 3), "bwd_ms": round(b_ms, 3),
                           "fwd_TFLOPs": round(flop_f / (f_ms * 1e-3) / 1e12, 1),
                           "bwd_TFLOPs": round(flop_b / (b_ms * 1e-3) / 1e12, 1)}
        tot_flop += flop_f + flop_b
        tot_ms += f_ms + b_ms
    step_ms = all_evs[0][0][0].elapsed_time(all_evs[-1][-1][2]) / steps
    tf = tot_flop / (step_ms * 1e-3) / 1e12
    res.update({"step_flop": tot_flop, "step_ms": round(step_ms, 3), "sum_of_calls_ms": round(tot_ms, 3),
                "fwd_bwd_TFLOPs": round(tf, 1), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)})
    del items, wsf, wsb
    torch.cuda.empty_cache()
    return res


def mid_tokens_leg(q, synth, dev, bf, n=20):
    """Forward and backward calls at token counts between the small-token
    kernels and full GEMM grids (64 and 256 tokens: the GEMMs split K), on the
    8B gate (4096 -> 14336) and down (14336 -> 4096) shapes at r = 64 and the
    q_proj shape (4096 -> 4096) at r = 16; the backward with the full workspace
    (expanded W_hat^T) and with the smallest (fused dX).  Each call is warmed
    up, then timed over n calls with events."""
    import torch
    res = {}
    for name, wid, pi in (("8b_gate", 3, 0), ("8b_down", 3, 2), ("q_proj", 4, 0)):
        wl = synth.WORKLOADS[wid]
        p = wl.projections[pi]
        n_out, n_in, r, alpha = p.out_features, p.in_features, wl.r, wl.alpha
        w = torch.from_numpy(synth.weight(wid, pi, n_out, n_in)).to(dev)
        W = q.nf4_quantize_weight(w)
        del w
        A = bf(synth.lora_A(wid, pi, r, n_in))
        B = bf(synth.lora_B(wid, pi, n_out, r))
        res[name] = {"out": n_out, "in": n_in, "r": r}
        for T in (64, 256):
            X = bf(synth.activations(wid, pi, T, n_in))
            dY = bf(synth.activations(wid, pi, T, n_out, "dY"))
            Y = torch.empty(T, n_out, dtype=torch.bfloat16, device=dev)
            dX = torch.empty(T, n_in, dtype=torch.bfloat16, device=dev)
            dA = torch.empty(r, n_in, dtype=torch.float32, device=dev)
            dB = torch.empty(n_out, r, dtype=torch.float32, device=dev)
            wf = q.make_workspace(q.qlora_workspace_bytes(T, n_in, n_out, r, False), dev)
            wb = q.make_workspace(q.qlora_workspace_bytes(T, n_in, n_out, r, True), dev)
            wm = q.make_workspace(q.qlora_workspace_bytes_bwd_min(T, n_in, [n_out], r), dev)

            def timed(fn):
                for _ in range(4):
                    fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(n):
                    fn()
                e1.record()
                e1.synchronize()
                return e0.elapsed_time(e1) / n * 1e3

            f_us = timed(lambda: q.qlora_linear_fwd(W, X, A, B, r, alpha, Y=Y, ws=wf))
            b_us = timed(lambda: q.qlora_linear_bwd(W, X, dY, A, B, r, alpha, dX, dA, dB, ws=wb))
            m_us = timed(lambda: q.qlora_linear_bwd(W, X, dY, A, B, r, alpha, dX, dA, dB, ws=wm))
            flop_f = 2 * T * n_in * n_out + 2 * T * r * (n_in + n_out)
            flop_b = 2 * T * n_in * n_out + 4 * T * r * (n_in + n_out)
            res[name][f"T{T}"] = {"fwd_us": round(f_us, 1), "bwd_us": round(b_us, 1),
                                  "bwd_min_workspace_us": round(m_us, 1),
                                  "fwd_TFLOPs": round(flop_f / (f_us * 1e-6) / 1e12, 1),
                                  "bwd_TFLOPs": round(flop_b / (b_us * 1e-6) / 1e12, 1),
                                  "bwd_workspace_bytes": {"full": int(wb.numel()), "min": int(wm.numel())}}
            del X, dY, Y, dX, dA, dB, wf, wb, wm
        del W
    torch.cuda.empty_cache()
    return res


def grouped_step_leg(q, synth, dev, bf, wid, groups, steps, step_flop, bwd_min=False):
    """The fwd + bwd step of workload `wid` with the projections that share
    their input X as one multi-projection call each way (`groups`: lists of
    projection indices, e.g. q|k|v then o): one LoRA down-projection pass over
    X, one GEMM launch over the group's stacked weights, one dX GEMM over
    their concatenated outputs.  bwd_min: the backward gets the smallest
    workspace it accepts, so its dX GEMM dequantizes the weight tiles while
    staging them instead of expanding W_hat^T.  2 untimed steps, then `steps`
    timed steps with events around every call."""
    import torch
    wl = synth.WORKLOADS[wid]
    T, r, alpha = wl.tokens[0], wl.r, wl.alpha
    items = []
    ws_f = ws_b = 0
    for g in groups:
        projs = [wl.projections[i] for i in g]
        n_in = projs[0].in_features
        outs = [p.out_features for p in projs]
        Ws, As, Bs = [], [], []
        for i, p in zip(g, projs):
            w = torch.from_numpy(synth.weight(wid, i, p.out_features, n_in)).to(dev)
            Ws.append(q.nf4_quantize_weight(w))
            del w
            As.append(bf(synth.lora_A(wid, i, r, n_in)))
            Bs.append(bf(synth.lora_B(wid, i, p.out_features, r)))
        N = sum(outs)
        items.append({"name": "|".join(p.name for p in projs), "Ws": Ws, "As": As, "Bs": Bs,
                      "X": bf(synth.activations(wid, g[0], T, n_in)),
                      "dY": bf(synth.activations(wid, g[0], T, N, "dY")),
                      "Y": torch.empty(T, N, dtype=torch.bfloat16, device=dev),
                      "dX": torch.empty(T, n_in, dtype=torch.bfloat16, device=dev),
                      "dAs": [torch.empty(r, n_in, dtype=torch.float32, device=dev) for _ in g],
                      "dBs": [torch.empty(o, r, dtype=torch.float32, device=dev) for o in outs]})
        ws_f = max(ws_f, q.qlora_workspace_bytes_multi(T, n_in, outs, r, False))
        need_b = (q.qlora_workspace_bytes_bwd_min(T, n_in, outs, r) if bwd_min
                  else q.qlora_workspace_bytes_multi(T, n_in, outs, r, True))
        ws_b = max(ws_b, need_b)
    wsf, wsb = q.make_workspace(ws_f, dev), q.make_workspace(ws_b, dev)

    def run(evs=None):
        for j, it in enumerate(items):
            if evs is not None:
                evs[j][0].record()
            q.qlora_linear_fwd_multi(it["Ws"], it["X"], it["As"], it["Bs"], r, alpha, Y=it["Y"], ws=wsf)
            if evs is not None:
                evs[j][1].record()
            q.qlora_linear_bwd_multi(it["Ws"], it["X"], it["dY"], it["As"], it["Bs"], r, alpha, dX=it["dX"],
                                     dAs=it["dAs"], dBs=it["dBs"], ws=wsb)
            if evs is not None:
                evs[j][2].record()

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    all_evs = [[(mk(), mk(), mk()) for _ in items] for _ in range(steps)]
    for k in range(steps):
        run(all_evs[k])
    torch.cuda.synchronize()
    res = {"T": T, "r": r, "steps": steps, "bwd_workspace_bytes": int(ws_b)}
    for j, it in enumerate(items):
        f_ms = sum(all_evs[k][j][0].elapsed_time(all_evs[k][j][1]) for k in range(steps)) / steps
        b_ms = sum(all_evs[k][j][1].elapsed_time(all_evs[k][j][2]) for k in range(steps)) / steps
        res[it["name"]] = {"fwd_ms": round(f_ms, 3), "bwd_ms": round(b_ms, 3)}
    step_ms = all_evs[0][0][0].elapsed_time(all_evs[-1][-1][2]) / steps
    tf = step_flop / (step_ms * 1e-3) / 1e12
    res.update({"step_ms": round(step_ms, 3), "fwd_bwd_TFLOPs": round(tf, 1),
                "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)})
    del items, wsf, wsb
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
