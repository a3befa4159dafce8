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
fwd+bwd TFLOP/s of the 8B-MLP projections (gate, up 4096 -> 14336, down
14336 -> 4096; T = 4096, r = 64) -- the large-token half of the metric;
skipped with --no-train.

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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pool", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--counters-probe", action="store_true",
                    help="only run the T=16 small-token forward over the weight pool and a "
                         "256 MiB copy (for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes)")
    ap.add_argument("--mlp-probe", action="store_true",
                    help="only run the 8B-MLP fwd + bwd leg and print its figures (for rocprofv3 "
                         "--pmc passes over the large-token GEMMs)")
    return ap.parse_args()


# Sources that define the small-token forward kernel; the HBM traffic recorded
# from hardware counters is reported only while they are unchanged.
DECODE_SOURCES = ("bit_nf4_quantized_20_amd/csrc/k_decode.hip",
                  "bit_nf4_quantized_20_amd/csrc/nf4_format.hpp",
                  "bit_nf4_quantized_20_amd/csrc/common.hpp",
                  "bit_nf4_quantized_20_amd/build.py")
TRAFFIC_RECORD = "profiles/k_decode_fwd_split_qproj4096x4096_T16_traffic.md"
COPY_BYTES = 256 << 20


def decode_fingerprint():
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
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
    wl = synth.WORKLOADS[2]
    proj = wl.projections[0]
    n_out, n_in, r, alpha = proj.out_features, proj.in_features, wl.r, wl.alpha

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

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
        print(json.dumps(train_leg(q, synth, dev, bf)), flush=True)
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

    extra = {
        "fwd_T1": {"us_per_call": round(us1, 3), "GB_per_s": round(b1 / (us1 * 1e-6) / 1e9, 1),
                   "algorithmic_bytes": b1},
        "fwd_T16": {"us_per_call": round(us16, 3), "GB_per_s": round(ach16, 1),
                    "algorithmic_bytes": b16},
        "eager_us_per_call": {"T1": round(eager_us(X1, Y1, 200), 2),
                              "T16": round(eager_us(X16, Y16, 200), 2)},
        "timing": "HIP graph replay of back-to-back calls (events on the library's stream)",
        "weight_pool_bytes": int(P * n_out * n_in * NF4_BYTES_PER_WEIGHT),
    }

    # ------------------------------------------------------------ quantize
    codes, aq, sc = pool[0].codes, pool[0].absmax_q, pool[0].absmax_scale
    for _ in range(3):
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
        for _ in range(3):
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
    extra["merge_8b_gate"] = merge_leg(q, synth, dev, bf)

    # ------------------------------------------- q|k|v at decode sizes
    extra["qkv8b_decode"] = qkv_decode_leg(q, synth, dev, bf)

    # ------------------------------ MLP-sized weights at decode sizes
    extra["mlp_weights_decode"] = mlp_decode_leg(q, synth, dev, bf)

    # ------------------------------------------- large-token fwd + bwd
    if not args.no_train:
        extra["mlp8b_fwd_bwd"] = train_leg(q, synth, dev, bf)

    # --------------------------------------------------------- cpu baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w_host, pool[0], n_out, n_in, r, alpha, X1, X16, A, B, b1 + b16)

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
        "wall_s_timed_region": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


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


def merge_leg(q, synth, dev, bf):
    """qlora_merge of the 8B-MLP gate projection (14336 x 4096 NF4, r = 64):
    W_merged = bf16(W_hat + (alpha/r) B A), HBM-bound (codes + absmax read,
    2 B per weight written)."""
    import torch
    wl = synth.WORKLOADS[3]
    p = wl.projections[0]
    r, alpha = wl.r, wl.alpha
    n_out, n_in = p.out_features, p.in_features
    W = q.nf4_quantize_weight(torch.from_numpy(synth.weight(3, 0, n_out, n_in)).to(dev))
    A = bf(synth.lora_A(3, 0, r, n_in))
    B = bf(synth.lora_B(3, 0, n_out, r))
    out = torch.empty(n_out, n_in, dtype=torch.bfloat16, device=dev)
    ws = q.make_workspace(q.qlora_merge_workspace_bytes(n_in, n_out, r), dev)
    for _ in range(3):
        q.qlora_merge(W, A, B, r, alpha, out=out, ws=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    n = 20
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
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "decode T=16 x %d, copy %d B x 4" % (len(pool), COPY_BYTES),
                      "sources_sha256": decode_fingerprint()}), flush=True)


def train_leg(q, synth, dev, bf):
    """fwd + bwd of the 8B-MLP projections (gate and up 4096 -> 14336, down
    14336 -> 4096; T = 4096, r = 64, alpha = 128): per projection and for the
    three together.  Each call is warmed up, then timed over 20 calls."""
    import torch
    wl = synth.WORKLOADS[3]
    T, r, alpha = wl.tokens[0], wl.r, wl.alpha
    res = {"T": T, "r": r, "alpha": alpha}
    tot_flop, tot_ms, tot_dms = 0.0, 0.0, 0.0

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

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
        wsf = q.make_workspace(q.qlora_workspace_bytes(T, n_in, n_out, r, False), dev)
        wsb = q.make_workspace(q.qlora_workspace_bytes(T, n_in, n_out, r, True), dev)

        def fwd():
            q.qlora_linear_fwd(W, X, A, B, r, alpha, Y=Y, ws=wsf)

        def bwd():
            q.qlora_linear_bwd(W, X, dY, A, B, r, alpha, dX=dX, dA=dA, dB=dB, ws=wsb)

        for _ in range(8):
            fwd()
            bwd()
        ms_f = timed(fwd, 20)
        ms_b = timed(bwd, 20)
        flop_f = 2 * T * n_in * n_out + 2 * T * r * (n_in + n_out)
        flop_b = 2 * T * n_in * n_out + 4 * T * r * (n_in + n_out)
        res[p.name] = {"out": n_out, "in": n_in, "fwd_ms": round(ms_f, 3), "bwd_ms": round(ms_b, 3),
                       "fwd_TFLOPs": round(flop_f / (ms_f * 1e-3) / 1e12, 1),
                       "bwd_TFLOPs": round(flop_b / (ms_b * 1e-3) / 1e12, 1),
                       "fwd_bwd_TFLOPs": round((flop_f + flop_b) / ((ms_f + ms_b) * 1e-3) / 1e12, 1)}
        tot_flop += flop_f + flop_b
        tot_ms += ms_f + ms_b

        # the same step with LoRA dropout (p = 0.05, a fresh seeded keep mask)
        keep = torch.from_numpy(synth.keep_mask(synth.seed_for(3, pi, "keep"), T, n_in, DROPOUT_P)).to(dev)
        wdf = q.make_workspace(q.qlora_workspace_bytes_dropout(T, n_in, n_out, r, False), dev)

        def dfwd():
            q.qlora_linear_fwd_dropout(W, X, keep, DROPOUT_P, A, B, r, alpha, Y=Y, ws=wdf)

        def dbwd():
            q.qlora_linear_bwd_dropout(W, X, dY, keep, DROPOUT_P, A, B, r, alpha, dX=dX, dA=dA, dB=dB,
                                       ws=wsb)

        for _ in range(8):
            dfwd()
            dbwd()
        dms_f = timed(dfwd, 20)
        dms_b = timed(dbwd, 20)
        res[p.name]["dropout_fwd_ms"] = round(dms_f, 3)
        res[p.name]["dropout_bwd_ms"] = round(dms_b, 3)
        tot_dms += dms_f + dms_b
        del W, X, dY, Y, dX, wsf, wsb, wdf, keep
    tf = tot_flop / (tot_ms * 1e-3) / 1e12
    res["mlp_fwd_bwd_ms"] = round(tot_ms, 3)
    res["mlp_fwd_bwd_TFLOPs"] = round(tf, 1)
    res["frac_of_bf16_peak"] = round(tf / BF16_PEAK_TFLOPS, 4)
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

    for _ in range(8):
        fwd2()
        bwd2()
    ms_f = timed(fwd2, 20)
    ms_b = timed(bwd2, 20)
    flop_f = 2 * T * n_in * N + 2 * T * r * (2 * n_in + N)
    flop_b = 2 * T * n_in * N + 4 * T * r * (2 * n_in + N)
    res["gate_up_fused"] = {"fwd_ms": round(ms_f, 3), "bwd_ms": round(ms_b, 3),
                            "fwd_TFLOPs": round(flop_f / (ms_f * 1e-3) / 1e12, 1),
                            "bwd_TFLOPs": round(flop_b / (ms_b * 1e-3) / 1e12, 1)}
    d = res["down"]
    fused_ms = ms_f + ms_b + d["fwd_ms"] + d["bwd_ms"]
    tf2 = tot_flop / (fused_ms * 1e-3) / 1e12
    res["mlp_fused_fwd_bwd_ms"] = round(fused_ms, 3)
    res["mlp_fused_fwd_bwd_TFLOPs"] = round(tf2, 1)
    res["mlp_fused_frac_of_bf16_peak"] = round(tf2 / BF16_PEAK_TFLOPS, 4)

    # below 2048 tokens the forward keeps the dequantization inside the GEMM's
    # LDS staging (W_hat never written): gate and up at T = 1792 (7 x 112 tiles)
    Tf = 1792
    Xf = X[:Tf].contiguous()
    Yf = torch.empty(Tf, N, dtype=torch.bfloat16, device=dev)
    wsff = q.make_workspace(q.qlora_workspace_bytes_multi(Tf, n_in, outs, r, False), dev)

    def fwdf():
        q.qlora_linear_fwd_multi(Ws, Xf, As, Bs, r, alpha, Y=Yf, ws=wsff)

    for _ in range(8):
        fwdf()
    ms_ff = timed(fwdf, 20)
    flop_ff = 2 * Tf * n_in * N + 2 * Tf * r * (2 * n_in + N)
    tff = flop_ff / (ms_ff * 1e-3) / 1e12
    res["gate_up_fused_nf4_fwd_T1792"] = {"fwd_ms": round(ms_ff, 3), "fwd_TFLOPs": round(tff, 1),
                                          "frac_of_bf16_peak": round(tff / BF16_PEAK_TFLOPS, 4)}
    return res


def cpu_baseline(w_host, W, n_out, n_in, r, alpha, X1, X16, A, B, step_bytes):
    """The oracle (NumPy, fp64 BLAS) doing the same step: dequantize one NF4
    weight and run the T=1 and T=16 forwards; repeated for ~10 s."""
    import numpy as np
    import torch
    from oracle import dense, nf4

    def bits(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    codes = W.codes.cpu().numpy()
    aq = W.absmax_q.cpu().numpy()
    sc = W.absmax_scale.cpu().numpy()
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
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": round(step_bytes * n / dt / 1e9, 4), "unit": "GB/s", "cores": min(cores, threads),
            "kind": "oracle",
            "sample": f"{n} steps (dequantize + T=1 and T=16 forward, fp64 BLAS) of the same "
                      f"workload on one weight, {dt:.1f} s"}


if __name__ == "__main__":
    main()
