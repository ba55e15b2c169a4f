"""Benchmark of the DBF linear forward on one MI355X.

Workload (default): the 4096x4096 projection at about 1 bit per weight
(n = m = 4096, k = 2048), signs uniform +/-1, a, b ~ |N(0,1)|*0.02,
mid ~ |N(0,1)|, x ~ N(0,1) in fp16, batch 1.  One step is one full forward
(input scaling, both signed sums, middle and output scaling) of one layer.
The step rotates over R distinct copies of the layer's packed weights,
R * bytes >= 512 MB, so that the 256 MB Infinity Cache cannot hold them and
every step streams its weights from HBM.  x is resident in HBM before the
timed region starts.

Metric: packed-weight GB/s = (n*k + k*m)/8 + 2*(n + k + m) bytes per step,
divided by the wall time of the timed steps (events around K steps, after W
warm-up steps).  A secondary measurement covers the batch-2048 half of the
metric (TFLOP/s-equivalent = 2*batch*k*(n+m) per forward) on the 4096x4096
projection at about 2 bits per weight (k = 4096).

Also reported: the roofline of the dominant kernel, from per-launch HIP
events recorded by the library on the launch stream over a second pass of
the same steps, and the CPU oracle (fp64, dense reconstruction) timed on the
host on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix-core peak


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=4860)
    p.add_argument("--warmup", type=int, default=486)
    p.add_argument("--rotate-mb", type=int, default=512)
    p.add_argument("--mode", choices=("graph", "eager"), default="graph",
                   help="graph: the timed steps replay a captured HIP graph of forwards")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-secondary", action="store_true", help="skip the batch-2048 measurement")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="only run a plain device copy of this size (counter scaling) and exit")
    p.add_argument("--no-block", action="store_true", help="skip the decoder-block measurement")
    p.add_argument("--no-backward", action="store_true", help="skip the gradient measurement")
    p.add_argument("--all-configs", action="store_true",
                   help="instead of the headline line: one JSON line per workload layer and batch "
                        "(decode at batch 1 and 16, prefill at batch 2048)")
    p.add_argument("--no-bqq", action="store_true", help="skip the BQQ-form layer measurement")
    p.add_argument("--no-factorize", action="store_true", help="skip the factorization measurement")
    p.add_argument("--no-context", action="store_true", help="skip the fp16-matvec and device-copy context")
    p.add_argument("--factor-cpu", action="store_true",
                   help="also time the factorization oracle (one outer x one inner iteration) on the host")
    p.add_argument("--only", choices=("decode", "prefill", "block", "backward", "bqq", "factorize", "context"),
                   default=None,
                   help="run one leg only (for profiling)")
    p.add_argument("--decode-path", choices=("mfma", "table"), default="mfma",
                   help="decode kernels: matrix cores (default) or vector-ALU lookup tables")
    return p.parse_args()


def layer_copies(layer, count):
    import dbf_linear_fwd_amd as dbf
    return [dbf.Layer(layer.A, layer.B, layer.a, layer.mid, layer.b, max_batch=max(layer.X)) for _ in range(count)]


def time_steps(fwd, steps, warmup, mode):
    """Run `fwd(i)` for warm-up then timed steps; returns elapsed seconds of the timed steps."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fwd(i)
    torch.cuda.synchronize()
    if mode == "graph":
        # capture one pass over the rotation, replay it for the timed steps
        period = getattr(fwd, "period", 1)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(period):
                    fwd(i)
        stream.wait_stream(s)
        reps = max(1, steps // period)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3, reps * period
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fwd(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3, steps


def kernel_times(layers, fwd, steps):
    """Per-kernel average event time (ms) over `steps` eager steps."""
    import dbf_linear_fwd_amd as dbf
    import torch
    for L in layers:
        dbf.dbf_timing_enable(L.handle, True)
        dbf.dbf_timing_read(L.handle)
    torch.cuda.synchronize()
    for i in range(steps):
        fwd(i)
    torch.cuda.synchronize()
    tot = {}
    for L in layers:
        for name, v in dbf.dbf_timing_read(L.handle).items():
            t = tot.setdefault(name, [0, 0.0])
            t[0] += v["launches"]
            t[1] += v["total_ms"]
        dbf.dbf_timing_enable(L.handle, False)
    return {k: {"launches": v[0], "avg_us": 1e3 * v[1] / max(v[0], 1)} for k, v in tot.items()}


def decode_kernel_bytes(layer, batch):
    """Algorithmic bytes each decode kernel must move (signs + scales + activations)."""
    n, m, k = layer.n, layer.m, layer.k
    return {
        "decode_stage1": k * m // 8 + 2 * m + 2 * batch * m,
        "decode_stage2": n * k // 8 + 2 * k + 2 * n + 2 * batch * n,
    }


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    record (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's reading), or
    None when the kernel's source has changed since it was recorded."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    try:
        text = open(path).read()
        rec = json.loads(re.search(r"```json\n(.*?)```", text, re.S).group(1))
        k = rec["kernels"][kernel]
        src = open(os.path.join(ROOT, k["source"]), "rb").read()
    except (OSError, KeyError, AttributeError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest() != k["sha256"]:
        return None
    sc = rec["scale"]
    return 1024.0 * (k["FETCH_SIZE"] * sc["FETCH_SIZE"] + k["WRITE_SIZE"] * sc["WRITE_SIZE"])


def prefill_kernel_flops(layer, batch):
    n, m, k = layer.n, layer.m, layer.k
    return {"prefill_gemm1": 2 * batch * k * m, "prefill_gemm2": 2 * batch * k * n}


def cpu_baseline(layer, seconds):
    """The fp64 oracle (dense reconstruction + X W^T, one batch-1 forward per
    call) on the host, repeated for about `seconds`; GB/s of packed weights.
    Also its two parts on their own (the W reconstruction, 2nmk flops, and
    the product X W^T with W built, 2nm flops per batch row) and one forward
    on a single core."""
    from oracle import dbf_oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    X = layer.X[1]
    calls = 0
    t0 = time.perf_counter()
    while True:
        O.dense_forward(X, layer.A, layer.B, layer.a, layer.mid, layer.b)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = (layer.sign_bytes + layer.scale_bytes) * calls / el / 1e9
    t1 = time.perf_counter()
    W = O.dense_weight(layer.A, layer.B, layer.a, layer.mid, layer.b)
    w_s = time.perf_counter() - t1
    X64 = X.astype(np.float64)
    xw = []
    for _ in range(21):
        t2 = time.perf_counter()
        X64 @ W.T
        xw.append(time.perf_counter() - t2)
    del W
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t3 = time.perf_counter()
            O.dense_forward(X, layer.A, layer.B, layer.a, layer.mid, layer.b)
            one = time.perf_counter() - t3
    return {"value": gbs, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{calls} batch-1 forwards of the 4096x4096 k=2048 layer through the fp64 dense oracle "
                      f"(W rebuilt each call) in {el:.1f} s",
            "w_rebuild_s": round(w_s, 3), "xwt_median_ms": round(1e3 * float(np.median(xw)), 3),
            "one_core_forward_s": None if one is None else round(one, 3),
            "host_cpu_count": os.cpu_count()}


def block_leg(args):
    """The seven linears of a Llama-3-8B-shaped decoder block (q, k, v, o,
    gate, up, down; per-layer k) at batch 1, one after another on one stream,
    over enough copies of the block to stream from HBM: each layer on its own,
    and with the layers that share an input (q, k, v; gate, up) grouped into
    one pair of launches."""
    import torch

    import dbf_linear_fwd_amd as dbf
    from tests import inputs

    layers = inputs.config(5).layers
    by = {L.name: L for L in layers}
    block_bytes = sum(L.sign_bytes + L.scale_bytes for L in layers)
    R = max(1, -(-args.rotate_mb * (1 << 20) // block_bytes))
    print(f"[bench] block: 7 layers, {block_bytes / 2**20:.1f} MiB per block, {R} copies", file=sys.stderr, flush=True)
    copies = [{L.name: dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=1) for L in layers} for _ in range(R)]
    xs = {L.name: torch.from_numpy(L.X[1]).cuda() for L in layers}
    ys = {L.name: torch.empty((1, L.n), dtype=torch.float16, device="cuda") for L in layers}
    order = ["q", "k", "v", "o", "gate", "up", "down"]
    groups = [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]

    def per_layer(i):
        c = copies[i % R]
        for name in order:
            c[name].forward(xs[name], out=ys[name])
    per_layer.period = R

    def grouped(i):
        c = copies[i % R]
        for gr in groups:
            if len(gr) == 1:
                c[gr[0]].forward(xs[gr[0]], out=ys[gr[0]])
            else:
                dbf.forward_group([c[name] for name in gr], xs[gr[0]], [ys[name] for name in gr])
    grouped.period = R

    steps = max(R, min(args.steps // 7, 20 * R))
    res = {"workload": "Llama-3-8B-shaped decoder block of 7 DBF linears (q 4096x4096, k/v 1024x4096, o 4096x4096, "
                       "gate/up 14336x4096, down 4096x14336), k per layer from 1.0-2.3 bits/weight, batch 1",
           "block_bytes": block_bytes, "copies": R}
    for name, fn in (("per_layer", per_layer), ("grouped", grouped)):
        el, done = time_steps(fn, steps, min(args.warmup, 2 * R), args.mode)
        res[name] = {"us_per_block": el * 1e6 / done, "gbs": block_bytes * done / el / 1e9,
                     "launches_per_block": 14 if name == "per_layer" else 8}
        print(f"[bench] block {name}: {res[name]['us_per_block']:.1f} us per block, {res[name]['gbs']:.1f} GB/s",
              file=sys.stderr, flush=True)
    for c in copies:
        for H in c.values():
            H.close()
    torch.cuda.synchronize()
    return res


def backward_leg():
    """Gradients (dX, da, dmid, db) of the 4096x4096, k = 4096 projection at
    batch 2048: four sign products of 2*batch*k*(n or m) flops each (t, s, g,
    h) plus the batch reductions; TFLOP/s-equivalent = 4*batch*k*(n+m) per
    call over the call's time."""
    import torch

    import dbf_linear_fwd_amd as dbf
    from tests import inputs

    layer = inputs.config(3).layers[0]
    bt = 2048
    H = dbf.Layer(layer.A, layer.B, layer.a, layer.mid, layer.b, max_batch=bt, backward=True)
    rng = np.random.default_rng(11)
    x = torch.from_numpy(layer.X[bt]).cuda()
    dy = torch.from_numpy(rng.standard_normal((bt, layer.n)).astype(np.float16)).cuda()

    def step(i):
        H.backward(x, dy)
    el, done = time_steps(step, 30, 5, "eager")
    flops = 4 * bt * layer.k * (layer.n + layer.m)
    kt = kernel_times([H], step, 10)
    print(f"[bench] backward: {flops * done / el / 1e12:.1f} TFLOP/s-eq; kernels {kt}", file=sys.stderr, flush=True)
    H.close()
    return {"value": flops * done / el / 1e12, "unit": "TFLOP/s-eq", "ms_per_call": el * 1e3 / done,
            "kernels": kt, "workload": "gradients of the 4096x4096 projection, k=4096, batch 2048 "
                                       "(dX, da, dmid, db)"}


def all_configs(args):
    """Every layer of the five workloads: decode (batch 1 and 16, weights
    rotated over >= rotate-mb of copies, graph replay) and prefill (batch
    2048).  One JSON line each."""
    import torch

    import dbf_linear_fwd_amd as dbf
    from tests import inputs

    for cid in inputs.CONFIG_IDS:
        cfg = inputs.config(cid)
        for layer in cfg.layers:
            bytes_step = layer.sign_bytes + layer.scale_bytes
            # copies streamed from HBM (at most 256: the 256x256 correctness layer stays cache-resident)
            R = min(256, max(2, -(-args.rotate_mb * (1 << 20) // bytes_step)))
            copies = [dbf.Layer(layer.A, layer.B, layer.a, layer.mid, layer.b, max_batch=16) for _ in range(R)]
            for bt in (1, 16):
                X = layer.X.get(bt)
                if X is None:
                    X = np.random.default_rng(bt).standard_normal((bt, layer.m)).astype(np.float16)
                x = torch.from_numpy(X).cuda()
                y = torch.empty((bt, layer.n), dtype=torch.float16, device="cuda")

                def fwd(i):
                    copies[i % R].forward(x, out=y)
                fwd.period = R
                el, done = time_steps(fwd, max(R, min(args.steps, 10 * R)), min(args.warmup, R), "graph")
                print(json.dumps({"config": cid, "layer": layer.name, "n": layer.n, "m": layer.m, "k": layer.k,
                                  "batch": bt, "path": "decode", "us_per_forward": el * 1e6 / done,
                                  "packed_gbs": bytes_step * done / el / 1e9,
                                  "frac_of_hbm_peak": bytes_step * done / el / 1e9 / HBM_PEAK_GBS,
                                  "copies": R}), flush=True)
            for c in copies:
                c.close()
            del copies
            torch.cuda.synchronize()
            if 2048 in cfg.batches or cid == 3:
                bt = 2048
                L = dbf.Layer(layer.A, layer.B, layer.a, layer.mid, layer.b, max_batch=bt)
                X = layer.X.get(bt)
                if X is None:
                    X = np.random.default_rng(bt).standard_normal((bt, layer.m)).astype(np.float16)
                x = torch.from_numpy(X).cuda()
                y = torch.empty((bt, layer.n), dtype=torch.float16, device="cuda")

                def pf(i):
                    L.forward(x, out=y)
                el, done = time_steps(pf, 30, 5, "eager")
                flops = 2 * bt * layer.k * (layer.n + layer.m)
                print(json.dumps({"config": cid, "layer": layer.name, "n": layer.n, "m": layer.m, "k": layer.k,
                                  "batch": bt, "path": "prefill", "us_per_forward": el * 1e6 / done,
                                  "tflops_eq": flops * done / el / 1e12,
                                  "frac_of_mfma_peak": flops * done / el / 1e12 / MFMA_F16_PEAK_TFLOPS}),
                      flush=True)
                L.close()
                torch.cuda.synchronize()


def bqq_leg(args):
    """A BQQ-form layer (sum of scaled 0/1 matrix products plus rank-one
    terms) of shape 4096x4096 with p = 2 products of inner dimension 1024 --
    2 MiB of bits, the size of the 4096x4096, k = 2048 DBF layer: batch-1
    decode over rotated weight copies (GB/s of bits + scales per forward)
    and batch-2048 prefill (TFLOP/s-equivalent 2 * batch * p d (n + m))."""
    import torch

    import dbf_linear_fwd_amd as dbf
    from tests import inputs

    n, m, d, p = 4096, 4096, 1024, 2
    L = inputs.bqq_layer("bqq", n, m, d, p, 7300, (1, 2048))
    bytes_step = L.bit_bytes + 2 * (n + p * d + m) + 4 * (n + m)
    R = max(1, -(-args.rotate_mb * (1 << 20) // bytes_step))
    print(f"[bench] bqq: {n}x{m} d={d} p={p}, {R} copies", file=sys.stderr, flush=True)
    copies = [dbf.Layer.bqq(L.Y, L.Z, L.r, L.s, L.t, L.u, max_batch=1) for _ in range(R)]
    x = torch.from_numpy(L.X[1]).cuda()
    y = torch.empty((1, n), dtype=torch.float16, device="cuda")

    def fwd(i):
        copies[i % R].forward(x, out=y)
    fwd.period = R
    el, done = time_steps(fwd, max(R, min(args.steps, 10 * R)), min(args.warmup, R), args.mode)
    kt = kernel_times(copies, fwd, min(args.steps, 2 * R))
    res = {"workload": "BQQ-form layer 4096x4096, p=2 products of d=1024 (2 MiB of bits)",
           "decode_b1": {"us_per_forward": el * 1e6 / done, "gbs": bytes_step * done / el / 1e9,
                         "frac_of_hbm_peak": bytes_step * done / el / 1e9 / HBM_PEAK_GBS, "kernels": kt,
                         "bytes_per_forward": bytes_step, "copies": R}}
    print(f"[bench] bqq decode: {res['decode_b1']['us_per_forward']:.2f} us, {res['decode_b1']['gbs']:.1f} GB/s; "
          f"kernels {kt}", file=sys.stderr, flush=True)
    for c in copies:
        c.close()
    del copies
    torch.cuda.synchronize()
    bt = 2048
    H = dbf.Layer.bqq(L.Y, L.Z, L.r, L.s, L.t, L.u, max_batch=bt)
    x = torch.from_numpy(L.X[bt]).cuda()
    y = torch.empty((bt, n), dtype=torch.float16, device="cuda")

    def pf(i):
        H.forward(x, out=y)
    el, done = time_steps(pf, 30, 5, "eager")
    kt = kernel_times([H], pf, 10)
    flops = 2 * bt * p * d * (n + m)
    res["prefill_b2048"] = {"us_per_forward": el * 1e6 / done, "tflops_eq": flops * done / el / 1e12,
                            "frac_of_mfma_peak": flops * done / el / 1e12 / MFMA_F16_PEAK_TFLOPS, "kernels": kt}
    print(f"[bench] bqq prefill: {res['prefill_b2048']['tflops_eq']:.1f} TFLOP/s-eq; kernels {kt}",
          file=sys.stderr, flush=True)
    H.close()
    torch.cuda.synchronize()
    return res


def factorize_leg(args):
    """The factorization of a 4096x4096 matrix into DBF factors with k = 2048
    (about 1 bit per weight): 2 outer iterations of 4 ADMM steps with 8
    power-method steps per SVID, from a seeded random start; wall time per
    call (it synchronizes) and per outer iteration, and the error after each
    outer iteration.  W is a synthetic matrix of i.i.d. N(0, 0.02^2) entries
    (no trained weights are used)."""
    import torch

    import dbf_linear_fwd_amd as dbf

    n = m = 4096
    k = 2048
    g = torch.Generator(device="cpu").manual_seed(21)
    W = (0.02 * torch.randn((n, m), generator=g)).cuda()
    U0 = (torch.randn((n, k), generator=g) * (0.02 / k) ** 0.5).cuda()
    V0 = torch.randn((k, m), generator=g).cuda()
    outer, inner, power = 2, 4, 8
    dbf.factorize(W, k, U0, V0, outer=1, inner=1, power_iters=2)   # library warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    A, B, a, mid, b, err = dbf.factorize(W, k, U0, V0, outer=outer, inner=inner, power_iters=power)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    res = {"workload": f"DBF factorization of a {n}x{m} fp32 matrix (i.i.d. normal), k={k}, {outer} outer x "
                       f"{inner} ADMM iterations, {power} power-method steps per SVID",
           "seconds": el, "ms_per_outer_iteration": el * 1e3 / outer,
           "rel_err_per_outer": [float(e) for e in err.cpu()]}
    print(f"[bench] factorize: {el * 1e3:.1f} ms ({el * 1e3 / outer:.1f} ms per outer iteration), "
          f"err {res['rel_err_per_outer']}", file=sys.stderr, flush=True)
    if args.factor_cpu:
        from oracle import factor_oracle as FO
        t0 = time.perf_counter()
        FO.factorize(W.cpu().double().numpy(), k, U0.cpu().double().numpy(), V0.cpu().double().numpy(),
                     outer=1, inner=1, power_iters=power)
        cel = time.perf_counter() - t0
        res["cpu_oracle_one_outer_one_inner_s"] = cel
        print(f"[bench] factorize oracle (1 outer x 1 inner): {cel:.1f} s", file=sys.stderr, flush=True)
    del W, U0, V0, A, B
    torch.cuda.synchronize()
    return res


def fp16_context_leg(args):
    """Context for the pages' headline (DBF matvec speedup over an fp16
    matvec): on the same GPU, the batch-1 forward of fp16 dense 4096x4096
    and 14336x4096 layers (torch's library matvec) against the DBF decode of
    the 4096x4096 layer at k = 2048 (~1 bit/weight) and k = 4096 (~2
    bits/weight) and of the 14336x4096 MLP layer at k = 4800, each over >=
    rotate-mb of distinct weight copies replayed from a graph; and the
    bandwidth of a plain 1 GiB device copy (the attainable HBM rate)."""
    import torch

    import dbf_linear_fwd_amd as dbf
    from tests import inputs

    res = {}
    g = torch.Generator(device="cpu").manual_seed(5)

    def fp16_us(n, m):
        R = max(2, -(-args.rotate_mb * (1 << 20) // (2 * n * m)))
        Ws = [(0.02 * torch.randn((n, m), generator=g)).half().cuda() for _ in range(R)]
        x = torch.randn((1, m), generator=g).half().cuda()
        yy = torch.empty((1, n), dtype=torch.float16, device="cuda")

        def dense(i):
            torch.matmul(x, Ws[i % R].t(), out=yy)
        dense.period = R
        el, done = time_steps(dense, max(R, min(args.steps, 20 * R)), min(args.warmup, R), "graph")
        del Ws
        torch.cuda.empty_cache()
        return el * 1e6 / done, 2 * n * m * done / el / 1e9

    t16, gbs16 = fp16_us(4096, 4096)
    res["fp16_matvec_4096x4096_us"] = t16
    res["fp16_matvec_4096x4096_gbs"] = gbs16
    t16_up, gbs16_up = fp16_us(14336, 4096)
    res["fp16_matvec_14336x4096_us"] = t16_up
    res["fp16_matvec_14336x4096_gbs"] = gbs16_up
    for cid, li, tag, tref in ((2, 0, "4096x4096_k2048_1bit", t16), (3, 0, "4096x4096_k4096_2bit", t16),
                               (4, 0, "14336x4096_k4800_1.5bit", t16_up)):
        layer = inputs.config(cid).layers[li]
        y = torch.empty((1, layer.n), dtype=torch.float16, device="cuda")
        bytes_step = layer.sign_bytes + layer.scale_bytes
        Rd = max(1, -(-args.rotate_mb * (1 << 20) // bytes_step))
        copies = [dbf.Layer(layer.A, layer.B, layer.a, layer.mid, layer.b, max_batch=1) for _ in range(Rd)]
        xd = torch.from_numpy(layer.X[1]).cuda()

        def fwd(i):
            copies[i % Rd].forward(xd, out=y)
        fwd.period = Rd
        el, done = time_steps(fwd, max(Rd, min(args.steps, 10 * Rd)), min(args.warmup, Rd), "graph")
        td = el * 1e6 / done
        res[f"dbf_{tag}_us"] = td
        res[f"speedup_{tag}"] = tref / td
        for c in copies:
            c.close()
        del copies
        torch.cuda.synchronize()
    # the library's dense fp16 GEMM on the batch-2048 shape of the 4096x4096
    # layer: the MFMA rate a plain GEMM attains on this chip under this load
    Xg = torch.randn((2048, 4096), generator=g).half().cuda()
    Wg = (0.02 * torch.randn((4096, 4096), generator=g)).half().cuda()
    Yg = torch.empty((2048, 4096), dtype=torch.float16, device="cuda")
    for _ in range(5):
        torch.matmul(Xg, Wg.t(), out=Yg)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(50):
        torch.matmul(Xg, Wg.t(), out=Yg)
    e1.record()
    torch.cuda.synchronize()
    tg = e0.elapsed_time(e1) * 1e3 / 50
    res["fp16_gemm_2048x4096x4096_us"] = tg
    res["fp16_gemm_2048x4096x4096_tflops"] = 2 * 2048 * 4096 * 4096 / (tg * 1e-6) / 1e12
    del Xg, Wg, Yg
    buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(buf)
    dst.copy_(buf)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(buf)
    e1.record()
    torch.cuda.synchronize()
    res["device_copy_1GiB_gbs"] = 10 * 2 * buf.numel() * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del buf, dst
    torch.cuda.empty_cache()
    print(f"[bench] fp16 context: {res}", file=sys.stderr, flush=True)
    return res


def copy_probe(mb):
    import torch
    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path; see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch

    import dbf_linear_fwd_amd as dbf
    from tests import inputs

    torch.cuda.set_device(0)
    if args.copy_probe_mb:
        copy_probe(args.copy_probe_mb)
        return
    if args.all_configs:
        all_configs(args)
        return

    result = {}
    # ---------------------------------------------------------------- decode, batch 1 (headline)
    if args.only in (None, "decode"):
        cfg = inputs.config(2)
        layer = cfg.layers[0]
        bytes_step = layer.sign_bytes + layer.scale_bytes
        R = max(1, -(-args.rotate_mb * (1 << 20) // bytes_step))
        print(f"[bench] decode: {layer.n}x{layer.m} k={layer.k}, {R} weight copies "
              f"({R * bytes_step / 2**20:.0f} MiB), {args.steps} steps, mode={args.mode}", file=sys.stderr, flush=True)
        copies = layer_copies(layer, R)
        x = torch.from_numpy(layer.X[1]).cuda()
        y = torch.empty((1, layer.n), dtype=torch.float16, device="cuda")

        dpath = dbf.DBF_PATH_DECODE if args.decode_path == "mfma" else dbf.DBF_PATH_DECODE_TABLE

        def fwd(i):
            copies[i % R].forward(x, out=y, path=dpath)
        fwd.period = R

        el, done = time_steps(fwd, args.steps, args.warmup, args.mode)
        gbs = bytes_step * done / el / 1e9
        print(f"[bench] decode: {done} steps in {el * 1e3:.2f} ms -> {gbs:.1f} GB/s", file=sys.stderr, flush=True)
        el_e, done_e = time_steps(fwd, min(args.steps, 2 * R), min(args.warmup, R), "eager")
        kt = kernel_times(copies, fwd, min(args.steps, 2 * R))
        print(f"[bench] kernel event times: {kt}", file=sys.stderr, flush=True)
        # cold calls: each after a 512 MiB write (evicts the L2s and the
        # Infinity Cache); a GPU-side spin covers the host's enqueue, so the
        # events time the forward's kernels and the gap between them
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold = []
        for i in range(9):
            scrub.fill_(i & 255)
            torch.cuda.synchronize()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(200000)
            c0.record()
            fwd(i)
            c1.record()
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1) * 1e3)
        del scrub
        torch.cuda.empty_cache()
        print(f"[bench] cold calls (us): {[round(c, 1) for c in cold]}", file=sys.stderr, flush=True)
        kb = decode_kernel_bytes(layer, 1)
        if args.decode_path == "table":
            kb = {"table_" + kname.split("_", 1)[1]: v for kname, v in kb.items()}
        dom = max(kb, key=lambda kname: kt.get(kname, {"avg_us": 0})["avg_us"])
        ach = kb[dom] / (kt[dom]["avg_us"] * 1e-6) / 1e9
        result["decode"] = {
            "value": gbs, "ms_per_step": el * 1e3 / done, "steps": done,
            "eager_gbs": bytes_step * done_e / el_e / 1e9,
            "cold_call_us_median": float(np.median(cold)),
            "kernels": kt, "dominant": dom,
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS, "traffic": recorded_traffic(dom), "kernel": dom,
                         "algorithmic_bytes_per_launch": kb[dom]},
            "layer": layer, "copies": copies,
        }
        for c in copies:
            c.close()
        del copies
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- prefill, batch 2048 (secondary)
    if args.only in (None, "prefill") and not args.no_secondary:
        layer = inputs.config(3).layers[0]
        bt = 2048
        print(f"[bench] prefill: {layer.n}x{layer.m} k={layer.k} batch {bt}", file=sys.stderr, flush=True)
        L = dbf.Layer(layer.A, layer.B, layer.a, layer.mid, layer.b, max_batch=bt)
        x = torch.from_numpy(layer.X[bt]).cuda()
        y = torch.empty((bt, layer.n), dtype=torch.float16, device="cuda")

        def pf(i):
            L.forward(x, out=y)
        reps = 50
        el, done = time_steps(pf, reps, 10, "eager")
        flops = 2 * bt * layer.k * (layer.n + layer.m)
        tfs = flops * done / el / 1e12
        kt = kernel_times([L], pf, 20)
        kf = prefill_kernel_flops(layer, bt)
        dom = max(kf, key=lambda kname: kt.get(kname, {"avg_us": 0})["avg_us"])
        ach = kf[dom] / (kt[dom]["avg_us"] * 1e-6) / 1e12
        print(f"[bench] prefill: {tfs:.1f} TFLOP/s-eq; kernels {kt}", file=sys.stderr, flush=True)
        result["prefill"] = {
            "value": tfs, "unit": "TFLOP/s-eq", "ms_per_forward": el * 1e3 / done,
            "frac_of_mfma_peak": tfs / MFMA_F16_PEAK_TFLOPS, "kernels": kt,
            "roofline": {"bound": "mfma", "achieved": ach, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": ach / MFMA_F16_PEAK_TFLOPS, "traffic": recorded_traffic(dom), "kernel": dom,
                         "algorithmic_flops_per_launch": kf[dom]},
            "workload": "4096x4096 projection, k=4096 (~2 bits/weight), batch 2048",
        }
        L.close()

    # ---------------------------------------------------------------- gradients, batch 2048 (secondary)
    if args.only in (None, "backward") and not args.no_backward:
        result["backward"] = backward_leg()

    # ---------------------------------------------------------------- decoder block, batch 1 (secondary)
    if args.only in (None, "block") and not args.no_block:
        result["block"] = block_leg(args)

    # ---------------------------------------------------------------- BQQ-form layer (secondary)
    if args.only in (None, "bqq") and not args.no_bqq:
        result["bqq"] = bqq_leg(args)

    # ---------------------------------------------------------------- fp16 matvec and copy context
    if args.only in (None, "context") and not args.no_context:
        result["context"] = fp16_context_leg(args)

    # ---------------------------------------------------------------- factorization (secondary)
    if args.only in (None, "factorize") and not args.no_factorize:
        result["factorize"] = factorize_leg(args)

    if args.only is not None:
        print(json.dumps({k: {kk: vv for kk, vv in v.items() if kk not in ("layer", "copies")}
                          for k, v in result.items()}, default=str))
        return

    d = result["decode"]
    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(d["layer"], args.cpu_seconds)
    line = {
        "metric": "DBF linear packed-weight GB/s (% HBM peak) at batch 1; TFLOP/s-eq at batch 2048",
        "value": round(d["value"], 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": d["steps"],
        "warmup": args.warmup,
        "ms_per_step": d["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "DBF linear 4096x4096, k=2048 (~1 bit/weight), batch 1, fp16 I/O, "
                               f"{d['layer'].n}x{d['layer'].m}; weights rotated over >=512 MB; {args.mode}",
                   "n": d["layer"].n, "m": d["layer"].m, "k": d["layer"].k, "batch": 1,
                   "mode": args.mode},
        "frac_of_hbm_peak": d["value"] / HBM_PEAK_GBS,
        "roofline": d["roofline"],
        "cpu_baseline": cpu,
        "decode_kernels_us": d["kernels"],
        "eager_gbs": d["eager_gbs"],
        "cold_call_us_median": d["cold_call_us_median"],
    }
    if "prefill" in result:
        line["prefill_batch2048"] = result["prefill"]
    if "block" in result:
        line["decode_block_b1"] = result["block"]
    if "backward" in result:
        line["backward_batch2048"] = result["backward"]
    if "bqq" in result:
        line["bqq_form"] = result["bqq"]
    if "factorize" in result:
        line["factorization"] = result["factorize"]
    if "context" in result:
        line["context_same_gpu"] = result["context"]
    print(json.dumps(line))


if __name__ == "__main__":
    main()
