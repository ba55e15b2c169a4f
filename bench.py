"""Benchmark of the DBF linear forward on one MI355X.

Headline workload: a Llama-3-8B-shaped decoder block of seven DBF linears
(q 4096x4096, k and v 1024x4096, o 4096x4096, gate and up 14336x4096, down
4096x14336) with a per-layer middle dimension drawn for 1.0-2.3 bits per
weight, signs uniform +/-1, a, b ~ |N(0,1)|*0.02, mid ~ |N(0,1)|, x ~ N(0,1)
in fp16, batch 1.  One step is one forward of the whole block in its
dependency order on one stream: the layers that read the same input run as
one grouped forward (q, k, v; gate, up), the groups one after another.  The
steps rotate over R distinct copies of the block's packed weights,
R * bytes >= 512 MB, so that the 256 MB Infinity Cache cannot hold them and
every step streams its weights from HBM.  The inputs are resident in HBM
before the timed region starts.

Metric: packed-weight GB/s = the block's (n*k + k*m)/8 + 2*(n + k + m) bytes
per step, summed over its layers, times the steps, divided by the wall time
of exactly --steps steps (one replay of a captured HIP graph of those steps,
after --warmup untimed steps and one untimed replay that uploads the graph).
Before any timing the outputs of the timed handles are checked against the
fp64 oracle (every output of every layer, first and last copy); on a
mismatch the bench prints no number and exits with status 1.

Secondary measurements in the same line: the batch-2048 half of the metric
(TFLOP/s-equivalent = 2*batch*k*(n+m) per forward) on the MLP up and down
projections (14336x4096 and 4096x14336, k = 4800), also parity-checked
first; the roofline of the dominant decode kernel (per-launch HIP events on
the launch stream); one cold forward of each layer after a 512 MiB scrub;
the CPU oracle timed on the host on a bounded sample of the same workload
(all BLAS threads and one); gradients, the BQQ-form layer, the factorization,
and the GPU's attainable copy and streaming-read rates.
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
    p.add_argument("--steps", type=int, default=240, help="timed decoder-block forwards (exactly)")
    p.add_argument("--warmup", type=int, default=48)
    p.add_argument("--rotate-mb", type=int, default=512)
    p.add_argument("--mode", choices=("graph", "eager"), default="graph",
                   help="graph: the timed steps replay a captured HIP graph of forwards")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-secondary", action="store_true", help="skip the batch-2048 measurement")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="only run a plain device copy of this size (counter scaling) and exit")
    p.add_argument("--no-backward", action="store_true", help="skip the gradient measurement")
    p.add_argument("--all-configs", action="store_true",
                   help="instead of the headline line: one JSON line per workload layer and batch "
                        "(decode at batch 1 and 16, prefill at batch 2048)")
    p.add_argument("--no-bqq", action="store_true", help="skip the BQQ-form layer measurement")
    p.add_argument("--no-factorize", action="store_true", help="skip the factorization measurement")
    p.add_argument("--no-context", action="store_true", help="skip the device-copy context")
    p.add_argument("--factor-cpu", action="store_true",
                   help="also time the factorization oracle (one outer x one inner iteration) on the host")
    p.add_argument("--only", choices=("block", "layer", "prefill", "block_prefill", "backward", "bqq", "factorize",
                                      "context"),
                   default=None,
                   help="run one leg only (for profiling)")
    return p.parse_args()


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


def time_median(fwd, groups=5, per=10, warmup=20):
    """Eager steady state: `warmup` untimed steps (the clocks ramp up after an
    idle spell such as a CPU parity check), then `groups` timed groups of
    `per` steps; returns (seconds of the median group, per)."""
    import torch
    for i in range(warmup):
        fwd(i)
    torch.cuda.synchronize()
    ts = []
    for _ in range(groups):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(per):
            fwd(i)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    ts.sort()
    return ts[len(ts) // 2], per


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
    el, done = time_median(step)
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
    2048, steady state: the median of 5 groups of 10 forwards after 20
    untimed ones).  One JSON line each."""
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
                el, done = time_median(pf)
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
    el, done = time_median(pf)
    kt = kernel_times([H], pf, 10)
    flops = 2 * bt * p * d * (n + m)
    res["prefill_b2048"] = {"us_per_forward": el * 1e6 / done, "tflops_eq": flops * done / el / 1e12,
                            "frac_of_mfma_peak": flops * done / el / 1e12 / MFMA_F16_PEAK_TFLOPS, "kernels": kt}
    print(f"[bench] bqq prefill: {res['prefill_b2048']['tflops_eq']:.1f} TFLOP/s-eq; kernels {kt}",
          file=sys.stderr, flush=True)
    H.close()
    torch.cuda.synchronize()
    res["grouped_g128"] = bqq_grouped_leg(args)
    return res


def bqq_grouped_leg(args):
    """The same 4096x4096, p = 2, d = 1024 layer with group-wise scalars
    (one set per 128 input columns: 32 groups): batch-1 decode over rotated
    copies (GB/s of bits + per-forward scale and weight bytes) and
    batch-2048 prefill (TFLOP/s-equivalent 2 * batch * p d (n + m))."""
    import torch

    import dbf_linear_fwd_amd as dbf
    from tests import inputs

    n, m, d, p, g = 4096, 4096, 1024, 2, 128
    L = inputs.bqq_grouped_layer("bqqg", n, m, d, p, g, 8300, (1, 2048))
    # bits; per-term input scales, mid and a (fp16); row sums of the Y_i and the p + 1 statistic weights (fp32)
    bytes_step = L.bit_bytes + 2 * (p * m + p * d + n) + 4 * (p * n + (p + 1) * m)
    R = max(1, -(-args.rotate_mb * (1 << 20) // bytes_step))
    print(f"[bench] bqq grouped: {n}x{m} d={d} p={p} group={g}, {R} copies", file=sys.stderr, flush=True)
    copies = [dbf.Layer.bqq_grouped(L.Y, L.Z, L.r, L.s, L.t, L.u, g, max_batch=1) for _ in range(R)]
    x = torch.from_numpy(L.X[1]).cuda()
    y = torch.empty((1, n), dtype=torch.float16, device="cuda")

    def fwd(i):
        copies[i % R].forward(x, out=y)
    fwd.period = R
    el, done = time_steps(fwd, max(R, min(args.steps, 10 * R)), min(args.warmup, R), args.mode)
    kt = kernel_times(copies, fwd, min(args.steps, 2 * R))
    res = {"workload": "BQQ-form layer 4096x4096, p=2 products of d=1024, scalars per group of 128 input columns",
           "decode_b1": {"us_per_forward": el * 1e6 / done, "gbs": bytes_step * done / el / 1e9,
                         "frac_of_hbm_peak": bytes_step * done / el / 1e9 / HBM_PEAK_GBS, "kernels": kt,
                         "bytes_per_forward": bytes_step, "copies": R}}
    print(f"[bench] bqq grouped decode: {res['decode_b1']['us_per_forward']:.2f} us, "
          f"{res['decode_b1']['gbs']:.1f} GB/s; kernels {kt}", file=sys.stderr, flush=True)
    for c in copies:
        c.close()
    del copies
    torch.cuda.synchronize()
    bt = 2048
    H = dbf.Layer.bqq_grouped(L.Y, L.Z, L.r, L.s, L.t, L.u, g, max_batch=bt)
    x = torch.from_numpy(L.X[bt]).cuda()
    y = torch.empty((bt, n), dtype=torch.float16, device="cuda")

    def pf(i):
        H.forward(x, out=y)
    el, done = time_median(pf)
    kt = kernel_times([H], pf, 10)
    flops = 2 * bt * p * d * (n + m)
    res["prefill_b2048"] = {"us_per_forward": el * 1e6 / done, "tflops_eq": flops * done / el / 1e12,
                            "frac_of_mfma_peak": flops * done / el / 1e12 / MFMA_F16_PEAK_TFLOPS, "kernels": kt}
    print(f"[bench] bqq grouped prefill: {res['prefill_b2048']['tflops_eq']:.1f} TFLOP/s-eq; kernels {kt}",
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


def copy_probe(mb):
    import torch
    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 3}))




GROUPS = [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
TOL = 2e-3


def block_bytes_of(layers):
    return sum(L.sign_bytes + L.scale_bytes for L in layers)


def stage_bytes(layers, batch):
    """Algorithmic bytes of the two decode stages of a group of layers that
    share an input: stage 1 reads B's signs, b, mid and x; stage 2 reads A's
    signs and a and writes y (the intermediate is an implementation cost)."""
    m = layers[0].m
    s1 = sum(L.k * L.m // 8 + 2 * L.m + 2 * L.k for L in layers) + 2 * batch * m
    s2 = sum(L.n * L.k // 8 + 2 * L.n + 2 * batch * L.n for L in layers)
    return s1, s2


def row_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float((np.abs(got - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-300)).max())


class Block:
    """R copies of the decoder block's handles, with its inputs and outputs."""

    def __init__(self, rotate_mb, max_batch=1):
        import torch

        import dbf_linear_fwd_amd as dbf
        from tests import inputs
        self.layers = inputs.config(5).layers
        self.by = {L.name: L for L in self.layers}
        self.bytes = block_bytes_of(self.layers)
        self.R = max(1, -(-rotate_mb * (1 << 20) // self.bytes))
        self.copies = [{L.name: dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=max_batch) for L in self.layers}
                       for _ in range(self.R)]
        self.xs = {L.name: torch.from_numpy(L.X[1]).cuda() for L in self.layers}
        self.ys = {L.name: torch.empty((1, L.n), dtype=torch.float16, device="cuda") for L in self.layers}

    def step(self, i):
        """One block forward on copy i mod R: the groups in dependency order."""
        import dbf_linear_fwd_amd as dbf
        c = self.copies[i % self.R]
        for gr in GROUPS:
            if len(gr) == 1:
                c[gr[0]].forward(self.xs[gr[0]], out=self.ys[gr[0]])
            else:
                dbf.forward_group([c[n] for n in gr], self.xs[gr[0]], [self.ys[n] for n in gr])

    def parity(self):
        """Every output of every layer of the first and last copy against the
        fp64 oracle (per-row infinity-norm relative error); the worst one."""
        import torch

        from oracle import dbf_oracle as O
        worst = 0.0
        # (a group's layers read the input of its first layer)
        xin = {n: self.by[gr[0]].X[1] for gr in GROUPS for n in gr}
        refs = {L.name: O.sampled_forward(xin[L.name], L.A, L.B, L.a, L.mid, L.b, [0], np.arange(L.n))
                for L in self.layers}
        for ci in sorted({0, self.R - 1}):
            for y in self.ys.values():
                y.fill_(float("nan"))
            self.step(ci)
            torch.cuda.synchronize()
            for L in self.layers:
                worst = max(worst, row_rel_err(self.ys[L.name].cpu().numpy(), refs[L.name]))
        return worst

    def close(self):
        import torch
        for c in self.copies:
            for H in c.values():
                H.close()
        torch.cuda.synchronize()


def time_exact(step, steps, warmup, start=0):
    """`warmup` untimed eager steps, then exactly `steps` steps i = start +
    warmup, ... captured in one HIP graph; one untimed replay uploads the
    graph, one replay is timed with events.  Returns seconds."""
    import torch
    cur = torch.cuda.current_stream()
    for i in range(warmup):
        step(start + i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(cur)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                step(start + warmup + i)
    cur.wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3


# device-side spin ahead of each timed round of eager forwards (about 10 ms
# at 2 GHz: longer than the host takes to enqueue a round)
SPIN_CYCLES = 20_000_000


def block_kernel_times(blk, passes=3):
    """Per-launch time (us) of each decode kernel of the block, from HIP
    events riding on the launches: after one untimed round over all copies
    (the clocks settle after the idle spells of eager launching), `passes`
    rounds of eager steps over all copies, each giving an average per
    kernel; the median of the passes' averages is reported (one perturbed
    pass does not move it).  Each round is queued behind a short device-side
    spin, so that the host has enqueued the whole round before it starts and
    its kernels run back to back, as in the graph replay, rather than one
    at a time with the GPU idle between host calls."""
    import dbf_linear_fwd_amd as dbf
    import torch
    heads = {"qkv": "q", "o": "o", "gateup": "gate", "down": "down"}
    for i in range(blk.R):
        blk.step(i)
    torch.cuda.synchronize()
    runs = []
    for _ in range(passes):
        for c in blk.copies:
            for h in heads.values():
                dbf.dbf_timing_enable(c[h].handle, True)
                dbf.dbf_timing_read(c[h].handle)
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        for i in range(blk.R):
            blk.step(i)
        torch.cuda.synchronize()
        one = {}
        for gname, h in heads.items():
            tot = {}
            for c in blk.copies:
                for kname, v in dbf.dbf_timing_read(c[h].handle).items():
                    t = tot.setdefault(kname, [0, 0.0])
                    t[0] += v["launches"]
                    t[1] += v["total_ms"]
                dbf.dbf_timing_enable(c[h].handle, False)
            for kname, (n, ms) in tot.items():
                stage = 1 if kname.endswith("stage1") else 2
                one[f"{gname}_stage{stage}"] = (n, 1e3 * ms / max(n, 1))
        runs.append(one)
    out = {}
    for k in runs[0]:
        avgs = sorted(r[k][1] for r in runs)
        out[k] = {"launches": sum(r[k][0] for r in runs), "avg_us": avgs[len(avgs) // 2],
                  "pass_avgs_us": [r[k][1] for r in runs]}
    return out


def block_leg(args):
    """The headline: the decoder block at batch 1 (see the module docstring)."""
    blk = Block(args.rotate_mb)
    print(f"[bench] block: 7 layers, {blk.bytes / 2**20:.1f} MiB per block, {blk.R} copies", file=sys.stderr,
          flush=True)
    err = blk.parity()
    print(f"[bench] block parity: worst row rel err {err:.3e}", file=sys.stderr, flush=True)
    if not err <= TOL:
        blk.close()
        print(f"[bench] PARITY FAILED on the decoder block (worst row rel err {err:.3e} > {TOL}); no number",
              file=sys.stderr, flush=True)
        sys.exit(1)
    el = time_exact(blk.step, args.steps, args.warmup, start=0)
    gbs = blk.bytes * args.steps / el / 1e9
    print(f"[bench] block: {args.steps} steps in {el * 1e3:.2f} ms -> {gbs:.1f} GB/s "
          f"({el * 1e6 / args.steps:.1f} us per block)", file=sys.stderr, flush=True)
    # beside it, a longer steady state over whole rotations
    long_steps = 10 * blk.R
    el_long = time_exact(blk.step, long_steps, blk.R, start=args.steps)
    kt = block_kernel_times(blk)
    print(f"[bench] block kernels: {kt}", file=sys.stderr, flush=True)
    cold = cold_latency(blk)
    print(f"[bench] cold single-layer forwards after a 512 MiB scrub (us): {cold}", file=sys.stderr, flush=True)
    sb = {}
    for gr, gname in zip(GROUPS, ("qkv", "o", "gateup", "down")):
        s1, s2 = stage_bytes([blk.by[n] for n in gr], 1)
        sb[f"{gname}_stage1"], sb[f"{gname}_stage2"] = s1, s2
    # the dominant kernel: the stage with the most bytes per launch (gate/up's
    # second stage, also the longest launch in every kernel trace)
    dom = max(sb, key=lambda k: sb[k])
    ach = sb[dom] / (kt[dom]["avg_us"] * 1e-6) / 1e9
    res = {
        "value": gbs, "ms_per_step": el * 1e3 / args.steps, "steps": args.steps, "parity_worst_row_rel_err": err,
        "steady_state": {"steps": long_steps, "gbs": blk.bytes * long_steps / el_long / 1e9,
                         "us_per_block": el_long * 1e6 / long_steps},
        "kernels": {k: dict(v, bytes=sb[k], gbs=sb[k] / (v["avg_us"] * 1e-6) / 1e9) for k, v in kt.items()},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": recorded_traffic(dom), "kernel": dom,
                     "algorithmic_bytes_per_launch": sb[dom]},
        "block_bytes": blk.bytes, "copies": blk.R, "cold_us": cold,
    }
    blk.close()
    return res


def cold_latency(blk, reps=5, scrub_mb=512):
    """One batch-1 forward of each layer of the block, alone, after a
    512 MiB scrub write (nothing of the layer left in the caches): the median
    over `reps` tries of its wall time between events on the launch stream
    (launch gaps included), in us."""
    import torch
    scrub = torch.empty(scrub_mb << 18, dtype=torch.float32, device="cuda")
    c = blk.copies[0]
    out = {}
    for L in blk.layers:
        ts = []
        for _ in range(reps):
            scrub.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            c[L.name].forward(blk.xs[L.name], out=blk.ys[L.name])
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        out[L.name] = sorted(ts)[reps // 2]
    del scrub
    torch.cuda.empty_cache()
    return out


def layer_leg(args):
    """Context: the single 4096x4096, k = 2048 layer (about 1 bit per weight)
    at batch 1, steady state over rotated copies."""
    import torch

    import dbf_linear_fwd_amd as dbf
    from tests import inputs
    layer = inputs.config(2).layers[0]
    bytes_step = layer.sign_bytes + layer.scale_bytes
    R = max(1, -(-args.rotate_mb * (1 << 20) // bytes_step))
    copies = [dbf.Layer(layer.A, layer.B, layer.a, layer.mid, layer.b, max_batch=1) for _ in range(R)]
    x = torch.from_numpy(layer.X[1]).cuda()
    y = torch.empty((1, layer.n), dtype=torch.float16, device="cuda")

    def fwd(i):
        copies[i % R].forward(x, out=y)
    el = time_exact(fwd, 4 * R, R)
    kt = kernel_times(copies, fwd, 2 * R)
    res = {"workload": "DBF linear 4096x4096, k=2048 (~1 bit/weight), batch 1", "copies": R,
           "us_per_forward": el * 1e6 / (4 * R), "gbs": bytes_step * 4 * R / el / 1e9, "kernels": kt}
    print(f"[bench] layer 4096x4096 k2048: {res['us_per_forward']:.2f} us, {res['gbs']:.1f} GB/s; kernels {kt}",
          file=sys.stderr, flush=True)
    for c in copies:
        c.close()
    torch.cuda.synchronize()
    return res


def prefill_leg(args):
    """The batch-2048 half of the metric on the MLP up (14336x4096) and down
    (4096x14336) projections, k = 4800: outputs checked against the oracle
    first (the first and last row of every 128-row tile and 16 random rows,
    every output of each), then TFLOP/s-equivalent 2*batch*k*(n+m) per
    forward (the median of 5 groups of 10 forwards after 20 warm-ups), and
    the kernels' launch times."""
    import torch

    import dbf_linear_fwd_amd as dbf
    from oracle import dbf_oracle as O
    from tests import inputs
    bt = 2048
    out = {}
    tot_flops, tot_s = 0, 0.0
    kall = {}
    for layer in inputs.config(4).layers:
        L = dbf.Layer(layer.A, layer.B, layer.a, layer.mid, layer.b, max_batch=bt)
        X = layer.X[bt]
        x = torch.from_numpy(X).cuda()
        y = torch.empty((bt, layer.n), dtype=torch.float16, device="cuda")
        L.forward(x, out=y)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([np.arange(0, bt, 128), np.arange(127, bt, 128),
                                         np.random.default_rng(7).choice(bt, 16, replace=False)]))
        err = row_rel_err(y.cpu().numpy()[rows],
                          O.sampled_forward(X, layer.A, layer.B, layer.a, layer.mid, layer.b, rows,
                                            np.arange(layer.n)))
        print(f"[bench] prefill {layer.name} parity: worst row rel err {err:.3e} over {len(rows)} rows",
              file=sys.stderr, flush=True)
        if not err <= TOL:
            print(f"[bench] PARITY FAILED on prefill {layer.name}; no number", file=sys.stderr, flush=True)
            sys.exit(1)

        def pf(i):
            L.forward(x, out=y)
        el, done = time_median(pf)
        flops = 2 * bt * layer.k * (layer.n + layer.m)
        kt = kernel_times([L], pf, 10)
        kf = prefill_kernel_flops(layer, bt)
        out[layer.name] = {"us_per_forward": el * 1e6 / done, "tflops_eq": flops * done / el / 1e12,
                           "parity_worst_row_rel_err": err, "kernels": kt}
        for kname, v in kt.items():
            if kname in kf:
                kall[f"{layer.name}_{kname}"] = (kf[kname], v["avg_us"])
        tot_flops += flops * done
        tot_s += el
        print(f"[bench] prefill {layer.name}: {out[layer.name]['tflops_eq']:.1f} TFLOP/s-eq; kernels {kt}",
              file=sys.stderr, flush=True)
        L.close()
        torch.cuda.synchronize()
    dom = max(kall, key=lambda k: kall[k][1])
    ach = kall[dom][0] / (kall[dom][1] * 1e-6) / 1e12
    tfs = tot_flops / tot_s / 1e12
    return {"value": tfs, "unit": "TFLOP/s-eq", "frac_of_mfma_peak": tfs / MFMA_F16_PEAK_TFLOPS,
            "workload": "MLP up 14336x4096 and down 4096x14336 projections, k=4800 (~1.5 bits/weight), batch 2048",
            "layers": out,
            "roofline": {"bound": "mfma", "achieved": ach, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": ach / MFMA_F16_PEAK_TFLOPS, "traffic": recorded_traffic(dom),
                         "kernel": dom, "algorithmic_flops_per_launch": kall[dom][0]}}


def block_prefill_leg(args):
    """The decoder block at batch 2048: its seven layers with q/k/v and
    gate/up each as one grouped forward (one launch per product for the
    group), checked against the oracle first (the first and last row of every
    128-row tile and 16 random rows of every layer), then TFLOP/s-equivalent
    2*batch*k*(n+m) summed over the layers per block forward (the median of 5
    groups of 4 block forwards after 6 warm-ups); beside it the same block as
    seven separate layer forwards, and each group alone both ways."""
    import torch

    import dbf_linear_fwd_amd as dbf
    from oracle import dbf_oracle as O
    from tests import inputs
    bt = 2048
    layers = {L.name: L for L in inputs.config(5).layers}
    hs = {n: dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=bt) for n, L in layers.items()}
    xs = {n: torch.from_numpy(L.X[bt]).cuda() for n, L in layers.items()}
    ys = {n: torch.empty((bt, L.n), dtype=torch.float16, device="cuda") for n, L in layers.items()}

    def grouped(i):
        for gr in GROUPS:
            if len(gr) == 1:
                hs[gr[0]].forward(xs[gr[0]], out=ys[gr[0]])
            else:
                dbf.forward_group([hs[n] for n in gr], xs[gr[0]], [ys[n] for n in gr])

    def separate(i):
        for gr in GROUPS:
            for n in gr:
                hs[n].forward(xs[gr[0]], out=ys[n])
    grouped(0)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, bt, 128), np.arange(127, bt, 128),
                                     np.random.default_rng(11).choice(bt, 16, replace=False)]))
    worst = 0.0
    for gr in GROUPS:
        X = layers[gr[0]].X[bt]
        for n in gr:
            L = layers[n]
            err = row_rel_err(ys[n].cpu().numpy()[rows],
                              O.sampled_forward(X, L.A, L.B, L.a, L.mid, L.b, rows, np.arange(L.n)))
            worst = max(worst, err)
    print(f"[bench] block prefill parity: worst row rel err {worst:.3e} over {len(rows)} rows of each layer",
          file=sys.stderr, flush=True)
    if not worst <= TOL:
        print("[bench] PARITY FAILED on the block at batch 2048; no number", file=sys.stderr, flush=True)
        sys.exit(1)
    flops = sum(2 * bt * L.k * (L.n + L.m) for L in layers.values())
    el_g, done_g = time_median(grouped, per=4, warmup=6)
    el_s, done_s = time_median(separate, per=4, warmup=6)
    per_group = {}
    for gr in GROUPS:
        if len(gr) == 1:
            continue
        gf = sum(2 * bt * layers[n].k * (layers[n].n + layers[n].m) for n in gr)

        def one_grouped(i, gr=gr):
            dbf.forward_group([hs[n] for n in gr], xs[gr[0]], [ys[n] for n in gr])

        def one_separate(i, gr=gr):
            for n in gr:
                hs[n].forward(xs[gr[0]], out=ys[n])
        eg, dg = time_median(one_grouped, warmup=10)
        es, ds = time_median(one_separate, warmup=10)
        per_group["".join(gr)] = {"grouped_us": eg * 1e6 / dg, "grouped_tflops_eq": gf * dg / eg / 1e12,
                                  "separate_us": es * 1e6 / ds, "separate_tflops_eq": gf * ds / es / 1e12}
    res = {"workload": "Llama-3-8B-shaped decoder block of 7 DBF linears, batch 2048, q/k/v and gate/up grouped",
           "us_per_block": el_g * 1e6 / done_g, "tflops_eq": flops * done_g / el_g / 1e12,
           "separate_layers_us_per_block": el_s * 1e6 / done_s,
           "separate_layers_tflops_eq": flops * done_s / el_s / 1e12, "groups": per_group,
           "parity_worst_row_rel_err": worst}
    print(f"[bench] block prefill: {res['us_per_block']:.1f} us per block, {res['tflops_eq']:.1f} TFLOP/s-eq "
          f"(separate layers {res['separate_layers_us_per_block']:.1f} us, {res['separate_layers_tflops_eq']:.1f}); "
          f"groups {per_group}", file=sys.stderr, flush=True)
    for h in hs.values():
        h.close()
    torch.cuda.synchronize()
    return res


def cpu_baseline(seconds):
    """The fp64 oracle's factored forward (the §2.1 evaluation order) of the
    decoder block's seven layers at batch 1, on the host's BLAS threads,
    repeated for about `seconds`; GB/s of packed weights, the headline's unit.
    Beside it: the same on one BLAS thread (about a quarter of `seconds`), and
    the oracle's dense form on the block's q projection -- forming W once
    (2nmk fp64 flops) and one batch-1 X Wᵀ (the median of 5)."""
    from oracle import dbf_oracle as O
    from tests import inputs
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    layers = inputs.config(5).layers
    nbytes = block_bytes_of(layers)

    def run(limit_s):
        blocks = 0
        t0 = time.perf_counter()
        while True:
            for L in layers:
                O.factored_forward(L.X[1], L.A, L.B, L.a, L.mid, L.b)
            blocks += 1
            el = time.perf_counter() - t0
            if el >= limit_s:
                return blocks, el
    blocks, el = run(seconds)
    res = {"value": nbytes * blocks / el / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{blocks} batch-1 forwards of the decoder block's 7 layers through the fp64 oracle "
                     f"(factored evaluation order) in {el:.1f} s",
           "host_cpu_count": os.cpu_count()}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            b1, e1 = run(seconds / 4)
        res["one_core"] = {"value": nbytes * b1 / e1 / 1e9, "unit": "GB/s", "cores": 1,
                           "sample": f"{b1} block forwards in {e1:.1f} s"}
    q = layers[0]
    t0 = time.perf_counter()
    W = O.dense_weight(q.A, q.B, q.a, q.mid, q.b)
    w_s = time.perf_counter() - t0
    ts = []
    x = O.widen(q.X[1])
    for _ in range(5):
        t0 = time.perf_counter()
        _ = x @ W.T
        ts.append(time.perf_counter() - t0)
    res["dense_q_layer"] = {"layer": f"{q.n}x{q.m}, k={q.k}", "weight_s": w_s,
                            "weight_gflop": 2 * q.n * q.m * q.k / 1e9, "forward_ms": 1e3 * sorted(ts)[2],
                            "cores": int(threads)}
    return res


def context_leg():
    """The attainable HBM rates on this GPU: a plain 1 GiB device copy (read
    and write), and a streaming read of 1 GiB (torch's sum: one read of the
    buffer, a few bytes written)."""
    import torch
    buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(buf)
    dst.copy_(buf)
    torch.cuda.synchronize()

    def rate(fn, bytes_per_call, reps=10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return reps * bytes_per_call / (e0.elapsed_time(e1) / 1e3) / 1e9
    copy_gbs = rate(lambda: dst.copy_(buf), 2 * buf.numel() * 4)
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    torch.sum(buf, dim=0, out=acc)
    read_gbs = rate(lambda: torch.sum(buf, dim=0, out=acc), buf.numel() * 4)
    del buf, dst
    torch.cuda.empty_cache()
    return {"device_copy_1GiB_gbs": copy_gbs, "streaming_read_1GiB_gbs": read_gbs}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path; see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.copy_probe_mb:
        copy_probe(args.copy_probe_mb)
        return
    if args.all_configs:
        all_configs(args)
        return
    result = {}
    if args.only in (None, "block"):
        result["block"] = block_leg(args)
    if args.only in (None, "layer"):
        result["layer"] = layer_leg(args)
    if args.only in (None, "prefill") and not args.no_secondary:
        result["prefill"] = prefill_leg(args)
    if args.only in (None, "block_prefill") and not args.no_secondary:
        result["block_prefill"] = block_prefill_leg(args)
    if args.only in (None, "backward") and not args.no_backward:
        result["backward"] = backward_leg()
    if args.only in (None, "bqq") and not args.no_bqq:
        result["bqq"] = bqq_leg(args)
    if args.only in (None, "factorize") and not args.no_factorize:
        result["factorize"] = factorize_leg(args)
    if args.only in (None, "context") and not args.no_context:
        result["context"] = context_leg()
    if args.only is not None:
        print(json.dumps(result, default=str))
        return
    d = result["block"]
    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.cpu_seconds)
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
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped decoder block of 7 DBF linears (q 4096x4096, k/v 1024x4096, "
                               "o 4096x4096, gate/up 14336x4096, down 4096x14336), k per layer for 1.0-2.3 "
                               "bits/weight, batch 1, fp16 in and out; q/k/v and gate/up grouped, groups in "
                               "dependency order; weights rotated over >= 512 MB",
                   "batch": 1, "layers": 7, "block_bytes": d["block_bytes"], "copies": d["copies"]},
        "frac_of_hbm_peak": d["value"] / HBM_PEAK_GBS,
        "roofline": d["roofline"],
        "cpu_baseline": cpu,
        "parity_worst_row_rel_err": d["parity_worst_row_rel_err"],
        "decode_block_steady_state": d["steady_state"],
        "decode_kernels": d["kernels"],
        "decode_cold_layer_us": d["cold_us"],
    }
    if "prefill" in result:
        line["prefill_batch2048"] = result["prefill"]
    if "block_prefill" in result:
        line["block_batch2048"] = result["block_prefill"]
    if "layer" in result:
        line["decode_layer_4096x4096_k2048_b1"] = result["layer"]
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
