"""GPU parity: the HIP path against the fp64 CPU oracle on the same seeded inputs.

What is compared (the layer is W = diag(a) A diag(mid) B diag(b) with +/-1
factors and Y = X W^T, "Addition is almost all you need", gist.science
technical summary, §2.1):

* tolerance suites: per batch row, max_i |y_i - ŷ_i| / max_i |ŷ_i| <= 2e-3
  against the unrounded fp64 oracle (fp16 output, fp32 accumulation);
* integer sub-suite: activations in {-1, 0, 1} and scales in {1, 2} (or
  powers of two), where every partial sum is an exact integer on both sides;
  the fp16 bits must equal the oracle's single rounding, +0 and -0 equal;
* both kernel paths (decode for batch <= 16, matrix cores for any batch) on
  shapes that span several tiles and ragged tails, on the five workloads at
  full size (large batches on sampled rows), and on edge cases;
* determinism, batch-row independence, output guard regions, error paths.

Every case prints its name before it touches the GPU.
"""

import os
import sys

import numpy as np
import pytest

import dbf_linear_fwd_amd as dbf
from oracle import dbf_oracle as O
from tests import inputs

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _torch():
    import torch
    return torch


def run(layer, X, path=dbf.DBF_PATH_AUTO, max_batch=None):
    """Forward X (numpy fp16, batch x m) through a fresh handle; returns numpy fp16."""
    torch = _torch()
    mb = max_batch or max(1, X.shape[0])
    L = dbf.Layer(layer.A, layer.B, layer.a, layer.mid, layer.b, max_batch=mb)
    try:
        x = torch.from_numpy(np.ascontiguousarray(X)).cuda()
        y = L.forward(x, path=path)
        torch.cuda.synchronize()
        return y.cpu().numpy()
    finally:
        L.close()


def rel_rows(y16, ref64):
    y = y16.astype(np.float64)
    den = np.maximum(np.abs(ref64).max(axis=1), 1e-300)
    return (np.abs(y - ref64).max(axis=1) / den)


def assert_tol(y16, ref64, what):
    assert np.all(np.isfinite(y16.astype(np.float64))), f"{what}: non-finite output"
    r = rel_rows(y16, ref64)
    assert r.max() <= TOL, f"{what}: worst row rel err {r.max():.3e} (row {int(r.argmax())})"
    return float(r.max())


def assert_bits(y16, ref64, what):
    want = O.rne_fp16(ref64)
    got_bits = y16.view(np.uint16).copy()
    want_bits = want.view(np.uint16).copy()
    # +0 and -0 compare equal
    got_bits[(got_bits & 0x7FFF) == 0] = 0
    want_bits[(want_bits & 0x7FFF) == 0] = 0
    bad = np.argwhere(got_bits != want_bits)
    assert bad.size == 0, (f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: "
                           f"got {y16[tuple(bad[0])]} want {want[tuple(bad[0])]}")


def fp16_intermediate(path, batch) -> bool:
    """Whether the path rounds v = mid * t to fp16 once (prefill, and the
    matrix-core decode at batch 2..16) instead of keeping it in fp32 (the
    batch-1 int8 decode)."""
    return path == dbf.DBF_PATH_PREFILL or (path == dbf.DBF_PATH_DECODE and batch > 1)


def integer_preconditions(layer, X, prefill: bool):
    """The realized data keep every partial sum an exact integer in fp32 and
    (where the path rounds it to fp16: `prefill`) the intermediate v exact."""
    u, t, v, s, y = O.factored_intermediate(X, layer.A, layer.B, layer.a, layer.mid, layer.b)
    m, k = layer.m, layer.k
    assert np.all(np.abs(u) <= 4) and np.abs(t).max() + np.abs(u).sum(axis=1).max() < 2 ** 24
    assert np.abs(v).sum(axis=1).max() < 2 ** 24
    if prefill:
        assert np.abs(v).max() <= 2048, "intermediate would not be exact in fp16"
    assert np.abs(y).max() <= 65504


# --------------------------------------------------------------------------- small and ragged shapes

SHAPES = [
    # n, m, k
    (1, 1, 1),
    (3, 5, 7),
    (64, 64, 64),
    (65, 97, 33),
    (130, 200, 190),
    (256, 256, 128),
    (100, 1100, 70),   # m spans two decode chunks and a ragged tail
    (70, 300, 1500),   # k spans two decode chunks
]


def tile_rows(batch, seed, extra=16):
    """Rows of a large batch checked against the oracle: the first and last
    row of every 128-row tile of the prefill products, plus `extra` random
    rows."""
    rows = set()
    for t0 in range(0, batch, 128):
        rows.update((t0, min(t0 + 127, batch - 1)))
    rows.update(np.random.default_rng(seed).choice(batch, min(extra, batch), replace=False).tolist())
    return np.array(sorted(rows))


DECODE_PATHS = [dbf.DBF_PATH_DECODE]


@pytest.mark.parametrize("n,m,k", SHAPES)
@pytest.mark.parametrize("batch", [1, 3, 9, 16])
@pytest.mark.parametrize("path", DECODE_PATHS, ids=["mfma"])
def test_decode_small_shapes(gpu, n, m, k, batch, path):
    _say(f"decode path={path} n={n} m={m} k={k} batch={batch}")
    X, A, B, a, mid, b = inputs.tiny_case(1000 + n + m + k + batch, n, m, k, batch, signed_scales=True)
    L = inputs.Layer("s", n, m, k, A, B, a, mid, b, {})
    y = run(L, X, path)
    assert y.shape == (batch, n)
    assert_tol(y, O.dense_forward(X, A, B, a, mid, b), f"decode {n}x{m}x{k} b{batch}")


# Shapes whose row counts (k for stage 1, n for stage 2) exceed 4096 / 8192,
# so the decode kernels take their 32- and 64-row workgroup variants.
ROW_TILE_SHAPES = [
    # n, m, k
    (64, 96, 4160),     # stage 1: 32-row workgroups
    (4160, 96, 64),     # stage 2: 32-row workgroups
    (70, 100, 8256),    # stage 1: 64-row workgroups
    (8256, 130, 200),   # stage 2: 64-row workgroups, ragged n
    (70, 100, 16448),   # stage 1: more 64-row blocks (257) than CUs, so no read-ahead blocks
]


@pytest.mark.parametrize("n,m,k", ROW_TILE_SHAPES)
# 1: the int8 kernels (every k here is within their reduction limit); 6, 9: the
# single-plane f16 form
@pytest.mark.parametrize("batch", [1, 6, 9])
def test_decode_row_tile_variants(gpu, n, m, k, batch):
    _say(f"decode row tiles n={n} m={m} k={k} batch={batch}")
    X, A, B, a, mid, b = inputs.tiny_case(3000 + n + m + k + batch, n, m, k, batch, signed_scales=True)
    L = inputs.Layer("s", n, m, k, A, B, a, mid, b, {})
    y = run(L, X, dbf.DBF_PATH_DECODE)
    assert_tol(y, O.dense_forward(X, A, B, a, mid, b), f"decode row tiles {n}x{m}x{k} b{batch}")


@pytest.mark.parametrize("n,m,k", SHAPES)
@pytest.mark.parametrize("batch", [1, 17, 100])
def test_prefill_small_shapes(gpu, n, m, k, batch):
    _say(f"prefill n={n} m={m} k={k} batch={batch}")
    X, A, B, a, mid, b = inputs.tiny_case(2000 + n + m + k + batch, n, m, k, batch, signed_scales=True)
    L = inputs.Layer("s", n, m, k, A, B, a, mid, b, {})
    y = run(L, X, dbf.DBF_PATH_PREFILL)
    assert y.shape == (batch, n)
    assert_tol(y, O.dense_forward(X, A, B, a, mid, b), f"prefill {n}x{m}x{k} b{batch}")


# Intermediate batches on shapes whose prefill grids are small (a few
# 128 x 256 output tiles), so both products take the split-K form: stage 1
# (K = 4096) in 16 parts, stage 2 (K = 1024) in 4, ragged n.
SPLIT_SHAPE = (1000, 4096, 1000)


@pytest.mark.parametrize("batch", [17, 100, 130, 300])
def test_prefill_split_k(gpu, batch):
    n, m, k = SPLIT_SHAPE
    _say(f"prefill split-K n={n} m={m} k={k} batch={batch}")
    X, A, B, a, mid, b = inputs.tiny_case(4000 + batch, n, m, k, batch, signed_scales=True)
    L = inputs.Layer("s", n, m, k, A, B, a, mid, b, {})
    y = run(L, X, dbf.DBF_PATH_PREFILL)
    assert_tol(y, O.dense_forward(X, A, B, a, mid, b), f"prefill split-K b{batch}")


def test_prefill_split_k_determinism(gpu):
    """The parts are added in a fixed order and their count depends on the
    batch only through its 128-row tiles: repeated calls give identical bits,
    and so do batches within one tile count."""
    torch = _torch()
    n, m, k = SPLIT_SHAPE
    X, A, B, a, mid, b = inputs.tiny_case(4999, n, m, k, 256, signed_scales=True)
    H = dbf.Layer(A, B, a, mid, b, max_batch=256)
    try:
        x = torch.from_numpy(X).cuda()
        y100 = H.forward(x[:100], path=dbf.DBF_PATH_PREFILL).cpu().numpy()
        assert np.array_equal(y100.view(np.uint16),
                              H.forward(x[:100], path=dbf.DBF_PATH_PREFILL).cpu().numpy().view(np.uint16))
        y17 = H.forward(x[:17], path=dbf.DBF_PATH_PREFILL).cpu().numpy()
        assert np.array_equal(y17.view(np.uint16), y100[:17].view(np.uint16))
        y256 = H.forward(x, path=dbf.DBF_PATH_PREFILL).cpu().numpy()
        y130 = H.forward(x[:130], path=dbf.DBF_PATH_PREFILL).cpu().numpy()
        assert np.array_equal(y130.view(np.uint16), y256[:130].view(np.uint16))
    finally:
        H.close()


# A reduction wide enough (m spans at least 160 word pairs) that stage 1 of
# the matrix-core decode at batch >= 2 is cut into parts (3 here) whose sums
# the last part of each row block adds in order; ragged m.  Batches 2 and 5
# take the direct form, 9 and 16 the pipelined rounds.
WIDE_SHAPE = (300, 10300, 600)


@pytest.mark.parametrize("batch", [2, 5, 9, 16])
def test_decode_wide_reduction_parts(gpu, batch):
    n, m, k = WIDE_SHAPE
    _say(f"decode wide reduction n={n} m={m} k={k} batch={batch}")
    X, A, B, a, mid, b = inputs.tiny_case(4300 + batch, n, m, k, batch, signed_scales=True)
    L = inputs.Layer("w", n, m, k, A, B, a, mid, b, {})
    y = run(L, X, dbf.DBF_PATH_DECODE)
    assert_tol(y, O.dense_forward(X, A, B, a, mid, b), f"decode wide b{batch}")


def test_decode_wide_reduction_batch_independence(gpu):
    """The parts do not depend on the batch (2..16): sub-batches give the
    rows of the full batch bit for bit, repeated calls the same bits, and a
    grouped forward the layer's own bits."""
    torch = _torch()
    n, m, k = WIDE_SHAPE
    X, A, B, a, mid, b = inputs.tiny_case(4399, n, m, k, 16, signed_scales=True)
    H = dbf.Layer(A, B, a, mid, b, max_batch=16)
    H2 = dbf.Layer(A[:100], B, a[:100], mid, b, max_batch=16)
    try:
        _say("decode wide reduction batch independence")
        x = torch.from_numpy(X).cuda()
        y16 = H.forward(x, path=dbf.DBF_PATH_DECODE).cpu().numpy()
        assert np.array_equal(y16.view(np.uint16), H.forward(x, path=dbf.DBF_PATH_DECODE).cpu().numpy().view(np.uint16))
        for bt in (2, 5, 12):
            yb = H.forward(x[:bt], path=dbf.DBF_PATH_DECODE).cpu().numpy()
            assert np.array_equal(yb.view(np.uint16), y16[:bt].view(np.uint16)), f"batch {bt}"
        _say("decode wide reduction grouped")
        for bt in (1, 9):
            ys = dbf.forward_group([H, H2], x[:bt])
            assert np.array_equal(ys[0].cpu().numpy().view(np.uint16),
                                  H.forward(x[:bt], path=dbf.DBF_PATH_DECODE).cpu().numpy().view(np.uint16))
            assert np.array_equal(ys[1].cpu().numpy().view(np.uint16),
                                  H2.forward(x[:bt], path=dbf.DBF_PATH_DECODE).cpu().numpy().view(np.uint16))
    finally:
        H.close()
        H2.close()


# Large batches on a shape whose prefill grids are one wave of 128 x 256
# output tiles plus a small partial one: the first column tiles (at most 256
# tiles) run whole-K, the remaining columns split-K.  Stage 1: N = k = 4480
# (18 column tiles; the tail from column 4096 at batch 2048, from 4352 at
# batch 1920, ragged); stage 2: N = n = 4400 (18 column tiles, ragged tail).
HEAD_TAIL_SHAPE = (4400, 512, 4480)


@pytest.mark.parametrize("batch", [1920, 2048])
def test_prefill_head_tail(gpu, batch):
    n, m, k = HEAD_TAIL_SHAPE
    _say(f"prefill head/tail n={n} m={m} k={k} batch={batch}")
    X, A, B, a, mid, b = inputs.tiny_case(4100 + batch, n, m, k, batch, signed_scales=True)
    L = inputs.Layer("s", n, m, k, A, B, a, mid, b, {})
    y = run(L, X)
    assert_tol(y, O.dense_forward(X, A, B, a, mid, b), f"prefill head/tail b{batch}")


def test_prefill_head_tail_determinism(gpu):
    """The head/tail split depends on the batch only through its 128-row
    tiles: batches of one tile count give identical bits."""
    torch = _torch()
    n, m, k = HEAD_TAIL_SHAPE
    X, A, B, a, mid, b = inputs.tiny_case(4199, n, m, k, 2048, signed_scales=True)
    H = dbf.Layer(A, B, a, mid, b, max_batch=2048)
    try:
        _say("prefill head/tail determinism")
        x = torch.from_numpy(X).cuda()
        y2048 = H.forward(x).cpu().numpy()
        assert np.array_equal(y2048.view(np.uint16), H.forward(x).cpu().numpy().view(np.uint16))
        y1930 = H.forward(x[:1930]).cpu().numpy()
        assert np.array_equal(y1930.view(np.uint16), y2048[:1930].view(np.uint16))
    finally:
        H.close()


# --------------------------------------------------------------------------- integer sub-suite (bit-exact)

INT_SHAPES = [
    (1, 1, 1, 1),
    (65, 97, 33, 5),
    (256, 256, 128, 16),
    (300, 1100, 200, 9),
]


@pytest.mark.parametrize("n,m,k,batch", INT_SHAPES)
@pytest.mark.parametrize("path", [dbf.DBF_PATH_DECODE, dbf.DBF_PATH_PREFILL])
def test_integer_bit_exact_small(gpu, n, m, k, batch, path):
    _say(f"integer n={n} m={m} k={k} batch={batch} path={path}")
    L = inputs.integer_layer("i", n, m, k, 77 + n, (batch,), a_vals=(0.5, 1.0), mid_vals=(1.0, 2.0),
                             b_vals=(1.0, 2.0))
    X = L.X[batch]
    integer_preconditions(L, X, prefill=fp16_intermediate(path, batch))
    y = run(L, X, path)
    assert_bits(y, O.factored_forward(X, L.A, L.B, L.a, L.mid, L.b), f"integer {n}x{m}x{k}")


# Full-size shapes of the five workloads with small-integer values.  Where
# b, mid in {1, 2} could overflow fp16 at the output (the 14336-wide layers),
# b = mid = 1.
INT_FULL = [
    ("c1", 256, 256, 128, (1.0, 2.0)),
    ("c2", 4096, 4096, 2048, (1.0, 2.0)),
    ("c3", 4096, 4096, 4096, (1.0, 2.0)),
    ("c4-up", 14336, 4096, 4800, (1.0,)),
    ("c4-down", 4096, 14336, 4800, (1.0,)),
]
INT_FULL_CASES = [(1, dbf.DBF_PATH_DECODE), (16, dbf.DBF_PATH_DECODE), (16, dbf.DBF_PATH_PREFILL),
                  (2048, dbf.DBF_PATH_PREFILL)]
# the decoder-block layers (per-layer k), b = mid = 1 (the 14336-wide ones
# would overflow fp16 with 2s): batch 1 (int8 decode), 9 (matrix-core
# decode) and 2048 (prefill)
INT_C5 = [(f"c5-{name}", n, m, k, (1.0,)) for (name, n, m), k in zip(inputs.C5_LAYERS, inputs.c5_middle_dims(4))]
INT_C5_CASES = [(1, dbf.DBF_PATH_DECODE), (9, dbf.DBF_PATH_DECODE), (2048, dbf.DBF_PATH_PREFILL)]


def _int_full_params():
    out = []
    for c in INT_FULL:
        out += [(*c, b, p) for b, p in INT_FULL_CASES]
    for c in INT_C5:
        out += [(*c, b, p) for b, p in INT_C5_CASES]
    return out


@pytest.mark.parametrize("name,n,m,k,vals,batch,path", _int_full_params(),
                         ids=[f"{c[0]}-b{c[5]}-p{c[6]}" for c in _int_full_params()])
def test_integer_bit_exact_full_size(gpu, name, n, m, k, vals, batch, path):
    _say(f"integer full {name} batch={batch} path={path}")
    L = inputs.integer_layer(name, n, m, k, 5000 + n + k, (batch,), a_vals=(1.0,), mid_vals=vals, b_vals=vals)
    X = L.X[batch]
    rows = np.arange(batch) if batch <= 16 else tile_rows(batch, 1)
    ref = O.sampled_forward(X, L.A, L.B, L.a, L.mid, L.b, rows, np.arange(n))
    assert np.abs(ref).max() <= 65504
    if fp16_intermediate(path, batch):
        u, t, v, s, y = O.factored_intermediate(X[rows], L.A, L.B, L.a, L.mid, L.b)
        assert np.abs(v).max() <= 2048
    y = run(L, X, path)
    assert_bits(y[rows], ref, f"integer full {name} b{batch}")


# fp16 subnormals.  (a) Outputs on subnormals, ties included: a in {2^-24,
# 2^-23, 2^-20} with mid = 1/2 makes y = a * s with s = Σ_j ±t_j / 2; every
# t_j of a batch row has the parity of the row's count of nonzero x_l with
# odd b_l, so with k odd, s is a half-integer on the rows where that count is
# odd, and their outputs with a = 2^-24 lie halfway between two subnormals
# (they round to even).  (b)
# Subnormal intermediates: mid in {2^-20, 2^-19} puts v = t * mid (an fp16
# operand on the batch 2..16 decode and the prefill) on subnormals, with a in
# {2^10, 2^11} bringing y back to normal values.  Every value stays exact on
# both sides up to the single final rounding (v exact in fp16 where the path
# rounds it).  Batch 1 is the int8 decode, 9 the matrix-core decode, 17 and
# 100 the prefill.
SUBNORMAL_CASES = [
    ("subnormal-y", (2.0 ** -24, 2.0 ** -23, 2.0 ** -20), (0.5,), (1.0, 2.0)),
    ("subnormal-v", (1024.0, 2048.0), (2.0 ** -20, 2.0 ** -19), (1.0, 2.0)),
]


@pytest.mark.parametrize("n,m,k", [(65, 97, 33), (300, 1100, 201)])
@pytest.mark.parametrize("batch", [1, 9, 17, 100])
@pytest.mark.parametrize("case", range(len(SUBNORMAL_CASES)), ids=[c[0] for c in SUBNORMAL_CASES])
def test_fp16_subnormal_bit_exact(gpu, n, m, k, batch, case):
    name, a_vals, mid_vals, b_vals = SUBNORMAL_CASES[case]
    _say(f"{name} n={n} m={m} k={k} batch={batch}")
    L = inputs.integer_layer(name, n, m, k, 9100 + n + batch, (batch,), a_vals=a_vals, mid_vals=mid_vals,
                             b_vals=b_vals)
    X = L.X[batch]
    u, t, v, s, y = O.factored_intermediate(X, L.A, L.B, L.a, L.mid, L.b)
    assert np.abs(t).max() < 2 ** 20 and np.array_equal(t, np.round(t))
    assert np.array_equal(O.rne_fp16(v).astype(np.float64), v), "v must be exact in fp16"
    want = O.rne_fp16(y)
    tiny = np.abs(want.astype(np.float64)) < 2.0 ** -14
    if name == "subnormal-y":
        assert tiny.sum() > 0.25 * want.size, "most outputs should be subnormal"
        if batch >= 9:
            assert np.any(np.abs(y / 2.0 ** -24 - np.round(y / 2.0 ** -24)) == 0.5), "some outputs are ties"
    else:
        vs = np.abs(v[v != 0])
        assert np.mean(vs < 2.0 ** -14) > 0.25, "most intermediates should be subnormal"
    got = run(L, X)
    assert_bits(got, y, f"{name} {n}x{m}x{k} b{batch}")


# Large |x * b|: x in {-2048, 0, 2048} and b in {32, 64} make u = x * b reach
# 131072, past the fp16 range (the batch-1 decode holds u in fp32; the other
# paths fold b into the sign operand).  mid = 2^-10 and a = 2^-10 keep v and
# y inside fp16, v exact in it.
@pytest.mark.parametrize("batch", [1, 9, 100])
def test_large_input_products_bit_exact(gpu, batch):
    n, m, k = 65, 97, 33
    _say(f"large x*b n={n} m={m} k={k} batch={batch}")
    L = inputs.integer_layer("xb", n, m, k, 9300 + batch, (batch,), a_vals=(2.0 ** -10,), mid_vals=(2.0 ** -10,),
                             b_vals=(32.0, 64.0), x_vals=(-2048.0, 0.0, 2048.0))
    X = L.X[batch]
    u, t, v, s, y = O.factored_intermediate(X, L.A, L.B, L.a, L.mid, L.b)
    assert np.abs(u).max() > 65504 and np.abs(t).max() < 2 ** 24
    assert np.array_equal(O.rne_fp16(v).astype(np.float64), v) and np.abs(y).max() <= 65504
    got = run(L, X)
    assert np.all(np.isfinite(got.astype(np.float64)))
    assert_bits(got, y, f"large x*b b{batch}")


def test_forward_rejects_host_output(gpu):
    """An out= tensor in host memory (or on another device), a missing
    grouped output or a dX output of another batch is refused before anything
    is launched."""
    torch = _torch()
    _say("host out tensor")
    L = inputs.random_layer("h", 64, 96, 32, 3, 0.05, 1.0, 0.05, (2,))
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=4, backward=True)
    try:
        x = torch.from_numpy(L.X[2]).cuda()
        with pytest.raises(ValueError):
            H.forward(x, out=torch.empty((2, 64), dtype=torch.float16))
        # grouped outputs: in host memory, or fewer than the layers
        with pytest.raises(ValueError):
            dbf.forward_group([H, H], x, [torch.empty((2, 64), dtype=torch.float16, device="cuda"),
                                          torch.empty((2, 64), dtype=torch.float16)])
        with pytest.raises(ValueError):
            dbf.forward_group([H, H], x, [torch.empty((2, 64), dtype=torch.float16, device="cuda")])
        # dX output with another batch than dy (the kernel would write dy's rows)
        dy = torch.zeros((2, 64), dtype=torch.float16, device="cuda")
        with pytest.raises(ValueError):
            H.backward_data(dy, out=torch.empty((1, 96), dtype=torch.float16, device="cuda"))
        torch.cuda.synchronize()
    finally:
        H.close()


# --------------------------------------------------------------------------- the five workloads

def _workload_cases():
    cases = []
    for cid in inputs.CONFIG_IDS:
        for bt in {1: (1,), 2: (1, 16), 3: (1, 16, 2048), 4: (1, 2048), 5: (1, 2048)}[cid]:
            cases.append((cid, bt))
    return cases


@pytest.mark.parametrize("cid,batch", _workload_cases(), ids=[f"c{c}-b{b}" for c, b in _workload_cases()])
def test_workload_tolerance(gpu, cid, batch):
    cfg = inputs.config(cid)
    for L in cfg.layers:
        _say(f"workload c{cid} layer={L.name} batch={batch}")
        X = L.X[batch]
        rows = np.arange(batch) if batch <= 16 else tile_rows(batch, cid)
        ref = O.sampled_forward(X, L.A, L.B, L.a, L.mid, L.b, rows, np.arange(L.n))
        y = run(L, X)
        err = assert_tol(y[rows], ref, f"c{cid} {L.name} b{batch}")
        _say(f"  worst row rel err {err:.3e} over {len(rows)} rows")


# --------------------------------------------------------------------------- invariants and edge cases

def test_determinism_and_batch_independence(gpu):
    torch = _torch()
    L = inputs.random_layer("d", 1000, 1300, 600, 9, 0.05, 1.0, 0.05, (16, 40))
    for path, bt in ((dbf.DBF_PATH_DECODE, 16), (dbf.DBF_PATH_PREFILL, 40)):
        _say(f"determinism path={path} batch={bt}")
        X = L.X[bt]
        H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=bt)
        try:
            x = torch.from_numpy(X).cuda()
            y1 = H.forward(x, path=path).cpu().numpy()
            y2 = H.forward(x, path=path).cpu().numpy()
            assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
            if path == dbf.DBF_PATH_DECODE:
                # batch 2..16 share one kernel form (one fp16 plane; staged
                # in rounds or loaded directly, the MFMAs run in the same
                # order): every output column is summed in the same order,
                # identical bits
                for bsub in (2, 8, 9):
                    ys = H.forward(x[:bsub].clone(), path=path).cpu().numpy()
                    assert np.array_equal(ys.view(np.uint16), y1[:bsub].view(np.uint16)), f"batch {bsub}"
            for r in (0, 5, bt - 1):
                yr = H.forward(x[r:r + 1].clone(), path=path).cpu().numpy()
                if path == dbf.DBF_PATH_PREFILL:
                    # the same kernel code serves both batch sizes and every
                    # output column is summed in the same order: identical bits
                    assert np.array_equal(yr[0].view(np.uint16), y1[r].view(np.uint16)), f"row {r}"
                else:
                    # batch 1 keeps v in fp32 (exact sums of a 32-bit fixed
                    # point vector), batch 16 rounds it to fp16 once: equal
                    # within the parity tolerance (the exact path gives batch
                    # 1's bits at batch 2..4: test_decode_exact_rows_match_batch1)
                    d = np.abs(yr[0].astype(np.float64) - y1[r].astype(np.float64)).max()
                    assert d <= TOL * np.abs(y1[r].astype(np.float64)).max(), f"row {r}"
        finally:
            H.close()


# The batch-1 int8 kernels take reductions up to 32768 (64 superchunks of 512;
# the largest vector per thread and the largest digit buffer in LDS); one
# 128-column step past it, the layer runs batch 1 on the f16 kernels with v
# (and u) as hi/lo fp16 planes.  Both reductions: m (stage 1) and k (stage 2).
LIMIT_SHAPES = [
    # n, m, k, int8 at batch 1
    (64, 32768, 64, True),
    (64, 32896, 64, False),
    (80, 96, 32768, True),
    (80, 96, 32832, False),
]


@pytest.mark.parametrize("n,m,k,i8", LIMIT_SHAPES)
def test_batch1_reduction_limits(gpu, n, m, k, i8):
    """At and just past the int8 kernels' reduction limit: the oracle's values
    at batch 1 on the default path, and the same bits on the explicit decode
    path; the exact path serves the layer at batch 1 only where the int8
    kernels do."""
    torch = _torch()
    _say(f"batch-1 reduction limit n={n} m={m} k={k} int8={i8}")
    L = inputs.random_layer("lim", n, m, k, 9500 + m + k, 0.02, 1.0, 0.02, (1,))
    X = L.X[1]
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=1)
    try:
        x = torch.from_numpy(X).cuda()
        y = H.forward(x).cpu().numpy()
        assert_tol(y, O.dense_forward(X, L.A, L.B, L.a, L.mid, L.b), f"limit {n}x{m}x{k}")
        yd = H.forward(x, path=dbf.DBF_PATH_DECODE).cpu().numpy()
        assert np.array_equal(yd.view(np.uint16), y.view(np.uint16))
        if i8:
            ye = H.forward(x, path=dbf.DBF_PATH_DECODE_EXACT).cpu().numpy()
            assert np.array_equal(ye.view(np.uint16), y.view(np.uint16))
        else:
            out = torch.empty((1, n), dtype=torch.float16, device="cuda")
            with pytest.raises(dbf.DbfError) as e:
                dbf.dbf_linear_forward_ex(H.handle, x.data_ptr(), out.data_ptr(), 1, dbf.DBF_PATH_DECODE_EXACT, 0)
            assert e.value.status == dbf.DBF_ERR_UNSUPPORTED
        torch.cuda.synchronize()
    finally:
        H.close()


# Layers on which the exact path runs batch 2..4 (m and k_pad up to 8192):
# ragged sizes, m not a multiple of 8 (element-wise vector loads), the
# 4096x4096 projection at about 1 bit per weight, and the largest reduction
# that qualifies (m = 8192: 16 superchunks, two octets per thread).
ROWS_SHAPES = [
    # n, m, k
    (130, 200, 190),
    (77, 1001, 333),
    (4096, 4096, 2048),
    (300, 8192, 8192),
]


@pytest.mark.parametrize("n,m,k", ROWS_SHAPES)
def test_decode_exact_rows_match_batch1(gpu, n, m, k):
    """DBF_PATH_DECODE_EXACT runs batch 1..4 on the batch-1 int8 kernels with
    one fixed-point exponent per batch row: every row of the batch gives the
    bits of that row's own batch-1 forward (on either path), and the oracle's
    values."""
    torch = _torch()
    _say(f"int8 batch rows n={n} m={m} k={k}")
    L = inputs.random_layer("r", n, m, k, 9100 + n + m, 0.02, 1.0, 0.02, (4,))
    X = L.X[4]
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=4)
    try:
        x = torch.from_numpy(X).cuda()
        one = [H.forward(x[r:r + 1].clone()).cpu().numpy() for r in range(4)]
        exact = dbf.DBF_PATH_DECODE_EXACT
        for r in range(4):
            y1 = H.forward(x[r:r + 1].clone(), path=exact).cpu().numpy()
            assert np.array_equal(y1.view(np.uint16), one[r].view(np.uint16)), f"batch 1 row {r}"
        for bt in (2, 3, 4):
            y = H.forward(x[:bt].clone(), path=exact).cpu().numpy()
            for r in range(bt):
                assert np.array_equal(y[r].view(np.uint16), one[r][0].view(np.uint16)), f"batch {bt} row {r}"
            again = H.forward(x[:bt].clone(), path=exact).cpu().numpy()
            assert np.array_equal(again.view(np.uint16), y.view(np.uint16)), f"batch {bt} repeated"
        ref = O.sampled_forward(X, L.A, L.B, L.a, L.mid, L.b, np.arange(4), np.arange(n))
        assert_tol(y, ref, f"int8 batch 4 {n}x{m}x{k}")
    finally:
        H.close()


def test_decode_exact_unsupported_layers(gpu):
    """The exact path refuses batch 2..4 on a layer wider than 8192 and any
    batch on a 0/1 (BQQ-form) layer, and leaves the output untouched."""
    torch = _torch()
    _say("exact path: unsupported layers")
    L = inputs.random_layer("w", 64, 8320, 64, 11, 0.02, 1.0, 0.02, (2,))
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=2)
    Q = inputs.bqq_layer("q", 64, 96, 64, 2, 12, (2,))
    HQ = dbf.Layer.bqq(Q.Y, Q.Z, Q.r, Q.s, Q.t, Q.u, max_batch=2)
    try:
        x = torch.from_numpy(L.X[2]).cuda()
        y = torch.full((2, 64), 7.0, dtype=torch.float16, device="cuda")
        with pytest.raises(dbf.DbfError) as e:
            dbf.dbf_linear_forward_ex(H.handle, x.data_ptr(), y.data_ptr(), 2, dbf.DBF_PATH_DECODE_EXACT, 0)
        assert e.value.status == dbf.DBF_ERR_UNSUPPORTED
        y1 = H.forward(x[:1].clone(), path=dbf.DBF_PATH_DECODE_EXACT).cpu().numpy()   # batch 1: served
        assert np.array_equal(y1.view(np.uint16), H.forward(x[:1].clone()).cpu().numpy().view(np.uint16))
        xq = torch.from_numpy(Q.X[2]).cuda()
        with pytest.raises(dbf.DbfError) as e:
            dbf.dbf_linear_forward_ex(HQ.handle, xq.data_ptr(), y.data_ptr(), 1, dbf.DBF_PATH_DECODE_EXACT, 0)
        assert e.value.status == dbf.DBF_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert np.all(y.cpu().numpy() == 7.0)
    finally:
        H.close()
        HQ.close()


def test_output_guard_regions(gpu):
    """No write outside y: the output slice sits between two guard regions."""
    torch = _torch()
    L = inputs.random_layer("g", 333, 257, 129, 4, 0.05, 1.0, 0.05, (7, 33))
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=64)
    try:
        for bt, path in ((7, dbf.DBF_PATH_DECODE), (33, dbf.DBF_PATH_PREFILL)):
            _say(f"guard batch={bt} path={path}")
            guard = 4096
            buf = torch.full((guard * 2 + bt * L.n,), 12345.0, dtype=torch.float16, device="cuda")
            out = buf[guard:guard + bt * L.n].view(bt, L.n)
            x = torch.from_numpy(L.X[bt]).cuda()
            H.forward(x, out=out, path=path)
            torch.cuda.synchronize()
            b = buf.cpu().numpy()
            assert np.all(b[:guard] == np.float16(12345.0)) and np.all(b[-guard:] == np.float16(12345.0))
            assert_tol(out.cpu().numpy(), O.dense_forward(L.X[bt], L.A, L.B, L.a, L.mid, L.b), "guard")
    finally:
        H.close()


def test_sign_flip_symmetry_on_gpu(gpu):
    """Negating row i of A together with a_i leaves the output unchanged."""
    L = inputs.random_layer("f", 200, 300, 100, 6, 0.05, 1.0, 0.05, (4,))
    A2, a2 = L.A.copy(), L.a.copy()
    A2[[3, 50, 199]] *= -1
    a2[[3, 50, 199]] = -a2[[3, 50, 199]]
    L2 = inputs.Layer("f2", L.n, L.m, L.k, A2, L.B, a2, L.mid, L.b, L.X)
    for path in (dbf.DBF_PATH_DECODE, dbf.DBF_PATH_PREFILL):
        _say(f"sign flip path={path}")
        y1 = run(L, L.X[4], path)
        y2 = run(L2, L.X[4], path)
        assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_zero_input_and_zero_batch(gpu):
    torch = _torch()
    L = inputs.random_layer("z", 64, 96, 32, 2, 0.05, 1.0, 0.05, (3,))
    _say("zero input")
    for path in (dbf.DBF_PATH_DECODE, dbf.DBF_PATH_PREFILL):
        y = run(L, np.zeros((3, 96), np.float16), path)
        assert np.all(y.astype(np.float64) == 0)
    _say("zero batch")
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=4)
    try:
        x = torch.zeros((0, 96), dtype=torch.float16, device="cuda")
        y = H.forward(x)
        assert y.shape == (0, 64)
        dbf.dbf_linear_forward(H.handle, 0, 0, 0, 0)   # batch 0 with null pointers: no launch
    finally:
        H.close()


def test_error_paths_on_gpu(gpu):
    torch = _torch()
    L = inputs.random_layer("e", 64, 96, 32, 3, 0.05, 1.0, 0.05, (20,))
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=20)
    try:
        _say("error paths")
        x = torch.from_numpy(L.X[20]).cuda()
        y = torch.empty((20, 64), dtype=torch.float16, device="cuda")
        with pytest.raises(dbf.DbfError) as e:
            dbf.dbf_linear_forward(H.handle, x.data_ptr(), y.data_ptr(), 21, 0)
        assert e.value.status == dbf.DBF_ERR_INVALID_ARG
        with pytest.raises(dbf.DbfError):
            dbf.dbf_linear_forward(H.handle, x.data_ptr(), y.data_ptr(), -1, 0)
        with pytest.raises(dbf.DbfError):
            dbf.dbf_linear_forward_ex(H.handle, x.data_ptr(), y.data_ptr(), 20, dbf.DBF_PATH_DECODE, 0)
        with pytest.raises(dbf.DbfError) as e:   # the table path is no longer built
            dbf.dbf_linear_forward_ex(H.handle, x.data_ptr(), y.data_ptr(), 4, dbf.DBF_PATH_DECODE_TABLE, 0)
        assert e.value.status == dbf.DBF_ERR_UNSUPPORTED
        with pytest.raises(dbf.DbfError):
            dbf.dbf_linear_forward_ex(H.handle, x.data_ptr(), y.data_ptr(), 4, 7, 0)
        with pytest.raises(dbf.DbfError) as e:   # the exact path serves batch 1..4
            dbf.dbf_linear_forward_ex(H.handle, x.data_ptr(), y.data_ptr(), 5, dbf.DBF_PATH_DECODE_EXACT, 0)
        assert e.value.status == dbf.DBF_ERR_INVALID_ARG
        with pytest.raises(dbf.DbfError):   # misaligned output pointer
            dbf.dbf_linear_forward(H.handle, x.data_ptr(), y.data_ptr() + 2, 4, 0)
        info = H.info()
        assert (info["n"], info["m"], info["k"], info["max_batch"]) == (64, 96, 32, 20)
        assert info["k_pad"] == 64 and info["m_pad"] == 128 and info["n_pad"] == 64
    finally:
        H.close()


def _warm_library(L, flags=0):
    """One pack, forward and free, so that the runtime's one-time set-up on
    the library's first allocation and launch (code objects, heaps) is not
    counted as a leak by a test that compares free device memory."""
    torch = _torch()
    h = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=64, backward=bool(flags))
    x = torch.zeros((64, L.m), dtype=torch.float16, device="cuda")
    h.forward(x[:1])
    h.forward(x)
    torch.cuda.synchronize()
    h.close()
    torch.cuda.synchronize()


def test_injected_allocation_failure_leaks_nothing(gpu):
    torch = _torch()
    L = inputs.random_layer("o", 512, 512, 256, 3, 0.05, 1.0, 0.05, (1,))
    _warm_library(L)
    free0 = torch.cuda.mem_get_info()[0]
    try:
        for nth in range(1, 14):
            _say(f"inject allocation failure #{nth}")
            os.environ["DBF_TEST_FAIL_ALLOC"] = str(nth)
            with pytest.raises(dbf.DbfError) as e:
                dbf.dbf_pack(L.n, L.m, L.k, L.A, L.B, L.a, L.mid, L.b, 64)
            assert e.value.status == dbf.DBF_ERR_OOM
        os.environ["DBF_TEST_FAIL_ALLOC"] = "100"
        h = dbf.dbf_pack(L.n, L.m, L.k, L.A, L.B, L.a, L.mid, L.b, 64)   # a pack makes 13 allocations
        dbf.dbf_free(h)
    finally:
        os.environ.pop("DBF_TEST_FAIL_ALLOC", None)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert abs(free1 - free0) < (8 << 20), (free0, free1)


def test_timing_facility(gpu):
    torch = _torch()
    L = inputs.random_layer("t", 256, 256, 128, 3, 0.05, 1.0, 0.05, (1, 32))
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=32)
    try:
        _say("timing")
        dbf.dbf_timing_enable(H.handle, True)
        for bt in (1, 32):
            x = torch.from_numpy(L.X[bt]).cuda()
            for _ in range(3):
                H.forward(x)
        t = dbf.dbf_timing_read(H.handle)
        assert sum(v["launches"] for v in t.values()) >= 6
        assert all(v["total_ms"] > 0 for v in t.values())
        dbf.dbf_timing_enable(H.handle, False)
        assert dbf.dbf_timing_read(H.handle) == {}
    finally:
        H.close()


# --------------------------------------------------------------------------- layers sharing one input

GROUPS = [
    # (m, [(n, k), ...])
    (300, [(64, 64), (130, 190), (70, 33)]),
    (1100, [(257, 100), (64, 1500)]),
    (96, [(64, 64)]),
    (4096, [(4096, 2688), (1024, 1216), (1024, 1536)]),   # attention q/k/v shapes
    (640, [(130, 190), (64, 64), (300, 1000)]),          # m % 64 == 0: grouped products above batch 16
]


@pytest.mark.parametrize("gi", range(len(GROUPS)))
@pytest.mark.parametrize("batch", [1, 3, 9, 16, 40, 2048])
def test_group_forward_equals_single_layers(gpu, gi, batch):
    """One launch per stage for layers sharing x gives each layer's own
    forward bit for bit at decode batches (same kernel arithmetic) and the
    oracle's values at every batch.  Above batch 16 the grouped products sum
    each output over its whole K, where a layer's own product may cut K into
    parts: equal within the parity tolerance there."""
    torch = _torch()
    m, dims = GROUPS[gi]
    _say(f"group m={m} layers={dims} batch={batch}")
    rng = np.random.default_rng(100 + gi)
    big = m >= 4096
    # the attention-shaped group takes the block workload's value ranges
    X = (rng.standard_normal((batch, m)) if big else rng.uniform(-4, 4, size=(batch, m))).astype(np.float16)
    layers, hs = [], []
    try:
        for j, (n, k) in enumerate(dims):
            if big:
                Lr = inputs.random_layer("g", n, m, k, 7000 + 10 * gi + j, 0.02, 1.0, 0.02, ())
                A, B, a, mid, b = Lr.A, Lr.B, Lr.a, Lr.mid, Lr.b
            else:
                _, A, B, a, mid, b = inputs.tiny_case(7000 + 10 * gi + j, n, m, k, 1, signed_scales=True)
            layers.append((A, B, a, mid, b))
            hs.append(dbf.Layer(A, B, a, mid, b, max_batch=batch))
        x = torch.from_numpy(X).cuda()
        ys = dbf.forward_group(hs, x)
        torch.cuda.synchronize()
        for j, (H, y) in enumerate(zip(hs, ys)):
            single = H.forward(x).cpu().numpy()
            got = y.cpu().numpy()
            if batch <= 16:
                assert np.array_equal(got.view(np.uint16), single.view(np.uint16)), f"layer {j}"
            else:
                d = np.abs(got.astype(np.float64) - single.astype(np.float64)).max(axis=1)
                assert np.all(d <= TOL * np.abs(single.astype(np.float64)).max(axis=1)), f"layer {j} vs own forward"
            A, B, a, mid, b = layers[j]
            if A.shape[0] * m * A.shape[1] * batch <= 1 << 30:
                assert_tol(got, O.dense_forward(X, A, B, a, mid, b), f"group layer {j}")
            else:
                rows = np.arange(min(batch, 3)) if batch <= 16 else tile_rows(batch, 5 + j)
                ref = O.sampled_forward(X, A, B, a, mid, b, rows, np.arange(A.shape[0]))
                assert_tol(got[rows], ref, f"group layer {j} (sampled rows)")
    finally:
        for H in hs:
            H.close()


def test_group_forward_errors(gpu):
    torch = _torch()
    L1 = inputs.random_layer("g1", 64, 96, 32, 3, 0.05, 1.0, 0.05, (4,))
    L2 = inputs.random_layer("g2", 80, 96, 64, 4, 0.05, 1.0, 0.05, (4,))
    L3 = inputs.random_layer("g3", 64, 128, 32, 5, 0.05, 1.0, 0.05, (4,))
    H1 = dbf.Layer(L1.A, L1.B, L1.a, L1.mid, L1.b, max_batch=4)
    H2 = dbf.Layer(L2.A, L2.B, L2.a, L2.mid, L2.b, max_batch=2)
    H3 = dbf.Layer(L3.A, L3.B, L3.a, L3.mid, L3.b, max_batch=4)
    try:
        _say("group errors")
        x = torch.from_numpy(L1.X[4]).cuda()
        y1 = torch.empty((4, 64), dtype=torch.float16, device="cuda")
        y2 = torch.empty((4, 80), dtype=torch.float16, device="cuda")
        with pytest.raises(dbf.DbfError):   # differing input widths
            dbf.dbf_linear_forward_group([H1.handle, H3.handle], x.data_ptr(), [y1.data_ptr(), y2.data_ptr()], 4)
        with pytest.raises(dbf.DbfError):   # batch above one handle's max_batch
            dbf.dbf_linear_forward_group([H1.handle, H2.handle], x.data_ptr(), [y1.data_ptr(), y2.data_ptr()], 4)
        with pytest.raises(dbf.DbfError):   # empty group
            dbf.dbf_linear_forward_group([], x.data_ptr(), [], 4)
        with pytest.raises(dbf.DbfError):   # more than 8 layers
            dbf.dbf_linear_forward_group([H1.handle] * 9, x.data_ptr(), [y1.data_ptr()] * 9, 4)
        with pytest.raises(dbf.DbfError):   # misaligned output
            dbf.dbf_linear_forward_group([H1.handle], x.data_ptr(), [y1.data_ptr() + 2], 4)
        with pytest.raises(dbf.DbfError):   # null output
            dbf.dbf_linear_forward_group([H1.handle], x.data_ptr(), [0], 4)
        dbf.dbf_linear_forward_group([H1.handle, H2.handle], 0, [0, 0], 0)   # batch 0: no launch
        # batch 2 is within both max_batch values
        dbf.dbf_linear_forward_group([H1.handle, H2.handle], x.data_ptr(), [y1.data_ptr(), y2.data_ptr()], 2)
        torch.cuda.synchronize()
        assert_tol(y1[:2].cpu().numpy(), O.dense_forward(L1.X[4][:2], L1.A, L1.B, L1.a, L1.mid, L1.b), "group b2")
    finally:
        H1.close()
        H2.close()
        H3.close()


# --------------------------------------------------------------------------- gradients (fine-tuning of the factors)

def _vec_rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


BWD_SHAPES = [
    # n, m, k
    (1, 1, 1),
    (3, 5, 7),
    (64, 64, 64),
    (130, 200, 190),
    (257, 96, 130),
    (100, 1100, 70),
]


@pytest.mark.parametrize("n,m,k", BWD_SHAPES)
@pytest.mark.parametrize("batch", [1, 3, 17, 100])
def test_backward_data_matches_oracle_and_transposed_forward(gpu, n, m, k, batch):
    """dX = dY W: the oracle's value, and the same bits as the forward of a
    layer packed directly from the transposed factors (Bᵀ, Aᵀ, b, mid, a)."""
    torch = _torch()
    _say(f"backward data n={n} m={m} k={k} batch={batch}")
    _, A, B, a, mid, b = inputs.tiny_case(8000 + n + m + k, n, m, k, 1, signed_scales=True)
    dY = np.random.default_rng(batch + n).uniform(-4, 4, (batch, n)).astype(np.float16)
    H = dbf.Layer(A, B, a, mid, b, max_batch=batch, backward=True)
    Ht = dbf.Layer(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), b, mid, a, max_batch=batch)
    try:
        dy = torch.from_numpy(dY).cuda()
        dx = H.backward_data(dy).cpu().numpy()
        direct = Ht.forward(dy).cpu().numpy()
        assert np.array_equal(dx.view(np.uint16), direct.view(np.uint16))
        X0 = np.zeros((batch, m), np.float16)
        ref = O.backward(X0, dY, A, B, a, mid, b)[0]
        assert_tol(dx, ref, f"dX {n}x{m}x{k}")
    finally:
        H.close()
        Ht.close()


@pytest.mark.parametrize("n,m,k", BWD_SHAPES)
@pytest.mark.parametrize("batch", [1, 5, 70, 300])
def test_backward_gradients_match_oracle(gpu, n, m, k, batch):
    torch = _torch()
    _say(f"backward n={n} m={m} k={k} batch={batch}")
    X, A, B, a, mid, b = inputs.tiny_case(9000 + n + m + k + batch, n, m, k, batch, signed_scales=True)
    dY = np.random.default_rng(7 * batch + n).uniform(-4, 4, (batch, n)).astype(np.float16)
    H = dbf.Layer(A, B, a, mid, b, max_batch=batch, backward=True)
    try:
        x = torch.from_numpy(X).cuda()
        dy = torch.from_numpy(dY).cuda()
        dx, da, dmid, db = (t.cpu().numpy() for t in H.backward(x, dy))
        rdx, rda, rdmid, rdb = O.backward(X, dY, A, B, a, mid, b)
        assert_tol(dx, rdx, "dX")
        for name, got, ref in (("da", da, rda), ("dmid", dmid, rdmid), ("db", db, rdb)):
            err = _vec_rel(got, ref)
            assert err <= TOL, f"{name}: rel err {err:.3e}"
        # deterministic: a second call gives the same bits
        again = [t.cpu().numpy() for t in H.backward(x, dy)]
        for g1, g2 in zip((dx, da, dmid, db), again):
            assert np.array_equal(g1.view(np.uint8), g2.view(np.uint8))
    finally:
        H.close()


def test_backward_partial_outputs_and_errors(gpu):
    """Any of dx, da, dmid, db may be skipped; the rest are unchanged.  A
    handle packed without backward support refuses."""
    torch = _torch()
    n, m, k, bt = 130, 200, 190, 33
    X, A, B, a, mid, b = inputs.tiny_case(4242, n, m, k, bt, signed_scales=True)
    dY = np.random.default_rng(5).uniform(-4, 4, (bt, n)).astype(np.float16)
    H = dbf.Layer(A, B, a, mid, b, max_batch=bt, backward=True)
    H0 = dbf.Layer(A, B, a, mid, b, max_batch=bt)
    try:
        _say("backward partial outputs")
        x = torch.from_numpy(X).cuda()
        dy = torch.from_numpy(dY).cuda()
        full = [t.cpu().numpy() for t in H.backward(x, dy)]
        for keep in range(4):
            outs = [torch.full((bt, m), 7.0, dtype=torch.float16, device="cuda"),
                    torch.full((n,), 7.0, device="cuda"), torch.full((k,), 7.0, device="cuda"),
                    torch.full((m,), 7.0, device="cuda")]
            ptrs = [o.data_ptr() if i == keep else 0 for i, o in enumerate(outs)]
            dbf.dbf_linear_backward(H.handle, x.data_ptr(), dy.data_ptr(), *ptrs, bt,
                                    torch.cuda.current_stream().cuda_stream)
            got = outs[keep].cpu().numpy()
            assert np.array_equal(got.view(np.uint8), full[keep].view(np.uint8)), keep
        with pytest.raises(dbf.DbfError) as e:
            dbf.dbf_linear_backward_data(H0.handle, dy.data_ptr(), x.data_ptr(), bt)
        assert e.value.status == dbf.DBF_ERR_UNSUPPORTED
        with pytest.raises(ValueError):   # batch of dy differs from x (the binding's check)
            H.backward(x, torch.cat([dy, dy]))
        with pytest.raises(dbf.DbfError) as e:
            dbf.dbf_linear_backward(H.handle, x.data_ptr(), dy.data_ptr(), 0, 0, 0, 0, bt + 1, 0)
        assert e.value.status == dbf.DBF_ERR_INVALID_ARG
    finally:
        H.close()
        H0.close()


def test_backward_full_size_projection(gpu):
    """The 4096 x 4096, k = 2048 projection at batch 256 with its workload's
    value ranges and a unit-scale upstream gradient."""
    torch = _torch()
    L = inputs.config(2).layers[0]
    bt = 256
    rng = np.random.default_rng(3)
    X = rng.standard_normal((bt, L.m)).astype(np.float16)
    dY = rng.standard_normal((bt, L.n)).astype(np.float16)
    _say("backward full size 4096x4096 k2048 batch 256")
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=bt, backward=True)
    try:
        dx, da, dmid, db = (t.cpu().numpy() for t in H.backward(torch.from_numpy(X).cuda(), torch.from_numpy(dY).cuda()))
        rdx, rda, rdmid, rdb = O.backward(X, dY, L.A, L.B, L.a, L.mid, L.b)
        assert_tol(dx, rdx, "dX full")
        for name, got, ref in (("da", da, rda), ("dmid", dmid, rdmid), ("db", db, rdb)):
            err = _vec_rel(got, ref)
            _say(f"  {name} rel err {err:.3e}")
            assert err <= TOL, f"{name}: rel err {err:.3e}"
    finally:
        H.close()


def test_backward_pack_allocation_failures_leak_nothing(gpu):
    """dbf_pack_ex with DBF_PACK_BACKWARD: a failure at any of its device
    allocations (the layer's, the transposed layer's, the gradient workspace)
    returns DBF_ERR_OOM and frees everything already allocated."""
    torch = _torch()
    L = inputs.random_layer("ob", 300, 200, 130, 3, 0.05, 1.0, 0.05, (1,))
    _warm_library(L, dbf.DBF_PACK_BACKWARD)
    free0 = torch.cuda.mem_get_info()[0]
    try:
        n_alloc = 28   # 13 for the layer, 13 for the transposed layer, t and the batch-sum partials
        for nth in range(1, n_alloc + 1):
            _say(f"backward pack: inject allocation failure #{nth}")
            os.environ["DBF_TEST_FAIL_ALLOC"] = str(nth)
            with pytest.raises(dbf.DbfError) as e:
                dbf.dbf_pack(L.n, L.m, L.k, L.A, L.B, L.a, L.mid, L.b, 64, dbf.DBF_PACK_BACKWARD)
            assert e.value.status == dbf.DBF_ERR_OOM
        os.environ["DBF_TEST_FAIL_ALLOC"] = str(n_alloc + 1)
        h = dbf.dbf_pack(L.n, L.m, L.k, L.A, L.B, L.a, L.mid, L.b, 64, dbf.DBF_PACK_BACKWARD)
        info = dbf.dbf_get_info(h)
        assert info["workspace_bytes"] > 0 and info["packed_bytes"] > 0
        dbf.dbf_free(h)
    finally:
        os.environ.pop("DBF_TEST_FAIL_ALLOC", None)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert abs(free1 - free0) < (8 << 20), (free0, free1)


def test_graph_replay_of_prefill_and_backward(gpu):
    """Prefill forwards and gradient calls captured in a HIP graph and
    replayed several times, with eager work between the replays, give the
    eager results every time."""
    torch = _torch()
    n, m, k, bt = 320, 256, 192, 96
    X, A, B, a, mid, b = inputs.tiny_case(515, n, m, k, bt, signed_scales=True)
    dY = np.random.default_rng(9).uniform(-2, 2, (bt, n)).astype(np.float16)
    H = dbf.Layer(A, B, a, mid, b, max_batch=bt, backward=True)
    try:
        _say("graph replay prefill + backward")
        x = torch.from_numpy(X).cuda()
        dy = torch.from_numpy(dY).cuda()
        want_y = H.forward(x).cpu().numpy()
        want_g = [t.cpu().numpy() for t in H.backward(x, dy)]
        y = torch.empty((bt, n), dtype=torch.float16, device="cuda")
        dx = torch.empty((bt, m), dtype=torch.float16, device="cuda")
        da = torch.empty(n, dtype=torch.float32, device="cuda")
        dmid = torch.empty(k, dtype=torch.float32, device="cuda")
        db = torch.empty(m, dtype=torch.float32, device="cuda")
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                H.forward(x, out=y)
                dbf.dbf_linear_backward(H.handle, x.data_ptr(), dy.data_ptr(), dx.data_ptr(), da.data_ptr(),
                                        dmid.data_ptr(), db.data_ptr(), bt, s.cuda_stream)
        torch.cuda.current_stream().wait_stream(s)
        for rep in range(4):
            for t in (y, dx):
                t.fill_(3.0)
            for t in (da, dmid, db):
                t.fill_(3.0)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().view(np.uint16), want_y.view(np.uint16)), rep
            for got, want in zip((dx, da, dmid, db), want_g):
                assert np.array_equal(got.cpu().numpy().view(np.uint8), want.view(np.uint8)), rep
            H.forward(x)   # eager work between replays
            torch.cuda.synchronize()
    finally:
        H.close()


def test_graph_replay_of_decode_paths(gpu):
    """Decode forwards captured in one HIP graph and replayed several times,
    with eager work between the replays, give the eager bits every time: the
    batch-1 int8 kernels (single layer and a group sharing x), the exact path
    at batch 3, the f16 decode at batch 9 on a wide layer whose stage 1 is cut
    into ticketed reduction parts, and the no-allocation forward."""
    torch = _torch()
    _say("graph replay of the decode paths")
    m = 640
    L1 = inputs.random_layer("g1", 300, m, 190, 31, 0.02, 1.0, 0.02, (3,))
    L2 = inputs.random_layer("g2", 130, m, 260, 32, 0.02, 1.0, 0.02, ())
    LW = inputs.random_layer("gw", 200, 10300, 600, 33, 0.02, 1.0, 0.02, (9,))
    H1 = dbf.Layer(L1.A, L1.B, L1.a, L1.mid, L1.b, max_batch=3)
    H2 = dbf.Layer(L2.A, L2.B, L2.a, L2.mid, L2.b, max_batch=3)
    HW = dbf.Layer(LW.A, LW.B, LW.a, LW.mid, LW.b, max_batch=9)
    try:
        x3 = torch.from_numpy(L1.X[3]).cuda()
        x1 = x3[:1].clone()
        xw = torch.from_numpy(LW.X[9]).cuda()
        outs = {"single": torch.empty((1, 300), dtype=torch.float16, device="cuda"),
                "g1": torch.empty((1, 300), dtype=torch.float16, device="cuda"),
                "g2": torch.empty((1, 130), dtype=torch.float16, device="cuda"),
                "exact": torch.empty((3, 300), dtype=torch.float16, device="cuda"),
                "wide": torch.empty((9, 200), dtype=torch.float16, device="cuda"),
                "noalloc": torch.empty((1, 300), dtype=torch.float16, device="cuda")}

        def work(stream):
            H1.forward(x1, out=outs["single"])
            dbf.forward_group([H1, H2], x1, [outs["g1"], outs["g2"]])
            H1.forward(x3, out=outs["exact"], path=dbf.DBF_PATH_DECODE_EXACT)
            HW.forward(xw, out=outs["wide"])
            dbf.dbf_linear_forward_noalloc(H1.handle, x1.data_ptr(), outs["noalloc"].data_ptr(), 1, stream)
        work(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        want = {k: v.cpu().numpy().copy() for k, v in outs.items()}
        assert np.array_equal(want["noalloc"].view(np.uint16), want["single"].view(np.uint16))
        assert np.array_equal(want["exact"][0].view(np.uint16), want["single"][0].view(np.uint16))
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                work(s.cuda_stream)
        torch.cuda.current_stream().wait_stream(s)
        for rep in range(4):
            for t in outs.values():
                t.fill_(3.0)
            g.replay()
            torch.cuda.synchronize()
            for k, t in outs.items():
                assert np.array_equal(t.cpu().numpy().view(np.uint16), want[k].view(np.uint16)), (rep, k)
            HW.forward(xw)   # eager work between replays (the same tickets and partials)
            torch.cuda.synchronize()
    finally:
        H1.close()
        H2.close()
        HW.close()


def test_non_default_stream(gpu):
    """Forwards enqueued on a side stream give the default-stream results."""
    torch = _torch()
    L = inputs.random_layer("st", 500, 400, 300, 12, 0.05, 1.0, 0.05, (1, 7, 64))
    H = dbf.Layer(L.A, L.B, L.a, L.mid, L.b, max_batch=64)
    try:
        _say("side stream")
        for bt in (1, 7, 64):
            x = torch.from_numpy(L.X[bt]).cuda()
            want = H.forward(x).cpu().numpy()
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                y = H.forward(x)
            s.synchronize()
            assert np.array_equal(y.cpu().numpy().view(np.uint16), want.view(np.uint16)), bt
    finally:
        H.close()
