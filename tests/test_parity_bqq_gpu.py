"""GPU parity of the BQQ-form layer (dbf_bqq_pack) against its fp64 oracle.

The weight is W = Σ_i (r_i Y_i Z_i + s_i Y_i 1 + t_i 1 Z_i) + u 1 with 0/1
matrices Y_i, Z_i (TL;DR of "Binary Quadratic Quantization: Beyond
First-Order Quantization for Real-Valued Matrix Compression", sciencestack.ai
page) and the layer output rne16(X Wᵀ).  The same bars as the DBF layer:
per batch row, max |y - ŷ| / max |ŷ| <= 2e-3 against the unrounded oracle;
bit-exact fp16 on integer data (every partial sum an exact integer on both
sides, the intermediate exact in fp16 where the path rounds it); identical
bits on repeated calls.

Every case prints its name before it touches the GPU.
"""

import sys

import numpy as np
import pytest

import dbf_linear_fwd_amd as dbf
from oracle import bqq_oracle as Q
from oracle import dbf_oracle as O
from tests import inputs

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _run(L, X, path=dbf.DBF_PATH_AUTO, max_batch=None):
    import torch
    H = dbf.Layer.bqq(L.Y, L.Z, L.r, L.s, L.t, L.u, max_batch=max_batch or max(1, X.shape[0]))
    try:
        x = torch.from_numpy(np.ascontiguousarray(X)).cuda()
        y = H.forward(x, path=path)
        torch.cuda.synchronize()
        return y.cpu().numpy()
    finally:
        H.close()


def _assert_tol(y16, ref, what):
    y = y16.astype(np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    r = np.abs(y - ref).max(axis=1) / den
    assert r.max() <= TOL, f"{what}: worst row rel err {r.max():.3e} (row {int(r.argmax())})"
    return float(r.max())


def _assert_bits(y16, ref, what):
    want = O.rne_fp16(ref).view(np.uint16).copy()
    got = y16.view(np.uint16).copy()
    got[(got & 0x7FFF) == 0] = 0
    want[(want & 0x7FFF) == 0] = 0
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}"


SHAPES = [
    # n, m, d, p
    (1, 1, 1, 1),
    (65, 97, 33, 2),
    (130, 200, 70, 3),
    (256, 256, 64, 2),
    (300, 1100, 100, 2),   # m spans two decode rounds, ragged
    (70, 300, 700, 2),     # middle dimension p d = 1400, ragged
]


@pytest.mark.parametrize("n,m,d,p", SHAPES)
@pytest.mark.parametrize("batch", [1, 3, 9, 16, 17, 100])
def test_bqq_small_shapes(gpu, n, m, d, p, batch):
    _say(f"bqq n={n} m={m} d={d} p={p} batch={batch}")
    L = inputs.bqq_layer("s", n, m, d, p, 7000 + n + m + d + p, (batch,))
    X = L.X[batch]
    ref = Q.bqq_forward(X, L.Y, L.Z, L.r, L.s, L.t, L.u)
    _assert_tol(_run(L, X), ref, f"bqq {n}x{m} d{d} p{p} b{batch}")


@pytest.mark.parametrize("batch", [1, 9, 16])
def test_bqq_prefill_path_at_decode_batch(gpu, batch):
    L = inputs.bqq_layer("s", 300, 1100, 100, 2, 7100 + batch, (batch,))
    _say(f"bqq prefill path batch={batch}")
    X = L.X[batch]
    ref = Q.bqq_forward(X, L.Y, L.Z, L.r, L.s, L.t, L.u)
    _assert_tol(_run(L, X, dbf.DBF_PATH_PREFILL), ref, f"bqq prefill b{batch}")


# Small prefill grids: both products take the split-K form, the second with
# the affine term in the finish kernel.
@pytest.mark.parametrize("batch", [17, 130])
def test_bqq_split_k(gpu, batch):
    n, m, d, p = 1000, 4096, 512, 2
    _say(f"bqq split-K n={n} m={m} d={d} p={p} batch={batch}")
    L = inputs.bqq_layer("k", n, m, d, p, 7050 + batch, (batch,))
    X = L.X[batch]
    ref = Q.bqq_forward(X, L.Y, L.Z, L.r, L.s, L.t, L.u)
    _assert_tol(_run(L, X), ref, f"bqq split-K b{batch}")
    # integer data on a narrower layer (still split: K = 1024 and 512), s, t = ±1 so the output fits fp16
    Li = inputs.bqq_layer("ki", n, 1024, 256, p, 7060 + batch, (batch,), integer=True)
    Li.s = np.sign(Li.s).astype(np.float16)
    Li.t = np.sign(Li.t).astype(np.float16)
    Xi = Li.X[batch]
    _assert_bits(_run(Li, Xi), _integer_preconditions(Li, Xi, True), f"bqq split-K integer b{batch}")


# A large batch on a layer whose second product is one wave of output tiles
# plus a partial one (n = 4400: 18 column tiles of 256 at 16 row tiles): its
# tail columns take the split-K finish, with the affine term.
def test_bqq_head_tail(gpu):
    n, m, d, p, batch = 4400, 512, 2240, 2, 2048
    _say(f"bqq head/tail n={n} m={m} d={d} p={p} batch={batch}")
    L = inputs.bqq_layer("h", n, m, d, p, 7080, (batch,))
    X = L.X[batch]
    ref = Q.bqq_forward(X, L.Y, L.Z, L.r, L.s, L.t, L.u)
    _assert_tol(_run(L, X), ref, f"bqq head/tail b{batch}")


def _integer_preconditions(L, X, fp16_intermediate):
    """Every partial sum is an integer far inside fp32's exact range, the
    kernel's intermediate v = 2 r_i (Z_i x) is exact where it is rounded to
    fp16, and the output fits fp16."""
    X64 = X.astype(np.float64)
    v = np.concatenate([2.0 * float(L.r[i]) * (X64 @ L.Z[i].astype(np.float64).T) for i in range(L.p)], axis=1)
    assert np.abs(v).sum(axis=1).max() < 2 ** 24
    if fp16_intermediate:
        assert np.abs(v).max() <= 2048
    y = Q.bqq_forward(X, L.Y, L.Z, L.r, L.s, L.t, L.u)
    assert np.abs(y).max() <= 65504
    return y


@pytest.mark.parametrize("n,m,d,p,batch", [(65, 97, 33, 2, 1), (65, 97, 33, 2, 5), (130, 200, 70, 3, 9),
                                           (256, 256, 64, 2, 16), (256, 256, 64, 2, 100), (300, 600, 100, 2, 17)])
@pytest.mark.parametrize("path", [dbf.DBF_PATH_AUTO, dbf.DBF_PATH_PREFILL])
def test_bqq_integer_bit_exact(gpu, n, m, d, p, batch, path):
    _say(f"bqq integer n={n} m={m} d={d} p={p} batch={batch} path={path}")
    L = inputs.bqq_layer("i", n, m, d, p, 7200 + n + batch, (batch,), integer=True)
    X = L.X[batch]
    fp16_v = path == dbf.DBF_PATH_PREFILL or batch > 1
    ref = _integer_preconditions(L, X, fp16_v)
    _assert_bits(_run(L, X, path), ref, f"bqq integer {n}x{m} d{d} p{p} b{batch}")


# The 4096 x 4096 projection as two binary products with d = 1024 (the
# packed size of the 4096 x 4096, k = 2048 DBF layer: 2 MiB of bits).
FULL = (4096, 4096, 1024, 2)


@pytest.mark.parametrize("batch", [1, 16, 2048])
def test_bqq_full_size(gpu, batch):
    n, m, d, p = FULL
    _say(f"bqq full size {n}x{m} d={d} p={p} batch={batch}")
    L = inputs.bqq_layer("f", n, m, d, p, 7300, (batch,))
    X = L.X[batch]
    rows = np.arange(batch) if batch <= 16 else np.random.default_rng(2).choice(batch, 12, replace=False)
    W = Q.bqq_weight(L.Y, L.Z, L.r, L.s, L.t, L.u)
    ref = X[rows].astype(np.float64) @ W.T
    y = _run(L, X)
    err = _assert_tol(y[rows], ref, f"bqq full b{batch}")
    _say(f"  worst row rel err {err:.3e}")


def test_bqq_determinism_and_errors(gpu):
    import torch
    L = inputs.bqq_layer("d", 500, 700, 200, 2, 7400, (16, 40))
    H = dbf.Layer.bqq(L.Y, L.Z, L.r, L.s, L.t, L.u, max_batch=40)
    try:
        for bt in (16, 40):
            _say(f"bqq determinism batch={bt}")
            x = torch.from_numpy(L.X[bt]).cuda()
            y1 = H.forward(x).cpu().numpy()
            y2 = H.forward(x).cpu().numpy()
            assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
        _say("bqq unsupported entries")
        x = torch.from_numpy(L.X[16]).cuda()
        with pytest.raises(dbf.DbfError) as e:
            H.forward(x, path=dbf.DBF_PATH_DECODE_TABLE)
        assert e.value.status == dbf.DBF_ERR_UNSUPPORTED
        with pytest.raises(dbf.DbfError) as e:
            dbf.forward_group([H], x)
        assert e.value.status == dbf.DBF_ERR_UNSUPPORTED
        info = H.info()
        assert info["k"] == 400 and info["n"] == 500 and info["m"] == 700
    finally:
        H.close()


def test_bqq_matches_dbf_layer_of_the_same_weight(gpu):
    """r = 4 rho, s = t = -2 rho, u = d rho turns each 0/1 product into rho
    times a ±1 product: the BQQ layer and the DBF layer with A = 1 - 2Y,
    B = 1 - 2Z, mid = rho, a = b = 1 compute the same weight (by different
    kernels' numerics: compared within the tolerance)."""
    import torch
    n, m, d = 640, 900, 256
    rng = np.random.default_rng(7500)
    Y = rng.integers(0, 2, size=(1, n, d), dtype=np.uint8)
    Z = rng.integers(0, 2, size=(1, d, m), dtype=np.uint8)
    rho = np.float16(0.015625)
    X = rng.standard_normal((8, m)).astype(np.float16)
    _say("bqq vs dbf layer")
    Hq = dbf.Layer.bqq(Y, Z, [4 * rho], [-2 * rho], [-2 * rho], np.float16(d * float(rho)), max_batch=8)
    A = (1 - 2 * Y[0].astype(np.int8)).astype(np.int8)
    B = (1 - 2 * Z[0].astype(np.int8)).astype(np.int8)
    Hd = dbf.Layer(A, B, np.ones(n, np.float16), np.full(d, rho, np.float16), np.ones(m, np.float16), max_batch=8)
    try:
        x = torch.from_numpy(X).cuda()
        yq = Hq.forward(x).cpu().numpy()
        yd = Hd.forward(x).cpu().numpy()
    finally:
        Hq.close()
        Hd.close()
    ref = O.dense_forward(X, A, B, np.ones(n, np.float16), np.full(d, rho, np.float16), np.ones(m, np.float16))
    _assert_tol(yq, ref, "bqq form")
    _assert_tol(yd, ref, "dbf form")
