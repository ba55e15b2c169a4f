"""GPU parity of the BQQ-form layer with group-wise scalars
(dbf_bqq_pack_grouped) against its fp64 oracle.

On the columns l of input group h = l // group the weight is
Σ_i (r_i[h] Y_i Z_i + s_i[h] Y_i 1 + t_i[h] 1 Z_i)[:, l] + u[h] (the BQQ
TL;DR formula of "Binary Quadratic Quantization: Beyond First-Order
Quantization for Real-Valued Matrix Compression", sciencestack.ai page, with
the group-wise scaling the same TL;DR names, read as scalars per group of
input columns).  The bars of the other layers: per batch row, max |y - ŷ| /
max |ŷ| <= 2e-3 against the unrounded oracle; bit-exact fp16 on integer
data; identical bits on repeated calls; one group gives the bits of the
single-group layer.

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


def _layer(L, max_batch):
    return dbf.Layer.bqq_grouped(L.Y, L.Z, L.r, L.s, L.t, L.u, L.group, max_batch=max_batch)


def _run(L, X, path=dbf.DBF_PATH_AUTO, max_batch=None):
    import torch
    H = _layer(L, max_batch or max(1, X.shape[0]))
    try:
        x = torch.from_numpy(np.ascontiguousarray(X)).cuda()
        y = H.forward(x, path=path)
        torch.cuda.synchronize()
        return y.cpu().numpy()
    finally:
        H.close()


def _ref(L, X):
    return Q.bqq_forward_grouped(X, L.Y, L.Z, L.r, L.s, L.t, L.u, L.group)


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
    # n, m, d, p, group
    (16, 5, 64, 1, 2),        # three groups of 2, 2, 1 columns (n > 1: the row metric
                              # normalises by the row's largest output; a single output
                              # cancelling to near zero would measure the intermediate's
                              # fp16 rounding against that one small value)
    (65, 97, 64, 2, 32),      # ragged last group of one column
    (130, 200, 128, 3, 48),
    (300, 1100, 64, 2, 128),  # m spans two decode rounds
    (70, 300, 448, 2, 100),   # middle dimension p d = 896
]


@pytest.mark.parametrize("n,m,d,p,group", SHAPES)
@pytest.mark.parametrize("batch", [1, 3, 16, 17, 100])
def test_grouped_small_shapes(gpu, n, m, d, p, group, batch):
    _say(f"bqq grouped n={n} m={m} d={d} p={p} group={group} batch={batch}")
    L = inputs.bqq_grouped_layer("g", n, m, d, p, group, 8000 + n + m + d + p + group, (batch,))
    X = L.X[batch]
    _assert_tol(_run(L, X), _ref(L, X), f"grouped {n}x{m} d{d} p{p} g{group} b{batch}")


@pytest.mark.parametrize("batch", [1, 9])
def test_grouped_prefill_path_at_decode_batch(gpu, batch):
    L = inputs.bqq_grouped_layer("gp", 300, 1100, 64, 2, 128, 8100 + batch, (batch,))
    _say(f"bqq grouped prefill path batch={batch}")
    X = L.X[batch]
    _assert_tol(_run(L, X, dbf.DBF_PATH_PREFILL), _ref(L, X), f"grouped prefill b{batch}")


# Small prefill grids: the per-term first products and the second product
# take the split-K form (the affine term in the finish kernel).
@pytest.mark.parametrize("batch", [17, 130])
def test_grouped_split_k(gpu, batch):
    n, m, d, p, g = 1000, 4096, 512, 2, 256
    _say(f"bqq grouped split-K n={n} m={m} d={d} p={p} group={g} batch={batch}")
    L = inputs.bqq_grouped_layer("gk", n, m, d, p, g, 8050 + batch, (batch,))
    X = L.X[batch]
    _assert_tol(_run(L, X), _ref(L, X), f"grouped split-K b{batch}")


# Above the decode batches, the p first products run as one product over all
# p d rows of B when d is a multiple of 256 and m of 64 (each 256-column
# output tile takes its own term's input scale); otherwise one product per
# term.  Both forms, ragged groups, split-K and whole-K grids, and integer
# data bit-exact.
@pytest.mark.parametrize("n,m,d,p,group", [(200, 640, 256, 3, 64), (70, 300, 256, 2, 100), (130, 512, 256, 2, 48)])
@pytest.mark.parametrize("batch", [17, 300])
def test_grouped_stacked_first_products(gpu, n, m, d, p, group, batch):
    _say(f"bqq grouped stacked n={n} m={m} d={d} p={p} group={group} batch={batch}")
    L = inputs.bqq_grouped_layer("gs", n, m, d, p, group, 8400 + n + m + batch, (batch,))
    X = L.X[batch]
    _assert_tol(_run(L, X), _ref(L, X), f"grouped stacked {n}x{m} d{d} p{p} g{group} b{batch}")
    Li = inputs.bqq_grouped_layer("gsi", n, m, d, p, group, 8500 + n + m + batch, (batch,), integer=True)
    Xi = Li.X[batch]
    _assert_bits(_run(Li, Xi), _integer_preconditions(Li, Xi, True), f"grouped stacked integer b{batch}")


def _integer_preconditions(L, X, fp16_intermediate):
    """Integer data: the first stage's signed sums t_i = (1 - 2 Z_i)(b_i ⊙ x)
    (b_i[l] = r_i[l // group]) are integers, exact in fp16 where the path
    rounds them; every later sum is a multiple of 1/2 far inside fp32's
    exact range; the output fits fp16."""
    X64 = X.astype(np.float64)
    ng = L.ngroups
    b = np.stack([np.repeat(L.r[i].astype(np.float64), L.group)[:L.m] for i in range(L.p)])
    t = np.concatenate([(X64 * b[i]) @ (1 - 2 * L.Z[i].astype(np.float64)).T for i in range(L.p)], axis=1)
    assert np.abs(t).sum(axis=1).max() * 2 < 2 ** 24
    if fp16_intermediate:
        assert np.abs(t).max() <= 2048
    assert ng > 1
    y = _ref(L, X)
    assert np.abs(y).max() <= 65504
    return y


@pytest.mark.parametrize("n,m,d,p,group,batch", [(65, 97, 64, 2, 32, 1), (65, 97, 64, 2, 32, 5),
                                                 (130, 200, 128, 3, 48, 16), (130, 200, 128, 3, 48, 100),
                                                 (300, 600, 64, 2, 64, 17)])
@pytest.mark.parametrize("path", [dbf.DBF_PATH_AUTO, dbf.DBF_PATH_PREFILL])
def test_grouped_integer_bit_exact(gpu, n, m, d, p, group, batch, path):
    _say(f"bqq grouped integer n={n} m={m} d={d} p={p} group={group} batch={batch} path={path}")
    L = inputs.bqq_grouped_layer("gi", n, m, d, p, group, 8200 + n + batch, (batch,), integer=True)
    X = L.X[batch]
    fp16_t = path == dbf.DBF_PATH_PREFILL or batch > 1
    ref = _integer_preconditions(L, X, fp16_t)
    _assert_bits(_run(L, X, path), ref, f"grouped integer {n}x{m} d{d} p{p} g{group} b{batch}")


# The 4096 x 4096 projection as two binary products with d = 1024 and
# scalars per group of 128 input columns (32 groups).
FULL = (4096, 4096, 1024, 2, 128)


def _rows(batch):
    if batch <= 16:
        return np.arange(batch)
    tiles = np.concatenate([np.arange(0, batch, 128), np.arange(127, batch, 128)])
    return np.unique(np.concatenate([tiles, np.random.default_rng(3).choice(batch, 16, replace=False)]))


@pytest.mark.parametrize("batch", [1, 16, 2048])
def test_grouped_full_size(gpu, batch):
    n, m, d, p, g = FULL
    _say(f"bqq grouped full size {n}x{m} d={d} p={p} group={g} batch={batch}")
    L = inputs.bqq_grouped_layer("gf", n, m, d, p, g, 8300, (batch,))
    X = L.X[batch]
    rows = _rows(batch)
    W = Q.bqq_weight_grouped(L.Y, L.Z, L.r, L.s, L.t, L.u, g)
    ref = X[rows].astype(np.float64) @ W.T
    err = _assert_tol(_run(L, X)[rows], ref, f"grouped full b{batch}")
    _say(f"  worst row rel err {err:.3e}")


def test_one_group_is_the_single_group_layer(gpu):
    """group >= m: the grouped entry point packs the single-group form; the
    outputs carry the single-group layer's bits."""
    import torch
    L = inputs.bqq_layer("o", 200, 300, 70, 2, 8400, (1, 9, 40))
    r, s, t = (np.asarray(v)[:, None] for v in (L.r, L.s, L.t))
    Hg = dbf.Layer.bqq_grouped(L.Y, L.Z, r, s, t, [L.u], 300, max_batch=40)
    Hs = dbf.Layer.bqq(L.Y, L.Z, L.r, L.s, L.t, L.u, max_batch=40)
    try:
        for bt in (1, 9, 40):
            _say(f"bqq one group batch={bt}")
            x = torch.from_numpy(L.X[bt]).cuda()
            yg = Hg.forward(x).cpu().numpy()
            ys = Hs.forward(x).cpu().numpy()
            assert np.array_equal(yg.view(np.uint16), ys.view(np.uint16))
    finally:
        Hg.close()
        Hs.close()


def test_grouped_determinism_and_errors(gpu):
    import torch
    L = inputs.bqq_grouped_layer("gd", 500, 700, 192, 2, 64, 8500, (1, 16, 40))
    H = _layer(L, 40)
    try:
        for bt in (1, 16, 40):
            _say(f"bqq grouped determinism batch={bt}")
            x = torch.from_numpy(L.X[bt]).cuda()
            y1 = H.forward(x).cpu().numpy()
            y2 = H.forward(x).cpu().numpy()
            assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
        _say("bqq grouped unsupported entries")
        x = torch.from_numpy(L.X[16]).cuda()
        with pytest.raises(dbf.DbfError) as e:
            H.forward(x, path=dbf.DBF_PATH_DECODE)
        assert e.value.status == dbf.DBF_ERR_UNSUPPORTED
        with pytest.raises(dbf.DbfError) as e:
            dbf.forward_group([H], x)
        assert e.value.status == dbf.DBF_ERR_UNSUPPORTED
        y = torch.empty((16, L.n), dtype=torch.float16, device="cuda")
        st = dbf.lib().dbf_linear_forward_noalloc(H.handle, x.data_ptr(), y.data_ptr(), 16, None)
        assert st == dbf.DBF_ERR_UNSUPPORTED
        info = H.info()
        assert info["k"] == 384 and info["n"] == 500 and info["m"] == 700
    finally:
        H.close()
