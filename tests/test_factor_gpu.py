"""GPU factorization (dbf_factorize) against its fp64 CPU oracle.

Method: gist.science technical summary of "Addition is almost all you
need", §2.2 -- alternating minimization of the two factors, ADMM for each
constrained subproblem, SVID projection, importance scaling.  The GPU runs
in fp32 (rocBLAS GEMMs, Newton-Schulz inverse) and the oracle in fp64 with
an exact solver, so the iterations agree closely but not bit for bit; what
is compared is what the method fixes:
* a matrix that already is a DBF product is a fixed point: the signs are
  recovered exactly, with and without importance weights, at small and full
  size;
* from the same start on a noisy DBF matrix, the per-iteration errors agree
  with the oracle's and the signs agree almost everywhere (256 x 192 up to
  2048 x 2048 with k = 1024, with and without importance weights);
* repeated calls give identical bits;
* the factors pack into a layer whose forward matches the oracle's DBF
  forward of the same factors.
Every case prints its name before it touches the GPU.
"""

import sys

import numpy as np
import pytest

import dbf_linear_fwd_amd as dbf
from oracle import dbf_oracle as O
from oracle import factor_oracle as F

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _dbf_case(seed, n, m, k, noise=0.0, start_noise=0.0):
    rng = np.random.default_rng(seed)
    SA = np.where(rng.random((n, k)) < 0.5, -1.0, 1.0)
    SB = np.where(rng.random((k, m)) < 0.5, -1.0, 1.0)
    U = rng.uniform(0.5, 1.5, n)[:, None] * SA * rng.uniform(0.5, 1.5, k)[None, :]
    V = rng.uniform(0.5, 1.5, k)[:, None] * SB * rng.uniform(0.5, 1.5, m)[None, :]
    W = U @ V
    if noise:
        W = W + noise * np.linalg.norm(W) / np.sqrt(W.size) * rng.standard_normal(W.shape)
    U0 = U + start_noise * rng.standard_normal(U.shape)
    V0 = V + start_noise * rng.standard_normal(V.shape)
    return SA, SB, W, U0, V0


def _gpu(W, k, U0, V0, d_out=None, d_in=None, **kw):
    import torch
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()  # noqa
    out = dbf.factorize(t(W), k, t(U0), t(V0), d_out=t(d_out), d_in=t(d_in), **kw)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in out]


@pytest.mark.parametrize("importance", [False, True])
def test_dbf_matrix_is_a_fixed_point(gpu, importance):
    n, m, k = 300, 260, 64
    _say(f"factorize fixed point {n}x{m} k={k} importance={importance}")
    SA, SB, W, U0, V0 = _dbf_case(10, n, m, k)
    d_o = d_i = None
    if importance:
        rng = np.random.default_rng(11)
        d_o = rng.uniform(0.5, 2.0, n)
        d_i = rng.uniform(0.5, 2.0, m)
        W = W / d_o[:, None] / d_i[None, :]
    A, B, a, mid, b, err = _gpu(W, k, U0, V0, d_o, d_i, outer=2, inner=3, power_iters=6)
    assert np.array_equal(A, SA.astype(np.int8)) and np.array_equal(B, SB.astype(np.int8))
    assert err.max() < 1e-4, err
    What = F.dbf_from_factors(A, B, a, mid, b)
    assert np.linalg.norm(What - W) <= 2e-3 * np.linalg.norm(W)


def test_matches_the_oracle_on_a_noisy_dbf_matrix(gpu):
    n, m, k = 256, 192, 48
    _say(f"factorize vs oracle {n}x{m} k={k}")
    SA, SB, W, U0, V0 = _dbf_case(12, n, m, k, noise=0.02, start_noise=0.3)
    kw = dict(rho_rel=1.0, outer=3, inner=4, power_iters=8)
    A, B, a, mid, b, err = _gpu(W, k, U0, V0, **kw)
    Ao, Bo, ao, mido, bo, erro = F.factorize(W, k, U0, V0, **kw)
    _say(f"  gpu err {err.tolist()} oracle err {erro.tolist()}")
    assert np.allclose(err, erro, rtol=2e-3, atol=1e-5)
    assert (A == Ao).mean() > 0.995 and (B == Bo).mean() > 0.995
    Wg = F.dbf_from_factors(A, B, a, mid, b)
    Wo = F.dbf_from_factors(Ao, Bo, ao, mido, bo)
    assert np.linalg.norm(Wg - Wo) <= 5e-3 * np.linalg.norm(Wo)
    assert err[-1] < 0.05


# Larger iterate comparisons: ragged sizes with importance weights, and a
# 2048 x 2048 matrix at k = 1024 (a quarter of the full-size layer per side).
LARGE_CASES = [
    # n, m, k, importance, outer, inner
    (1024, 768, 384, True, 3, 4),
    (2048, 2048, 1024, False, 2, 3),
]


@pytest.mark.parametrize("n,m,k,importance,outer,inner", LARGE_CASES)
def test_matches_the_oracle_at_larger_sizes(gpu, n, m, k, importance, outer, inner):
    _say(f"factorize vs oracle {n}x{m} k={k} importance={importance}")
    SA, SB, W, U0, V0 = _dbf_case(17 + n, n, m, k, noise=0.02, start_noise=0.3)
    d_o = d_i = None
    if importance:
        rng = np.random.default_rng(18)
        d_o = rng.uniform(0.5, 2.0, n)
        d_i = rng.uniform(0.5, 2.0, m)
    kw = dict(rho_rel=1.0, outer=outer, inner=inner, power_iters=8)
    A, B, a, mid, b, err = _gpu(W, k, U0, V0, d_o, d_i, **kw)
    Ao, Bo, ao, mido, bo, erro = F.factorize(W, k, U0, V0, d_out=d_o, d_in=d_i, **kw)
    _say(f"  gpu err {err.tolist()} oracle err {erro.tolist()}")
    assert np.allclose(err, erro, rtol=2e-3, atol=1e-5)
    assert (A == Ao).mean() > 0.995 and (B == Bo).mean() > 0.995
    Wg = F.dbf_from_factors(A, B, a, mid, b)
    Wo = F.dbf_from_factors(Ao, Bo, ao, mido, bo)
    assert np.linalg.norm(Wg - Wo) <= 5e-3 * np.linalg.norm(Wo)


def test_repeated_calls_are_identical(gpu):
    _say("factorize determinism")
    SA, SB, W, U0, V0 = _dbf_case(13, 200, 150, 40, noise=0.05, start_noise=0.5)
    r1 = _gpu(W, 40, U0, V0, outer=2, inner=2, power_iters=5)
    r2 = _gpu(W, 40, U0, V0, outer=2, inner=2, power_iters=5)
    for x, y in zip(r1, r2):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_factors_pack_into_a_layer(gpu):
    import torch
    n, m, k = 384, 320, 96
    _say(f"factorize then pack and forward {n}x{m} k={k}")
    SA, SB, W, U0, V0 = _dbf_case(14, n, m, k, noise=0.05, start_noise=0.3)
    A, B, a, mid, b, err = _gpu(W, k, U0, V0, outer=2, inner=3, power_iters=6)
    H = dbf.Layer(A, B, a, mid, b, max_batch=8)
    try:
        X = np.random.default_rng(15).standard_normal((8, m)).astype(np.float16)
        y = H.forward(torch.from_numpy(X).cuda()).cpu().numpy().astype(np.float64)
    finally:
        H.close()
    ref = O.dense_forward(X, A, B, a, mid, b)
    r = np.abs(y - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert r.max() <= 2e-3
    # and the layer approximates the original matrix about as well as the factors do
    full = X.astype(np.float64) @ W.T
    assert np.linalg.norm(y - full) <= 3 * err[-1] * np.linalg.norm(full) + 1e-3 * np.linalg.norm(full)


def test_full_size_fixed_point(gpu):
    n, m, k = 4096, 4096, 2048
    _say(f"factorize fixed point full size {n}x{m} k={k}")
    SA, SB, W, U0, V0 = _dbf_case(16, n, m, k)
    A, B, a, mid, b, err = _gpu(W, k, U0, V0, outer=1, inner=2, power_iters=4)
    assert np.array_equal(A, SA.astype(np.int8)) and np.array_equal(B, SB.astype(np.int8))
    assert err.max() < 1e-4, err
