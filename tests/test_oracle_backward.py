"""Pins of the oracle's gradients (CPU).

The oracle's `backward` writes the derivatives of Y = X Wᵀ, W = diag(a) A
diag(mid) B diag(b), with respect to X, a, mid and b as matrix products.
They are pinned here to things other than themselves:

* exact rational brute force straight from the sum that defines Y;
* finite differences of the oracle's forward: the loss Σ dY ⊙ Y is linear
  in each of X, a, mid and b separately, so a step of 1 in one entry changes
  it by exactly that entry's gradient (up to fp64 rounding);
* the transpose identity: dX = dY W is the forward of the layer with factors
  (Bᵀ, Aᵀ, b, mid, a), computed through a different dense product;
* the k = 1 closed form of dmid;
* planted mistakes, each of which one of these checks must catch.
"""

import numpy as np
import pytest

from oracle import dbf_oracle as O
from tests import inputs


def _case(seed, n, m, k, bt):
    X, A, B, a, mid, b = inputs.tiny_case(seed, n, m, k, bt, signed_scales=True)
    dY = np.random.default_rng(seed + 1).uniform(-2, 2, (bt, n)).astype(np.float16)
    return X, dY, A, B, a, mid, b


def _loss(X, dY, A, B, a, mid, b):
    return float((O.widen(dY) * O.dense_forward(X, A, B, a, mid, b)).sum())


def _rel(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    return float(np.abs(x - y).max() / max(np.abs(y).max(), 1e-300))


def check_brute(fn, seed=11, shape=(3, 5, 4, 2)):
    n, m, k, bt = shape
    X, dY, A, B, a, mid, b = _case(seed, n, m, k, bt)
    got = fn(X, dY, A, B, a, mid, b)
    want = O.brute_force_backward(X, dY, A, B, a, mid, b)
    return all(_rel(g, np.array(w, dtype=np.float64)) <= 1e-13 for g, w in zip(got, want))


def check_fd(fn, seed=21, shape=(12, 15, 9, 3)):
    n, m, k, bt = shape
    X, dY, A, B, a, mid, b = _case(seed, n, m, k, bt)
    dX, da, dmid, db = fn(X, dY, A, B, a, mid, b)
    L0 = _loss(X, dY, A, B, a, mid, b)
    scale = max(abs(L0), 1.0)
    ok = True
    X64, a64, mid64, b64 = (O.widen(v) for v in (X, a, mid, b))
    for i in range(n):
        a2 = a64.copy(); a2[i] += 1.0
        ok &= abs(_loss(X, dY, A, B, a2, mid, b) - L0 - da[i]) <= 1e-10 * scale
    for j in range(k):
        m2 = mid64.copy(); m2[j] += 1.0
        ok &= abs(_loss(X, dY, A, B, a, m2, b) - L0 - dmid[j]) <= 1e-10 * scale
    for l in range(m):
        b2 = b64.copy(); b2[l] += 1.0
        ok &= abs(_loss(X, dY, A, B, a, mid, b2) - L0 - db[l]) <= 1e-10 * scale
    for r in range(bt):
        for l in range(0, m, 4):
            X2 = X64.copy(); X2[r, l] += 1.0
            ok &= abs(_loss(X2, dY, A, B, a, mid, b) - L0 - dX[r, l]) <= 1e-10 * scale
    return bool(ok)


def check_transpose(fn, seed=31, shape=(40, 50, 30, 4)):
    n, m, k, bt = shape
    X, dY, A, B, a, mid, b = _case(seed, n, m, k, bt)
    dX = fn(X, dY, A, B, a, mid, b)[0]
    want = O.dense_forward(dY, np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), b, mid, a)
    return _rel(dX, want) <= 1e-12


def check_k1(fn, seed=41, shape=(7, 9, 1, 3)):
    n, m, k, bt = shape
    X, dY, A, B, a, mid, b = _case(seed, n, m, k, bt)
    dmid = fn(X, dY, A, B, a, mid, b)[2]
    X64, dY64 = O.widen(X), O.widen(dY)
    t = X64 @ (B[0].astype(np.float64) * O.widen(b))           # (bt,)
    g = dY64 @ (O.widen(a) * A[:, 0].astype(np.float64))       # (bt,)
    return _rel(dmid, np.array([(g * t).sum()])) <= 1e-13


CHECKS = [check_brute, check_fd, check_transpose, check_k1]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_backward_pins(check):
    assert check(O.backward)


@pytest.mark.parametrize("seed,shape", [(1, (1, 1, 1, 1)), (2, (2, 3, 4, 2)), (3, (4, 2, 3, 3)), (4, (5, 6, 2, 1))])
def test_backward_brute_force_shapes(seed, shape):
    assert check_brute(O.backward, seed, shape)


def _mut_da_from_y(X, dY, A, B, a, mid, b):
    dX, da, dmid, db = O.backward(X, dY, A, B, a, mid, b)
    y = O.dense_forward(X, A, B, a, mid, b)
    return dX, (O.widen(dY) * y).sum(axis=0), dmid, db


def _mut_dmid_no_a(X, dY, A, B, a, mid, b):
    dX, da, dmid, db = O.backward(X, dY, A, B, a, mid, b)
    t = (O.widen(X) * O.widen(b)[None, :]) @ B.T.astype(np.float64)
    g = O.widen(dY) @ A.astype(np.float64)
    return dX, da, (g * t).sum(axis=0), db


def _mut_db_extra_b(X, dY, A, B, a, mid, b):
    dX, da, dmid, db = O.backward(X, dY, A, B, a, mid, b)
    return dX, da, dmid, db * O.widen(b)


def _mut_dx_transposed_factor(X, dY, A, B, a, mid, b):
    dX, da, dmid, db = O.backward(X, dY, A, B, a, mid, b)
    W = O.dense_weight(A, B, a, np.ones_like(O.widen(mid)), b)   # mid dropped
    return O.widen(dY) @ W, da, dmid, db


def _mut_dmid_sign(X, dY, A, B, a, mid, b):
    dX, da, dmid, db = O.backward(X, dY, A, B, a, mid, b)
    return dX, da, -dmid, db


MUTANTS = [_mut_da_from_y, _mut_dmid_no_a, _mut_db_extra_b, _mut_dx_transposed_factor, _mut_dmid_sign]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_backward_planted_mistakes_are_caught(mutant):
    assert not all(check(mutant) for check in CHECKS)
