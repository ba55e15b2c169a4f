"""Pins of the factorization oracle (oracle/factor_oracle.py): the SVID
projection against numpy's SVD and on exact rank-one inputs, the ADMM step
against its optimality condition, exact recovery of a matrix that already
is a DBF product (a fixed point of every step, with and without importance
weights), invariance under a uniform importance weight, the decrease of the
error on a noisy DBF matrix, and planted mistakes that must fail a pin.

Algorithm: gist.science technical summary of "Addition is almost all you
need", §2.2 (alternating minimization, ADMM, SVID projection, importance
scaling).
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import factor_oracle as F


def _dbf_factors(rng, n, m, k):
    SA = np.where(rng.random((n, k)) < 0.5, -1.0, 1.0)
    SB = np.where(rng.random((k, m)) < 0.5, -1.0, 1.0)
    a = rng.uniform(0.5, 1.5, n)
    cu = rng.uniform(0.5, 1.5, k)
    cv = rng.uniform(0.5, 1.5, k)
    b = rng.uniform(0.5, 1.5, m)
    U = a[:, None] * SA * cu[None, :]
    V = cv[:, None] * SB * b[None, :]
    return SA, SB, U, V


def test_svid_matches_svd_top_triplet():
    rng = np.random.default_rng(0)
    M = rng.standard_normal((40, 25))
    S, r, c = F.svid(M, 200)
    assert np.array_equal(S, np.where(M < 0, -1.0, 1.0))
    u, sv, vt = np.linalg.svd(np.abs(M))
    want = sv[0] * np.outer(np.abs(u[:, 0]), np.abs(vt[0]))
    assert np.allclose(np.outer(r, c), want, rtol=1e-9, atol=1e-12)
    assert np.all(r >= 0) and np.all(c >= 0)


def test_svid_reproduces_a_scaled_sign_matrix():
    rng = np.random.default_rng(1)
    S0 = np.where(rng.random((12, 7)) < 0.5, -1.0, 1.0)
    S0[3, 4] = 1.0
    r0 = rng.uniform(0.1, 2.0, 12)
    c0 = rng.uniform(0.1, 2.0, 7)
    M = S0 * np.outer(r0, c0)
    S, r, c = F.svid(M, 1)   # |M| has rank one: one power step is exact
    assert np.array_equal(S, S0)
    assert np.allclose(S * np.outer(r, c), M, rtol=1e-13, atol=1e-13)
    # sign(0) = +1
    assert np.array_equal(F.sign_pm1(np.array([0.0, -0.0, -1e-300, 2.0])), np.array([1.0, 1.0, -1.0, 1.0]))


def test_ridge_update_satisfies_its_optimality_condition():
    rng = np.random.default_rng(2)
    T = rng.standard_normal((9, 11))
    Y = rng.standard_normal((4, 11))
    Z = rng.standard_normal((9, 4))
    L = rng.standard_normal((9, 4))
    X = F.ridge_update(T, Y, Z, L, 0.7)
    grad = (X @ Y - T) @ Y.T + 0.7 * (X - Z + L)
    assert np.abs(grad).max() < 1e-10


def _dual_identity_fails():
    """Every ADMM iterate satisfies (X Y - T) Y^T + rho (L_new + Z_new - Z_old) = 0:
    the X step's optimality condition rewritten with the dual update
    L_new = L_old + X - Z_new (checked with the gradient formed here); and
    Z_new + L_new (= X + L_old, the projected matrix) has the signs of Z_new."""
    rng = np.random.default_rng(6)
    T = rng.standard_normal((14, 12))
    Y = rng.standard_normal((5, 12))
    X0 = np.where(rng.random((14, 5)) < 0.5, -1.0, 1.0) * 0.3
    hist = []
    F.admm_factor_step(T, Y, X0, 0.5, 6, 5, history=hist)
    Z_old = X0
    for rho, X, Z, L in hist:
        res = (X @ Y - T) @ Y.T + rho * (L + Z - Z_old)
        if np.abs(res).max() > 1e-9 * max(1.0, np.abs(T).max()):
            return True
        # Z + L_new = X + L_old is the matrix that was projected, and the
        # projection keeps its signs: sign(Z + L) = sign(Z) wherever Z != 0
        nz = Z != 0
        if not np.array_equal(np.sign(Z + L)[nz], np.sign(Z)[nz]):
            return True
        Z_old = Z
    return False


def test_admm_iterates_satisfy_the_dual_identity():
    assert not _dual_identity_fails()


def _recovery_failures(rho_rel=1.0, importance=False):
    rng = np.random.default_rng(3)
    n, m, k = 24, 20, 8
    SA, SB, U, V = _dbf_factors(rng, n, m, k)
    W = U @ V
    d_o = d_i = None
    U0, V0 = U, V
    if importance:
        d_o = rng.uniform(0.5, 2.0, n)
        d_i = rng.uniform(0.5, 2.0, m)
        W = W / d_o[:, None] / d_i[None, :]          # the scaled matrix d_o W d_i is U V
    A, B, a, mid, b, err = F.factorize(W, k, U0, V0, rho_rel, outer=2, inner=3, power_iters=4, d_out=d_o,
                                       d_in=d_i)
    bad = []
    if not (np.array_equal(A, SA.astype(np.int8)) and np.array_equal(B, SB.astype(np.int8))):
        bad.append("signs")
    if np.abs(err).max() > 1e-12:
        bad.append("error")
    What = F.dbf_from_factors(A, B, a, mid, b)
    if np.linalg.norm(What - W) > 2e-3 * np.linalg.norm(W):   # fp16 scales
        bad.append("weight")
    return bad


def test_a_dbf_matrix_is_a_fixed_point():
    assert _recovery_failures() == []
    assert _recovery_failures(rho_rel=0.1) == []


def test_a_dbf_matrix_is_a_fixed_point_under_importance_weights():
    assert _recovery_failures(importance=True) == []


def test_uniform_importance_changes_nothing():
    rng = np.random.default_rng(4)
    n, m, k = 30, 26, 10
    W = rng.standard_normal((n, m))
    U0 = rng.standard_normal((n, k))
    V0 = rng.standard_normal((k, m))
    r1 = F.factorize(W, k, U0, V0, outer=2, inner=2, power_iters=6)
    r2 = F.factorize(W, k, 4.0 * U0, V0, outer=2, inner=2, power_iters=6, d_out=np.full(n, 4.0))
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])
    assert np.allclose(r1[5], r2[5], rtol=1e-9)


def test_error_drops_on_a_noisy_dbf_matrix():
    rng = np.random.default_rng(5)
    n, m, k = 64, 48, 16
    SA, SB, U, V = _dbf_factors(rng, n, m, k)
    W = U @ V
    W = W + 0.01 * np.linalg.norm(W) / np.sqrt(W.size) * rng.standard_normal(W.shape)
    U0 = U + 0.3 * rng.standard_normal(U.shape)
    V0 = V + 0.3 * rng.standard_normal(V.shape)
    start = np.linalg.norm(W - U0 @ V0) / np.linalg.norm(W)
    A, B, a, mid, b, err = F.factorize(W, k, U0, V0, outer=3, inner=4, power_iters=8)
    assert err[-1] < 0.05 < start
    assert err[-1] <= err[0] + 1e-12


def test_planted_mistakes_fail_a_pin(monkeypatch):
    real_ridge = F.ridge_update
    real_svid = F.svid
    mutants = {
        "dual sign": lambda: monkeypatch.setattr(
            F, "admm_factor_step", _step_with(lambda L, X, Z: L - X + Z)),
        "no penalty in X step": lambda: monkeypatch.setattr(
            F, "ridge_update", lambda T, Y, Z, L, rho: real_ridge(T, Y, Z, L, 0.0 * rho + 1e-300)),
        "projection of X alone": lambda: monkeypatch.setattr(
            F, "admm_factor_step", _step_with(None, project_x_only=True)),
        "sign flipped in SVID": lambda: monkeypatch.setattr(
            F, "svid", lambda M, it: (lambda S, r, c: (-S, r, c))(*real_svid(M, it))),
    }
    for name, plant in mutants.items():
        with monkeypatch.context() as mp:   # noqa: F841  (undo after each mutant)
            plant()
            failed = _recovery_failures() != [] or _recovery_failures(importance=True) != [] or \
                _noisy_fails() or _dual_identity_fails()
            monkeypatch.undo()
            assert failed, f"planted mistake '{name}' passed every pin"


def _noisy_fails():
    try:
        test_error_drops_on_a_noisy_dbf_matrix()
        return False
    except AssertionError:
        return True


def _step_with(dual, project_x_only=False):
    def step(T, Y, X0, rho_rel, inner, power_iters, history=None):
        T = np.asarray(T, dtype=np.float64)
        Y = np.asarray(Y, dtype=np.float64)
        k = Y.shape[0]
        rho = rho_rel * np.trace(Y @ Y.T) / k
        Z = np.asarray(X0, dtype=np.float64).copy()
        L = np.zeros_like(Z)
        S = r = c = None
        for _ in range(inner):
            X = F.ridge_update(T, Y, Z, L, rho)
            S, r, c = F.svid(X if project_x_only else X + L, power_iters)
            Z = S * np.outer(r, c)
            L = dual(L, X, Z) if dual else L + X - Z
            if history is not None:
                history.append((rho, X, Z, L))
        return Z, S, r, c
    return step
