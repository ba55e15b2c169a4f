"""CPU oracle for the DBF factorization of a weight matrix (the step before
the forward: W -> a, A, mid, B, b).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module.  The product path never imports, links or calls anything here,
and this file shares no code, tables or helpers with it.

What is computed
----------------
Source: technical summary (gist.science) of "Addition is almost all you
need", §2.2 (optimization algorithm), and the TL;DR of the same paper on its
sciencestack.ai page (an ADMM-based optimization with importance weighting).
§2.2 names four ingredients and no further detail:
  1. alternating minimization: fix one factor, optimize the other, in turn;
  2. ADMM for the constrained subproblem;
  3. projection onto the constraint set (a sign matrix with a rank-one
     scaling) by SVID, the sign-value-independent decomposition of OneBit;
  4. importance-based scaling of the rows and columns of the error.
This oracle writes them out in that order, in the plainest form they allow
(each reading below is also listed with the library's other readings):

* Problem.  W (n x m) ~ U V with U = diag(a) A diag(c_u) (n x k) and
  V = diag(c_v) B diag(b) (k x m), A and B of +/-1: the DBF weight with
  mid = c_u ⊙ c_v.  Importance: with row weights d_o (n) and column weights
  d_i (m), the error is measured as || diag(d_o) (W - U V) diag(d_i) ||_F;
  this is the plain error of the scaled matrix T = diag(d_o) W diag(d_i),
  whose factors are unscaled at the end (a / d_o, b / d_i).
* Alternating minimization.  Each outer iteration updates U with V fixed,
  then V with U fixed; the V step is the U step applied to the transposed
  problem T^T ~ V^T U^T.
* ADMM for  min_X ||T - X Y||_F^2  s.t.  X in S  (S = sign matrices with a
  rank-one scaling), split as X = Z with Z in S, scaled dual L, penalty rho:
      X <- argmin ||T - X Y||^2 + rho ||X - Z + L||^2
         = (T Y^T + rho (Z - L)) (Y Y^T + rho I)^{-1}
      Z <- SVID(X + L)
      L <- L + X - Z
  starting from Z = the current (feasible) factor, L = 0; after the inner
  iterations the factor becomes Z.  rho = rho_rel * trace(Y Y^T) / k.
* SVID(M) = sign(M) ⊙ (sigma u v^T), where sigma u v^T is the leading
  rank-one term of |M|, found by `power_iters` steps of the power method
  from u = 1/sqrt(rows) (v <- |M|^T u / ||.||, u <- |M| v, sigma = ||u||,
  u <- u / sigma).  sign(0) = +1.  Pinned against numpy's SVD.
* Start: the factors U0, V0 are inputs (random numbers the method draws
  are passed in).
* Output scales in fp16: a and b are divided by their RMS and mid takes the
  two RMS factors, then all three are rounded to fp16 once.

The objective is reported after each outer iteration as
||T - U V||_F / ||T||_F.  No step of this heuristic guarantees a decrease
(ADMM with a non-convex projection); tests check the decrease over the run
and exact recovery of a matrix that already is a DBF product.
"""

from __future__ import annotations

import numpy as np

__all__ = ["sign_pm1", "svid", "ridge_update", "admm_factor_step", "factorize", "dbf_from_factors"]


def sign_pm1(M) -> np.ndarray:
    """+1 where M >= 0, -1 where M < 0 (sign(0) = +1)."""
    M = np.asarray(M)
    return np.where(M < 0, -1.0, 1.0)


def svid(M, power_iters: int):
    """SVID of M: (S, r, c) with S = sign(M) and r c^T the power-method
    rank-one approximation of |M| (r = sigma u, c = v, both >= 0)."""
    M = np.asarray(M, dtype=np.float64)
    S = sign_pm1(M)
    Mabs = np.abs(M)
    rows, cols = Mabs.shape
    u = np.full(rows, 1.0 / np.sqrt(rows))
    v = np.zeros(cols)
    sigma = 0.0
    for _ in range(power_iters):
        v = Mabs.T @ u
        nv = np.linalg.norm(v)
        if nv == 0.0:
            return S, np.zeros(rows), np.zeros(cols)
        v = v / nv
        u = Mabs @ v
        sigma = np.linalg.norm(u)
        u = u / sigma
    return S, sigma * u, v


def ridge_update(T, Y, Z, L, rho: float) -> np.ndarray:
    """The ADMM X step: argmin_X ||T - X Y||_F^2 + rho ||X - Z + L||_F^2,
    i.e. X (Y Y^T + rho I) = T Y^T + rho (Z - L), solved with a library
    solver (the matrix is symmetric, so X^T = H^{-1} (T Y^T + rho (Z - L))^T)."""
    Y = np.asarray(Y, dtype=np.float64)
    H = Y @ Y.T + rho * np.eye(Y.shape[0])
    return np.linalg.solve(H, (np.asarray(T, dtype=np.float64) @ Y.T + rho * (Z - L)).T).T


def admm_factor_step(T, Y, X0, rho_rel: float, inner: int, power_iters: int, history=None):
    """ADMM for min_X ||T - X Y||_F^2 with X a sign matrix with rank-one
    scaling, from the feasible X0.  Returns (Z, S, r, c) with Z = S ⊙ r c^T.
    With a list `history`, appends (rho, X, Z, L) after every inner iteration."""
    T = np.asarray(T, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    k = Y.shape[0]
    rho = rho_rel * np.trace(Y @ Y.T) / k
    Z = np.asarray(X0, dtype=np.float64).copy()
    L = np.zeros_like(Z)
    S, r, c = sign_pm1(Z), None, None
    for _ in range(inner):
        X = ridge_update(T, Y, Z, L, rho)
        S, r, c = svid(X + L, power_iters)
        Z = S * np.outer(r, c)
        L = L + X - Z
        if history is not None:
            history.append((rho, X, Z, L))
    return Z, S, r, c


def factorize(W, k: int, U0, V0, rho_rel: float = 1.0, outer: int = 2, inner: int = 4, power_iters: int = 8,
              d_out=None, d_in=None):
    """The DBF factorization of W (n x m) with middle dimension k.

    Returns (A, B, a, mid, b, err): A (n x k) and B (k x m) as int8 +/-1,
    a, mid, b as fp16, and err[t] = ||T - U V||_F / ||T||_F after outer
    iteration t (T the importance-scaled W)."""
    W = np.asarray(W, dtype=np.float64)
    n, m = W.shape
    d_o = np.ones(n) if d_out is None else np.asarray(d_out, dtype=np.float64)
    d_i = np.ones(m) if d_in is None else np.asarray(d_in, dtype=np.float64)
    T = d_o[:, None] * W * d_i[None, :]
    tnorm = np.linalg.norm(T)
    U = np.asarray(U0, dtype=np.float64)
    V = np.asarray(V0, dtype=np.float64)
    assert U.shape == (n, k) and V.shape == (k, m)
    err = []
    SA = a_u = c_u = SBt = b_v = c_v = None
    for _ in range(outer):
        U, SA, a_u, c_u = admm_factor_step(T, V, U, rho_rel, inner, power_iters)
        Vt, SBt, b_v, c_v = admm_factor_step(T.T, U.T, V.T, rho_rel, inner, power_iters)
        V = Vt.T
        err.append(float(np.linalg.norm(T - U @ V) / tnorm))
    a = a_u / d_o
    b = b_v / d_i
    mid = c_u * c_v
    ra = np.sqrt(np.mean(a * a))
    rb = np.sqrt(np.mean(b * b))
    if ra > 0 and rb > 0:
        a, b, mid = a / ra, b / rb, mid * ra * rb
    A = SA.astype(np.int8)
    B = SBt.T.astype(np.int8)
    return (A, B, a.astype(np.float16), mid.astype(np.float16), b.astype(np.float16), np.asarray(err))


def dbf_from_factors(A, B, a, mid, b) -> np.ndarray:
    """The DBF weight diag(a) A diag(mid) B diag(b) in fp64."""
    a64, mid64, b64 = (np.asarray(v).astype(np.float64) for v in (a, mid, b))
    return (a64[:, None] * np.asarray(A, dtype=np.float64) * mid64[None, :]) @ (
        np.asarray(B, dtype=np.float64) * b64[None, :])
