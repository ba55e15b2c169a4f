"""CPU oracle for the Double Binary Factorization (DBF) linear-layer forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  The product path (the HIP library and its Python binding)
never imports, links or calls anything here, and this file shares no code,
tables or helpers with it.

What is computed
----------------
Source: "Addition is almost all you need: Compressing large language models
with double binary factorization", technical summary (gist.science), §2.1
(mathematical formulation), and Figure 1's caption on the sciencestack.ai
page of the same paper.

* A weight matrix W of shape n x m (n = output features, m = input features)
  is approximated by the product of two factors: the left factor is the
  n x k sign matrix A (entries +1/-1) with its rows scaled by the fp16 vector
  a (length n) and its columns scaled by the fp16 vector ``mid`` (length k);
  the right factor is the k x m sign matrix B with its columns scaled by the
  fp16 vector b (length m).  In matrix form:
  W = diag(a) A diag(mid) B diag(b).
  (The pages call the middle vector ``m``; it is named ``mid`` here because
  ``m`` is also the input width.)
* For a layer input X (batch x m, fp16) the layer output is X W^T
  (batch x n).  §2.1 evaluates it right to left without forming W: scale the
  columns of X by b, multiply by B^T, scale by mid, multiply by A^T, scale
  by a.  Every product with a sign matrix is a signed sum.

Gradients (``backward``, ``brute_force_backward``): the derivatives of the
same function with respect to X, a, mid and b, for fine-tuning the factors
(gist.science technical summary, §4 and §5), written as the plain
definition; pinned in tests/test_oracle_backward.py.

Readings where the pages are silent:
* The output is fp16, obtained by one round-to-nearest-even from the exact
  (here: fp64) value.  The pages state fp16 only for X and the scales.
* There is no flush-to-zero; subnormal fp16 values are ordinary values.

Precision of this oracle
------------------------
Inputs are fp16 and the signs are +/-1, so widening to fp64 is exact.  Each
fp64 product a_i*mid_j*b_l*x_l carries at most 44 significant bits, so the
fp64 results below differ from the exact rational value only by sum
rounding, a relative error of order (k + m) * 2**-53, some eleven orders of
magnitude below the fp16 output rounding.  When every input is a small
integer (or a power of two times one) and every partial sum stays below
2**53, the fp64 results are exact.  ``brute_force`` evaluates the definition
in exact rational arithmetic for tiny shapes.

Every function here is pinned by the CPU tests against something other than
itself: exact rational brute force, a worked example computed by hand, the
k = 1 closed form, the Walsh-Hadamard special case (an independent fast
transform), sign-gauge symmetries, linearity and an exhaustive check of the
fp16 rounding against an integer-arithmetic definition.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = [
    "widen",
    "rne_fp16",
    "dense_weight",
    "dense_forward",
    "factored_forward",
    "factored_intermediate",
    "sampled_forward",
    "brute_force",
    "backward",
    "brute_force_backward",
]


def _check_signs(S: np.ndarray, name: str) -> np.ndarray:
    S = np.asarray(S)
    if S.ndim != 2:
        raise ValueError(f"{name} must be 2-D, got shape {S.shape}")
    if not np.all((S == 1) | (S == -1)):
        raise ValueError(f"{name} must hold only +1 and -1")
    return S.astype(np.float64)


def widen(v) -> np.ndarray:
    """fp16 (or any narrower float) -> fp64.  Exact for fp16 inputs."""
    return np.asarray(v).astype(np.float64)


def rne_fp16(y) -> np.ndarray:
    """Round fp64 values to fp16, nearest-even, in a single step.

    numpy converts float64 to float16 directly (no detour through float32,
    which would round twice).  Overflow goes to +/-inf like IEEE 754
    binary16.  Pinned exhaustively against an integer-arithmetic rounding
    rule in the CPU tests.
    """
    return np.asarray(y, dtype=np.float64).astype(np.float16)


def _shapes(X, A, B, a, mid, b):
    A64 = _check_signs(A, "A")
    B64 = _check_signs(B, "B")
    n, k = A64.shape
    k2, m = B64.shape
    if k2 != k:
        raise ValueError(f"A is {A64.shape} but B is {B64.shape}: middle dims differ")
    a64, mid64, b64 = widen(a), widen(mid), widen(b)
    if a64.shape != (n,) or mid64.shape != (k,) or b64.shape != (m,):
        raise ValueError("scale vectors must have lengths n, k, m")
    X64 = widen(X)
    if X64.ndim != 2 or X64.shape[1] != m:
        raise ValueError(f"X must be batch x {m}, got {X64.shape}")
    return X64, A64, B64, a64, mid64, b64


def dense_weight(A, B, a, mid, b) -> np.ndarray:
    """W = (a ⊙ A ⊙ midᵀ)(B ⊙ bᵀ) in fp64 (§2.1, the factorized form of W).

    A column vector multiplied elementwise into a matrix scales its rows, a
    row vector scales its columns: L[i, j] = a[i] * A[i, j] * mid[j] and
    R[j, l] = B[j, l] * b[l].  The matrix product is a library matmul.
    """
    A64 = _check_signs(A, "A")
    B64 = _check_signs(B, "B")
    a64, mid64, b64 = widen(a), widen(mid), widen(b)
    L = a64[:, None] * A64 * mid64[None, :]
    R = B64 * b64[None, :]
    return L @ R


def dense_forward(X, A, B, a, mid, b) -> np.ndarray:
    """Y = X Wᵀ in fp64 with W reconstructed densely (the plain definition).

    Returns the unrounded fp64 result, shape (batch, n).  Round it with
    ``rne_fp16`` to get the fp16 layer output.
    """
    X64, A64, B64, a64, mid64, b64 = _shapes(X, A, B, a, mid, b)
    W = dense_weight(A64, B64, a64, mid64, b64)
    return X64 @ W.T


def factored_intermediate(X, A, B, a, mid, b):
    """The intermediates of the §2.1 evaluation order, in fp64.

    Returns (u, t, v, s, y):
      u = X ⊙ bᵀ        (batch x m)  input columns scaled by b
      t = u Bᵀ          (batch x k)  first signed sum
      v = t ⊙ midᵀ      (batch x k)  middle scaling
      s = v Aᵀ          (batch x n)  second signed sum
      y = s ⊙ aᵀ        (batch x n)  output scaling (unrounded)
    """
    X64, A64, B64, a64, mid64, b64 = _shapes(X, A, B, a, mid, b)
    u = X64 * b64[None, :]
    t = u @ B64.T
    v = t * mid64[None, :]
    s = v @ A64.T
    y = s * a64[None, :]
    return u, t, v, s, y


def factored_forward(X, A, B, a, mid, b) -> np.ndarray:
    """Y by the §2.1 evaluation order ((((X⊙bᵀ)Bᵀ)⊙midᵀ)Aᵀ)⊙aᵀ, fp64, unrounded."""
    return factored_intermediate(X, A, B, a, mid, b)[-1]


def sampled_forward(X, A, B, a, mid, b, rows, cols) -> np.ndarray:
    """Selected outputs y[r, i] for r in ``rows`` and i in ``cols``, fp64.

    For full-size layers where forming W or the whole output is too slow:
    for each selected batch row r it forms t = B (b ⊙ x_r) and
    v = mid ⊙ t once, then y[r, i] = a[i] * <A[i, :], v> for each selected
    output i.  Returns an array of shape (len(rows), len(cols)).
    """
    A = np.asarray(A)
    B = np.asarray(B)
    a64, mid64, b64 = widen(a), widen(mid), widen(b)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    U = widen(np.asarray(X)[rows]) * b64[None, :]          # (R, m)
    T = np.empty((B.shape[0], len(rows)), dtype=np.float64)
    # 256 middle channels at a time keeps the fp64 copy of B small
    step = 256
    for j0 in range(0, B.shape[0], step):
        T[j0:j0 + step] = _check_signs(B[j0:j0 + step], "B") @ U.T
    V = T * mid64[:, None]                                  # (k, R)
    Asub = _check_signs(A[cols], "A rows")                  # (C, k)
    return (a64[cols][:, None] * (Asub @ V)).T              # (R, C)


def brute_force(X, A, B, a, mid, b):
    """Exact rational Y[r][i] = Σ_l X[r,l] W[i,l], W[i,l] = Σ_j a_i A_ij mid_j B_jl b_l.

    Triple loops in ``fractions.Fraction`` straight from the definition of W
    as a product of the two scaled factors; for tiny shapes only.  Returns a
    list of lists of Fractions, shape (batch, n).
    """
    A = np.asarray(A)
    B = np.asarray(B)
    n, k = A.shape
    m = B.shape[1]
    if n * k * m > 20000:
        raise ValueError("brute_force is for tiny shapes only")
    fa = [Fraction(float(v)) for v in np.asarray(a, dtype=np.float64)]
    fmid = [Fraction(float(v)) for v in np.asarray(mid, dtype=np.float64)]
    fb = [Fraction(float(v)) for v in np.asarray(b, dtype=np.float64)]
    W = [[Fraction(0)] * m for _ in range(n)]
    for i in range(n):
        for l in range(m):
            acc = Fraction(0)
            for j in range(k):
                acc += fa[i] * int(A[i, j]) * fmid[j] * int(B[j, l]) * fb[l]
            W[i][l] = acc
    Xf = np.asarray(X, dtype=np.float64)
    out = []
    for r in range(Xf.shape[0]):
        xr = [Fraction(float(v)) for v in Xf[r]]
        out.append([sum((xr[l] * W[i][l] for l in range(m)), Fraction(0)) for i in range(n)])
    return out


def backward(X, dY, A, B, a, mid, b):
    """Gradients of the layer for an upstream gradient dY = dL/dY, in fp64.

    The pages fine-tune the factors after factorization (gist.science
    technical summary, §4: tuning of the discrete parameters improves
    accuracy; §5: the memory cost of fine-tuning binary factors is open).
    For the fp16 parameters of Y = X Wᵀ with W = diag(a) A diag(mid) B
    diag(b), i.e. Y[r,i] = a_i Σ_j A_ij mid_j Σ_l B_jl b_l X[r,l]:

      dX[r,l]  = Σ_i dY[r,i] W[i,l]                    dX = dY W
      da[i]    = Σ_r dY[r,i] s[r,i]                    s = ((X ⊙ bᵀ) Bᵀ ⊙ midᵀ) Aᵀ
      dmid[j]  = Σ_r g[r,j] t[r,j]                     t = (X ⊙ bᵀ) Bᵀ,  g = (dY ⊙ aᵀ) A
      db[l]    = Σ_r h[r,l] X[r,l]                     h = (g ⊙ midᵀ) B

    (each line is the derivative of the sum above with respect to one
    factor, the others held fixed).  Returns (dX, da, dmid, db), unrounded.
    """
    X64, A64, B64, a64, mid64, b64 = _shapes(X, A, B, a, mid, b)
    dY64 = widen(dY)
    if dY64.shape != (X64.shape[0], A64.shape[0]):
        raise ValueError(f"dY must be batch x n = {(X64.shape[0], A64.shape[0])}, got {dY64.shape}")
    W = dense_weight(A64, B64, a64, mid64, b64)
    dX = dY64 @ W
    t = (X64 * b64[None, :]) @ B64.T
    s = (t * mid64[None, :]) @ A64.T
    g = (dY64 * a64[None, :]) @ A64
    h = (g * mid64[None, :]) @ B64
    da = (dY64 * s).sum(axis=0)
    dmid = (g * t).sum(axis=0)
    db = (h * X64).sum(axis=0)
    return dX, da, dmid, db


def brute_force_backward(X, dY, A, B, a, mid, b):
    """Exact rational gradients straight from Y[r,i] = Σ_j Σ_l a_i A_ij mid_j
    B_jl b_l X[r,l]: each gradient entry is the sum, over the terms of the
    loss Σ_r Σ_i dY[r,i] Y[r,i], of the term's factor other than the
    parameter.  Tiny shapes only.  Returns lists of Fractions (dX as a list of
    rows)."""
    A = np.asarray(A)
    B = np.asarray(B)
    n, k = A.shape
    m = B.shape[1]
    bt = np.asarray(X).shape[0]
    if bt * n * k * m > 20000:
        raise ValueError("brute_force_backward is for tiny shapes only")
    F = lambda v: [Fraction(float(x)) for x in np.asarray(v, dtype=np.float64).ravel()]
    fa, fmid, fb = F(a), F(mid), F(b)
    Xf = [F(row) for row in np.asarray(X, dtype=np.float64)]
    Gf = [F(row) for row in np.asarray(dY, dtype=np.float64)]
    dX = [[Fraction(0)] * m for _ in range(bt)]
    da = [Fraction(0)] * n
    dmid = [Fraction(0)] * k
    db = [Fraction(0)] * m
    for r in range(bt):
        for i in range(n):
            for j in range(k):
                for l in range(m):
                    sign = int(A[i, j]) * int(B[j, l])
                    w = Gf[r][i] * sign          # dL/dY[r,i] times the signs of the term
                    dX[r][l] += w * fa[i] * fmid[j] * fb[l]
                    da[i] += w * fmid[j] * fb[l] * Xf[r][l]
                    dmid[j] += w * fa[i] * fb[l] * Xf[r][l]
                    db[l] += w * fa[i] * fmid[j] * Xf[r][l]
    return dX, da, dmid, db

