"""CPU oracle for the forward of a binary-quadratic (BQQ-form) weight matrix.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module.  The product path (the HIP library and its Python binding)
never imports, links or calls anything here, and this file shares no code,
tables or helpers with it.

What is computed
----------------
Source: "Binary Quadratic Quantization: Beyond First-Order Quantization for
Real-Valued Matrix Compression", TL;DR on its sciencestack.ai page (the
formula for W).  It writes a real matrix as a sum of p binary matrix
products, each with its own scalings, plus a constant:

    W = Σ_{i<p} ( r_i Y_i Z_i + s_i Y_i 1_Z + t_i 1_Y Z_i ) + u 1

with Y_i of shape n x d and Z_i of shape d x m binary, 1_Z the d x m matrix
of ones, 1_Y the n x d matrix of ones and 1 the n x m matrix of ones.  As a
layer weight (n outputs, m inputs), the output for an input X (batch x m)
is X W^T, the same contract as the DBF layer.

Readings where the page is silent (each is listed with the others of the
library):
* "binary" means entries in {0, 1} (the method builds on polynomial
  unconstrained binary optimization, whose variables are 0/1).
* r_i, s_i, t_i and u are one scalar each per term (one scaling group),
  given as fp16 like the DBF scales.
* Group-wise scaling (the same TL;DR names it as a way to cut parameter
  overhead, and the page's Figure 2 is captioned as a figure on ways of
  scaling the weights; the page gives no formula): the m input columns fall into
  groups of ``group`` consecutive columns (the last group may be shorter),
  and every group h has scalars of its own, r_i[h], s_i[h], t_i[h] (i < p)
  and u[h]; the binary matrices Y_i and Z_i are shared by all groups.  On
  the columns l of group h,

      W[:, l] = Σ_{i<p} ( r_i[h] Y_i Z_i + s_i[h] Y_i 1_Z + t_i[h] 1_Y Z_i )[:, l] + u[h]

  so one group covering all columns is the form above.  Groups run along
  the input dimension, as the groups of weight quantizers usually do, and a
  group's scalars serve every output row (the low overhead the TL;DR
  names: 3 p + 1 scalars per group).
* The output is fp16, one round-to-nearest-even of the exact value.

Precision: inputs are fp16 or 0/1, so widening to fp64 is exact; the fp64
results differ from the exact rational value only by sum rounding (relative
order (p d + m) 2**-53).  ``brute_force`` evaluates the definition entry by
entry in exact rational arithmetic for tiny shapes.

Pinned by the CPU tests (tests/test_oracle_bqq.py) against exact rational
brute force, a hand-worked 2 x 2 example, the all-ones closed form, each
term on its own in closed form, and the identity that turns a 0/1 product
into a ±1 product (checked against the separately pinned DBF oracle).  The
group-wise form is pinned against its own entry-by-entry rational brute
force (ragged last group included), a hand-worked two-group example, the
sum of single-group layers over the column blocks, and the single-group
form when every group has the same scalars.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = ["bqq_weight", "bqq_forward", "brute_force", "group_columns", "bqq_weight_grouped",
           "bqq_forward_grouped", "brute_force_grouped"]


def _check_binary(M, name: str, ndim: int = 3) -> np.ndarray:
    M = np.asarray(M)
    if M.ndim != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {M.shape}")
    if not np.all((M == 0) | (M == 1)):
        raise ValueError(f"{name} must hold only 0 and 1")
    return M.astype(np.float64)


def _parts(Y, Z, r, s, t, u):
    Y64 = _check_binary(Y, "Y")
    Z64 = _check_binary(Z, "Z")
    p, n, d = Y64.shape
    p2, d2, m = Z64.shape
    if (p2, d2) != (p, d):
        raise ValueError(f"Y is {Y64.shape} but Z is {Z64.shape}")
    r64, s64, t64 = (np.asarray(v).astype(np.float64) for v in (r, s, t))
    if r64.shape != (p,) or s64.shape != (p,) or t64.shape != (p,):
        raise ValueError("r, s, t must have one value per term")
    u64 = float(np.asarray(u).astype(np.float64))
    return Y64, Z64, r64, s64, t64, u64, p, n, d, m


def bqq_weight(Y, Z, r, s, t, u) -> np.ndarray:
    """W of the formula above in fp64, the ones-matrices formed explicitly.

    Y: (p, n, d) of 0/1; Z: (p, d, m) of 0/1; r, s, t: (p,); u: scalar.
    The matrix products are library matmuls.
    """
    Y64, Z64, r64, s64, t64, u64, p, n, d, m = _parts(Y, Z, r, s, t, u)
    ones_Z = np.ones((d, m))
    ones_Y = np.ones((n, d))
    W = u64 * np.ones((n, m))
    for i in range(p):
        W += r64[i] * (Y64[i] @ Z64[i]) + s64[i] * (Y64[i] @ ones_Z) + t64[i] * (ones_Y @ Z64[i])
    return W


def bqq_forward(X, Y, Z, r, s, t, u) -> np.ndarray:
    """X Wᵀ in fp64 with W from ``bqq_weight`` (unrounded, shape (batch, n))."""
    W = bqq_weight(Y, Z, r, s, t, u)
    X64 = np.asarray(X).astype(np.float64)
    if X64.ndim != 2 or X64.shape[1] != W.shape[1]:
        raise ValueError(f"X must be batch x {W.shape[1]}, got {X64.shape}")
    return X64 @ W.T


def brute_force(X, Y, Z, r, s, t, u):
    """Exact rational X Wᵀ, W entry by entry from the formula; tiny shapes.

    W[o][l] = Σ_i ( r_i Σ_j Y_i[o][j] Z_i[j][l] + s_i Σ_j Y_i[o][j]
                    + t_i Σ_j Z_i[j][l] ) + u
    (the (o, l) entry of Y_i 1_Z is row o of Y_i summed, that of 1_Y Z_i is
    column l of Z_i summed).  Returns a list of lists of Fractions.
    """
    Y = np.asarray(Y)
    Z = np.asarray(Z)
    p, n, d = Y.shape
    m = Z.shape[2]
    fr = lambda v: Fraction(float(v))  # noqa: E731  (fp16 -> exact binary fraction)
    R = [fr(v) for v in np.asarray(r)]
    S = [fr(v) for v in np.asarray(s)]
    T = [fr(v) for v in np.asarray(t)]
    U = fr(np.asarray(u))
    W = [[U for _ in range(m)] for _ in range(n)]
    for o in range(n):
        for l in range(m):
            acc = U
            for i in range(p):
                yz = sum(int(Y[i, o, j]) * int(Z[i, j, l]) for j in range(d))
                ysum = sum(int(Y[i, o, j]) for j in range(d))
                zsum = sum(int(Z[i, j, l]) for j in range(d))
                acc += R[i] * yz + S[i] * ysum + T[i] * zsum
            W[o][l] = acc
    X = np.asarray(X)
    out = []
    for row in X:
        xr = [fr(v) for v in row]
        out.append([sum((W[o][l] * xr[l] for l in range(m)), Fraction(0)) for o in range(n)])
    return out


# --------------------------------------------------------------------------- group-wise scaling

def group_columns(m: int, group: int):
    """The column ranges [start, stop) of the groups: ``group`` consecutive
    columns each, the last one shorter when ``group`` does not divide m."""
    if group < 1 or m < 1:
        raise ValueError("m and group must be positive")
    return [(c, min(m, c + group)) for c in range(0, m, group)]


def bqq_weight_grouped(Y, Z, r, s, t, u, group: int) -> np.ndarray:
    """W of the group-wise form in fp64, group by group.

    Y: (p, n, d) of 0/1; Z: (p, d, m) of 0/1; r, s, t: (p, ngroups);
    u: (ngroups,), with ngroups = ceil(m / group).  On the columns of group
    h the weight is the single-group formula with r_i[h], s_i[h], t_i[h],
    u[h], the ones-matrices formed explicitly at the group's width.
    """
    Y64 = _check_binary(Y, "Y")
    Z64 = _check_binary(Z, "Z")
    p, n, d = Y64.shape
    p2, d2, m = Z64.shape
    if (p2, d2) != (p, d):
        raise ValueError(f"Y is {Y64.shape} but Z is {Z64.shape}")
    cols = group_columns(m, group)
    ng = len(cols)
    r64, s64, t64 = (np.asarray(v).astype(np.float64) for v in (r, s, t))
    u64 = np.asarray(u).astype(np.float64)
    if r64.shape != (p, ng) or s64.shape != (p, ng) or t64.shape != (p, ng) or u64.shape != (ng,):
        raise ValueError(f"r, s, t must be ({p}, {ng}) and u ({ng},) for m = {m}, group = {group}")
    W = np.empty((n, m))
    for h, (c0, c1) in enumerate(cols):
        w = c1 - c0
        Wh = u64[h] * np.ones((n, w))
        for i in range(p):
            Wh += (r64[i, h] * (Y64[i] @ Z64[i][:, c0:c1]) + s64[i, h] * (Y64[i] @ np.ones((d, w)))
                   + t64[i, h] * (np.ones((n, d)) @ Z64[i][:, c0:c1]))
        W[:, c0:c1] = Wh
    return W


def bqq_forward_grouped(X, Y, Z, r, s, t, u, group: int) -> np.ndarray:
    """X Wᵀ in fp64 with W from ``bqq_weight_grouped`` (unrounded)."""
    W = bqq_weight_grouped(Y, Z, r, s, t, u, group)
    X64 = np.asarray(X).astype(np.float64)
    if X64.ndim != 2 or X64.shape[1] != W.shape[1]:
        raise ValueError(f"X must be batch x {W.shape[1]}, got {X64.shape}")
    return X64 @ W.T


def brute_force_grouped(X, Y, Z, r, s, t, u, group: int):
    """Exact rational X Wᵀ of the group-wise form, entry by entry; tiny shapes.

    W[o][l] = Σ_i ( r_i[h] Σ_j Y_i[o][j] Z_i[j][l] + s_i[h] Σ_j Y_i[o][j]
                    + t_i[h] Σ_j Z_i[j][l] ) + u[h],   h = l // group.
    Returns a list of lists of Fractions.
    """
    Y = np.asarray(Y)
    Z = np.asarray(Z)
    p, n, d = Y.shape
    m = Z.shape[2]
    fr = lambda v: Fraction(float(v))  # noqa: E731
    R = [[fr(v) for v in row] for row in np.asarray(r)]
    S = [[fr(v) for v in row] for row in np.asarray(s)]
    T = [[fr(v) for v in row] for row in np.asarray(t)]
    U = [fr(v) for v in np.asarray(u)]
    W = [[Fraction(0)] * m for _ in range(n)]
    for o in range(n):
        for l in range(m):
            h = l // group
            acc = U[h]
            for i in range(p):
                yz = sum(int(Y[i, o, j]) * int(Z[i, j, l]) for j in range(d))
                ysum = sum(int(Y[i, o, j]) for j in range(d))
                zsum = sum(int(Z[i, j, l]) for j in range(d))
                acc += R[i][h] * yz + S[i][h] * ysum + T[i][h] * zsum
            W[o][l] = acc
    out = []
    for row in np.asarray(X):
        xr = [fr(v) for v in row]
        out.append([sum((W[o][l] * xr[l] for l in range(m)), Fraction(0)) for o in range(n)])
    return out
