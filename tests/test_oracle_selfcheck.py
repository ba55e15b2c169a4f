"""Pins for the CPU oracle, checked against things other than the oracle itself.

Citations: the DBF form of W and its evaluation order are from "Addition is
almost all you need: Compressing large language models with double binary
factorization", gist.science technical summary, §2.1.

* exact rational brute force on tiny shapes (and stored exact results under
  tests/golden written by a script that calls only the oracle);
* a worked example computed by hand, non-square so a transposed operand fails;
* the k = 1 rank-one closed form;
* the Sylvester-Hadamard special case, checked with an independent fast
  Walsh-Hadamard transform (with a column permutation, so that B and B^T
  differ);
* the sign-gauge symmetries of the factorization;
* homogeneity, linearity and batch-row independence;
* an exhaustive check of the fp16 rounding helper against an integer
  round-half-to-even rule;
* mutation checks: plausible mistakes planted into copies of the oracle are
  caught by these pins.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import dbf_oracle as O
from tests import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- helpers

def _rand_fp16(rng, size, lo=-2.0, hi=2.0):
    return rng.uniform(lo, hi, size=size).astype(np.float16)


_tiny_case = inputs.tiny_case


def _rel_rows(y, ref):
    """Per-row max-norm relative difference."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    return (np.abs(y - ref).max(axis=1) / den).max()


def rne16_int(x: float) -> float:
    """Round a finite fp64 value to the fp16 grid, ties to even, with integers.

    Independent of numpy's conversion: the fp16 grid has spacing 2**-24 below
    2**-14 and 2**(e-10) in the binade [2**e, 2**(e+1)); values whose rounded
    magnitude reaches 2**16 overflow to infinity.
    """
    if x == 0.0:
        return x
    sign = -1.0 if x < 0 else 1.0
    num, den = abs(x).as_integer_ratio()           # den is a power of two
    # exponent e with 2**e <= |x| < 2**(e+1)
    e = num.bit_length() - den.bit_length()
    if Fraction(num, den) < Fraction(2) ** e:
        e -= 1
    g = -24 if e < -14 else e - 10                  # grid exponent
    # q = |x| / 2**g, split into integer part and remainder
    scaled = Fraction(num, den) / (Fraction(2) ** g)
    q = scaled.numerator // scaled.denominator
    r = scaled - q
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and q % 2 == 1):
        q += 1
    val = q * (2.0 ** g)
    if val >= 65536.0:
        return sign * math.inf
    return sign * val


# --------------------------------------------------------------------------- fp16 rounding

def test_rne_fp16_exhaustive():
    """All finite fp16 values, every midpoint between neighbours, and the fp64
    neighbours of each midpoint round as the integer rule says."""
    allbits = np.arange(0, 0x7C00, dtype=np.uint16)        # +0 .. max finite
    vals = allbits.view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0                     # exact in fp64
    top = np.array([65504.0 + 16.0])                        # tie above max finite
    pts = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf), top,
                          np.nextafter(top, 0)])
    pts = np.concatenate([pts, -pts])
    got = O.rne_fp16(pts).astype(np.float64)
    want = np.array([rne16_int(float(p)) for p in pts])
    both_inf = np.isinf(got) & np.isinf(want) & (np.sign(got) == np.sign(want))
    assert np.all((got == want) | both_inf)
    # spot values: ties to even at 2049 -> 2048 and 2051 -> 2052, overflow boundary
    assert float(O.rne_fp16(2049.0)) == 2048.0
    assert float(O.rne_fp16(2051.0)) == 2052.0
    assert float(O.rne_fp16(65519.99)) == 65504.0
    assert math.isinf(float(O.rne_fp16(65520.0)))
    # a single rounding: via fp32 this value would round twice and land on 1.0
    assert float(O.rne_fp16(1 + 2 ** -11 + 2 ** -40)) == 1 + 2 ** -10


# --------------------------------------------------------------------------- worked example

def test_worked_example_by_hand():
    """n=2 outputs, m=3 inputs, k=2, two batch rows, evaluated by hand.

    A = [[1,-1],[-1,-1]], B = [[1,1,-1],[-1,1,1]], a = [2, 1/2], mid = [1, 3],
    b = [1, 2, 1/4].
    Row 1: X = [1, -2, 4]   -> u = X⊙b = [1, -4, 1]
           t = B u = [1-4-1, -1-4+1] = [-4, -4];  v = t⊙mid = [-4, -12]
           s = A v = [-4+12, 4+12] = [8, 16];     y = s⊙a = [16, 8]
    Row 2: X = [1/2, 1, -1] -> u = [1/2, 2, -1/4]
           t = [1/2+2+1/4, -1/2+2-1/4] = [11/4, 5/4]; v = [11/4, 15/4]
           s = [11/4-15/4, -11/4-15/4] = [-1, -13/2];  y = [-2, -13/4]
    The dense route agrees: W = [[8, -8, -2], [1, -4, -1/4]].
    """
    A = np.array([[1, -1], [-1, -1]], dtype=np.int8)
    B = np.array([[1, 1, -1], [-1, 1, 1]], dtype=np.int8)
    a = np.array([2, 0.5], dtype=np.float16)
    mid = np.array([1, 3], dtype=np.float16)
    b = np.array([1, 2, 0.25], dtype=np.float16)
    X = np.array([[1, -2, 4], [0.5, 1, -1]], dtype=np.float16)
    want = np.array([[16.0, 8.0], [-2.0, -3.25]])
    assert np.array_equal(O.dense_weight(A, B, a, mid, b),
                          np.array([[8.0, -8.0, -2.0], [1.0, -4.0, -0.25]]))
    assert np.array_equal(O.dense_forward(X, A, B, a, mid, b), want)
    assert np.array_equal(O.factored_forward(X, A, B, a, mid, b), want)
    u, t, v, s, y = O.factored_intermediate(X, A, B, a, mid, b)
    assert np.array_equal(t, [[-4, -4], [2.75, 1.25]])
    assert np.array_equal(s, [[8, 16], [-1, -6.5]])
    assert np.array_equal(O.sampled_forward(X, A, B, a, mid, b, [1, 0], [1]), [[-3.25], [8.0]])
    assert [[float(f) for f in row] for row in O.brute_force(X, A, B, a, mid, b)] == want.tolist()


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed,n,m,k,batch", [
    (0, 1, 1, 1, 1), (1, 2, 3, 4, 2), (2, 5, 4, 3, 3), (3, 6, 6, 6, 2), (4, 3, 5, 6, 1),
    (5, 6, 2, 5, 3),
])
def test_brute_force_matches_dense_and_factored(seed, n, m, k, batch):
    X, A, B, a, mid, b = _tiny_case(seed, n, m, k, batch)
    exact = O.brute_force(X, A, B, a, mid, b)
    ex = np.array([[float(f) for f in row] for row in exact])
    for f in (O.dense_forward, O.factored_forward):
        y = f(X, A, B, a, mid, b)
        scale = np.abs(ex).max() + 1e-300
        assert np.abs(y - ex).max() <= 1e-14 * scale
        # the fp16 result matches exact rounding unless the exact value sits
        # within fp64 noise of a rounding boundary
        r16 = O.rne_fp16(y).astype(np.float64)
        for rr in range(ex.shape[0]):
            for ii in range(ex.shape[1]):
                want = rne16_int(float(exact[rr][ii]))
                if r16[rr, ii] != want:
                    lo, hi = sorted([r16[rr, ii], want])
                    boundary = (lo + hi) / 2
                    assert abs(float(exact[rr][ii]) - boundary) <= 1e-13 * abs(boundary)


def test_golden_exact_results():
    """Stored exact rational results (written by tests/golden/make_golden.py,
    which calls only the oracle's exact brute force)."""
    with open(os.path.join(GOLDEN, "brute_force_cases.json")) as fh:
        cases = json.load(fh)
    assert len(cases) >= 3
    for case in cases:
        X, A, B, a, mid, b = _tiny_case(case["seed"], case["n"], case["m"], case["k"], case["batch"])
        want = np.array([[float(Fraction(s)) for s in row] for row in case["y_exact"]])
        y = O.dense_forward(X, A, B, a, mid, b)
        assert np.abs(y - want).max() <= 1e-14 * (np.abs(want).max() + 1e-300)
        assert np.array_equal(O.rne_fp16(y).view(np.uint16),
                              np.array(case["y_fp16_bits"], dtype=np.uint16))


# --------------------------------------------------------------------------- closed forms

def test_k1_rank_one_closed_form():
    """With k = 1, Y[r, i] = mid_0 * a_i * A_i0 * sum_l B_0l b_l X_rl."""
    rng = np.random.default_rng(11)
    n, m, batch = 37, 53, 4
    A = (1 - 2 * rng.integers(0, 2, size=(n, 1))).astype(np.int8)
    B = (1 - 2 * rng.integers(0, 2, size=(1, m))).astype(np.int8)
    a, mid, b = _rand_fp16(rng, n), _rand_fp16(rng, 1), _rand_fp16(rng, m)
    X = _rand_fp16(rng, (batch, m))
    col = a.astype(np.float64) * A[:, 0]                         # (n,)
    row = X.astype(np.float64) @ (B[0] * b.astype(np.float64))  # (batch,)
    want = float(mid[0]) * np.outer(row, col)
    for f in (O.dense_forward, O.factored_forward):
        assert _rel_rows(f(X, A, B, a, mid, b), want) < 1e-14


def _sylvester(p):
    H = np.array([[1]], dtype=np.int8)
    for _ in range(p):
        H = np.block([[H, H], [H, -H]]).astype(np.int8)
    return H


def _fwht(v):
    """Fast Walsh-Hadamard transform (Sylvester order), unnormalised, along the last axis."""
    v = np.array(v, dtype=np.float64)
    n = v.shape[-1]
    h = 1
    while h < n:
        v = v.reshape(v.shape[:-1] + (n // (2 * h), 2, h))
        x, y = v[..., 0, :].copy(), v[..., 1, :].copy()
        v[..., 0, :], v[..., 1, :] = x + y, x - y
        v = v.reshape(v.shape[:-3] + (n,))
        h *= 2
    return v


def test_hadamard_special_case():
    """B = H P (Sylvester Hadamard, columns permuted) and A = H: the two signed
    sums are fast Walsh-Hadamard transforms: Y = a ⊙ FWHT(mid ⊙ FWHT(P(b ⊙ x)))."""
    p = 6
    N = 1 << p
    rng = np.random.default_rng(5)
    H = _sylvester(p)
    perm = rng.permutation(N)
    B = np.ascontiguousarray(H[:, perm])       # column l of B is column perm[l] of H
    A = H.copy()
    a, mid, b = _rand_fp16(rng, N), _rand_fp16(rng, N), _rand_fp16(rng, N)
    X = _rand_fp16(rng, (3, N))
    u = X.astype(np.float64) * b.astype(np.float64)
    Pu = np.zeros_like(u)
    Pu[:, perm] = u                            # (H P u)_j = sum_l H[j, perm[l]] u_l
    want = a.astype(np.float64) * _fwht(mid.astype(np.float64) * _fwht(Pu))
    for f in (O.dense_forward, O.factored_forward):
        assert _rel_rows(f(X, A, B, a, mid, b), want) < 1e-13


# --------------------------------------------------------------------------- invariants

def test_sign_gauge_symmetries_bitwise():
    X, A, B, a, mid, b = _tiny_case(21, 17, 23, 9, 3)
    base = O.dense_forward(X, A, B, a, mid, b)
    i, j, l = 4, 2, 7
    # row i of A with a_i
    A1, a1 = A.copy(), a.copy(); A1[i] *= -1; a1[i] = -a1[i]
    # column j of A with row j of B
    A2, B2 = A.copy(), B.copy(); A2[:, j] *= -1; B2[j] *= -1
    # row j of B with mid_j
    B3, mid3 = B.copy(), mid.copy(); B3[j] *= -1; mid3[j] = -mid3[j]
    # column l of B with b_l
    B4, b4 = B.copy(), b.copy(); B4[:, l] *= -1; b4[l] = -b4[l]
    for args in ((X, A1, B, a1, mid, b), (X, A2, B2, a, mid, b), (X, A, B3, a, mid3, b),
                 (X, A, B4, a, mid, b4)):
        assert np.array_equal(O.rne_fp16(O.dense_forward(*args)).view(np.uint16),
                              O.rne_fp16(base).view(np.uint16))
        assert _rel_rows(O.dense_forward(*args), base) < 1e-15
    # flipping only one member of a pair changes the output
    assert not np.allclose(O.dense_forward(X, A1, B, a, mid, b), base)


def test_homogeneity_linearity_batch_independence():
    X, A, B, a, mid, b = _tiny_case(31, 19, 29, 13, 4)
    base = O.dense_forward(X, A, B, a, mid, b)
    # powers of two scale exactly
    assert np.array_equal(O.dense_forward((X.astype(np.float64) * 4).astype(np.float16), A, B, a, mid, b),
                          base * 4)
    assert np.array_equal(O.dense_forward(np.zeros_like(X), A, B, a, mid, b), np.zeros_like(base))
    # linear in each scale vector (small-integer values keep fp64 exact)
    rng = np.random.default_rng(3)
    ai = lambda n: rng.integers(-3, 4, size=n).astype(np.float16)
    Xi = rng.integers(-3, 4, size=X.shape).astype(np.float16)
    a1, a2, m1, m2, b1, b2 = ai(19), ai(19), ai(13), ai(13), ai(29), ai(29)
    f = O.dense_forward
    assert np.array_equal(f(Xi, A, B, a1 + a2, m1, b1), f(Xi, A, B, a1, m1, b1) + f(Xi, A, B, a2, m1, b1))
    assert np.array_equal(f(Xi, A, B, a1, m1 + m2, b1), f(Xi, A, B, a1, m1, b1) + f(Xi, A, B, a1, m2, b1))
    assert np.array_equal(f(Xi, A, B, a1, m1, b1 + b2), f(Xi, A, B, a1, m1, b1) + f(Xi, A, B, a1, m1, b2))
    # each batch row alone gives the same result as inside the batch (BLAS may
    # sum a single row in another order, so agreement is to fp64 rounding)
    for r in range(X.shape[0]):
        assert _rel_rows(f(X[r:r + 1], A, B, a, mid, b), base[r:r + 1]) < 1e-14
    for r in range(Xi.shape[0]):
        assert np.array_equal(f(Xi[r:r + 1], A, B, a1, m1, b1)[0], f(Xi, A, B, a1, m1, b1)[r])


def test_dense_equals_factored_and_sampled_moderate():
    """Associativity (dense W route == §2.1 right-to-left route) at a moderate
    size, and the one-by-one sampled outputs used at full sizes."""
    L = inputs.random_layer("t", 96, 160, 64, 7, 0.05, 1.0, 0.05, (5,))
    X = L.X[5]
    d = O.dense_forward(X, L.A, L.B, L.a, L.mid, L.b)
    fz = O.factored_forward(X, L.A, L.B, L.a, L.mid, L.b)
    assert _rel_rows(fz, d) < 1e-13
    rows, cols = [4, 0, 2], [95, 0, 17, 64]
    s = O.sampled_forward(X, L.A, L.B, L.a, L.mid, L.b, rows, cols)
    assert np.abs(s - d[np.ix_(rows, cols)]).max() <= 1e-13 * np.abs(d).max()


def test_integer_inputs_are_exact():
    """Small-integer inputs: dense and factored agree bit for bit and are integers."""
    L = inputs.integer_layer("i", 64, 96, 32, 9, (3,), a_vals=(0.5, 1.0))
    X = L.X[3]
    d = O.dense_forward(X, L.A, L.B, L.a, L.mid, L.b)
    fz = O.factored_forward(X, L.A, L.B, L.a, L.mid, L.b)
    assert np.array_equal(d, fz)
    assert np.array_equal(d * 2, np.round(d * 2))


def test_input_validation():
    X, A, B, a, mid, b = _tiny_case(1, 2, 3, 4, 1)
    A0 = A.copy(); A0[0, 0] = 0
    with pytest.raises(ValueError):
        O.dense_forward(X, A0, B, a, mid, b)
    with pytest.raises(ValueError):
        O.dense_forward(X, A, B[:3], a, mid, b)
    with pytest.raises(ValueError):
        O.dense_forward(X[:, :2], A, B, a, mid, b)


# --------------------------------------------------------------------------- mutation checks

def _pin_outcomes(forward):
    """Run the value pins (worked example, brute force on a non-square and a
    square shape) on a candidate forward.  Returns one of "pass", "fail"
    (a wrong value) or "error" (an exception, e.g. a shape mismatch) per pin."""
    out = []

    def run(fn):
        try:
            out.append("pass" if fn() else "fail")
        except Exception:
            out.append("error")

    def worked():
        A = np.array([[1, -1], [-1, -1]], dtype=np.int8)
        B = np.array([[1, 1, -1], [-1, 1, 1]], dtype=np.int8)
        a = np.array([2, 0.5], dtype=np.float16)
        mid = np.array([1, 3], dtype=np.float16)
        b = np.array([1, 2, 0.25], dtype=np.float16)
        X = np.array([[1, -2, 4], [0.5, 1, -1]], dtype=np.float16)
        return np.array_equal(forward(X, A, B, a, mid, b), [[16.0, 8.0], [-2.0, -3.25]])

    def brute(seed, n, m, k):
        X, A, B, a, mid, b = _tiny_case(seed, n, m, k, 2)
        ex = np.array([[float(f) for f in r] for r in O.brute_force(X, A, B, a, mid, b)])
        y = np.asarray(forward(X, A, B, a, mid, b))
        return y.shape == ex.shape and np.abs(y - ex).max() <= 1e-12 * np.abs(ex).max()

    run(worked)
    run(lambda: brute(2, 5, 4, 3))
    run(lambda: brute(3, 6, 6, 6))
    return out


def _mutants():
    w = O.widen

    def transposed_B(X, A, B, a, mid, b):
        # B where B^T belongs (shape-compatible only when k == m)
        return (((w(X) * w(b)) @ w(B)) * w(mid)) @ w(A).T * w(a)

    def transposed_A(X, A, B, a, mid, b):
        # A where A^T belongs (shape-compatible only when n == k)
        return (((w(X) * w(b)) @ w(B).T) * w(mid)) @ w(A) * w(a)

    def dropped_b(X, A, B, a, mid, b):
        return ((w(X) @ w(B).T) * w(mid)) @ w(A).T * w(a)

    def dropped_mid(X, A, B, a, mid, b):
        return ((w(X) * w(b)) @ w(B).T) @ w(A).T * w(a)

    def squared_mid(X, A, B, a, mid, b):
        return (((w(X) * w(b)) @ w(B).T) * w(mid) ** 2) @ w(A).T * w(a)

    def sign_flipped_A(X, A, B, a, mid, b):
        return (((w(X) * w(b)) @ w(B).T) * w(mid)) @ (-w(A)).T * w(a)

    def a_scales_columns_of_left_factor(X, A, B, a, mid, b):
        # a applied along the middle axis (shape-compatible only when n == k)
        L = w(A) * w(a)[None, :] * w(mid)[None, :]
        return w(X) @ (L @ (w(B) * w(b)[None, :])).T

    def shifted_b_index(X, A, B, a, mid, b):
        return (((w(X) * np.roll(w(b), 1)) @ w(B).T) * w(mid)) @ w(A).T * w(a)

    def shifted_middle_index(X, A, B, a, mid, b):
        return (((w(X) * w(b)) @ w(B).T) * np.roll(w(mid), 1)) @ w(A).T * w(a)

    return [transposed_B, transposed_A, dropped_b, dropped_mid, squared_mid, sign_flipped_A,
            a_scales_columns_of_left_factor, shifted_b_index, shifted_middle_index]


def test_oracle_pins_pass():
    assert _pin_outcomes(O.dense_forward) == ["pass"] * 3
    assert _pin_outcomes(O.factored_forward) == ["pass"] * 3


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught(mutant):
    """Each mistake gives a wrong value on at least one pin (not merely a shape error)."""
    assert "fail" in _pin_outcomes(mutant)
