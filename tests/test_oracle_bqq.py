"""Pins of the BQQ-form oracle (oracle/bqq_oracle.py) against things other
than itself: exact rational brute force, a 2 x 2 example worked by hand, the
all-ones closed form, each term of the formula on its own in closed form,
and the identity that turns a product of 0/1 matrices into a product of ±1
matrices, checked against the separately pinned DBF oracle.  A mutation
check shows that plausible mistakes in the formula fail at least one pin.

Formula: TL;DR of "Binary Quadratic Quantization: Beyond First-Order
Quantization for Real-Valued Matrix Compression" (sciencestack.ai page).
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import bqq_oracle as Q
from oracle import dbf_oracle as O
from tests import inputs


def _f16(v):
    return np.asarray(v, dtype=np.float64).astype(np.float16)


def _forward_with(weight_fn, X, Y, Z, r, s, t, u):
    return np.asarray(X, dtype=np.float64) @ weight_fn(Y, Z, r, s, t, u).T


def _random_case(seed, p, n, d, m, batch):
    rng = np.random.default_rng(seed)
    Y = rng.integers(0, 2, size=(p, n, d), dtype=np.uint8)
    Z = rng.integers(0, 2, size=(p, d, m), dtype=np.uint8)
    r, s, t = (_f16(rng.uniform(-2, 2, size=p)) for _ in range(3))
    u = _f16(rng.uniform(-2, 2))
    X = _f16(rng.uniform(-3, 3, size=(batch, m)))
    return X, Y, Z, r, s, t, u


def _pin_failures(weight_fn):
    """Run every pin with `weight_fn` as the weight builder; return the names
    of the pins that fail."""
    bad = []

    # exact rational brute force on tiny random shapes (square, so that a
    # transposed operand would still type-check)
    for seed, (p, n, d, m) in enumerate([(1, 3, 3, 3), (2, 4, 3, 4), (3, 2, 2, 2), (2, 3, 4, 3)]):
        X, Y, Z, r, s, t, u = _random_case(seed, p, n, d, m, 2)
        want = np.array([[float(v) for v in row] for row in Q.brute_force(X, Y, Z, r, s, t, u)])
        got = _forward_with(weight_fn, X, Y, Z, r, s, t, u)
        if not np.allclose(got, want, rtol=1e-12, atol=1e-12):
            bad.append(f"brute force {seed}")

    # hand-worked: Y = [[1,0],[1,1]], Z = [[0,1],[1,1]], r = 2, s = 1, t = -1, u = 0.5
    #   Y Z = [[0,1],[1,2]], Y 1 = [[1,1],[2,2]], 1 Z = [[1,2],[1,2]]
    #   W = [[0.5, 1.5], [3.5, 4.5]];  x = [1, -2]  ->  y = [-2.5, -5.5]
    Y = np.array([[[1, 0], [1, 1]]], dtype=np.uint8)
    Z = np.array([[[0, 1], [1, 1]]], dtype=np.uint8)
    W = weight_fn(Y, Z, _f16([2.0]), _f16([1.0]), _f16([-1.0]), _f16(0.5))
    if not np.array_equal(W, np.array([[0.5, 1.5], [3.5, 4.5]])):
        bad.append("hand-worked W")
    y = _forward_with(weight_fn, _f16([[1.0, -2.0]]), Y, Z, _f16([2.0]), _f16([1.0]), _f16([-1.0]), _f16(0.5))
    if not np.array_equal(y, np.array([[-2.5, -5.5]])):
        bad.append("hand-worked y")

    # all ones: every entry of W is sum_i d (r_i + s_i + t_i) + u
    p, n, d, m = 2, 3, 5, 4
    rng = np.random.default_rng(11)
    r, s, t = (_f16(rng.uniform(-1, 1, size=p)) for _ in range(3))
    u = _f16(0.25)
    W = weight_fn(np.ones((p, n, d), np.uint8), np.ones((p, d, m), np.uint8), r, s, t, u)
    const = sum(d * (float(r[i]) + float(s[i]) + float(t[i])) for i in range(p)) + float(u)
    if not np.allclose(W, const, rtol=0, atol=1e-12):
        bad.append("all ones")

    # each term on its own, in closed form with explicit loops
    p, n, d, m = 3, 4, 5, 6
    X, Y, Z, r, s, t, u = _random_case(21, p, n, d, m, 3)
    zero = _f16(np.zeros(p))
    Xf = X.astype(np.float64)
    # s only: y[b][o] = sum_i s_i (row o of Y_i summed) (sum of x_b)
    got = _forward_with(weight_fn, X, Y, Z, zero, s, zero, _f16(0))
    want = np.zeros((3, n))
    for b in range(3):
        for o in range(n):
            want[b, o] = sum(float(s[i]) * int(Y[i, o, :].sum()) for i in range(p)) * Xf[b].sum()
    if not np.allclose(got, want, rtol=1e-12, atol=1e-12):
        bad.append("s term")
    # t only: y[b][o] = sum_i t_i sum_l (column l of Z_i summed) x_b[l], the same for every o
    got = _forward_with(weight_fn, X, Y, Z, zero, zero, t, _f16(0))
    want = np.zeros((3, n))
    for b in range(3):
        val = sum(float(t[i]) * sum(int(Z[i, :, l].sum()) * Xf[b, l] for l in range(m)) for i in range(p))
        want[b, :] = val
    if not np.allclose(got, want, rtol=1e-12, atol=1e-12):
        bad.append("t term")
    # u only: y[b][o] = u (sum of x_b)
    got = _forward_with(weight_fn, X, Y, Z, zero, zero, zero, _f16(1.5))
    if not np.allclose(got, 1.5 * Xf.sum(axis=1, keepdims=True) * np.ones((1, n)), rtol=1e-12, atol=1e-12):
        bad.append("u term")

    # 0/1 -> ±1: with A = 1 - 2 Y and B = 1 - 2 Z (entries ±1),
    #   A B = d 1 - 2 (1_Y Z) - 2 (Y 1_Z) + 4 Y Z,
    # so the terms r = 4 rho, s = t = -2 rho, u = d rho sum to rho A B: the DBF
    # weight with a = 1, mid = rho, b = 1 (one DBF product per term).
    p, n, d, m = 2, 7, 6, 5
    rng = np.random.default_rng(31)
    Y = rng.integers(0, 2, size=(p, n, d), dtype=np.uint8)
    Z = rng.integers(0, 2, size=(p, d, m), dtype=np.uint8)
    rho = np.array([0.5, -0.25])
    X = _f16(rng.uniform(-3, 3, size=(4, m)))
    got = _forward_with(weight_fn, X, Y, Z, _f16(4 * rho), _f16(-2 * rho), _f16(-2 * rho), _f16(d * rho.sum()))
    want = np.zeros((4, n))
    for i in range(p):
        A = (1 - 2 * Y[i].astype(np.int8)).astype(np.int8)
        B = (1 - 2 * Z[i].astype(np.int8)).astype(np.int8)
        want += O.dense_forward(X, A, B, np.ones(n, np.float16), _f16(np.full(d, rho[i])), np.ones(m, np.float16))
    if not np.allclose(got, want, rtol=1e-12, atol=1e-12):
        bad.append("±1 identity")
    return bad


def test_oracle_meets_every_pin():
    assert _pin_failures(Q.bqq_weight) == []


def _mutant(kind):
    def weight(Y, Z, r, s, t, u):
        Y = np.asarray(Y, dtype=np.float64)
        Z = np.asarray(Z, dtype=np.float64)
        p, n, d = Y.shape
        m = Z.shape[2]
        W = float(u) * np.ones((n, m))
        if kind == "no_u":
            W[:] = 0
        for i in range(p):
            ri, si, ti = float(r[i]), float(s[i]), float(t[i])
            yz = Y[i] @ Z[i]
            y1 = Y[i] @ np.ones((d, m))
            z1 = np.ones((n, d)) @ Z[i]
            if kind == "s_t_swapped":
                si, ti = ti, si
            if kind == "s_sign":
                si = -si
            if kind == "drop_t":
                ti = 0.0
            if kind == "first_term_only" and i > 0:
                continue
            W += ri * yz + si * y1 + ti * z1
        return W
    return weight


@pytest.mark.parametrize("kind", ["no_u", "s_t_swapped", "s_sign", "drop_t", "first_term_only"])
def test_pins_catch_plausible_mistakes(kind):
    assert _pin_failures(_mutant(kind)) != [], f"mutant {kind} passed every pin"


def test_integer_layer_values_are_exact_in_fp64():
    """The integer layers of the GPU tests: fp64 forward equals the rational
    brute force exactly on a slice small enough to enumerate."""
    L = inputs.bqq_layer("i", 6, 9, 5, 2, 3, (2,), integer=True)
    X = L.X[2]
    got = Q.bqq_forward(X, L.Y, L.Z, L.r, L.s, L.t, L.u)
    want = np.array([[float(v) for v in row] for row in Q.brute_force(X, L.Y, L.Z, L.r, L.s, L.t, L.u)])
    assert np.array_equal(got, want)


def test_synthetic_layer_is_centred():
    """With zero jitter the generator's scalars make every term a ±1 product
    (the identity above), so W has zero-mean entries of size about sigma."""
    L = inputs.bqq_layer("c", 64, 96, 128, 2, 5, (1,), sigma=0.02, jitter=0.0)
    W = Q.bqq_weight(L.Y, L.Z, L.r, L.s, L.t, L.u)
    assert abs(W.mean()) < 0.1 * W.std()
    assert 0.005 < W.std() < 0.08


# --------------------------------------------------------------------------- group-wise scaling

def _random_grouped(seed, p, n, d, m, group, batch):
    rng = np.random.default_rng(seed)
    ng = -(-m // group)
    Y = rng.integers(0, 2, size=(p, n, d), dtype=np.uint8)
    Z = rng.integers(0, 2, size=(p, d, m), dtype=np.uint8)
    r, s, t = (_f16(rng.uniform(-2, 2, size=(p, ng))) for _ in range(3))
    u = _f16(rng.uniform(-2, 2, size=ng))
    X = _f16(rng.uniform(-3, 3, size=(batch, m)))
    return X, Y, Z, r, s, t, u


def _grouped_pin_failures(weight_fn):
    """Run every pin of the group-wise form with `weight_fn(Y, Z, r, s, t, u,
    group)` as the weight builder; return the names of the pins that fail."""
    bad = []

    def fwd(X, Y, Z, r, s, t, u, g):
        return np.asarray(X, dtype=np.float64) @ weight_fn(Y, Z, r, s, t, u, g).T

    # exact rational brute force; ragged last groups (m not a multiple of group)
    for seed, (p, n, d, m, g) in enumerate([(1, 3, 3, 4, 2), (2, 4, 3, 5, 2), (2, 3, 4, 7, 3), (3, 2, 2, 5, 4)]):
        X, Y, Z, r, s, t, u = _random_grouped(100 + seed, p, n, d, m, g, 2)
        want = np.array([[float(v) for v in row] for row in Q.brute_force_grouped(X, Y, Z, r, s, t, u, g)])
        if not np.allclose(fwd(X, Y, Z, r, s, t, u, g), want, rtol=1e-12, atol=1e-12):
            bad.append(f"grouped brute force {seed}")

    # hand-worked, two groups of two columns, p = 1:
    #   Y = [[1,0],[1,1]], Z = [[0,1,1,0],[1,1,0,1]]
    #   Y Z = [[0,1,1,0],[1,2,1,1]], rows of Y summed [1, 2], columns of Z summed [1, 2, 1, 1]
    #   group 0 (columns 0, 1): r = 2, s = 1, t = -1, u = 0.5
    #   group 1 (columns 2, 3): r = -1, s = 0.5, t = 2, u = -1
    #   W = [[0.5, 1.5, 0.5, 1.5], [3.5, 4.5, 1.0, 1.0]];  x = [1, -2, 2, 1] -> y = [0, -2.5]
    Y = np.array([[[1, 0], [1, 1]]], dtype=np.uint8)
    Z = np.array([[[0, 1, 1, 0], [1, 1, 0, 1]]], dtype=np.uint8)
    r, s, t = _f16([[2.0, -1.0]]), _f16([[1.0, 0.5]]), _f16([[-1.0, 2.0]])
    u = _f16([0.5, -1.0])
    if not np.array_equal(weight_fn(Y, Z, r, s, t, u, 2), np.array([[0.5, 1.5, 0.5, 1.5], [3.5, 4.5, 1.0, 1.0]])):
        bad.append("grouped hand-worked W")
    if not np.array_equal(fwd(_f16([[1.0, -2.0, 2.0, 1.0]]), Y, Z, r, s, t, u, 2), np.array([[0.0, -2.5]])):
        bad.append("grouped hand-worked y")

    # the layer is the sum over column blocks of single-group layers, each
    # on its block of the input (single-group form: pinned above)
    p, n, d, m, g = 2, 5, 6, 11, 4
    X, Y, Z, r, s, t, u = _random_grouped(7, p, n, d, m, g, 3)
    want = np.zeros((3, n))
    for h, c0 in enumerate(range(0, m, g)):
        c1 = min(m, c0 + g)
        want += Q.bqq_forward(X[:, c0:c1], Y, Z[:, :, c0:c1], r[:, h], s[:, h], t[:, h], u[h])
    if not np.allclose(fwd(X, Y, Z, r, s, t, u, g), want, rtol=1e-12, atol=1e-12):
        bad.append("sum of column blocks")

    # the same scalars in every group: the single-group form
    X, Y, Z, r, s, t, u = _random_case(8, 2, 4, 5, 9, 2)
    rg, sg, tg = (np.repeat(v[:, None], 3, axis=1) for v in (r, s, t))
    if not np.allclose(fwd(X, Y, Z, rg, sg, tg, np.repeat(u, 3), 4), Q.bqq_forward(X, Y, Z, r, s, t, u),
                       rtol=1e-12, atol=1e-12):
        bad.append("equal groups")
    return bad


def test_grouped_oracle_meets_every_pin():
    assert _grouped_pin_failures(Q.bqq_weight_grouped) == []


def test_group_columns():
    assert Q.group_columns(10, 4) == [(0, 4), (4, 8), (8, 10)]
    assert Q.group_columns(8, 8) == [(0, 8)]
    assert Q.group_columns(3, 5) == [(0, 3)]


def _grouped_mutant(kind):
    def weight(Y, Z, r, s, t, u, group):
        Y = np.asarray(Y, dtype=np.float64)
        Z = np.asarray(Z, dtype=np.float64)
        p, n, d = Y.shape
        m = Z.shape[2]
        W = np.zeros((n, m))
        for l in range(m):
            h = l // group
            if kind == "group_off_by_one":
                h = min((l + 1) // group, r.shape[1] - 1)
            hs = 0 if kind == "s_first_group" else h
            W[:, l] = float(u[h])
            for i in range(p):
                ri = float(r[i, h])
                if kind == "r_by_row":
                    ri = float(r[i, min(i, r.shape[1] - 1)])
                W[:, l] += ri * (Y[i] @ Z[i][:, l]) + float(s[i, hs]) * Y[i].sum(axis=1) + float(t[i, h]) * Z[i][:, l].sum()
        return W
    return weight


@pytest.mark.parametrize("kind", ["group_off_by_one", "s_first_group", "r_by_row"])
def test_grouped_pins_catch_plausible_mistakes(kind):
    assert _grouped_pin_failures(_grouped_mutant(kind)) != [], f"mutant {kind} passed every pin"


def test_grouped_mutant_control():
    """The mutant builder with no mutation meets every pin (so the pins test
    the mutations, not the builder)."""
    assert _grouped_pin_failures(_grouped_mutant("none")) == []


def test_grouped_synthetic_layer_is_centred_per_group():
    """With zero jitter every group's columns are ±1 products scaled by that
    group's rho: zero-mean entries of size about sigma in each group."""
    L = inputs.bqq_grouped_layer("g", 64, 96, 128, 2, 32, 5, (1,), sigma=0.02, jitter=0.0)
    W = Q.bqq_weight_grouped(L.Y, L.Z, L.r, L.s, L.t, L.u, L.group)
    for c0, c1 in Q.group_columns(L.m, L.group):
        Wg = W[:, c0:c1]
        assert abs(Wg.mean()) < 0.15 * Wg.std()
        assert 0.005 < Wg.std() < 0.08


def test_grouped_integer_layer_values_are_exact_in_fp64():
    L = inputs.bqq_grouped_layer("gi", 5, 11, 4, 2, 4, 9, (2,), integer=True)
    X = L.X[2]
    got = Q.bqq_forward_grouped(X, L.Y, L.Z, L.r, L.s, L.t, L.u, L.group)
    want = np.array([[float(v) for v in row] for row in Q.brute_force_grouped(X, L.Y, L.Z, L.r, L.s, L.t, L.u,
                                                                              L.group)])
    assert np.array_equal(got, want)
