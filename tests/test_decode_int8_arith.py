"""Host model of the batch-1 decode arithmetic (CPU only).

The batch-1 kernels (decode_i8.hip) compute each stage's signed sum
s_r = Σ_l sign_rl u_l as an exact integer sum of a fixed-point vector on the
int8 matrix cores: q_l = rne(u_l 2^S) as four balanced base-256 digits in the
product's columns, the sign words of dbf_layout_signs_dec AND 0x01010101 << j
as the int8 operand (values 0 or 2^j, -128 for j = 7), one accumulator per j,
folded as Z_c = Σ_j ±acc_j >> j, Z = Σ_c Z_c 256^c, s = U - 2 Z with
U = Σ_l q_l.  This test runs those steps in numpy on the library's own layout
(an int8 product is a plain integer matrix product) and checks them against
the fp64 oracle: the stage results equal the exact signed sums of the
quantized vector, and the two-stage result is within the parity tolerance.
It pins the arithmetic the kernels implement, not the kernels.
"""

import numpy as np
import pytest

import dbf_linear_fwd_amd as dbf
from oracle import dbf_oracle as O
from tests import inputs


def quantize(u: np.ndarray):
    """q = rne(u 2^S) with 2^29 <= max |u 2^S| < 2^30 (S = 0 for a zero vector)."""
    mx = float(np.abs(u).max()) if u.size else 0.0
    if mx == 0.0:
        return np.zeros(u.shape, np.int64), 0
    _, E = np.frexp(mx)
    S = 30 - int(E)
    return np.rint(np.ldexp(u.astype(np.float64), S)).astype(np.int64), S


def digits(q: np.ndarray) -> np.ndarray:
    """Balanced base-256 digits d0..d3 in [-128, 127] with q = Σ d_c 256^c."""
    e = ((q.astype(np.int64) + 0x808080) & 0xFFFFFFFF) ^ 0x808080
    d = np.stack([(e >> (8 * c)) & 0xFF for c in range(4)], axis=-1).astype(np.int64)
    return np.where(d >= 128, d - 256, d)


def stage_model(S_signs: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Signed sums s = S_signs @ u the kernel's way, as exact float results s 2^-S."""
    rows, K = S_signs.shape
    rows_pad, cols_pad = -(-rows // 16) * 16, -(-K // 128) * 128
    lay = dbf.dbf_layout_signs_dec(dbf.dbf_pack_signs(S_signs), K, rows_pad, cols_pad).astype(np.uint64)
    q, S = quantize(u)
    assert np.abs(q).max(initial=0) < 2 ** 30
    qp = np.zeros(cols_pad, np.int64)
    qp[:K] = q
    dg = digits(qp)                                   # [K, 4]
    assert np.array_equal((dg * (256 ** np.arange(4))).sum(axis=1), qp)
    U = int(qp.sum())
    nsc = -(-cols_pad // 512)
    out = np.zeros(rows_pad)
    for T in range(rows_pad // 16):
        acc = np.zeros((8, 16, 4), np.int64)          # [j][row][digit column]
        for s in range(nsc):
            W = 4 if s + 1 < nsc else (cols_pad - 512 * s) // 128
            base = T * cols_pad // 2 + 256 * s
            for j in range(8):
                A = np.zeros((16, 64), np.int64)      # rows x (g, i, b)
                B = np.zeros((64, 4), np.int64)
                for g in range(4):
                    for i in range(4):
                        for b in range(4):
                            kk = g * 16 + i * 4 + b
                            col = 512 * s + 128 * i + 16 * j + 4 * g + b
                            B[kk] = dg[col] if col < cols_pad else 0
                            if i < W:
                                words = lay[base + W * (np.arange(16) + 16 * g) + i]
                                byte = (words >> np.uint64(8 * b)) & np.uint64(0xFF)
                                v = (byte & np.uint64(1 << j)).astype(np.int64)
                                A[:, kk] = np.where(v >= 128, v - 256, v)   # int8
                acc[j] += A @ B
        Zc = np.zeros((16, 4), np.int64)
        for j in range(8):
            assert np.all(acc[j] % (1 << j) == 0)
            Zc += (acc[j] >> j) * (-1 if j == 7 else 1)
        Z = (Zc * (256 ** np.arange(4))).sum(axis=1)
        out[16 * T:16 * T + 16] = np.ldexp((U - 2 * Z).astype(np.float64), -S)
    return out[:rows], q, S


@pytest.mark.parametrize("rows,K", [(16, 128), (20, 300), (33, 700), (48, 1408), (7, 1030)])
def test_stage_is_exact_signed_sum_of_quantized_vector(rows, K):
    rng = np.random.default_rng(rows + K)
    Sg = (1 - 2 * rng.integers(0, 2, size=(rows, K))).astype(np.int8)
    u = (rng.standard_normal(K) * 3).astype(np.float32).astype(np.float64)
    got, q, S = stage_model(Sg, u)
    exact = (Sg.astype(np.int64) @ q).astype(np.float64) * 2.0 ** -S
    assert np.array_equal(got, exact)
    # and close to the unquantized sum: |error| <= K * 2^-(S+1)
    assert np.abs(got - Sg.astype(np.float64) @ u).max() <= K * 2.0 ** -(S + 1)


def test_two_stage_model_matches_oracle():
    L = inputs.random_layer("m", 40, 300, 200, 11, 0.05, 1.0, 0.05, (1,))
    x = L.X[1][0].astype(np.float64)
    u = (x * L.b.astype(np.float64)).astype(np.float32).astype(np.float64)   # exact in fp32
    t, _, _ = stage_model(L.B, u)
    v = (t * L.mid.astype(np.float64)).astype(np.float32).astype(np.float64)
    s, _, _ = stage_model(L.A, v)
    y = O.rne_fp16(s * L.a.astype(np.float64))
    ref = O.dense_forward(L.X[1], L.A, L.B, L.a, L.mid, L.b)[0]
    err = np.abs(y.astype(np.float64) - ref).max() / np.abs(ref).max()
    assert err <= 2e-3, err


def test_integer_inputs_are_exact():
    L = inputs.integer_layer("i", 50, 260, 130, 5, (1,), a_vals=(1.0,), mid_vals=(1.0, 2.0), b_vals=(1.0, 2.0))
    x = L.X[1][0].astype(np.float64)
    t, _, _ = stage_model(L.B, x * L.b.astype(np.float64))
    s, _, _ = stage_model(L.A, t * L.mid.astype(np.float64))
    y = O.rne_fp16(s * L.a.astype(np.float64))
    ref = O.rne_fp16(O.dense_forward(L.X[1], L.A, L.B, L.a, L.mid, L.b)[0])
    assert np.array_equal(y.view(np.uint16), ref.view(np.uint16))
