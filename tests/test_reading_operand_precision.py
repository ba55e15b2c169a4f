"""Evidence for the choice of 16-bit operand type on the matrix-core path.

The pages state the activations and scales in fp16 and say nothing about the
operand type of the products.  The matrix cores take both operands in one
16-bit type, so the prefill path must round its activation operand (X, and
T = t ⊙ mid between the two products) and its scaled sign operand (±b) to
that type.  This test simulates the two candidates in numpy on a layer drawn
like the 4096-wide workloads (a, b ~ |N(0,1)|·0.02, mid ~ |N(0,1)|,
x ~ N(0,1)) and measures the per-row ∞-norm relative error against the fp64
oracle:

* fp16 operands: X and ±b are exact; T is rounded once to fp16;
* bf16 operands: X, ±b and T are each rounded to bf16 (8 significant bits).

fp16 stays well inside the 2e-3 bound and bf16 does not, which is why the
kernels use f16 x f16 -> f32 products.  Accumulation is simulated in fp64
(fp32 accumulation adds errors near 1e-6 here, far below either figure).
"""

import numpy as np

from oracle import dbf_oracle as O
from tests import inputs

TOL = 2e-3


def _bf16(v):
    """Round float64 values to bf16 (round to nearest, ties to even) and back:
    to fp32 first (exact for the fp16-derived and product values here up to
    fp32 rounding), then the upper 16 bits with the carry of the lower 16."""
    f = np.asarray(v, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _rel_rows(y, ref):
    return (np.abs(y - ref).max(axis=1) / np.abs(ref).max(axis=1)).max()


def _simulate(X, A, B, a, mid, b, rnd):
    """y = rne16(a ⊙ (rnd(t ⊙ mid) Aᵀ)) with t = rnd(X) (B ⊙ rnd(b))ᵀ."""
    X64, A64, B64 = (np.asarray(v, dtype=np.float64) for v in (X, A, B))
    a64, mid64, b64 = (np.asarray(v).astype(np.float64) for v in (a, mid, b))
    t = rnd(X64) @ (B64 * rnd(b64)[None, :]).T
    T = rnd(t * mid64[None, :])
    return O.rne_fp16(a64[None, :] * (T @ A64.T)).astype(np.float64)


def test_fp16_operands_meet_the_bound_and_bf16_do_not():
    n, m, k, batch = 512, 1024, 512, 16
    L = inputs.random_layer("p", n, m, k, 12, 0.02, 1.0, 0.02, (batch,))
    X = L.X[batch]
    ref = O.dense_forward(X, L.A, L.B, L.a, L.mid, L.b)
    fp16 = _simulate(X, L.A, L.B, L.a, L.mid, L.b, lambda v: np.asarray(v, dtype=np.float64).astype(np.float16))
    bf16 = _simulate(X, L.A, L.B, L.a, L.mid, L.b, _bf16)
    e16, eb = _rel_rows(fp16, ref), _rel_rows(bf16, ref)
    print(f"worst row rel err: fp16 operands {e16:.2e}, bf16 operands {eb:.2e}")
    assert e16 < 0.5 * TOL
    assert eb > TOL


def test_bf16_rounding_helper():
    """The helper against values whose bf16 rounding is known by hand."""
    got = _bf16([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -3.0, 1.0 + 2.0 ** -7])
    want = [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0, -3.0, 1.0 + 2.0 ** -7]
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to the even 1.0;
    # 1 + 3·2^-8 is the midpoint of 1 + 2^-7 and 1 + 2^-6: ties to the even 1 + 2^-6
    assert np.array_equal(got, want)
