"""Seeded synthetic inputs for the DBF linear forward.

This module is the only piece shared by the oracle side and the GPU side of
the tests and the bench.  It holds data generation only -- no step of the
DBF computation -- so that neither side can lean on the other's arithmetic.

The layer shapes follow the projections of a Llama-3-8B decoder block (the
models the DBF paper evaluates on, per the experiments section of the
gist.science technical summary of "Addition is almost all you need").  No
trained weights are used: signs are i.i.d. uniform +/-1 and the scales are
half-normal, so the inputs have the shapes and value ranges of the paper's
workloads but not their values.

Draw order inside one layer, with one ``numpy.random.Generator(PCG64)``:
A bits (n x k), B bits (k x m), a, mid, b, then X for each listed batch
size in order.  Signs are ``1 - 2 * integers(0, 2)``; scales are
``|standard_normal| * sigma`` rounded to fp16; X is ``standard_normal``
rounded to fp16.
"""

from __future__ import annotations

import dataclasses
import functools
import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

__all__ = [
    "Layer",
    "Config",
    "config",
    "CONFIG_IDS",
    "random_layer",
    "integer_layer",
    "random_x",
    "integer_x",
    "C5_LAYERS",
    "tiny_case",
    "BqqLayer",
    "bqq_layer",
]


@dataclasses.dataclass
class Layer:
    name: str
    n: int                      # output features
    m: int                      # input features
    k: int                      # middle dimension
    A: np.ndarray               # int8 (n, k), entries +/-1
    B: np.ndarray               # int8 (k, m), entries +/-1
    a: np.ndarray               # float16 (n,)
    mid: np.ndarray             # float16 (k,)
    b: np.ndarray               # float16 (m,)
    X: Dict[int, np.ndarray]    # batch -> float16 (batch, m)

    @property
    def sign_bytes(self) -> int:
        """Bytes of the signs at one bit each: (n*k + k*m) / 8."""
        return (self.n * self.k + self.k * self.m) // 8

    @property
    def scale_bytes(self) -> int:
        return 2 * (self.n + self.k + self.m)


@dataclasses.dataclass
class Config:
    cid: int
    description: str
    layers: List[Layer]
    batches: Tuple[int, ...]


def _signs(rng: np.random.Generator, shape) -> np.ndarray:
    bits = rng.integers(0, 2, size=shape, dtype=np.int8)
    return (1 - 2 * bits).astype(np.int8)


def _halfnormal16(rng: np.random.Generator, size: int, sigma: float) -> np.ndarray:
    return (np.abs(rng.standard_normal(size)) * sigma).astype(np.float16)


def random_x(rng: np.random.Generator, batch: int, m: int) -> np.ndarray:
    return rng.standard_normal((batch, m)).astype(np.float16)


def random_layer(name: str, n: int, m: int, k: int, seed, sig_a: float, sig_mid: float,
                 sig_b: float, batches: Sequence[int]) -> Layer:
    """One layer with the draw order stated in the module docstring.

    ``seed`` is an int or a ``numpy.random.SeedSequence``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    A = _signs(rng, (n, k))
    B = _signs(rng, (k, m))
    a = _halfnormal16(rng, n, sig_a)
    mid = _halfnormal16(rng, k, sig_mid)
    b = _halfnormal16(rng, m, sig_b)
    X = {bt: random_x(rng, bt, m) for bt in batches}
    return Layer(name, n, m, k, A, B, a, mid, b, X)


def integer_x(rng: np.random.Generator, batch: int, m: int,
              values: Sequence[float] = (-1.0, 0.0, 1.0)) -> np.ndarray:
    return rng.choice(np.asarray(values, dtype=np.float64), size=(batch, m)).astype(np.float16)


def integer_layer(name: str, n: int, m: int, k: int, seed, batches: Sequence[int],
                  a_vals=(1.0,), mid_vals=(1.0, 2.0), b_vals=(1.0, 2.0),
                  x_vals=(-1.0, 0.0, 1.0)) -> Layer:
    """A layer whose activations and scales are small integers (or powers of two).

    With such values every partial sum of either signed sum is an integer
    well inside fp32's exact range, so any summation order gives the same
    exact value; the tests check the realized ranges before relying on it.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    A = _signs(rng, (n, k))
    B = _signs(rng, (k, m))
    a = rng.choice(np.asarray(a_vals), size=n).astype(np.float16)
    mid = rng.choice(np.asarray(mid_vals), size=k).astype(np.float16)
    b = rng.choice(np.asarray(b_vals), size=m).astype(np.float16)
    X = {bt: integer_x(rng, bt, m, x_vals) for bt in batches}
    return Layer(name, n, m, k, A, B, a, mid, b, X)


def tiny_case(seed: int, n: int, m: int, k: int, batch: int, signed_scales: bool = True):
    """Small random case with signed (or non-negative) fp16 scales.

    Returns (X, A, B, a, mid, b).  Scales are uniform in [-2, 2) (or [0, 2)),
    X uniform in [-4, 4), all rounded to fp16.
    """
    rng = np.random.default_rng(seed)
    A = (1 - 2 * rng.integers(0, 2, size=(n, k))).astype(np.int8)
    B = (1 - 2 * rng.integers(0, 2, size=(k, m))).astype(np.int8)
    lo = -2.0 if signed_scales else 0.0
    a = rng.uniform(lo, 2.0, size=n).astype(np.float16)
    mid = rng.uniform(lo, 2.0, size=k).astype(np.float16)
    b = rng.uniform(lo, 2.0, size=m).astype(np.float16)
    X = rng.uniform(-4.0, 4.0, size=(batch, m)).astype(np.float16)
    return X, A, B, a, mid, b


# Llama-3-8B decoder-block projections: (name, n = out, m = in).
C5_LAYERS = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 14336, 4096),
    ("up", 14336, 4096),
    ("down", 4096, 14336),
)


def c5_middle_dims(seed: int = 4) -> List[int]:
    """Per-layer middle dimension for the decoder-block workload.

    For each layer in the order q, k, v, o, gate, up, down, a target
    bits-per-weight beta ~ U[1.0, 2.3] is drawn from one generator, and
    k = 64 * ceil(beta * n * m / (n + m) / 64): the signs then take about
    beta bits per weight.  This stands in for the paper's layer-budget search,
    which needs a trained model.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ks = []
    for _, n, m in C5_LAYERS:
        beta = rng.uniform(1.0, 2.3)
        ks.append(64 * math.ceil(beta * n * m / (n + m) / 64))
    return ks


CONFIG_IDS = (1, 2, 3, 4, 5)


@functools.lru_cache(maxsize=2)
def config(cid: int) -> Config:
    """The five workloads, numbered 1..5 (1 = the small correctness case)."""
    if cid == 1:
        L = random_layer("c1", 256, 256, 128, 0, 0.05, 0.05, 0.05, (1,))
        return Config(1, "single layer 256x256, k=128", [L], (1,))
    if cid == 2:
        L = random_layer("c2", 4096, 4096, 2048, 1, 0.02, 1.0, 0.02, (1, 16))
        return Config(2, "4096x4096 projection, k=2048 (~1 bit/weight)", [L], (1, 16))
    if cid == 3:
        L = random_layer("c3", 4096, 4096, 4096, 2, 0.02, 1.0, 0.02, (1, 16, 2048))
        return Config(3, "4096x4096 projection, k=4096 (~2 bits/weight)", [L], (1, 16, 2048))
    if cid == 4:
        ss = np.random.SeedSequence(3).spawn(2)
        up = random_layer("up", 14336, 4096, 4800, ss[0], 0.02, 0.02, 0.02, (1, 2048))
        down = random_layer("down", 4096, 14336, 4800, ss[1], 0.02, 0.02, 0.02, (1, 2048))
        return Config(4, "MLP up 14336x4096 and down 4096x14336, k=4800", [up, down], (1, 2048))
    if cid == 5:
        ks = c5_middle_dims(4)
        ss = np.random.SeedSequence(4).spawn(len(C5_LAYERS))
        layers = [random_layer(name, n, m, k, ss[i], 0.02, 1.0, 0.02, (1, 2048))
                  for i, ((name, n, m), k) in enumerate(zip(C5_LAYERS, ks))]
        return Config(5, "Llama-3-8B-shaped block of 7 DBF linears, per-layer k", layers, (1, 2048))
    raise ValueError(f"unknown config {cid}")


# --------------------------------------------------------------------------- binary-quadratic (BQQ-form) layers

@dataclasses.dataclass
class BqqLayer:
    name: str
    n: int                      # output features
    m: int                      # input features
    d: int                      # inner dimension of each binary product
    p: int                      # number of binary products
    Y: np.ndarray               # uint8 (p, n, d), entries 0/1
    Z: np.ndarray               # uint8 (p, d, m), entries 0/1
    r: np.ndarray               # float16 (p,)
    s: np.ndarray               # float16 (p,)
    t: np.ndarray               # float16 (p,)
    u: np.float16
    X: Dict[int, np.ndarray]    # batch -> float16 (batch, m)

    @property
    def bit_bytes(self) -> int:
        return self.p * self.d * (self.n + self.m) // 8


def bqq_layer(name: str, n: int, m: int, d: int, p: int, seed, batches: Sequence[int],
              sigma: float = 0.02, jitter: float = 0.05, integer: bool = False) -> BqqLayer:
    """A seeded BQQ-form layer.

    Draw order with one ``Generator(PCG64(seed))``: Y bits (p, n, d), Z bits
    (p, d, m), then per term rho_i ~ U[0.5, 1.5] * sigma / sqrt(d) and the
    jitters e_s, e_t (p each) and e_u ~ U[-jitter, jitter], then X per batch.
    The scalars are r = 4 rho, s = -2 rho (1 + e_s), t = -2 rho (1 + e_t),
    u = d * sum(rho) * (1 + e_u), rounded to fp16: with zero jitter a term is
    rho times a product of two +/-1 matrices (centred entries of size
    sigma, like trained weights); the jitter keeps every term of the formula
    in play.  ``integer=True`` instead draws r, s, t from {-2, -1, 1, 2}, u
    from {-4, ..., 4} and X from {-1, 0, 1}, so every partial sum is a small
    integer (exact in fp32 in any order).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    Y = rng.integers(0, 2, size=(p, n, d), dtype=np.uint8)
    Z = rng.integers(0, 2, size=(p, d, m), dtype=np.uint8)
    if integer:
        r = rng.choice([-2.0, -1.0, 1.0, 2.0], size=p).astype(np.float16)
        s = rng.choice([-2.0, -1.0, 1.0, 2.0], size=p).astype(np.float16)
        t = rng.choice([-2.0, -1.0, 1.0, 2.0], size=p).astype(np.float16)
        u = np.float16(rng.integers(-4, 5))
        X = {bt: integer_x(rng, bt, m) for bt in batches}
    else:
        rho = rng.uniform(0.5, 1.5, size=p) * sigma / math.sqrt(d)
        e_s = rng.uniform(-jitter, jitter, size=p)
        e_t = rng.uniform(-jitter, jitter, size=p)
        e_u = rng.uniform(-jitter, jitter)
        r = (4.0 * rho).astype(np.float16)
        s = (-2.0 * rho * (1.0 + e_s)).astype(np.float16)
        t = (-2.0 * rho * (1.0 + e_t)).astype(np.float16)
        u = np.float16(d * rho.sum() * (1.0 + e_u))
        X = {bt: random_x(rng, bt, m) for bt in batches}
    return BqqLayer(name, n, m, d, p, Y, Z, r, s, t, u, X)


@dataclasses.dataclass
class BqqGroupedLayer:
    name: str
    n: int                      # output features
    m: int                      # input features
    d: int                      # inner dimension of each binary product
    p: int                      # number of binary products
    group: int                  # input columns per scaling group (the last may be shorter)
    Y: np.ndarray               # uint8 (p, n, d), entries 0/1
    Z: np.ndarray               # uint8 (p, d, m), entries 0/1
    r: np.ndarray               # float16 (p, ngroups)
    s: np.ndarray               # float16 (p, ngroups)
    t: np.ndarray               # float16 (p, ngroups)
    u: np.ndarray               # float16 (ngroups,)
    X: Dict[int, np.ndarray]    # batch -> float16 (batch, m)

    @property
    def ngroups(self) -> int:
        return -(-self.m // self.group)

    @property
    def bit_bytes(self) -> int:
        return self.p * self.d * (self.n + self.m) // 8


def bqq_grouped_layer(name: str, n: int, m: int, d: int, p: int, group: int, seed, batches: Sequence[int],
                      sigma: float = 0.02, jitter: float = 0.05, integer: bool = False) -> BqqGroupedLayer:
    """A seeded BQQ-form layer with group-wise scalars (ngroups = ceil(m /
    group) groups of input columns).

    Draw order with one ``Generator(PCG64(seed))``: Y bits (p, n, d), Z bits
    (p, d, m), then rho ~ U[0.5, 1.5] * sigma / sqrt(d) of shape (p,
    ngroups), the jitters e_s, e_t (p, ngroups) and e_u (ngroups,) ~
    U[-jitter, jitter], then X per batch.  Per group the scalars follow
    ``bqq_layer``: r = 4 rho, s = -2 rho (1 + e_s), t = -2 rho (1 + e_t),
    u = d * sum_i rho (1 + e_u), rounded to fp16, so each group's columns are
    centred with entries of size sigma.  ``integer=True`` draws r, s, t from
    {-2, -1, 1, 2}, u from {-4, ..., 4} and X from {-1, 0, 1}.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ng = -(-m // group)
    Y = rng.integers(0, 2, size=(p, n, d), dtype=np.uint8)
    Z = rng.integers(0, 2, size=(p, d, m), dtype=np.uint8)
    if integer:
        r = rng.choice([-2.0, -1.0, 1.0, 2.0], size=(p, ng)).astype(np.float16)
        s = rng.choice([-2.0, -1.0, 1.0, 2.0], size=(p, ng)).astype(np.float16)
        t = rng.choice([-2.0, -1.0, 1.0, 2.0], size=(p, ng)).astype(np.float16)
        u = rng.integers(-4, 5, size=ng).astype(np.float16)
        X = {bt: integer_x(rng, bt, m) for bt in batches}
    else:
        rho = rng.uniform(0.5, 1.5, size=(p, ng)) * sigma / math.sqrt(d)
        e_s = rng.uniform(-jitter, jitter, size=(p, ng))
        e_t = rng.uniform(-jitter, jitter, size=(p, ng))
        e_u = rng.uniform(-jitter, jitter, size=ng)
        r = (4.0 * rho).astype(np.float16)
        s = (-2.0 * rho * (1.0 + e_s)).astype(np.float16)
        t = (-2.0 * rho * (1.0 + e_t)).astype(np.float16)
        u = (d * rho.sum(axis=0) * (1.0 + e_u)).astype(np.float16)
        X = {bt: random_x(rng, bt, m) for bt in batches}
    return BqqGroupedLayer(name, n, m, d, p, group, Y, Z, r, s, t, u, X)
