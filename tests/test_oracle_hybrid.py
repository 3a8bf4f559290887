"""Pins of the oracle's HYBRID_SHARD two-level reduce and of rounding the
collectives' outputs to the reduce dtype (CPU only).

The pages ("Building GPT from Scratch -- Part 8: FSDP", sections "Sharding
Strategies" and "HYBRID_SHARD: The Multi-Node Strategy") shard within a node
and all-reduce across nodes; they print no arithmetic for it. Pinned here by
the special case that reduces to the flat reduce, exact integer arithmetic
(with an integer round-to-nearest-even written independently of the
oracle's bit-pattern rounding), hand-worked fp32 and bf16 cases whose
answers follow from the IEEE formats, and summation error bounds.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import zs_oracle as O


def to_bf16_bits(x):
    """torch's cast, an independent route to bf16 bits."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rne_int(n: int, bits: int) -> int:
    """Integer n rounded to `bits` significant bits, ties to even."""
    if n == 0:
        return 0
    a = abs(n)
    k = max(0, a.bit_length() - bits)
    q, r = divmod(a, 1 << k)
    half = 1 << k >> 1 if k else 0
    if k and (r > half or (r == half and q & 1)):
        q += 1
    return (q << k) * (1 if n > 0 else -1)


def test_rne_int_itself():
    assert rne_int(257, 8) == 256          # halfway between 256 and 258: 256 has the even quotient
    assert rne_int(259, 8) == 260          # tie between 258 and 260: 260 has the even quotient
    assert rne_int(258, 8) == 258
    assert rne_int(-771, 8) == -772        # 771 = 192.75 * 4: rounds up to 193 * 4
    assert rne_int(255, 8) == 255


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32])
def test_one_replica_without_rounding_is_the_flat_reduce(dtype):
    rng = np.random.default_rng(3)
    for D in (1, 2, 5, 8):
        x = rng.standard_normal((D, 999)).astype(np.float32) * 1e-3
        cs = [to_bf16_bits(r) for r in x] if dtype == O.BF16 else list(x)
        a = O.reduce_shard_hybrid(cs, dtype, 1, False)
        b = O.reduce_shard(cs, dtype)
        assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("R,D", [(1, 1), (1, 8), (2, 1), (2, 4), (4, 8), (8, 2)])
@pytest.mark.parametrize("rnd", [False, True])
def test_exact_small_integers(R, D, rnd):
    """Every partial sum stays a bf16-exact integer: no rounding anywhere."""
    rng = np.random.default_rng(R * 100 + D)
    ints = rng.integers(-3, 4, size=(R * D, 501))
    cs = [to_bf16_bits(r) for r in ints]
    g = O.reduce_shard_hybrid(cs, O.BF16, R, rnd)
    want = [Fraction(int(s), R * D) for s in ints.sum(axis=0)]
    assert all(Fraction(float(a)) == b for a, b in zip(g, want))


@pytest.mark.parametrize("R,D", [(2, 4), (4, 8), (3, 2)])
def test_rounded_integer_sums(R, D):
    """bf16 integers whose node sums need more than 8 significant bits: each
    node sum is rounded to 8 bits, then the total, then scaled (R*D is a
    power of two, or 6 for which the scale is applied as float32(1/6))."""
    rng = np.random.default_rng(R + 10 * D)
    ints = rng.integers(-255, 256, size=(R * D, 400))     # exact in bf16 (8 bits)
    cs = [to_bf16_bits(r) for r in ints]
    g = O.reduce_shard_hybrid(cs, O.BF16, R, True)
    for e in range(ints.shape[1]):
        nodes = [rne_int(int(ints[j * D:(j + 1) * D, e].sum()), 8) for j in range(R)]
        total = 0
        for s in nodes:                                     # fp32 fold is exact for these
            total += s
        total = rne_int(total, 8)
        scale = np.float32(1.0 / (R * D))
        want = np.float32(np.float32(total) * scale)
        assert g[e] == want, (e, nodes, total)


def test_fp32_rounding_is_identity():
    rng = np.random.default_rng(9)
    cs = list(rng.standard_normal((8, 1000)).astype(np.float32))
    a = O.reduce_shard_hybrid(cs, O.FP32, 2, True)
    b = O.reduce_shard_hybrid(cs, O.FP32, 2, False)
    assert a.tobytes() == b.tobytes()


def test_two_level_order_differs_from_flat_fold():
    """fp32, R = 2 nodes of D = 2: node 0 holds (1, 2^25), node 1 (-2^25, 1).
    Node 0: 1 + 2^25 rounds to 2^25 (spacing 4 there). Node 1: 1 - 2^25 =
    -(2^25 - 1) is halfway between -2^25 and -(2^25 - 2) (spacing 2); ties go
    to the even significand, -2^25. The nodes cancel: 0. The flat rank-order
    fold gives ((1 + 2^25) - 2^25) + 1 = 1, so a mean of 1/4."""
    big = np.float32(2.0 ** 25)
    cs = [np.array([1.0], np.float32), np.array([big]), np.array([-big]),
          np.array([1.0], np.float32)]
    assert O.reduce_shard_hybrid(cs, O.FP32, 2, False)[0] == 0.0
    assert O.reduce_shard(cs, O.FP32)[0] == np.float32(0.25)


def test_bf16_rounding_ties_to_even():
    """1 + 2^-8 is half a bf16 step above 1 (the step at 1 is 2^-7): it rounds
    to 1. 1 + 3 * 2^-8 is halfway between 1 + 2^-7 (odd significand) and
    1 + 2^-6: it rounds up."""
    one, eps8 = np.float32(1.0), np.float32(2.0 ** -8)
    cs = [to_bf16_bits([one, one + np.float32(2.0 ** -7)]), to_bf16_bits([eps8, eps8])]
    g = O.reduce_shard_hybrid(cs, O.BF16, 1, True)
    assert g[0] == np.float32(0.5)
    assert g[1] == np.float32((1.0 + 2.0 ** -6) / 2)
    g0 = O.reduce_shard_hybrid(cs, O.BF16, 1, False)
    assert g0[0] == np.float32((1.0 + 2.0 ** -8) / 2)


@pytest.mark.parametrize("rnd", [False, True])
def test_error_bound_against_exact_sum(rnd):
    """Any summation order of n terms in fp32 errs by at most (n-1) u sum|c|;
    each rounding to bf16 adds at most 2^-8 of the running magnitude."""
    rng = np.random.default_rng(11)
    R, D = 4, 8
    x = rng.standard_normal((R * D, 3000)).astype(np.float32)
    cs = [to_bf16_bits(r) for r in x]
    w = np.stack([O.bf16_widen(c) for c in cs]).astype(np.float64)
    g = O.reduce_shard_hybrid(cs, O.BF16, R, rnd).astype(np.float64) * (R * D)
    exact = np.array([math.fsum(w[:, e]) for e in range(w.shape[1])])
    mag = np.abs(w).sum(axis=0)
    u = 2.0 ** -24
    bound = (R * D - 1) * u * mag * 1.01
    if rnd:
        bound = bound + (R + 1) * 2.0 ** -8 * mag * 1.01
    assert np.all(np.abs(g - exact) <= bound + 1e-30)
    if rnd:
        # a rounded total is a bf16 value before the exact power-of-two scale
        assert np.array_equal(O.round_to_dtype(g.astype(np.float32), O.BF16), g.astype(np.float32))


def test_rank_step_hybrid_reduces_to_rank_step():
    rng = np.random.default_rng(5)
    S = 2000
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    cs = [to_bf16_bits(rng.standard_normal(S) * 1e-3) for _ in range(8)]
    hp = O.AdamWHP(3e-4, 0.9, 0.95, 1e-8, 0.1, 1)
    a = O.rank_step_hybrid(p, m, v, cs, O.BF16, hp, 1, False)
    b = O.rank_step(p, m, v, cs, O.BF16, hp)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()
    # with R = 2 the reduced gradient, and so the step, generally differs
    c = O.rank_step_hybrid(p, m, v, cs, O.BF16, hp, 2, True)
    assert c[0].tobytes() != b[0].tobytes()
