"""Pins of the oracle's reduce-scatter arithmetic (CPU only).

Pinned by exact integer arithmetic, the fixed rank-order left fold on an
order-adversarial input, a summation error bound against math.fsum, the
reduce-scatter diagram of "Building GPT from Scratch -- Part 8: FSDP", and
the identity between the concatenated reduce-scatter and the all-reduce.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import zs_oracle as O

U = 2.0 ** -24


def to_bf16_bits(x):
    """torch's cast, an independent route to bf16 bits."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("D", [1, 2, 4, 8, 16, 32, 64])
def test_exact_integer_contributions(D):
    rng = np.random.default_rng(D)
    S = 777
    ints = rng.integers(-128, 129, size=(D, S))
    contribs = [to_bf16_bits(ints[k]) for k in range(D)]
    g = O.reduce_shard(contribs, O.BF16)
    want = [Fraction(int(s), D) for s in ints.sum(axis=0)]
    assert all(Fraction(float(a)) == b for a, b in zip(g, want))


def test_d1_is_exact_widening():
    rng = np.random.default_rng(0)
    h = rng.integers(0, 65536, size=5000).astype(np.uint16)
    h = h[(h & 0x7F80) != 0x7F80]                     # finite patterns
    g = O.reduce_shard([h], O.BF16)
    back = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert g.tobytes() == back.tobytes()
    f = rng.standard_normal(100).astype(np.float32)
    assert O.reduce_shard([f], O.FP32).tobytes() == f.tobytes()


def test_rank_order_left_fold():
    """(2^25, 1, -2^25, 1): the left fold from c_0 gives 1, so g = 1/4.
    Reversed order or a pairwise tree give 0; the exact sum gives 1/2."""
    c = [to_bf16_bits([v]) for v in (2.0 ** 25, 1.0, -(2.0 ** 25), 1.0)]
    assert float(O.reduce_shard(c, O.BF16)[0]) == 0.25
    assert float(O.reduce_shard(c[::-1], O.BF16)[0]) == 0.0


def test_negative_zero_fold():
    nz = to_bf16_bits([-0.0])
    g = O.reduce_shard([nz, nz, nz], O.BF16)
    assert np.signbit(g[0]) and g[0] == 0.0
    pz = to_bf16_bits([0.0])
    assert not np.signbit(O.reduce_shard([nz, pz], O.BF16)[0])


@pytest.mark.parametrize("D", [3, 5, 8, 16, 31])
def test_summation_error_bound_fp32(D):
    rng = np.random.default_rng(100 + D)
    S = 2000
    x = (rng.standard_normal((D, S)) * 1e-3).astype(np.float32)
    x[:, :200] *= 1e4                                  # mixed magnitudes
    x[-1, 200:400] = -x[:-1, 200:400].sum(axis=0)      # heavy cancellation
    g = O.reduce_shard(list(x), O.FP32).astype(np.float64)
    for i in range(S):
        exact = math.fsum(float(v) for v in x[:, i]) / D
        absum = sum(abs(float(v)) for v in x[:, i]) / D
        # recursive summation (D-1)u*sum|x| plus the rounded 1/D and the product
        bound = (D - 1) * U * 1.01 * absum + 2.01 * U * abs(exact) + 1e-45
        assert abs(g[i] - exact) <= bound, (i, g[i], exact, bound)


def test_reduce_scatter_diagram():
    """Rank r gets the sum over k of g_k restricted to block r (times 1/D)."""
    rows = read_golden("collective_diagrams.txt")
    before = {int(r[1]): r[2].split() for r in rows if r[0] == "reducescatter.before"}
    after = {int(r[1]): r[2].split() for r in rows if r[0] == "reducescatter.after"}
    D = len(before)
    rng = np.random.default_rng(7)
    S = 5
    val = {}
    for k in range(D):
        for sym in before[k]:
            val[sym] = rng.integers(-100, 101, size=S)
    full = [np.concatenate([val[s] for s in before[k]]) for k in range(D)]
    for r in range(D):
        assert after[r][0] == "sum"
        contribs = [to_bf16_bits(full[k][r * S:(r + 1) * S]) for k in range(D)]
        g = O.reduce_shard(contribs, O.BF16)
        want = sum(val[s] for s in after[r][1:])
        assert np.array_equal(g * D, want.astype(np.float32))


def test_concat_of_reduce_scatter_equals_all_reduce():
    """Rank r's reduce on slice r of every rank's full-unit gradient,
    concatenated over r, equals the all-reduce mean of the full gradients."""
    rng = np.random.default_rng(11)
    for D, dt in ((4, O.BF16), (8, O.BF16), (16, O.FP32), (3, O.FP32)):
        N = 1001
        _, _, N_pad, S = O.unit_layout([N], D)
        G = [(rng.standard_normal(N) * 1e-3).astype(np.float32) for _ in range(D)]
        Gp = [np.concatenate([x, np.zeros(N_pad - N, np.float32)]) for x in G]
        if dt == O.BF16:
            Gp = [to_bf16_bits(x) for x in Gp]
        allred = O.reduce_shard(Gp, dt)
        rs = np.concatenate([O.reduce_shard([x[r * S:(r + 1) * S] for x in Gp], dt)
                             for r in range(D)])
        assert rs.tobytes() == allred.tobytes()
        assert not allred[N:].any()                     # pad gradient stays +0


def test_inv_d_is_multiplied_not_divided():
    """Reading taken: the sum is multiplied by float32(1/D). For D = 3 the
    product s * float32(1/3) is exact in double (24 x 24 bits), so one
    rounding to float32 gives the expected value; some s make it differ from
    the correctly rounded s / 3, and the oracle must give the product."""
    inv3 = np.float32(1.0 / 3.0)
    found = 0
    for s in range(1, 4000):
        x = np.float32(s) * np.float32(1.0009765625)       # 11-bit mantissas
        prod = np.float32(float(Fraction(float(x)) * Fraction(float(inv3))))
        quot = np.float32(float(Fraction(float(x)) / 3))
        g = O.reduce_shard([np.array([x], np.float32), np.zeros(1, np.float32),
                            np.zeros(1, np.float32)], O.FP32)[0]
        assert g.tobytes() == prod.tobytes()
        found += prod != quot
    assert found > 0


# ------------------------------------------------- an explicit multiplier
@pytest.mark.parametrize("D", [1, 3, 8, 32])
def test_scale_one_is_the_plain_sum(D):
    """scale = 1: the reduce-scatter diagram's sum itself, exact for small
    integers (a closed form: Python's integer sum)."""
    rng = np.random.default_rng(200 + D)
    ints = rng.integers(-128, 129, size=(D, 500))
    g = O.reduce_shard([to_bf16_bits(ints[k]) for k in range(D)], O.BF16, scale=1.0)
    assert [float(x) for x in g] == [float(s) for s in ints.sum(axis=0)]


@pytest.mark.parametrize("scale, den", [(0.25, 4), (0.5, 2), (2.0 ** -10, 1024)])
def test_power_of_two_scale_is_exact(scale, den):
    rng = np.random.default_rng(den)
    ints = rng.integers(-1000, 1001, size=(5, 300))
    g = O.reduce_shard([ints[k].astype(np.float32) for k in range(5)], O.FP32, scale=scale)
    want = [Fraction(int(s), den) for s in ints.sum(axis=0)]
    assert all(Fraction(float(a)) == b for a, b in zip(g, want))


def test_scale_is_rounded_to_fp32_once():
    """1/3 is not an fp32 number: the multiplier is float32(1/3), and for an
    exact integer sum s the result is the fp32 rounding of s * float32(1/3),
    computed here exactly with fractions."""
    ints = np.arange(-40, 41, dtype=np.int64).reshape(1, -1).repeat(3, axis=0)
    g = O.reduce_shard([r.astype(np.float32) for r in ints], O.FP32, scale=1.0 / 3.0)
    third = Fraction(float(np.float32(1.0 / 3.0)))
    for a, s in zip(g, ints.sum(axis=0)):
        exact = Fraction(int(s)) * third       # fits a double exactly (< 31 significant bits)
        assert float(a) == float(np.float32(float(exact)))


def test_default_scale_is_one_over_d():
    rng = np.random.default_rng(9)
    x = [(rng.standard_normal(256) * 1e-3).astype(np.float32) for _ in range(7)]
    assert O.reduce_shard(x, O.FP32).tobytes() == O.reduce_shard(x, O.FP32, scale=1.0 / 7).tobytes()


@pytest.mark.parametrize("rnd", [False, True])
def test_hybrid_scale_one_is_the_integer_sum(rnd):
    """HYBRID_SHARD with scale = 1 on small integers: every partial sum is an
    integer below 2^8, exact in bf16, so rounding changes nothing and the
    result is Python's integer sum over all R * D contributions."""
    rng = np.random.default_rng(31)
    R, D = 4, 8
    ints = rng.integers(-7, 8, size=(R * D, 400))
    c = [to_bf16_bits(ints[k]) for k in range(R * D)]
    g = O.reduce_shard_hybrid(c, O.BF16, R, rnd, scale=1.0)
    assert [float(x) for x in g] == [float(s) for s in ints.sum(axis=0)]
