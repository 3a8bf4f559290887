"""Pins of the oracle's AdamW step (CPU only).

The pages name Adam/AdamW with an fp32 master copy and fp32 moments and
print no equations. The oracle is pinned here by Adam's closed forms (step
1, and a constant gradient at every step), the exact special cases g = 0,
lr = 0 and wd = 0, an error bound against an independent float64
evaluation, and the "same math as unsharded" statement of "Building GPT from
Scratch -- Part 8: FSDP" (TL;DR, "Key Takeaways"): all D rank steps, then
gathered, equal one unsharded step on the all-reduce-mean gradient.
"""
import math

import numpy as np
import pytest

from oracle import zs_oracle as O
import workloads as W

U = 2.0 ** -24
HP = dict(W.ADAMW_HP)


def hp(step, **kw):
    d = dict(HP)
    d.update(kw)
    return O.AdamWHP(step=step, **d)


def f64_adamw(p, m, v, g, lr, b1, b2, eps, wd, t):
    """Adam with bias correction and decoupled decay, all in float64 with
    exact scalar factors (pow from the math library)."""
    p, m, v, g = (np.asarray(a, np.float64) for a in (p, m, v, g))
    m1 = b1 * m + (1 - b1) * g
    v1 = b2 * v + (1 - b2) * g * g
    mhat = m1 / (1 - b1 ** t)
    vhat = v1 / (1 - b2 ** t)
    p2 = p * (1 - lr * wd) - lr * mhat / (np.sqrt(vhat) + eps)
    return p2, m1, v1


def rand_state(rng, n):
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    return p, g


def test_step1_closed_form():
    """t = 1: m_hat = g and v_hat = g^2, so the update is lr*g/(|g|+eps)."""
    rng = np.random.default_rng(0)
    n = 20000
    p, g = rand_state(rng, n)
    z = np.zeros(n, np.float32)
    p1, m1, v1, w1 = O.adamw_step(p, z, z, g, hp(1))
    lr, wd, eps = HP["lr"], HP["weight_decay"], HP["eps"]
    gd = g.astype(np.float64)
    want = p.astype(np.float64) * (1 - lr * wd) - lr * gd / (np.abs(gd) + eps)
    upd = lr * np.abs(gd) / (np.abs(gd) + eps)
    err = np.abs(p1 - want)
    assert np.all(err <= 8 * U * (np.abs(p) + upd) + 1e-45)
    assert np.allclose(m1, (1 - HP["beta1"]) * gd, rtol=4 * U * 8, atol=0)
    assert np.allclose(v1, (1 - HP["beta2"]) * gd * gd, rtol=8 * U * 8, atol=0)
    assert np.array_equal(w1, O.bf16_round(p1))


def test_constant_gradient_every_step():
    """With g fixed, m_t = (1-b1^t) g, v_t = (1-b2^t) g^2 and every update is
    lr*g/(|g|+eps): p_t = p_{t-1}(1-lr wd) - lr g/(|g|+eps)."""
    rng = np.random.default_rng(1)
    n = 5000
    p, g = rand_state(rng, n)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    lr, wd, eps, b1, b2 = (HP[k] for k in ("lr", "weight_decay", "eps", "beta1", "beta2"))
    gd = g.astype(np.float64)
    pd = p.astype(np.float64)
    step_upd = lr * gd / (np.abs(gd) + eps)
    for t in range(1, 31):
        p, m, v, _ = O.adamw_step(p, m, v, g, hp(t))
        pd = pd * (1 - lr * wd) - step_upd
        assert np.allclose(m, (1 - b1 ** t) * gd, rtol=2e-6 * t, atol=0)
        assert np.allclose(v, (1 - b2 ** t) * gd * gd, rtol=2e-6 * t, atol=0)
        # rounding of each step accumulates; bound it by t steps of a few ulps
        tol = t * 16 * U * (np.abs(pd) + np.abs(step_upd)) + 1e-30
        assert np.all(np.abs(p - pd) <= tol), t


def test_zero_gradient_is_pure_decay():
    rng = np.random.default_rng(2)
    p, _ = rand_state(rng, 3000)
    z = np.zeros_like(p)
    for t in (1, 2, 7):
        p1, m1, v1, w = O.adamw_step(p, z, z, z, hp(t))
        dec = np.float32(1.0 - HP["lr"] * HP["weight_decay"])
        assert p1.tobytes() == (p * dec).astype(np.float32).tobytes()
        assert not m1.any() and not v1.any()
        assert np.array_equal(w, O.bf16_round(p1))


def test_zero_lr_leaves_params():
    rng = np.random.default_rng(3)
    p, g = rand_state(rng, 3000)
    m = (g * 0.5).astype(np.float32)
    v = (g * g).astype(np.float32)
    p1, m1, v1, _ = O.adamw_step(p, m, v, g, hp(4, lr=0.0))
    assert p1.tobytes() == p.tobytes()
    assert not np.array_equal(m1, m)                 # moments still move


def test_zero_wd_has_no_decay_factor():
    k = O.adamw_constants(hp(3, weight_decay=0.0))
    assert k["DEC"] == np.float32(1.0)
    rng = np.random.default_rng(4)
    p, _ = rand_state(rng, 100)
    z = np.zeros_like(p)
    assert O.adamw_step(p, z, z, z, hp(3, weight_decay=0.0))[0].tobytes() == p.tobytes()


def test_constants_double_then_float():
    """Each constant is rounded from double once: float32(1 - 0.9) is
    0x3DCCCCCD, whereas 1.0f - 0.9f would be 0x3DCCCCD0."""
    k = O.adamw_constants(hp(1))
    assert k["B1c"].view(np.uint32) == 0x3DCCCCCD
    assert (np.float32(1.0) - np.float32(0.9)).view(np.uint32) == 0x3DCCCCD0
    # beta^t by repeated multiplication agrees with pow to well within fp32
    for t in (1, 2, 10, 1000):
        k = O.adamw_constants(hp(t))
        want = HP["lr"] / (1 - HP["beta1"] ** t)
        assert abs(float(k["SS"]) - want) <= U * want
        assert abs(float(k["BC2S"]) - math.sqrt(1 - HP["beta2"] ** t)) <= U


def test_step_below_one_rejected():
    with pytest.raises(ValueError):
        O.adamw_constants(hp(0))


@pytest.mark.parametrize("t", [1, 2, 5, 50])
def test_error_bound_against_float64(t):
    """fp32 oracle vs float64 Adam on the same fp32 inputs, one step. A
    dropped term, a wrong sign or a swapped operand moves p by about the
    update (lr ~ 3e-4 against |p| ~ 0.02), far beyond this bound."""
    rng = np.random.default_rng(10 + t)
    n = 20000
    p, g = rand_state(rng, n)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = (rng.standard_normal(n) ** 2 * 1e-6).astype(np.float32)
    p32, m32, v32, _ = O.adamw_step(p, m, v, g, hp(t))
    p64, m64, v64 = f64_adamw(p, m, v, g, HP["lr"], HP["beta1"], HP["beta2"],
                              HP["eps"], HP["weight_decay"], t)
    b1, b2, lr = HP["beta1"], HP["beta2"], HP["lr"]
    mag_m = np.abs(b1 * m.astype(np.float64)) + np.abs((1 - b1) * g.astype(np.float64))
    den = np.sqrt(v64 / (1 - b2 ** t)) + HP["eps"]
    mag_u = lr / (1 - b1 ** t) * mag_m / den
    assert np.all(np.abs(m32 - m64) <= 3 * U * mag_m + 1e-45)
    assert np.all(np.abs(v32 - v64) <= 4 * U * np.abs(v64) + 1e-45)
    assert np.all(np.abs(p32 - p64) <= 3 * U * np.abs(p) + 12 * U * mag_u + 1e-45)
    # and the plausible mistakes do fail it
    bad = p64 + 2 * lr * m64 / den / (1 - b1 ** t)     # wrong sign of the update
    assert not np.all(np.abs(p32 - bad) <= 3 * U * np.abs(p) + 12 * U * mag_u)


def test_sharded_equals_unsharded():
    """All D rank steps, gathered, equal one D = 1 step on the all-reduce
    mean gradient, bit for bit, over several steps."""
    rng = np.random.default_rng(20)
    numels = [300, 17, 1024, 5, 999]
    D = 4
    _, N, N_pad, S = O.unit_layout(numels, D)
    ts = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in numels]
    shards_p = O.pack_flat(ts, D)
    shards_m = [np.zeros(S, np.float32) for _ in range(D)]
    shards_v = [np.zeros(S, np.float32) for _ in range(D)]
    flat_p = O.gather_unit(shards_p)
    flat_m = np.zeros(N_pad, np.float32)
    flat_v = np.zeros(N_pad, np.float32)
    to_bits = lambda x: O.bf16_round(x.astype(np.float32))
    for t in range(1, 6):
        full_grads = [to_bits(np.concatenate([rng.standard_normal(N) * 1e-3,
                                              np.zeros(N_pad - N)]))
                      for _ in range(D)]
        ws = []
        for r in range(D):
            c = [G[r * S:(r + 1) * S] for G in full_grads]
            shards_p[r], shards_m[r], shards_v[r], w = O.rank_step(
                shards_p[r], shards_m[r], shards_v[r], c, O.BF16, hp(t))
            ws.append(w)
        g_all = O.reduce_shard(full_grads, O.BF16)
        flat_p, flat_m, flat_v, flat_w = O.rank_step(flat_p, flat_m, flat_v,
                                                     [g_all], O.FP32, hp(t))
        assert O.gather_unit(shards_p).tobytes() == flat_p.tobytes()
        assert O.gather_unit(shards_m).tobytes() == flat_m.tobytes()
        assert O.gather_unit(shards_v).tobytes() == flat_v.tobytes()
        assert O.gather_unit(ws).tobytes() == flat_w.tobytes()
        assert not flat_p[N:].any() and not flat_w[N:].any()   # pad stays +0


def test_fused_equals_unfused():
    """rank_step (reduce then step) equals a step fed the reduced gradient as
    a single fp32 contribution: the 1/1 scale is exact."""
    rng = np.random.default_rng(21)
    n = 4000
    p, _ = rand_state(rng, n)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    c = [O.bf16_round((rng.standard_normal(n) * 1e-3).astype(np.float32)) for _ in range(8)]
    a = O.rank_step(p, m, v, c, O.BF16, hp(1))
    b = O.rank_step(p, m, v, [O.reduce_shard(c, O.BF16)], O.FP32, hp(1))
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()
