"""The host (ZeRO-Offload) AdamW step, zs_adamw_step_host, against the CPU
oracle: bit-exact on ragged sizes, several thread counts, several steps,
special values (zeros, signed zeros, denormal gradients and moments, huge
and NaN values), and with the caller's FPU set to flush denormals. Runs on
the host only: no GPU is needed."""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from oracle import zs_oracle as O

HP = W.ADAMW_HP


def host_state(S, seed):
    g = torch.Generator().manual_seed(seed)
    p = (torch.randn(S, generator=g) * 0.02).contiguous()
    return p, torch.zeros(S), torch.zeros(S), torch.zeros(S, dtype=torch.int16)


def grads(S, seed, specials=False):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(S, generator=g) * 1e-3
    if specials and S >= 16:
        vals = torch.tensor([0.0, -0.0, 1e-40, -1e-42, 3e38, -3e38, 1e-45, 2.0 ** -126,
                             float("nan"), 7.0, -1e-30, 1e30], dtype=torch.float32)
        idx = torch.randint(0, S, (min(S, 4000),), generator=g)
        x[idx] = vals[torch.randint(0, len(vals), (idx.numel(),), generator=g)]
    return x


def check(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        both_nan = np.isnan(a) & np.isnan(b)
        ne = (a.view(np.uint32) != b.view(np.uint32)) & ~both_nan
    else:
        ne = a.view(np.uint16) != b.view(np.uint16)
    assert not ne.any(), f"{what}: {int(ne.sum())} elements differ, first at {np.flatnonzero(ne)[0]}"


@pytest.mark.parametrize("S", [1, 7, 63, 64, 65, 1000, 1_000_003])
@pytest.mark.parametrize("threads", [1, 3, 16])
def test_host_step_matches_oracle(S, threads):
    p, m, v, w = host_state(S, S)
    op, om, ov = p.numpy().copy(), m.numpy().copy(), v.numpy().copy()
    for t in (1, 2, 3):
        g = grads(S, 100 * t + S, specials=(t == 2))
        hp = dict(step=t, **HP)
        zs.zs_adamw_step_host(p, m, v, w, g, hp, threads=threads)
        with np.errstate(all="ignore"):      # the specials overflow g * g to inf
            op, om, ov, ow = O.adamw_step(op, om, ov, g.numpy(), O.AdamWHP(**hp))
        check(p.numpy(), op, f"p step {t}")
        check(m.numpy(), om, f"m step {t}")
        check(v.numpy(), ov, f"v step {t}")
        check(w.numpy().view(np.uint16), ow, f"w step {t}")


def test_denormals_kept_when_the_caller_flushes():
    S = 4099
    p, m, v, w = host_state(S, 1)
    p[:100] = 1e-39                      # denormal parameters
    g = grads(S, 2)
    g[100:200] = 1e-41                   # denormal gradients: g*g underflows, m keeps them
    op, om, ov, ow = O.adamw_step(p.numpy().copy(), m.numpy().copy(), v.numpy().copy(), g.numpy(),
                                  O.AdamWHP(step=1, **HP))
    assert torch.set_flush_denormal(True)
    try:
        zs.zs_adamw_step_host(p, m, v, w, g, dict(step=1, **HP), threads=1)
    finally:
        torch.set_flush_denormal(False)
    check(p.numpy(), op, "p")
    check(m.numpy(), om, "m")
    check(w.numpy().view(np.uint16), ow, "w")
    assert (np.abs(om[100:200]) > 0).all() and (np.abs(om[100:200]) < 1.2e-38).all()


def test_host_step_argument_errors():
    S = 100
    p, m, v, w = host_state(S, 0)
    g = grads(S, 1)
    with pytest.raises(zs.ZsError) as e:
        zs.zs_adamw_step_host(p, m, v, w, g, dict(step=1, **HP), threads=0)
    assert e.value.status == zs.ZS_EINVAL
    with pytest.raises(zs.ZsError) as e:
        zs.zs_adamw_step_host(p, p, v, w, g, dict(step=1, **HP))
    assert e.value.status == zs.ZS_EALIAS
    with pytest.raises(zs.ZsError) as e:
        zs.zs_adamw_step_host(p, m, v, w, g, dict(step=0, **HP))
    assert e.value.status == zs.ZS_EINVAL
    with pytest.raises(ValueError):
        zs.zs_adamw_step_host(p, m, v, w, g[:50], dict(step=1, **HP))


@pytest.mark.slow
def test_host_working_shard_rounding_all_fp32_patterns():
    """lr = 0, no weight decay, zero gradient: the host step leaves p
    unchanged and writes w = RNE(p); every one of the 2^32 fp32 patterns.
    Each chunk is checked against torch's CPU cast, which test_oracle_bf16
    pins equal to the oracle's bf16_round over the same 2^32 patterns (that
    is the faster route); every 16th chunk also against bf16_round itself."""
    chunk = 1 << 22          # temporaries small enough to be reused, not faulted in afresh
    hp = dict(lr=0.0, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, step=1)
    m = torch.zeros(chunk)
    v = torch.zeros(chunk)
    g = torch.zeros(chunk)
    w = torch.empty(chunk, dtype=torch.int16)
    p = torch.empty(chunk)
    for a in range(0, 1 << 32, chunk):
        bits = np.arange(a, a + chunk, dtype=np.uint32)
        p.numpy().view(np.uint32)[:] = bits
        m.zero_()
        v.zero_()
        zs.zs_adamw_step_host(p, m, v, w, g, hp, threads=8)
        got = w.numpy().view(np.uint16)
        want = torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16).view(torch.int16)
        want = want.numpy().view(np.uint16)
        nan = (bits & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if (a // chunk) % 16 == 0:
            assert not np.any((want != O.bf16_round(bits.view(np.float32))) & ~nan)
        bad = (got != want) & ~nan
        if bad.any():
            i = np.flatnonzero(bad)
            raise AssertionError(f"{i.size} patterns differ near {a:#x}, first {bits[i[0]]:#010x}")
        assert (((got[nan] & 0x7FFF) > 0x7F80) & ((got[nan] >> 15) == (bits[nan] >> 31))).all()
        assert not np.any((p.numpy().view(np.uint32) != bits) & ~nan)


def test_concurrent_callers_share_the_worker_pool():
    """Several host threads call the host step at once (ctypes drops the
    GIL for the call), each on its own state with its own hyperparameters,
    while other threads make calls that fail with their own messages: every
    result equals the oracle's and every thread reads only its own error."""
    import ctypes
    import threading
    lib = zs.load()
    i64 = ctypes.c_int64
    n_step, n_err, rounds = 6, 4, 5
    results, errors = {}, []

    def stepper(j):
        try:
            S = 200_003 + 977 * j
            p, m, v, w = host_state(S, 50 + j)
            op, om, ov = p.numpy().copy(), m.numpy().copy(), v.numpy().copy()
            for t in range(1, rounds + 1):
                g = grads(S, 1000 * j + t)
                hp = dict(HP, lr=HP["lr"] * (1 + j), step=t)
                zs.zs_adamw_step_host(p, m, v, w, g, hp, threads=1 + j % 4)
                op, om, ov, ow = O.adamw_step(op, om, ov, g.numpy(), O.AdamWHP(**hp))
            results[j] = (p.numpy(), m.numpy(), v.numpy(), w.numpy().view(np.uint16),
                          op, om, ov, ow)
        except Exception as e:  # reported below, on the main thread
            errors.append(f"stepper {j}: {e!r}")

    def failer(j):
        try:
            for _ in range(200):
                # D outside 1..ZS_MAX_D: the message names this thread's D
                D = 1000 + j
                numels = (i64 * 1)(5)
                off = (i64 * 2)()
                a, b, c = i64(), i64(), i64()
                st = lib.zs_unit_layout(numels, 1, D, off, a, b, c)
                msg = lib.zs_last_error().decode()
                if st != zs.ZS_EINVAL or f"D = {D}" not in msg:
                    errors.append(f"failer {j}: status {st}, message {msg!r}")
                    return
        except Exception as e:
            errors.append(f"failer {j}: {e!r}")

    ths = [threading.Thread(target=stepper, args=(j,)) for j in range(n_step)]
    ths += [threading.Thread(target=failer, args=(j,)) for j in range(n_err)]
    for th in ths:
        th.start()
    for th in ths:
        th.join()
    assert not errors, errors
    assert sorted(results) == list(range(n_step))
    for j, (p, m, v, w, op, om, ov, ow) in results.items():
        check(p, op, f"thread {j} p")
        check(m, om, f"thread {j} m")
        check(v, ov, f"thread {j} v")
        check(w, ow, f"thread {j} w")


def test_step_constants_over_sequences_of_step_counts():
    """The library keeps the beta powers it computed last on each thread and
    advances from them; every order of step counts (forward, repeated, back
    to an earlier step, large, with other betas in between) gives the
    oracle's constants: the host step's results are the oracle's bit for
    bit."""
    S = 4099
    seq = [(1, HP), (2, HP), (2, HP), (200_000, HP), (200_001, HP), (5, HP),
           (5, dict(HP, beta2=0.99999)), (70_000, dict(HP, beta2=0.99999)),
           (70_000, HP), (3, dict(HP, beta1=0.0, beta2=0.0)), (4, dict(HP, beta1=0.0, beta2=0.0)),
           (123_456, HP)]
    for i, (t, hpd) in enumerate(seq):
        p, m, v, w = host_state(S, 300 + i)
        m.copy_(grads(S, 400 + i)); v.copy_(grads(S, 500 + i).square())
        g = grads(S, 600 + i)
        op, om, ov = p.numpy().copy(), m.numpy().copy(), v.numpy().copy()
        hp = dict(hpd, step=t)
        zs.zs_adamw_step_host(p, m, v, w, g, hp, threads=2)
        op, om, ov, ow = O.adamw_step(op, om, ov, g.numpy(), O.AdamWHP(**hp))
        check(p.numpy(), op, f"p at {i}: step {t}")
        check(v.numpy(), ov, f"v at {i}: step {t}")
        check(w.numpy().view(np.uint16), ow, f"w at {i}: step {t}")
