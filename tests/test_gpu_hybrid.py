"""GPU parity of the HYBRID_SHARD / reduce-dtype-rounded reduce and step
(zs_reduce_shard_ex, zs_adamw_step_ex) against the CPU oracle
(reduce_shard_hybrid, rank_step_hybrid): bit-exact, at sizes with several
tiles and a ragged tail, on aligned and misaligned buffers, for both reduce
dtypes, and at the full size of the 4-node x 8-GPU LLaMA-7B HYBRID_SHARD
rank shard on sampled positions.
"""
import time

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from oracle import zs_oracle as O
from gpu_util import check_bf16, check_f32, device, sample_indices, to_np

pytestmark = pytest.mark.gpu

HP = W.ADAMW_HP


def contribs(n, S, dtype, seed, dev, offset=0, scale=W.GRAD_SCALE):
    """n contributions of S elements; offset > 0 makes them views that start
    `offset` elements into a larger buffer (misaligned for the vector path)."""
    out = []
    for k in range(n):
        x = W.normal_f32(S + offset, scale, seed * 100 + k, dev)
        x = W.as_bf16_bits(x) if dtype == O.BF16 else x
        out.append(x[offset:])
    return out


def state(S, seed, dev, offset=0):
    p = W.master_init(S + offset, seed, dev)[offset:]
    m = torch.zeros(S + offset, device=dev)[offset:]
    v = torch.zeros(S + offset, device=dev)[offset:]
    w = torch.zeros(S + offset, dtype=torch.int16, device=dev)[offset:]
    return p, m, v, w


CASES = [(1, 8, False), (1, 8, True), (2, 4, False), (2, 4, True), (4, 8, True),
         (4, 8, False), (3, 3, True), (8, 8, True), (2, 16, True), (2, 32, False), (5, 1, True)]


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32])
@pytest.mark.parametrize("R,D,rnd", CASES)
@pytest.mark.parametrize("offset", [0, 1])
def test_reduce_ex_matches_oracle(dtype, R, D, rnd, offset):
    dev = device()
    S = 3 * 2048 * 8 + 5
    cs = contribs(R * D, S, dtype, 10 * R + D, dev, offset)
    out = torch.empty(S + offset, device=dev)[offset:]
    zs.zs_reduce_shard_ex(cs, out, replicas=R, round_to_reduce_dtype=rnd)
    want = O.reduce_shard_hybrid([to_np(c) for c in cs], dtype, R, rnd)
    check_f32(to_np(out), want, f"reduce R={R} D={D} rnd={rnd}", exact=True)


SCALES = [1.0, 0.5, 1.0 / 3.0, 2.0 ** -20, 1024.0]


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32])
@pytest.mark.parametrize("R,D,rnd", [(1, 8, False), (1, 5, False), (2, 4, True), (4, 8, True)])
@pytest.mark.parametrize("scale", SCALES)
def test_reduce_ex_scale_matches_oracle(dtype, R, D, rnd, scale):
    """An explicit multiplier in place of 1/(R*D): 1 is the reduce-scatter's
    plain sum, the others scale it (rounded to fp32 once)."""
    dev = device()
    S = 2 * 2048 * 8 + 29
    cs = contribs(R * D, S, dtype, 300 + 10 * R + D, dev)
    out = torch.empty(S, device=dev)
    zs.zs_reduce_shard_ex(cs, out, replicas=R, round_to_reduce_dtype=rnd, scale=scale)
    want = O.reduce_shard_hybrid([to_np(c) for c in cs], dtype, R, rnd, scale=scale)
    check_f32(to_np(out), want, f"reduce R={R} D={D} rnd={rnd} scale={scale}", exact=True)


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32])
@pytest.mark.parametrize("R,D,rnd", [(1, 8, False), (2, 4, True), (3, 3, False)])
@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("offset", [0, 1])
def test_adamw_ex_scale_matches_oracle(dtype, R, D, rnd, scale, offset):
    dev = device()
    S = 2048 * 8 + 77
    p, m, v, w = state(S, 50 + R + D, dev, offset)
    op, om, ov = to_np(p), np.zeros(S, np.float32), np.zeros(S, np.float32)
    for t in (1, 2):
        cs = contribs(R * D, S, dtype, 700 * t + 10 * R + D, dev, offset)
        hp = dict(step=t, **HP)
        zs.zs_adamw_step_ex(p, m, v, w, cs, hp, replicas=R, round_to_reduce_dtype=rnd,
                            scale=scale)
        op, om, ov, ow = O.rank_step_hybrid(op, om, ov, [to_np(c) for c in cs], dtype,
                                            O.AdamWHP(**hp), R, rnd, scale=scale)
    torch.cuda.synchronize()
    what = f"R={R} D={D} rnd={rnd} scale={scale} off={offset}"
    check_f32(to_np(p), op, what + " p", exact=True)
    check_f32(to_np(m), om, what + " m", exact=True)
    check_f32(to_np(v), ov, what + " v", exact=True)
    check_bf16(to_np(w), ow, what + " w", exact=True)


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32])
@pytest.mark.parametrize("R,D,rnd", [(1, 8, False), (2, 4, True)])
def test_keep_working_shard_hint_changes_no_bits(dtype, R, D, rnd):
    """ZS_W_KEEP (cache-allocating stores of the working shard) gives the
    same p, m, v and w as the default non-temporal stores, and the oracle's."""
    dev = device()
    S = 3 * 1024 * 8 + 19
    a = state(S, 60 + R + D, dev)
    b = [t.clone() for t in a]
    op, om, ov = to_np(a[0]), np.zeros(S, np.float32), np.zeros(S, np.float32)
    for t in (1, 2):
        cs = contribs(R * D, S, dtype, 500 * t + R + D, dev)
        hp = dict(step=t, **HP)
        zs.zs_adamw_step_ex(*a, cs, hp, replicas=R, round_to_reduce_dtype=rnd)
        zs.zs_adamw_step_ex(*b, cs, hp, replicas=R, round_to_reduce_dtype=rnd,
                            keep_working_shard=True)
        op, om, ov, ow = O.rank_step_hybrid(op, om, ov, [to_np(c) for c in cs], dtype,
                                            O.AdamWHP(**hp), R, rnd)
    torch.cuda.synchronize()
    for x, y, name in zip(a, b, "pmvw"):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y), name
    check_f32(to_np(b[0]), op, "keep p", exact=True)
    check_bf16(to_np(b[3]), ow, "keep w", exact=True)


def test_scale_zero_means_the_mean():
    """scale = 0 (the default) and scale = 1/(R*D) give the same bits."""
    dev = device()
    S = 4096 + 3
    cs = contribs(6, S, O.BF16, 901, dev)
    a, b = torch.empty(S, device=dev), torch.empty(S, device=dev)
    zs.zs_reduce_shard_ex(cs, a, replicas=2)
    zs.zs_reduce_shard_ex(cs, b, replicas=2, scale=1.0 / 6.0)
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32])
@pytest.mark.parametrize("R,D,rnd", CASES)
@pytest.mark.parametrize("offset", [0, 1])
def test_adamw_ex_matches_oracle(dtype, R, D, rnd, offset):
    dev = device()
    S = 2 * 2048 * 8 + 13
    p, m, v, w = state(S, 7 + R + D, dev, offset)
    op, om, ov = to_np(p), np.zeros(S, np.float32), np.zeros(S, np.float32)
    for t in (1, 2, 3):
        cs = contribs(R * D, S, dtype, 1000 * t + 10 * R + D, dev, offset)
        hp = dict(step=t, **HP)
        zs.zs_adamw_step_ex(p, m, v, w, cs, hp, replicas=R, round_to_reduce_dtype=rnd)
        op, om, ov, ow = O.rank_step_hybrid(op, om, ov, [to_np(c) for c in cs], dtype,
                                            O.AdamWHP(**hp), R, rnd)
    torch.cuda.synchronize()
    what = f"R={R} D={D} rnd={rnd} off={offset}"
    check_f32(to_np(p), op, what + " p", exact=True)
    check_f32(to_np(m), om, what + " m", exact=True)
    check_f32(to_np(v), ov, what + " v", exact=True)
    check_bf16(to_np(w), ow, what + " w", exact=True)


def test_rounding_ties_and_cancellation():
    """Contributions drawn from a few bf16 values so that node sums land on
    bf16 rounding ties and cancel exactly, plus fp32 values that make the
    two-level order differ from the flat fold."""
    dev = device()
    S = 4096 + 7
    rng = np.random.default_rng(0)
    vals = np.array([1.0, 2.0 ** -8, -1.0, 3 * 2.0 ** -9, 2.0 ** 25, -2.0 ** 25, 0.0, -0.0],
                    np.float32)
    R, D = 4, 4
    xs = vals[rng.integers(0, len(vals), size=(R * D, S))]
    for dtype in (O.BF16, O.FP32):
        cs = []
        for x in xs:
            t = torch.from_numpy(x).to(dev)
            cs.append(W.as_bf16_bits(t) if dtype == O.BF16 else t)
        for rnd in (False, True):
            out = torch.empty(S, device=dev)
            zs.zs_reduce_shard_ex(cs, out, replicas=R, round_to_reduce_dtype=rnd)
            want = O.reduce_shard_hybrid([to_np(c) for c in cs], dtype, R, rnd)
            check_f32(to_np(out), want, f"ties {dtype} rnd={rnd}", exact=True)
            assert np.array_equal(np.signbit(to_np(out)), np.signbit(want))


def test_flat_options_equal_plain_entry_points():
    dev = device()
    S = 50000
    cs = contribs(8, S, O.BF16, 3, dev)
    a, b = state(S, 1, dev), state(S, 1, dev)
    zs.zs_adamw_step(*a, cs, dict(step=1, **HP))
    zs.zs_adamw_step_ex(*b, cs, dict(step=1, **HP), replicas=1, round_to_reduce_dtype=False)
    ga, gb = torch.empty(S, device=dev), torch.empty(S, device=dev)
    zs.zs_reduce_shard(cs, ga)
    zs.zs_reduce_shard_ex(cs, gb)
    torch.cuda.synchronize()
    for x, y in zip(a + (ga,), b + (gb,)):
        assert to_np(x).tobytes() == to_np(y).tobytes()


def test_fused_equals_unfused_hybrid():
    """zs_reduce_shard_ex then zs_adamw_step on its fp32 output == zs_adamw_step_ex."""
    dev = device()
    S = 40000 + 3
    cs = contribs(32, S, O.BF16, 9, dev)
    a, b = state(S, 2, dev), state(S, 2, dev)
    hp = dict(step=4, **HP)
    zs.zs_adamw_step_ex(*a, cs, hp, replicas=4, round_to_reduce_dtype=True)
    g = torch.empty(S, device=dev)
    zs.zs_reduce_shard_ex(cs, g, replicas=4, round_to_reduce_dtype=True)
    zs.zs_adamw_step(*b, [g], hp)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert to_np(x).tobytes() == to_np(y).tobytes()


def test_hybrid_errors():
    dev = device()
    S = 100
    cs = contribs(8, S, O.BF16, 1, dev)
    p, m, v, w = state(S, 1, dev)
    with pytest.raises(ValueError):
        zs.zs_adamw_step_ex(p, m, v, w, cs, dict(step=1, **HP), replicas=3)
    with pytest.raises(zs.ZsError) as e:
        zs.zs_adamw_step_ex(p, m, v, w, cs * 9, dict(step=1, **HP), replicas=9)
    assert e.value.status == zs.ZS_EINVAL and "exceeds" in zs.zs_last_error()
    g = torch.empty(S, device=dev)
    with pytest.raises(zs.ZsError) as e:
        zs.zs_reduce_shard_ex(cs[:4] + [g[:S].view(torch.int16)[:S]] * 4, g, replicas=2)
    assert e.value.status == zs.ZS_EALIAS


def test_llama7b_hybrid_full_size_sampled():
    """The rank-0 shard of LLaMA-7B under HYBRID_SHARD (4 nodes x 8 GPUs):
    one bucket per unit (33), 32 bf16 contributions per bucket, collectives
    held in bf16, 3 steps; every bucket checked on sampled positions."""
    dev = device()
    w = W.get("llama7b_hybrid")
    R, D = w.replicas, w.D
    sizes = [zs.zs_unit_layout(u.numels, D)[3] for u in w.units]
    S = sum(sizes)
    starts = np.concatenate([[0], np.cumsum(sizes)])
    print(f"[{time.strftime('%H:%M:%S')}] llama7b_hybrid S={S}", flush=True)
    p = W.master_init(S, 6000, dev)
    m = torch.zeros(S, device=dev)
    v = torch.zeros(S, device=dev)
    ws = torch.zeros(S, dtype=torch.int16, device=dev)
    idx = [sample_indices(sz, 20000, 60 + b, dev) for b, sz in enumerate(sizes)]
    ref = []
    for b, sz in enumerate(sizes):
        sl = slice(int(starts[b]), int(starts[b + 1]))
        ref.append([to_np(p[sl][idx[b]]), np.zeros(idx[b].numel(), np.float32),
                    np.zeros(idx[b].numel(), np.float32), None])
    bmax = max(sizes)
    pool = torch.empty((R * D, bmax), dtype=torch.int16, device=dev)
    for t in range(1, w.steps + 1):
        hp = dict(step=t, **HP)
        for b, sz in enumerate(sizes):
            for k in range(R * D):
                pool[k, :sz].copy_(W.contribution(w, sz, t, b, k, dev))
            cs = [pool[k, :sz] for k in range(R * D)]
            sl = slice(int(starts[b]), int(starts[b + 1]))
            zs.zs_adamw_step_ex(p[sl], m[sl], v[sl], ws[sl], cs, hp, replicas=R,
                                round_to_reduce_dtype=w.round_reduce)
            r = ref[b]
            r[0], r[1], r[2], r[3] = O.rank_step_hybrid(
                r[0], r[1], r[2], [to_np(c[idx[b]]) for c in cs], O.BF16, O.AdamWHP(**hp), R,
                w.round_reduce)
        torch.cuda.synchronize()
        print(f"[{time.strftime('%H:%M:%S')}] step {t} done", flush=True)
    for b, sz in enumerate(sizes):
        sl = slice(int(starts[b]), int(starts[b + 1]))
        what = f"bucket {b}"
        check_f32(to_np(p[sl][idx[b]]), ref[b][0], what + " p", exact=True)
        check_f32(to_np(m[sl][idx[b]]), ref[b][1], what + " m", exact=True)
        check_f32(to_np(v[sl][idx[b]]), ref[b][2], what + " v", exact=True)
        check_bf16(to_np(ws[sl][idx[b]]), ref[b][3], what + " w", exact=True)
