"""zs_step_pipelined_static -- the pipelined step with its staging in the
library's own device array, for callers that cannot allocate -- against the
existing zs_step_pipelined on identical state and sources, bit for bit, over
two calls in a row, the second on smaller inputs. Buckets larger than one
64 MiB staging slot go through the array in pieces; the cases cover that
split, a ragged tail, an empty bucket, a misaligned bucket, pinned host
sources and both reduce dtypes. One bucket is also checked against the
oracle."""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from gpu_util import check_bf16, check_f32, device, to_np
from oracle import zs_oracle as O

pytestmark = pytest.mark.gpu


def sources(sizes, n, code, seed, dev, host):
    out = []
    for b, S in enumerate(sizes):
        row = []
        for k in range(n):
            x = W.normal_f32(S, W.GRAD_SCALE, seed * 1000 + 64 * b + k, dev)
            x = W.as_bf16_bits(x) if code == zs.ZS_BF16 else x
            if host:
                h = torch.empty(S, dtype=x.dtype, pin_memory=True)
                h.copy_(x)
                x = h
            row.append(x)
        out.append(row)
    return out


def states(sizes, seed, dev, offsets):
    out = []
    for b, (S, off) in enumerate(zip(sizes, offsets)):
        p = W.master_init(S + off, seed + b, dev)[off:]
        m = torch.zeros(S + off, device=dev)[off:]
        v = torch.zeros(S + off, device=dev)[off:]
        w = torch.zeros(S + off, dtype=torch.int16, device=dev)[off:]
        out.append([p, m, v, w])
    return out


def clone(st):
    return [[t.clone() for t in b] for b in st]


def one_call(sizes, n, code, seed, host, offsets, steps, dev, compute, transfer):
    src = sources(sizes, n, code, seed, dev, host)
    ref = states(sizes, seed, dev, offsets)
    new = clone(ref)
    init = clone(ref)
    dt = torch.int16 if code == zs.ZS_BF16 else torch.float32
    smax = max(sizes)
    staging = (torch.empty((n, smax), dtype=dt, device=dev),
               torch.empty((n, smax), dtype=dt, device=dev))
    for t in range(1, steps + 1):
        hp = dict(step=t, **W.ADAMW_HP)
        zs.zs_step_pipelined([(*ref[b], src[b]) for b in range(len(sizes))], staging, hp,
                             compute, transfer)
        zs.zs_step_pipelined_static([(*new[b], src[b]) for b in range(len(sizes))], hp,
                                    compute, transfer)
    torch.cuda.synchronize()
    for b, S in enumerate(sizes):
        what = f"bucket {b} (S={S}, n={n}, host={host})"
        for j, name in enumerate(("p", "m", "v")):
            check_f32(to_np(new[b][j]), to_np(ref[b][j]), f"{what} {name}", exact=True)
        check_bf16(to_np(new[b][3]), to_np(ref[b][3]), f"{what} w", exact=True)
    return src, init, new


def test_static_staging_matches_pipelined_two_calls():
    dev = device()
    compute, transfer = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    # call 1: 8 bf16 contributions; 5,000,000 elements is more than one slot
    # (pieces of 4,194,304), then a ragged bucket, an empty one and one whose
    # arrays start one element off 16 bytes
    sizes1 = [5_000_000, 1_000_003, 0, 300_001]
    src, init, new = one_call(sizes1, 8, zs.ZS_BF16, 11, False, [0, 0, 0, 1], 2, dev,
                              compute, transfer)
    # the ragged bucket against the oracle as well (two steps)
    b = 1
    op, om, ov = to_np(init[b][0]), np.zeros(sizes1[b], np.float32), np.zeros(sizes1[b], np.float32)
    for t in (1, 2):
        op, om, ov, ow = O.rank_step(op, om, ov, [to_np(c) for c in src[b]], O.BF16,
                                     O.AdamWHP(step=t, **W.ADAMW_HP))
    check_f32(to_np(new[b][0]), op, "oracle p", exact=True)
    check_bf16(to_np(new[b][3]), ow, "oracle w", exact=True)
    del src, init, new
    # call 2, smaller: 3 fp32 contributions from pinned host memory
    one_call([100_000, 4_097], 3, zs.ZS_F32, 12, True, [0, 0], 1, dev, compute, transfer)


def test_static_staging_many_pieces():
    """64 fp32 contributions: pieces of 262,144 elements, three per bucket."""
    dev = device()
    compute, transfer = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    one_call([600_000], 64, zs.ZS_F32, 13, False, [0], 1, dev, compute, transfer)
    one_call([262_144, 10], 64, zs.ZS_F32, 14, False, [0, 0], 1, dev, compute, transfer)


def test_static_staging_argument_errors():
    dev = device()
    p = torch.zeros(1024, device=dev)
    m, v = torch.zeros_like(p), torch.zeros_like(p)
    w = torch.zeros(1024, dtype=torch.int16, device=dev)
    c = [torch.zeros(1024, dtype=torch.int16, device=dev) for _ in range(2)]
    with pytest.raises(zs.ZsError):
        zs.zs_step_pipelined_static([(p, m, v, w, c)], dict(step=0, **W.ADAMW_HP))
    with pytest.raises(zs.ZsError):                   # a source over p
        zs.zs_step_pipelined_static([(p, m, v, w, [c[0], p.view(torch.int16)[:1024]])],
                                    dict(step=1, **W.ADAMW_HP))
