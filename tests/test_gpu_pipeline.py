"""GPU parity of the pipelined shard step (zs_step_pipelined) against the
CPU oracle: a sequence of buckets whose contributions are copied into two
alternating staging slots on one stream while the fused step runs on
another. The arithmetic is the fused step's, so every bucket must match the
oracle's rank step bit for bit, whatever the overlap did to the timing.
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from oracle import zs_oracle as O
from gpu_util import check_bf16, check_f32, device, to_np

pytestmark = pytest.mark.gpu

HP = W.ADAMW_HP


class Shard:
    """One bucket's device state and the oracle's copy of it."""

    def __init__(self, S, seed, dev):
        self.p = W.master_init(S, seed, dev)
        self.m = torch.zeros(S, device=dev)
        self.v = torch.zeros(S, device=dev)
        self.w = torch.full((S,), 0x7F7F, dtype=torch.int16, device=dev)
        self.op, self.om, self.ov = to_np(self.p), np.zeros(S, np.float32), np.zeros(S, np.float32)
        self.ow = None

    def oracle_step(self, sources, dtype, t):
        cs = [to_np(c) for c in sources]
        self.op, self.om, self.ov, self.ow = O.rank_step(
            self.op, self.om, self.ov, cs, dtype, O.AdamWHP(step=t, **HP))

    def check(self, what):
        if self.p.numel() == 0:
            return
        check_f32(to_np(self.p), self.op, what + " p", exact=True)
        check_f32(to_np(self.m), self.om, what + " m", exact=True)
        check_f32(to_np(self.v), self.ov, what + " v", exact=True)
        check_bf16(to_np(self.w), self.ow, what + " w", exact=True)


def make_sources(n, S, dtype, seed, dev, host):
    if dtype == O.BF16:
        cs = [W.as_bf16_bits(W.normal_f32(S, W.GRAD_SCALE, seed * 100 + k, dev)) for k in range(n)]
    else:
        cs = [W.normal_f32(S, W.GRAD_SCALE, seed * 100 + k, dev) for k in range(n)]
    if host:
        pinned = []
        for c in cs:
            h = torch.empty(c.shape, dtype=c.dtype, pin_memory=True)
            h.copy_(c)
            pinned.append(h)
        cs = pinned
    return cs


def run_pipeline(sizes, n_contrib, dtype, steps, host, staging_len=None, same_stream=False,
                 seed=0):
    dev = device()
    tdt = torch.int16 if dtype == O.BF16 else torch.float32
    shards = [Shard(S, 500 + seed * 50 + b, dev) for b, S in enumerate(sizes)]
    L = staging_len if staging_len is not None else max(sizes)
    staging = (torch.empty((n_contrib, L), dtype=tdt, device=dev),
               torch.empty((n_contrib, L), dtype=tdt, device=dev))
    compute = torch.cuda.Stream(device=dev)
    transfer = compute if same_stream else torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        srcs = [make_sources(n_contrib, S, dtype, 1000 * seed + 10 * t + b, dev, host)
                for b, S in enumerate(sizes)]
        torch.cuda.synchronize()
        buckets = [(s.p, s.m, s.v, s.w, src) for s, src in zip(shards, srcs)]
        zs.zs_step_pipelined(buckets, staging, dict(step=t, **HP), compute, transfer)
        # the library's streams are unknown to torch's caching allocators:
        # keep every source alive until the copies are done
        torch.cuda.synchronize()
        for s, src in zip(shards, srcs):
            s.oracle_step(src, dtype, t)
    torch.cuda.synchronize()
    for b, s in enumerate(shards):
        s.check(f"bucket {b} (S={sizes[b]})")


RAGGED = [4096, 1000, 0, 8 * 1024 + 3, 17, 2048, 5000, 1]


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32])
def test_pipeline_device_sources(dtype):
    run_pipeline(RAGGED, 4, dtype, steps=3, host=False)


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32])
def test_pipeline_pinned_host_sources(dtype):
    run_pipeline(RAGGED, 3, dtype, steps=2, host=True, seed=1)


def test_pipeline_unaligned_staging_slots():
    """A staging length that is not a multiple of 8 puts contribution q's
    slot offset off 16-byte alignment: the element-wise kernel runs."""
    run_pipeline([333, 4096, 77], 5, O.BF16, steps=2, host=False, staging_len=4099, seed=2)


def test_pipeline_one_stream_and_many_contributions():
    run_pipeline([20000, 12345, 8], 16, O.BF16, steps=2, host=False, same_stream=True, seed=3)


def test_pipeline_back_to_back_calls_share_staging():
    """Two calls enqueued without a host sync in between: the second call's
    copies must wait for the first call's steps to release the slots."""
    dev = device()
    sizes = [300000, 250000, 310000]
    n = 8
    shards = [Shard(S, 900 + b, dev) for b, S in enumerate(sizes)]
    staging = (torch.empty((n, max(sizes)), dtype=torch.int16, device=dev),
               torch.empty((n, max(sizes)), dtype=torch.int16, device=dev))
    compute, transfer = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    srcs = {t: [make_sources(n, S, O.BF16, 7000 + 10 * t + b, dev, False)
                for b, S in enumerate(sizes)] for t in (1, 2, 3)}
    torch.cuda.synchronize()
    for t in (1, 2, 3):
        zs.zs_step_pipelined([(s.p, s.m, s.v, s.w, src) for s, src in zip(shards, srcs[t])],
                             staging, dict(step=t, **HP), compute, transfer)
    torch.cuda.synchronize()
    for t in (1, 2, 3):
        for s, src in zip(shards, srcs[t]):
            s.oracle_step(src, O.BF16, t)
    for b, s in enumerate(shards):
        s.check(f"bucket {b}")


def test_pipeline_matches_adamw_step_per_bucket():
    """The same buckets stepped by zs_adamw_step one by one give the same bits."""
    dev = device()
    sizes = [5000, 4096, 123]
    a = [Shard(S, 40 + b, dev) for b, S in enumerate(sizes)]
    b_ = [Shard(S, 40 + b, dev) for b, S in enumerate(sizes)]
    srcs = [make_sources(8, S, O.BF16, 300 + i, dev, False) for i, S in enumerate(sizes)]
    staging = (torch.empty((8, 5000), dtype=torch.int16, device=dev),
               torch.empty((8, 5000), dtype=torch.int16, device=dev))
    zs.zs_step_pipelined([(s.p, s.m, s.v, s.w, src) for s, src in zip(a, srcs)], staging,
                         dict(step=1, **HP))
    for s, src in zip(b_, srcs):
        zs.zs_adamw_step(s.p, s.m, s.v, s.w, src, dict(step=1, **HP))
    torch.cuda.synchronize()
    for x, y in zip(a, b_):
        for f in ("p", "m", "v", "w"):
            assert to_np(getattr(x, f)).tobytes() == to_np(getattr(y, f)).tobytes(), f


def test_pipeline_errors():
    dev = device()
    s = Shard(1000, 1, dev)
    src = make_sources(2, 1000, O.BF16, 5, dev, False)
    small = (torch.empty((2, 999), dtype=torch.int16, device=dev),
             torch.empty((2, 999), dtype=torch.int16, device=dev))
    with pytest.raises(zs.ZsError) as e:
        zs.zs_step_pipelined([(s.p, s.m, s.v, s.w, src)], small, dict(step=1, **HP))
    assert e.value.status == zs.ZS_EINVAL and "staging_len" in zs.zs_last_error()
    ok = (torch.empty((2, 1000), dtype=torch.int16, device=dev),
          torch.empty((2, 1000), dtype=torch.int16, device=dev))
    with pytest.raises(zs.ZsError) as e:   # a source inside a staging slot
        zs.zs_step_pipelined([(s.p, s.m, s.v, s.w, [ok[0][1], src[1]])], ok, dict(step=1, **HP))
    assert e.value.status == zs.ZS_EALIAS
    with pytest.raises(zs.ZsError) as e:   # two buckets sharing p
        zs.zs_step_pipelined([(s.p, s.m, s.v, s.w, src), (s.p, s.m.clone(), s.v.clone(),
                                                          s.w.clone(), src)], ok, dict(step=1, **HP))
    assert e.value.status == zs.ZS_EALIAS
    with pytest.raises(ValueError):        # pageable host memory is refused by the binding
        zs.zs_step_pipelined([(s.p, s.m, s.v, s.w, [c.cpu() for c in src])], ok, dict(step=1, **HP))
    zs.zs_step_pipelined([], ok, dict(step=1, **HP))    # no buckets: nothing to do
    torch.cuda.synchronize()
