"""GPU: zs_adamw_step_timed, the fused step whose kernel launch carries two
timing events, and zs_stream_ceiling_timed. The step's results are the
oracle's (and zs_adamw_step_ex's) bit for bit on aligned and misaligned
buffers, flat and HYBRID_SHARD; the events hold each kernel's own start and
end: a positive time no longer than the time between plain events recorded
around the same call."""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from oracle import zs_oracle as O
from gpu_util import check_bf16, check_f32, device, to_np

pytestmark = pytest.mark.gpu

HP = W.ADAMW_HP


def inputs(S, n, dtype, seed, dev, offset):
    cs = []
    for k in range(n):
        x = W.normal_f32(S + offset, W.GRAD_SCALE, seed * 100 + k, dev)
        x = W.as_bf16_bits(x) if dtype == O.BF16 else x
        cs.append(x[offset:])
    p = W.master_init(S + offset, seed, dev)[offset:]
    m = torch.zeros(S + offset, device=dev)[offset:]
    v = torch.zeros(S + offset, device=dev)[offset:]
    w = torch.zeros(S + offset, dtype=torch.int16, device=dev)[offset:]
    return p, m, v, w, cs


def timing_events():
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for x in e:
        x.record()                     # creates the event
    return e


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32])
@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("R,D", [(1, 8), (1, 5), (4, 8)])
def test_timed_step_matches_oracle(dtype, offset, R, D):
    dev = device()
    S = 3 * 2048 * 8 + 77
    p, m, v, w, cs = inputs(S, R * D, dtype, 31 + D, dev, offset)
    snap = (to_np(p), to_np(m), to_np(v), [to_np(c) for c in cs])
    start, stop = timing_events()
    h = zs.AdamWHP(step=3, **HP)
    zs.zs_adamw_step_timed(p, m, v, w, cs, h, start, stop, replicas=R,
                           keep_working_shard=(offset == 0))
    torch.cuda.synchronize()
    p0, m0, v0, c0 = snap
    if R == 1:
        want = O.rank_step(p0, m0, v0, c0, dtype, O.AdamWHP(step=3, **HP))
    else:
        want = O.rank_step_hybrid(p0, m0, v0, c0, dtype, O.AdamWHP(step=3, **HP), R, False)
    for name, got, ref in zip("pmv", (p, m, v), want[:3]):
        check_f32(to_np(got), ref, f"timed {name} R={R} D={D}", exact=True)
    check_bf16(to_np(w), want[3], f"timed w R={R} D={D}", exact=True)
    assert start.elapsed_time(stop) > 0.0


def test_timed_step_equals_untimed_and_times_the_kernel():
    dev = device()
    S = 106_956_800 // 8                # a 13.4M-param shard: a kernel of about 0.1 ms
    pa, ma, va, wa, cs = inputs(S, 8, O.BF16, 7, dev, 0)
    pb, mb, vb, wb = pa.clone(), ma.clone(), va.clone(), wa.clone()
    h = zs.AdamWHP(step=1, **HP)
    start, stop = timing_events()
    outer = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    kernel_ms, outer_ms = [], []
    for t in range(1, 6):
        h = zs.AdamWHP(step=t, **HP)
        outer[0].record()
        zs.zs_adamw_step_timed(pa, ma, va, wa, cs, h, start, stop)
        outer[1].record()
        zs.zs_adamw_step_ex(pb, mb, vb, wb, cs, h)
        torch.cuda.synchronize()
        kernel_ms.append(start.elapsed_time(stop))
        outer_ms.append(outer[0].elapsed_time(outer[1]))
    for a, b in ((pa, pb), (ma, mb), (va, vb), (wa, wb)):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b)
    # the kernel's own time: positive, and within the plain events around the call
    for k, o in zip(kernel_ms, outer_ms):
        assert 0.0 < k <= o * 1.0001 + 1e-3, (kernel_ms, outer_ms)
    assert np.median(kernel_ms) > 0.02, kernel_ms


def test_timed_step_rejects_missing_or_shared_events():
    dev = device()
    p, m, v, w, cs = inputs(4096, 2, O.BF16, 3, dev, 0)
    e0, e1 = timing_events()
    h = zs.AdamWHP(step=1, **HP)
    with pytest.raises(ValueError):
        zs.zs_adamw_step_timed(p, m, v, w, cs, h, torch.cuda.Event(enable_timing=True), e1)
    with pytest.raises(zs.ZsError):
        zs.zs_adamw_step_timed(p, m, v, w, cs, h, e0, e0)


def test_timed_ceiling_times_its_kernel():
    dev = device()
    S = 106_956_800 // 8
    p, m, v, w, cs = inputs(S, 8, O.BF16, 9, dev, 0)
    start, stop = timing_events()
    outer = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(3):
        outer[0].record()
        zs.zs_stream_ceiling_timed(p, m, v, w, cs, start, stop)
        outer[1].record()
        torch.cuda.synchronize()
        k, o = start.elapsed_time(stop), outer[0].elapsed_time(outer[1])
        assert 0.02 < k <= o * 1.0001 + 1e-3, (k, o)
