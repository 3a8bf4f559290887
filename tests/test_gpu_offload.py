"""GPU parity of the ZeRO-Offload step (zs_offload_step): device reduce,
gradient down in chunks, host AdamW, working shard up -- bit-identical to
the device step zs_adamw_step and to the oracle's rank step, over several
steps, for both reduce dtypes, chunk sizes that do and do not divide S,
pinned and pageable host buffers, and one or two streams."""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from oracle import zs_oracle as O
from gpu_util import check_bf16, check_f32, device, to_np

pytestmark = pytest.mark.gpu

HP = W.ADAMW_HP


def host(n, dtype, pinned):
    return torch.zeros(n, dtype=dtype, pin_memory=pinned)


@pytest.mark.parametrize("dtype", [O.BF16, O.FP32])
@pytest.mark.parametrize("S,chunk,pinned,two_streams",
                         [(1_000_003, 1 << 18, True, True), (777_777, 777_777, True, False),
                          (50_001, 4096, False, True), (8, 3, True, True)])
def test_offload_matches_device_step_and_oracle(dtype, S, chunk, pinned, two_streams):
    dev = device()
    D = 8
    p0 = W.master_init(S, 31, dev)
    # device reference state
    pd, md, vd = p0.clone(), torch.zeros(S, device=dev), torch.zeros(S, device=dev)
    wd = torch.zeros(S, dtype=torch.int16, device=dev)
    # offload state: p, m, v on the host
    ph, mh, vh = host(S, torch.float32, pinned), host(S, torch.float32, pinned), host(S, torch.float32, pinned)
    ph.copy_(p0)
    wh = host(S, torch.int16, pinned)
    gh = host(S, torch.float32, pinned)
    gdev = torch.empty(S, device=dev)
    wdev = torch.zeros(S, dtype=torch.int16, device=dev)
    op, om, ov = to_np(p0), np.zeros(S, np.float32), np.zeros(S, np.float32)
    stream = torch.cuda.Stream(device=dev)
    h2d = torch.cuda.Stream(device=dev) if two_streams else stream
    for t in (1, 2, 3):
        if dtype == O.BF16:
            cs = [W.as_bf16_bits(W.normal_f32(S, W.GRAD_SCALE, 70 * t + k, dev)) for k in range(D)]
        else:
            cs = [W.normal_f32(S, W.GRAD_SCALE, 70 * t + k, dev) for k in range(D)]
        torch.cuda.synchronize()
        hp = dict(step=t, **HP)
        zs.zs_offload_step(cs, gdev, gh, ph, mh, vh, wh, wdev, hp, threads=8, chunk=chunk,
                           stream=stream, h2d_stream=h2d)
        h2d.synchronize()
        stream.synchronize()
        zs.zs_adamw_step(pd, md, vd, wd, cs, hp)
        op, om, ov, ow = O.rank_step(op, om, ov, [to_np(c) for c in cs], dtype, O.AdamWHP(**hp))
        torch.cuda.synchronize()
        what = f"S={S} chunk={chunk} step {t}"
        check_f32(ph.numpy(), op, what + " p", exact=True)
        check_f32(mh.numpy(), om, what + " m", exact=True)
        check_f32(vh.numpy(), ov, what + " v", exact=True)
        check_bf16(to_np(wdev), ow, what + " w", exact=True)
        assert ph.numpy().tobytes() == to_np(pd).tobytes()
        assert to_np(wdev).tobytes() == to_np(wd).tobytes()
        check_f32(gh.numpy(), O.reduce_shard([to_np(c) for c in cs], dtype), what + " g", exact=True)


def test_offload_errors():
    dev = device()
    S = 1000
    cs = [W.as_bf16_bits(W.normal_f32(S, 1e-3, k, dev)) for k in range(2)]
    gdev = torch.empty(S, device=dev)
    wdev = torch.empty(S, dtype=torch.int16, device=dev)
    ph, mh, vh, gh = (torch.zeros(S) for _ in range(4))
    wh = torch.zeros(S, dtype=torch.int16)
    with pytest.raises(zs.ZsError) as e:
        zs.zs_offload_step(cs, gdev, gh, ph, mh, vh, wh, wdev, dict(step=1, **HP), chunk=0)
    assert e.value.status == zs.ZS_EINVAL
    with pytest.raises(zs.ZsError) as e:
        zs.zs_offload_step(cs, gdev, gh, ph, ph, vh, wh, wdev, dict(step=1, **HP))
    assert e.value.status == zs.ZS_EALIAS
    with pytest.raises(zs.ZsError) as e:
        zs.zs_offload_step(cs, gdev, gh, ph, mh, vh, wh, gdev[:S // 2].view(torch.int16),
                           dict(step=1, **HP))
    assert e.value.status == zs.ZS_EALIAS
    torch.cuda.synchronize()
