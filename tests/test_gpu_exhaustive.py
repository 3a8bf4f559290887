"""The fused kernel's fp32 -> bf16 rounding of the working shard, over every
one of the 2^32 fp32 bit patterns, against the oracle's bf16_round (itself
pinned against torch's CPU cast over the same 2^32 patterns).

With lr = 0, weight decay 0 and a zero gradient the step leaves p unchanged
(p * 1 - 0 * (0 / eps) = p exactly, denormals and signed zeros included), so
the bf16 working shard it writes is exactly the rounding of p. One launch
over S = 2^32 elements also exercises 64-bit indexing past 2^31.
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
from oracle import zs_oracle as O
from gpu_util import device

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28


def test_working_shard_rounding_all_fp32_patterns():
    dev = device()
    S = 1 << 32
    p = torch.empty(S, dtype=torch.int32, device=dev)
    for a in range(0, S, CHUNK):                  # p's bits are 0 .. 2^32 - 1 in order
        torch.arange(a - (1 << 31), a - (1 << 31) + CHUNK, dtype=torch.int32, device=dev,
                     out=p[a:a + CHUNK])
    p = p.view(torch.float32)
    m = torch.zeros(S, device=dev)
    v = torch.zeros(S, device=dev)
    w = torch.empty(S, dtype=torch.int16, device=dev)
    g = torch.zeros(S, dtype=torch.int16, device=dev)    # one bf16 contribution of +0
    zs.zs_adamw_step(p, m, v, w, [g], dict(lr=0.0, beta1=0.9, beta2=0.95, eps=1e-8,
                                            weight_decay=0.0, step=1))
    torch.cuda.synchronize()
    for a in range(0, S, CHUNK):
        # element i holds the int32 value i - 2^31, whose bit pattern is i ^ 0x80000000
        bits = np.arange(a, a + CHUNK, dtype=np.uint64).astype(np.uint32) ^ np.uint32(0x80000000)
        x = bits.view(np.float32)
        want = O.bf16_round(x)
        got = w[a:a + CHUNK].cpu().numpy().view(np.uint16)
        nan = (bits & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        bad = np.flatnonzero((got != want) & ~nan)
        assert bad.size == 0, f"chunk at {a}: {bad.size} patterns differ, first bits {bits[bad[0]]:#010x}"
        # NaNs stay NaNs with their sign (their payload bits are the hardware's)
        assert (((got[nan] & 0x7FFF) > 0x7F80) & ((got[nan] >> 15) == (bits[nan] >> 31))).all()
        pb = p[a:a + CHUNK].cpu().numpy().view(np.uint32)
        assert np.array_equal(pb[~nan], bits[~nan]), f"p changed in chunk at {a}"
        print(f"patterns {a:#011x}..{a + CHUNK - 1:#011x} ok", flush=True)
    del p, m, v, w, g
    torch.cuda.empty_cache()


def test_element_at_a_time_path_past_the_grid_cap():
    """Buffers one element off 16-byte alignment take the element-at-a-time
    kernels, one lane per element; at S = 2^32 + 4099 their grid is capped
    at 2^24 - 1 workgroups of 256 (the launch's thread count must fit in 32
    bits) and the kernels loop in grid-stride order over the rest. The fused
    step and the reduce are checked against the oracle on sampled positions,
    both ends, and every element around the first stride boundary
    (2^32 - 256) and past 2^32."""
    from gpu_util import SampledRank, sample_indices, to_np, check_f32
    dev = device()
    S = (1 << 32) + 4099
    stride = ((1 << 32) - 1) // 256 * 256          # threads of the capped grid: 2^32 - 256
    gen = torch.Generator(device=dev)
    gen.manual_seed(321)

    def fill_normal(t, std):
        for a in range(0, S, CHUNK):
            b = min(S, a + CHUNK)
            torch.randn(b - a, generator=gen, device=dev, out=t[a:b]).mul_(std)

    p = torch.empty(S + 1, device=dev)[1:]          # 4 bytes off: not 16-byte aligned
    fill_normal(p, 0.02)
    m = torch.zeros(S + 1, device=dev)[1:]
    v = torch.zeros(S + 1, device=dev)[1:]
    w = torch.empty(S + 1, dtype=torch.int16, device=dev)[1:]
    c = torch.empty(S, dtype=torch.int16, device=dev)
    tmp = torch.empty(CHUNK, device=dev)
    for a in range(0, S, CHUNK):
        b = min(S, a + CHUNK)
        torch.randn(b - a, generator=gen, device=dev, out=tmp[:b - a]).mul_(1e-3)
        c[a:b].copy_(tmp[:b - a].to(torch.bfloat16).view(torch.int16))
    del tmp
    extra = torch.cat([torch.arange(stride - 300, stride + 300, device=dev),
                       torch.arange((1 << 32) - 300, (1 << 32) + 300, device=dev)])
    idx = torch.unique(torch.cat([sample_indices(S, 100_000, 77, dev), extra]))
    orc = SampledRank(idx, p, m, v)
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    zs.zs_adamw_step(p, m, v, w, [c], hp)
    orc.step([c], O.BF16, O.AdamWHP(**hp))
    orc.check(p, m, v, w, "S = 2^32 + 4099, misaligned")
    del m, v, w
    out = torch.empty(S + 1, device=dev)[1:]
    zs.zs_reduce_shard([c, c], out)
    want = O.reduce_shard([to_np(c[idx]), to_np(c[idx])], O.BF16)
    check_f32(to_np(out[idx]), want, "reduce S = 2^32 + 4099, misaligned", exact=True)
    del p, c, out
    torch.cuda.empty_cache()
