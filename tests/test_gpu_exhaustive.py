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
