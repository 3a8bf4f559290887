"""The measurement aid zs_stream_ceiling writes the documented placeholders
(p + m, v, p, XOR of the contributions' 16-byte vectors) over the first
8 * floor(S / 8) elements and touches nothing else."""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from gpu_util import device, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,n", [("bf16", 8), ("bf16", 3), ("f32", 4)])
def test_stream_ceiling_placeholders(dtype, n):
    dev = device()
    S = 8 * 5000 + 5
    p = W.master_init(S, 1, dev)
    m = W.master_init(S, 2, dev)
    v = W.master_init(S, 3, dev)
    w = torch.zeros(S, dtype=torch.int16, device=dev)
    cs = [W.normal_f32(S, 1e-3, 10 + k, dev) for k in range(n)]
    if dtype == "bf16":
        cs = [W.as_bf16_bits(c) for c in cs]
    p0, m0, v0 = to_np(p), to_np(m), to_np(v)
    zs.zs_stream_ceiling(p, m, v, w, cs)
    torch.cuda.synchronize()
    L = 8 * (S // 8)
    assert to_np(p)[:L].tobytes() == (p0[:L] + m0[:L]).astype(np.float32).tobytes()
    assert to_np(m)[:L].tobytes() == v0[:L].tobytes()
    assert to_np(v)[:L].tobytes() == p0[:L].tobytes()
    assert to_np(p)[L:].tobytes() == p0[L:].tobytes()
    words = [np.ascontiguousarray(to_np(c)[:L]).view(np.uint32) for c in cs]
    per_vec = 4 if dtype == "bf16" else 8          # u32 words per 8 elements of one contribution
    x = np.zeros((L // 8, 4), np.uint32)
    for wd in words:
        blk = wd[:L // 8 * per_vec].reshape(L // 8, per_vec // 4, 4)
        for h in range(per_vec // 4):
            x ^= blk[:, h, :]
    assert np.ascontiguousarray(to_np(w)[:L]).view(np.uint32).tobytes() == x.reshape(-1).tobytes()
