"""The measurement aid zs_stream_ceiling writes the documented placeholders
over the first 1024 * floor(S / 1024) elements (whole tile pairs) and touches
nothing else: p + m into p, v into m, p into v, and into w the first two
words of each 16-byte XOR of the contributions, in the lane maps of the
fused kernel."""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from gpu_util import device, to_np

pytestmark = pytest.mark.gpu

PAIR = 1024          # elements the kernel moves per wavefront and iteration


def expected_w_words(words, dtype, L):
    """u32 words of w[:L] from the contributions' u32 words (first L elements)."""
    x = np.zeros_like(words[0])
    for wd in words:
        x ^= wd
    if dtype == "f32":
        # split map: lane vectors are 4 consecutive fp32 elements; the first two
        # words of each XORed vector land in the 4 bf16 slots of w
        return x.reshape(L // 4, 4)[:, :2].reshape(-1)
    # bf16: per tile, lane l XORs words 4l .. 4l+3 (8 elements); LDS entry k
    # holds lane k >> 1's vector, XORed with 1 when k is odd; w's elements
    # 4k .. 4k+3 get the entry's first two words
    xt = x.reshape(L // 512, 64, 4)
    k = np.arange(128)
    ent = xt[:, k >> 1, :2] ^ (k & 1).astype(np.uint32)[None, :, None]
    return ent.reshape(-1)


@pytest.mark.parametrize("dtype,n", [("bf16", 8), ("bf16", 3), ("f32", 4)])
@pytest.mark.parametrize("S", [1024 * 39 + 69, 1024 * 38 + 512, 300])
def test_stream_ceiling_placeholders(dtype, n, S):
    dev = device()
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
    L = PAIR * (S // PAIR)
    assert to_np(p)[:L].tobytes() == (p0[:L] + m0[:L]).astype(np.float32).tobytes()
    assert to_np(m)[:L].tobytes() == v0[:L].tobytes()
    assert to_np(v)[:L].tobytes() == p0[:L].tobytes()
    assert to_np(p)[L:].tobytes() == p0[L:].tobytes()
    assert to_np(m)[L:].tobytes() == m0[L:].tobytes()
    assert to_np(v)[L:].tobytes() == v0[L:].tobytes()
    assert not to_np(w)[L:].any()
    if L:
        words = [np.ascontiguousarray(to_np(c)[:L]).view(np.uint32) for c in cs]
        want = expected_w_words(words, dtype, L)
        assert np.ascontiguousarray(to_np(w)[:L]).view(np.uint32).tobytes() == want.tobytes()


@pytest.mark.parametrize("per_cu", [0, 1, 3])
def test_hbm_probe_write_copy_read(per_cu):
    dev = device()
    n = (1 << 20) + 48                                  # bytes, a multiple of 16
    guard = 4096
    big = torch.zeros(n + guard, dtype=torch.uint8, device=dev)
    zs.zs_hbm_probe(zs.ZS_PROBE_WRITE, big[:n], blocks_per_cu=per_cu)
    torch.cuda.synchronize()
    words = to_np(big[:n].view(torch.int32)).view(np.uint32).reshape(-1, 4)
    vec = np.arange(n // 16, dtype=np.uint64)
    assert np.array_equal(words[:, 0], (vec & 0xffffffff).astype(np.uint32))
    assert np.array_equal(words[:, 1], (vec >> 32).astype(np.uint32))
    assert np.all(words[:, 2] == 0x5a5a5a5a) and np.all(words[:, 3] == 0)
    assert not to_np(big[n:]).any()

    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev)
    dst = torch.zeros(n + guard, dtype=torch.uint8, device=dev)
    zs.zs_hbm_probe(zs.ZS_PROBE_COPY, src, dst[:n], blocks_per_cu=per_cu)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src) and not to_np(dst[n:]).any()

    before = src.clone()
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    zs.zs_hbm_probe(zs.ZS_PROBE_READ, src, sink, blocks_per_cu=per_cu)
    torch.cuda.synchronize()
    assert torch.equal(src, before)

    two = torch.randint(0, 256, (2 * n,), dtype=torch.uint8, device=dev)
    out = torch.zeros(n + guard, dtype=torch.uint8, device=dev)
    zs.zs_hbm_probe(zs.ZS_PROBE_TRIAD, two, out[:n], blocks_per_cu=per_cu)
    torch.cuda.synchronize()
    want = np.bitwise_xor(to_np(two[:n]), to_np(two[n:]))
    assert np.array_equal(to_np(out[:n]), want) and not to_np(out[n:]).any()
