"""GPU parity of the D -> D2 re-shard kernel (zs_reshard) and the shard
checkpoints (zs_shard_save / zs_shard_load / zs_shard_load_resharded)
against the CPU oracle: re-sharded shards equal the oracle's reshard bit
for bit; a run saved after 5 steps and resumed for 5 more equals 10 steps
straight and the oracle's 10 steps, at the same D and re-sharded to other
D; corrupt or mismatched files are refused.
"""
import os

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from oracle import zs_oracle as O
from gpu_util import check_bits, device, to_np

pytestmark = pytest.mark.gpu

HP = W.ADAMW_HP


def ceil_div(a, b):
    return -(-a // b)


# ------------------------------------------------------------ zs_reshard
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("seed", range(8))
def test_reshard_random(dtype, seed):
    dev = device()
    rng = np.random.default_rng(seed)
    N = int(rng.choice([1, 5, 63, 1000, 4097, 70001, 300000 + seed]))
    D = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 64]))
    D2 = int(rng.choice([1, 2, 3, 5, 8, 12, 32, 64]))
    tdt = torch.int16 if dtype == "bf16" else torch.float32
    flat = torch.randint(-30000, 30000, (N,), device=dev).to(tdt) if dtype == "bf16" else \
        torch.randn(N, device=dev)
    S, S2 = ceil_div(N, D), ceil_div(N, D2)
    off = seed % 3                          # shards as views at element offsets
    src_buf = torch.zeros(D * (S + 3), dtype=tdt, device=dev)
    src = [src_buf[r * (S + 3) + off:r * (S + 3) + off + S] for r in range(D)]
    want_src = O.pack_flat([to_np(flat)], D)
    for r in range(D):
        src[r].copy_(torch.from_numpy(want_src[r].view(np.int16) if dtype == "bf16"
                                      else want_src[r]).to(dev))
    dst_buf = torch.full((D2 * (S2 + 5),), 77, dtype=tdt, device=dev)
    dst = [dst_buf[r * (S2 + 5) + 1:r * (S2 + 5) + 1 + S2] for r in range(D2)]
    zs.zs_reshard(src, N, dst)
    want = O.reshard([to_np(s) for s in src], N, D2)
    for r in range(D2):
        check_bits(to_np(dst[r]), want[r], f"reshard N={N} D={D}->{D2} shard {r}")


def test_reshard_llama7b_block_full_size():
    """One LLaMA-7B block unit (202,383,360 fp32 elements) from D=8 to D2=12."""
    dev = device()
    unit = W.get("llama7b_block").units[0]
    N = unit.numel
    flat = W.master_init(N, 11, dev)
    src = list(torch.chunk(flat, 8))
    dst = [torch.empty(ceil_div(N, 12), device=dev) for _ in range(12)]
    zs.zs_reshard(src, N, dst)
    want = O.reshard([to_np(s) for s in src], N, 12)
    for r in range(12):
        check_bits(to_np(dst[r]), want[r], f"shard {r}")


def test_reshard_errors():
    dev = device()
    a = [torch.zeros(10, device=dev) for _ in range(4)]
    b = [torch.zeros(14, device=dev) for _ in range(3)]
    with pytest.raises(zs.ZsError) as e:
        zs.zs_reshard(a, 40, b)              # S2 must be ceil(40/3) = 14: ok; S = 10 ok
        torch.cuda.synchronize()
        zs.zs_reshard(a, 41, b)              # S must be ceil(41/4) = 11
    assert e.value.status == zs.ZS_EINVAL
    with pytest.raises(zs.ZsError) as e:
        zs.zs_reshard(a, 40, [a[0][:10], a[1][:10], a[2][:10], a[3][:10]])
    assert e.value.status == zs.ZS_EALIAS


# ------------------------------------------------------------ checkpoints
class Run:
    """D ranks' shard states of one unit on the GPU, and the oracle's copy."""

    def __init__(self, N, D, dev, seed=0):
        self.N, self.D, self.S = N, D, ceil_div(N, D)
        flat = W.master_init(N, 900 + seed, dev)
        self.p = [torch.empty(self.S, device=dev) for _ in range(D)]
        zs.zs_pack_flat([flat], D, self.p)
        self.m = [torch.zeros(self.S, device=dev) for _ in range(D)]
        self.v = [torch.zeros(self.S, device=dev) for _ in range(D)]
        self.w = [torch.zeros(self.S, dtype=torch.int16, device=dev) for _ in range(D)]
        self.op = O.pack_flat([to_np(flat)], D)
        self.om = [np.zeros(self.S, np.float32) for _ in range(D)]
        self.ov = [np.zeros(self.S, np.float32) for _ in range(D)]
        self.ow = [O.bf16_round(x) for x in self.op]

    def step(self, t, dev):
        """One step: D full-unit bf16 gradients, rank r reduces its slice."""
        grads = [W.as_bf16_bits(W.normal_f32(self.D * self.S, W.GRAD_SCALE, 5000 + 100 * t + k, dev))
                 for k in range(self.D)]
        for r in range(self.D):
            cs = [g[r * self.S:(r + 1) * self.S] for g in grads]
            zs.zs_adamw_step(self.p[r], self.m[r], self.v[r], self.w[r], cs, dict(step=t, **HP))
            self.op[r], self.om[r], self.ov[r], self.ow[r] = O.rank_step(
                self.op[r], self.om[r], self.ov[r], [to_np(c) for c in cs], O.BF16,
                O.AdamWHP(step=t, **HP))
        torch.cuda.synchronize()

    def save(self, d, t):
        paths = [os.path.join(d, f"rank{r}.zss") for r in range(self.D)]
        for r in range(self.D):
            zs.zs_shard_save(paths[r], r, self.D, self.N, t, self.p[r], self.m[r], self.v[r], self.w[r])
        return paths

    def check(self, what):
        for r in range(self.D):
            for name, g, o in (("p", self.p, self.op), ("m", self.m, self.om), ("v", self.v, self.ov),
                               ("w", self.w, self.ow)):
                check_bits(to_np(g[r]), o[r], f"{what} rank {r} {name}")


def fresh_like(run, dev):
    return ([torch.full((run.S,), 3.0, device=dev) for _ in range(run.D)],
            [torch.full((run.S,), 3.0, device=dev) for _ in range(run.D)],
            [torch.full((run.S,), 3.0, device=dev) for _ in range(run.D)],
            [torch.full((run.S,), 5, dtype=torch.int16, device=dev) for _ in range(run.D)])


def test_save_and_resume_same_d(tmp_path):
    dev = device()
    straight = Run(3_281_408 + 5, 4, dev)       # the 3.3M GPT's size plus a ragged tail
    resumed = Run(3_281_408 + 5, 4, dev)
    for t in range(1, 6):
        straight.step(t, dev)
        resumed.step(t, dev)
    paths = resumed.save(str(tmp_path), 5)
    p, m, v, w = fresh_like(resumed, dev)
    for r in range(4):
        info = zs.zs_shard_load(paths[r], p[r], m[r], v[r], w[r])
        assert info == dict(rank=r, D=4, N=resumed.N, S=resumed.S, step=5)
        assert zs.zs_shard_info_read(paths[r]) == info
    resumed.p, resumed.m, resumed.v, resumed.w = p, m, v, w
    for t in range(6, 11):
        straight.step(t, dev)
        resumed.step(t, dev)
    straight.check("straight 10 steps vs oracle")
    resumed.check("5 + 5 steps vs oracle")
    for r in range(4):
        for a, b in ((straight.p, resumed.p), (straight.m, resumed.m), (straight.v, resumed.v),
                     (straight.w, resumed.w)):
            assert to_np(a[r]).tobytes() == to_np(b[r]).tobytes()


@pytest.mark.parametrize("D2", [1, 3, 4, 7])
def test_save_and_resume_resharded(tmp_path, D2):
    """Saved at D=4 after 5 steps, loaded at D2, stepped 5 more with D2
    contributions: equal to the oracle re-sharding its own state."""
    dev = device()
    run = Run(1_000_003, 4, dev, seed=1)
    for t in range(1, 6):
        run.step(t, dev)
    paths = run.save(str(tmp_path), 5)
    N, S2 = run.N, ceil_div(run.N, D2)
    new = Run.__new__(Run)
    new.N, new.D, new.S = N, D2, S2
    new.p = [torch.empty(S2, device=dev) for _ in range(D2)]
    new.m = [torch.empty(S2, device=dev) for _ in range(D2)]
    new.v = [torch.empty(S2, device=dev) for _ in range(D2)]
    new.w = [torch.empty(S2, dtype=torch.int16, device=dev) for _ in range(D2)]
    for r in range(D2):
        info = zs.zs_shard_load_resharded(paths, r, D2, new.p[r], new.m[r], new.v[r], new.w[r])
        assert info == dict(rank=r, D=D2, N=N, S=S2, step=5)
    new.op = O.reshard(run.op, N, D2)
    new.om = O.reshard(run.om, N, D2)
    new.ov = O.reshard(run.ov, N, D2)
    new.ow = O.reshard(run.ow, N, D2)
    new.check(f"loaded at D2={D2}")
    for t in range(6, 11):
        new.step(t, dev)
    new.check(f"resumed at D2={D2}, 10 steps")


def test_multi_block_files_and_partial_reads(tmp_path):
    """Arrays of 80 MB (5 CRC blocks, 2 staging windows): loads that start
    and end mid-block and cross windows."""
    dev = device()
    N, D = 80_000_003, 4
    run = Run(N, D, dev, seed=2)
    run.step(1, dev)
    paths = run.save(str(tmp_path), 1)
    for D2 in (3, 5):
        S2 = ceil_div(N, D2)
        want = O.reshard(run.op, N, D2), O.reshard(run.ow, N, D2)
        for r in range(D2):
            p = torch.empty(S2, device=dev)
            m = torch.empty(S2, device=dev)
            v = torch.empty(S2, device=dev)
            w = torch.empty(S2, dtype=torch.int16, device=dev)
            zs.zs_shard_load_resharded(paths, r, D2, p, m, v, w)
            check_bits(to_np(p), want[0][r], f"D2={D2} rank {r} p")
            check_bits(to_np(w), want[1][r], f"D2={D2} rank {r} w")


def test_corrupt_and_mismatched_files(tmp_path):
    dev = device()
    run = Run(100_003, 2, dev, seed=3)
    run.step(1, dev)
    a = run.save(str(tmp_path), 1)
    other = tmp_path / "other"
    other.mkdir()
    run.step(2, dev)
    b = run.save(str(other), 2)
    p, m, v, w = (x[0] for x in fresh_like(run, dev))
    # files of two different checkpoints
    with pytest.raises(zs.ZsError) as e:
        zs.zs_shard_load_resharded([a[0], b[1]], 0, 3, p[:ceil_div(run.N, 3)], m[:ceil_div(run.N, 3)],
                                   v[:ceil_div(run.N, 3)], w[:ceil_div(run.N, 3)])
    assert e.value.status == zs.ZS_EIO
    # ranks in the wrong order
    with pytest.raises(zs.ZsError) as e:
        zs.zs_shard_load_resharded([a[1], a[0]], 0, 2, p, m, v, w)
    assert e.value.status == zs.ZS_EIO
    # a flipped data byte
    raw = bytearray(open(a[0], "rb").read())
    raw[4096 + 12345] ^= 0x10
    bad = tmp_path / "bad.zss"
    bad.write_bytes(bytes(raw))
    with pytest.raises(zs.ZsError) as e:
        zs.zs_shard_load(str(bad), p, m, v, w)
    assert e.value.status == zs.ZS_EIO and "checksum" in zs.zs_last_error()
    # a flipped header byte
    raw = bytearray(open(a[0], "rb").read())
    raw[30] ^= 1
    bad.write_bytes(bytes(raw))
    with pytest.raises(zs.ZsError) as e:
        zs.zs_shard_info_read(str(bad))
    assert e.value.status == zs.ZS_EIO
    # a truncated file
    bad.write_bytes(open(a[0], "rb").read()[:5000])
    with pytest.raises(zs.ZsError) as e:
        zs.zs_shard_load(str(bad), p, m, v, w)
    assert e.value.status == zs.ZS_EIO
    # wrong buffer length for a same-D load
    with pytest.raises(zs.ZsError) as e:
        zs.zs_shard_load(a[0], p[:-1], m[:-1], v[:-1], w[:-1])
    assert e.value.status == zs.ZS_EINVAL
    # the intact file still loads
    zs.zs_shard_load(a[0], p, m, v, w)
    torch.cuda.synchronize()
