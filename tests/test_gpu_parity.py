"""GPU parity of every entry point against the CPU oracle, at sizes the
oracle finishes in seconds: several tiles, ragged tails, every alignment,
D from 1 to 64, both reduce dtypes, and the degenerate cases.

Bar: pack, gather and the bf16 bit moves are bit-exact; p, m, v within
rel 1e-6 and w within 1 bf16 ulp of the oracle, and, because the kernels
follow the oracle's operation order, also bit-identical (checked too).
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zs_amd as zs
import workloads as W
from oracle import zs_oracle as O
from gpu_util import (check_bf16, check_bits, check_f32, device, to_np)

pytestmark = pytest.mark.gpu

HP = W.ADAMW_HP


def bf16_contribs(n, S, seed, dev, scale=W.GRAD_SCALE):
    return [W.as_bf16_bits(W.normal_f32(S, scale, seed * 100 + k, dev)) for k in range(n)]


def f32_contribs(n, S, seed, dev, scale=W.GRAD_SCALE):
    return [W.normal_f32(S, scale, seed * 100 + k, dev) for k in range(n)]


def oracle_dtype(code):
    return O.BF16 if code == zs.ZS_BF16 else O.FP32


# ------------------------------------------------------------------ pack
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("seed", range(6))
def test_pack_and_gather_random_units(dtype, seed):
    dev = device()
    rng = np.random.default_rng(seed)
    unit = W.small_random_unit(rng, max_tensors=14, max_numel=40000)
    D = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 16, 31, 64]))
    ts = W.tensor_values(unit, dtype, 1000 + seed, dev)
    _, N, N_pad, S = zs.zs_unit_layout(unit.numels, D)
    tdt = torch.int16 if dtype == "bf16" else torch.float32
    shards = [torch.full((S,), 77, dtype=tdt, device=dev) for _ in range(D)]
    if S:
        zs.zs_pack_flat([t.reshape(-1) for t in ts], D, shards)
    want = O.pack_flat([to_np(t) for t in ts], D)
    for r in range(D):
        check_bits(to_np(shards[r]), want[r], f"shard {r} (D={D}, N={N})")
    flat = torch.full((N_pad,), 55, dtype=tdt, device=dev)
    if S:
        zs.zs_gather_unit(shards, flat)
    check_bits(to_np(flat), O.gather_unit(want), "gather")
    for t, view in zip(ts, O.unit_views(to_np(flat), [tuple(t.shape) for t in ts])):
        check_bits(to_np(t).reshape(-1), view.reshape(-1), "tensor view")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_every_source_alignment(dtype):
    """Tensors as views at every element offset of one buffer, and shard
    lengths that put every shard boundary at a different alignment."""
    dev = device()
    tdt = torch.int16 if dtype == "bf16" else torch.float32
    base = torch.arange(1, 200000, device=dev).to(tdt)
    for D in (3, 8):
        ts, pos = [], 0
        for j, n in enumerate([9, 1, 1000, 33, 4097, 2, 0, 515, 8191]):
            pos += j % 8 + 1
            ts.append(base[pos:pos + n])
            pos += n
        numels = [t.numel() for t in ts]
        _, N, N_pad, S = zs.zs_unit_layout(numels, D)
        shards = [torch.empty(S, dtype=tdt, device=dev) for _ in range(D)]
        zs.zs_pack_flat(ts, D, shards)
        want = O.pack_flat([to_np(t) for t in ts], D)
        for r in range(D):
            check_bits(to_np(shards[r]), want[r], f"shard {r} D={D}")
        # gather into a misaligned flat view
        buf = torch.zeros(N_pad + 8, dtype=tdt, device=dev)
        for off in (1, 3):
            flat = buf[off:off + N_pad]
            zs.zs_gather_unit(shards, flat)
            check_bits(to_np(flat), O.gather_unit(want), f"gather off={off}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [63, 64, 65, 300, 4097])
def test_pack_many_tensors(dtype, T):
    """Long tensor tables (up to 4,097 entries) for the search of each work
    item's first tensor; a third of the tensors are empty and many hold one
    element, so that runs of table entries end at the same flat offset, and
    the sources sit at assorted alignments."""
    dev = device()
    rng = np.random.default_rng(T)
    tdt = torch.int16 if dtype == "bf16" else torch.float32
    numels = [int(x) for x in rng.choice([0, 0, 1, 3, 17, 700, 5000], size=T)]
    base = torch.arange(1, sum(numels) + 8 * T + 8, device=dev).to(tdt)
    ts, pos = [], 0
    for j, n in enumerate(numels):
        pos += j % 3                       # sources at assorted alignments
        ts.append(base[pos:pos + n])
        pos += n
    for D in (1, 5, 16):
        _, N, N_pad, S = zs.zs_unit_layout(numels, D)
        if S == 0:
            continue
        shards = [torch.full((S,), 77, dtype=tdt, device=dev) for _ in range(D)]
        zs.zs_pack_flat(ts, D, shards)
        want = O.pack_flat([to_np(t) for t in ts], D)
        for r in range(D):
            check_bits(to_np(shards[r]), want[r], f"T={T} D={D} shard {r}")


def test_pack_gpt3m_unit():
    """The 3.3M-parameter GPT unit (43 tensors), fp32 and bf16, D = 4."""
    dev = device()
    w = W.get("gpt3m")
    unit = w.units[0]
    for dtype in ("f32", "bf16"):
        ts = W.tensor_values(unit, dtype, 1, dev)
        _, N, N_pad, S = zs.zs_unit_layout(unit.numels, w.D)
        tdt = torch.int16 if dtype == "bf16" else torch.float32
        shards = [torch.empty(S, dtype=tdt, device=dev) for _ in range(w.D)]
        zs.zs_pack_flat([t.reshape(-1) for t in ts], w.D, shards)
        want = O.pack_flat([to_np(t) for t in ts], w.D)
        for r in range(w.D):
            check_bits(to_np(shards[r]), want[r], f"{dtype} shard {r}")


def test_pack_pad_written_as_zero_and_nothing_else():
    """The pad is +0 and bytes outside the shards (canaries) are untouched."""
    dev = device()
    D, numels = 8, [5, 6]                     # N = 11 -> S = 2, pad 5, shards 6, 7 all pad
    ts = [torch.full((n,), -1.5, device=dev) for n in numels]
    _, N, N_pad, S = zs.zs_unit_layout(numels, D)
    guard = 64
    bufs = [torch.full((S + 2 * guard,), 9.25, device=dev) for _ in range(D)]
    shards = [b[guard:guard + S] for b in bufs]
    zs.zs_pack_flat(ts, D, shards)
    flat = np.concatenate([to_np(s) for s in shards])
    assert np.all(flat[:N] == -1.5) and flat[N:].tobytes() == bytes(4 * (N_pad - N))
    for b in bufs:
        g = to_np(b)
        assert np.all(g[:guard] == 9.25) and np.all(g[guard + S:] == 9.25)


# --------------------------------------------------------------- reduce
@pytest.mark.parametrize("code", [zs.ZS_BF16, zs.ZS_F32])
@pytest.mark.parametrize("D", [1, 2, 3, 4, 5, 8, 13, 16, 32, 64])
def test_reduce_vs_oracle(code, D):
    dev = device()
    for S in (1, 7, 8, 9, 1000, 65537, 262147):
        gen = bf16_contribs if code == zs.ZS_BF16 else f32_contribs
        cs = gen(D, S, D * 7 + S % 97, dev)
        out = torch.empty(S, device=dev)
        zs.zs_reduce_shard(cs, out)
        want = O.reduce_shard([to_np(c) for c in cs], oracle_dtype(code))
        check_f32(to_np(out), want, f"reduce D={D} S={S}", exact=True)


def test_reduce_rank_order_adversarial():
    """(2^25, 1, -2^25, 1) folded left to right from c_0 is 1: g = 1/4."""
    dev = device()
    vals = [2.0 ** 25, 1.0, -(2.0 ** 25), 1.0]
    S = 1031
    cs = [W.as_bf16_bits(torch.full((S,), v, device=dev)) for v in vals]
    out = torch.empty(S, device=dev)
    zs.zs_reduce_shard(cs, out)
    assert torch.all(out == 0.25)
    zs.zs_reduce_shard(cs[::-1], out)
    assert torch.all(out == 0.0)


def test_reduce_misaligned_buffers():
    dev = device()
    S, D = 5003, 6
    for code in (zs.ZS_BF16, zs.ZS_F32):
        tdt = torch.int16 if code == zs.ZS_BF16 else torch.float32
        bufs = [torch.zeros(S + 16, dtype=tdt, device=dev) for _ in range(D)]
        src = (bf16_contribs if code == zs.ZS_BF16 else f32_contribs)(D, S, 3, dev)
        cs = []
        for k in range(D):
            v = bufs[k][k + 1:k + 1 + S]
            v.copy_(src[k])
            cs.append(v)
        ob = torch.zeros(S + 4, device=dev)
        out = ob[1:1 + S]
        zs.zs_reduce_shard(cs, out)
        want = O.reduce_shard([to_np(c) for c in cs], oracle_dtype(code))
        check_f32(to_np(out), want, "reduce misaligned", exact=True)


# ---------------------------------------------------------------- AdamW
def run_steps(D, S, code, steps, dev, seed=0, hp=None, contrib_scale=W.GRAD_SCALE,
              p_init=None, views=None):
    """Run `steps` fused steps on the GPU and the oracle side by side and
    compare after every step."""
    hp = dict(HP if hp is None else hp)
    p = p_init.clone() if p_init is not None else W.master_init(S, 10 + seed, dev)
    m = torch.zeros(S, device=dev)
    v = torch.zeros(S, device=dev)
    w = torch.empty(S, dtype=torch.int16, device=dev)
    if views is not None:
        p, m, v, w = views(p, m, v, w)
    op, om, ov = to_np(p), to_np(m), to_np(v)
    gen = bf16_contribs if code == zs.ZS_BF16 else f32_contribs
    for t in range(1, steps + 1):
        cs = gen(D, S, 1000 * seed + t, dev, contrib_scale)
        zs.zs_adamw_step(p, m, v, w, cs, zs.AdamWHP(step=t, **hp))
        op, om, ov, ow = O.rank_step(op, om, ov, [to_np(c) for c in cs], oracle_dtype(code),
                                     O.AdamWHP(step=t, **hp))
        tag = f"D={D} S={S} step {t}"
        check_f32(to_np(p), op, tag + " p", exact=True)
        check_f32(to_np(m), om, tag + " m", exact=True)
        check_f32(to_np(v), ov, tag + " v", exact=True)
        check_bf16(to_np(w), ow, tag + " w", exact=True)
    return p, m, v, w


@pytest.mark.parametrize("code", [zs.ZS_BF16, zs.ZS_F32])
@pytest.mark.parametrize("D", [1, 2, 3, 4, 8, 16, 32, 64])
def test_adamw_vs_oracle(code, D):
    dev = device()
    for S in (1, 9, 4096 + 5, 100003):
        run_steps(D, S, code, 3, dev, seed=D)


# The tiled kernels take two adjacent 512-element tiles per wavefront; the
# elements past the last whole tile pair go to the last workgroup, one per
# lane. Sizes around those edges, and one of 2,441 tile pairs plus a tail.
# The long folds (16 and 32 contributions) run their batches of 8 in a loop.
TILE_EDGE_SIZES = (511, 512, 513, 1024, 1536, 1537, 3 * 1024 + 511, 2_500_517)


@pytest.mark.parametrize("code,D", [(zs.ZS_BF16, 8), (zs.ZS_F32, 4), (zs.ZS_BF16, 3),
                                    (zs.ZS_BF16, 16), (zs.ZS_F32, 16), (zs.ZS_BF16, 32)])
def test_adamw_tile_edges(code, D):
    dev = device()
    for S in TILE_EDGE_SIZES:
        run_steps(D, S, code, 2, dev, seed=S % 101)


@pytest.mark.parametrize("code,D", [(zs.ZS_BF16, 8), (zs.ZS_F32, 4), (zs.ZS_F32, 5)])
def test_reduce_tile_edges(code, D):
    dev = device()
    gen = bf16_contribs if code == zs.ZS_BF16 else f32_contribs
    for S in TILE_EDGE_SIZES:
        cs = gen(D, S, S % 89, dev)
        out = torch.empty(S, device=dev)
        zs.zs_reduce_shard(cs, out)
        want = O.reduce_shard([to_np(c) for c in cs], oracle_dtype(code))
        check_f32(to_np(out), want, f"reduce D={D} S={S}", exact=True)


def test_adamw_many_steps_gpt3m_shard():
    """The 3.3M GPT rank shard (S = 820,352), D = 4, all 10 steps."""
    run_steps(4, 820_352, zs.ZS_BF16, 10, device(), seed=5)


def test_adamw_misaligned_buffers():
    """Views at element offsets force the element-at-a-time kernel."""
    dev = device()

    def views(p, m, v, w):
        S = p.numel()
        out = []
        for t, off in ((p, 1), (m, 2), (v, 3), (w, 1)):
            b = torch.zeros(S + 8, dtype=t.dtype, device=dev)
            b[off:off + S].copy_(t)
            out.append(b[off:off + S])
        return out

    run_steps(8, 30011, zs.ZS_BF16, 2, dev, seed=9, views=views)


def test_fused_equals_unfused():
    """zs_reduce_shard then zs_adamw_step on its fp32 output, vs the fused
    call: identical bits."""
    dev = device()
    S, D = 70001, 8
    p0 = W.master_init(S, 3, dev)
    cs = bf16_contribs(D, S, 77, dev)
    st = []
    for fused in (True, False):
        p, m, v = p0.clone(), torch.zeros(S, device=dev), torch.zeros(S, device=dev)
        w = torch.empty(S, dtype=torch.int16, device=dev)
        for t in (1, 2, 3):
            hp = zs.AdamWHP(step=t, **HP)
            if fused:
                zs.zs_adamw_step(p, m, v, w, cs, hp)
            else:
                g = torch.empty(S, device=dev)
                zs.zs_reduce_shard(cs, g)
                zs.zs_adamw_step(p, m, v, w, [g], hp)
        st.append([to_np(x) for x in (p, m, v, w)])
    for a, b in zip(*st):
        check_bits(a, b, "fused vs unfused")


def test_adamw_special_values():
    """g = 0 (exact decay), lr = 0 (p unchanged), -0, denormal and huge p
    (bf16 rounding to inf), large gradients."""
    dev = device()
    S = 4099
    specials = np.array([0.0, -0.0, 1e-40, -1e-40, 3.3e38, -3.3e38, 1.0, -2.5, 1e-20, 0.02],
                        np.float32)
    p0 = torch.from_numpy(np.resize(specials, S)).to(dev)
    run_steps(4, S, zs.ZS_BF16, 2, dev, seed=1, p_init=p0)
    run_steps(4, S, zs.ZS_BF16, 2, dev, seed=2, p_init=p0, contrib_scale=0.0)
    run_steps(4, S, zs.ZS_F32, 2, dev, seed=3, p_init=p0, hp=dict(HP, lr=0.0))
    run_steps(4, S, zs.ZS_F32, 2, dev, seed=4, p_init=p0, hp=dict(HP, weight_decay=0.0))
    run_steps(2, S, zs.ZS_F32, 2, dev, seed=5, p_init=p0, contrib_scale=1e30)
    run_steps(3, S, zs.ZS_F32, 1, dev, seed=6, p_init=p0, contrib_scale=1e-41)


def test_adamw_extreme_hyperparameters():
    dev = device()
    run_steps(4, 5000, zs.ZS_BF16, 2, dev, seed=7,
              hp=dict(lr=1.0, beta1=0.0, beta2=0.0, eps=0.0, weight_decay=0.5))
    run_steps(4, 5000, zs.ZS_BF16, 2, dev, seed=8,
              hp=dict(lr=1e-2, beta1=0.999999, beta2=0.9999999, eps=1e-3, weight_decay=0.0))


def test_adamw_large_step_counter():
    dev = device()
    S = 3000
    p = W.master_init(S, 1, dev)
    m = W.normal_f32(S, 1e-3, 2, dev)
    v = W.normal_f32(S, 1e-3, 3, dev).square_()
    w = torch.empty(S, dtype=torch.int16, device=dev)
    cs = bf16_contribs(8, S, 5, dev)
    want = O.rank_step(to_np(p), to_np(m), to_np(v), [to_np(c) for c in cs], O.BF16,
                       O.AdamWHP(step=123456, **HP))
    zs.zs_adamw_step(p, m, v, w, cs, zs.AdamWHP(step=123456, **HP))
    check_f32(to_np(p), want[0], "p", exact=True)
    check_bf16(to_np(w), want[3], "w", exact=True)


def test_adamw_canaries_and_determinism():
    """Nothing outside p, m, v, w is written; two runs give the same bits."""
    dev = device()
    S, D, guard = 12347, 8, 256
    runs = []
    for _ in range(2):
        bufs = {k: torch.full((S + 2 * guard,), 4.5, device=dev) for k in "pmv"}
        wb = torch.full((S + 2 * guard,), 0x1234, dtype=torch.int16, device=dev)
        p, m, v = (bufs[k][guard:guard + S] for k in "pmv")
        p.copy_(W.master_init(S, 1, dev))
        m.zero_()
        v.zero_()
        w = wb[guard:guard + S]
        cs = bf16_contribs(D, S, 11, dev)
        for t in (1, 2):
            zs.zs_adamw_step(p, m, v, w, cs, zs.AdamWHP(step=t, **HP))
        for b in bufs.values():
            g = to_np(b)
            assert np.all(g[:guard] == 4.5) and np.all(g[guard + S:] == 4.5)
        g = to_np(wb)
        assert np.all(g[:guard] == 0x1234) and np.all(g[guard + S:] == 0x1234)
        runs.append([to_np(x) for x in (p, m, v, w)])
    for a, b in zip(*runs):
        check_bits(a, b, "determinism")


def test_errors_on_real_buffers():
    dev = device()
    S = 1000
    p = torch.zeros(S, device=dev)
    m = torch.zeros(S, device=dev)
    w = torch.empty(S, dtype=torch.int16, device=dev)
    c = torch.zeros(S, dtype=torch.int16, device=dev)
    with pytest.raises(zs.ZsError) as e:
        zs.zs_adamw_step(p, p, m, w, [c], zs.AdamWHP(step=1, **HP))
    assert e.value.status == zs.ZS_EALIAS
    with pytest.raises(zs.ZsError) as e:
        zs.zs_adamw_step(p, m, torch.zeros(S, device=dev), w, [w], zs.AdamWHP(step=1, **HP))
    assert e.value.status == zs.ZS_EALIAS
    with pytest.raises(zs.ZsError) as e:
        zs.zs_adamw_step(p, m, torch.zeros(S, device=dev), w, [c], zs.AdamWHP(step=0, **HP))
    assert e.value.status == zs.ZS_EINVAL
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [torch.int16, torch.float32])
def test_gather_in_place_shards(dtype):
    """Shards that sit exactly in their own slot of the unit buffer (an
    in-place all-gather) are left alone; the others are copied in; the result
    equals the out-of-place gather."""
    dev = device()
    for S in (70001, 70000):            # a general (per-shard) and an aligned (one-launch) gather
        _gather_in_place_case(dev, dtype, 8, S)


def _gather_in_place_case(dev, dtype, D, S):
    src = [torch.randint(-30000, 30000, (S,), device=dev).to(dtype) for _ in range(D)]
    want = torch.cat(src)
    for in_place in (set(), {0}, {0, 3, 7}, set(range(D))):
        flat = torch.full((D * S,), -7, device=dev).to(dtype)
        shards = []
        for r in range(D):
            if r in in_place:
                flat[r * S:(r + 1) * S].copy_(src[r])
                shards.append(flat[r * S:(r + 1) * S])
            else:
                shards.append(src[r])
        zs.zs_gather_unit(shards, flat)
        torch.cuda.synchronize()
        assert torch.equal(flat, want), (S, sorted(in_place))


def test_gather_in_place_d64_last_shard():
    """The in-place mask at its widest: D = 64 with shard 63 (the mask's top
    bit) and shard 0 in place, both gather paths."""
    dev = device()
    for S in (1000, 1001):
        D = 64
        src = [torch.randint(-30000, 30000, (S,), device=dev).to(torch.int16) for _ in range(D)]
        flat = torch.full((D * S,), -7, dtype=torch.int16, device=dev)
        shards = list(src)
        for r in (0, 63):
            flat[r * S:(r + 1) * S].copy_(src[r])
            shards[r] = flat[r * S:(r + 1) * S]
        zs.zs_gather_unit(shards, flat)
        torch.cuda.synchronize()
        assert torch.equal(flat, torch.cat(src)), S


def test_native_bfloat16_tensors():
    """Callers may pass torch.bfloat16 tensors wherever bf16 bits are taken
    (tensors to pack, shards, contributions, the working shard, the unit
    buffer): the results are the bits of the int16 path and the oracle's."""
    dev = device()
    D, numels = 4, [300, 4097, 1, 2048]
    ts = [W.normal_f32(n, 0.02, 70 + j, dev).to(torch.bfloat16) for j, n in enumerate(numels)]
    _, N, N_pad, S = zs.zs_unit_layout(numels, D)
    sh_b = [torch.empty(S, dtype=torch.bfloat16, device=dev) for _ in range(D)]
    sh_i = [torch.empty(S, dtype=torch.int16, device=dev) for _ in range(D)]
    zs.zs_pack_flat(ts, D, sh_b)
    zs.zs_pack_flat([t.view(torch.int16) for t in ts], D, sh_i)
    want = O.pack_flat([to_np(t) for t in ts], D)
    for r in range(D):
        check_bits(to_np(sh_b[r]), want[r], f"bfloat16 shard {r}")
        check_bits(to_np(sh_i[r]), want[r], f"int16 shard {r}")
    # fused step: bfloat16 contributions and working shard
    cs = [W.normal_f32(S, W.GRAD_SCALE, 90 + k, dev).to(torch.bfloat16) for k in range(D)]
    p0 = W.master_init(S, 11, dev)
    pb, mb, vb = p0.clone(), torch.zeros(S, device=dev), torch.zeros(S, device=dev)
    pi, mi, vi = p0.clone(), torch.zeros(S, device=dev), torch.zeros(S, device=dev)
    wb = torch.empty(S, dtype=torch.bfloat16, device=dev)
    wi = torch.empty(S, dtype=torch.int16, device=dev)
    hp = zs.AdamWHP(step=1, **HP)
    zs.zs_adamw_step(pb, mb, vb, wb, cs, hp)
    zs.zs_adamw_step(pi, mi, vi, wi, [c.view(torch.int16) for c in cs], hp)
    op, om, ov, ow = O.rank_step(to_np(p0), np.zeros(S, np.float32), np.zeros(S, np.float32),
                                 [to_np(c) for c in cs], O.BF16, O.AdamWHP(step=1, **HP))
    for got, what in ((pb, "p"), (pi, "p int16")):
        check_f32(to_np(got), op, what, exact=True)
    check_bf16(to_np(wb), ow, "w bfloat16", exact=True)
    check_bf16(to_np(wi), ow, "w int16", exact=True)
    # gather into a bfloat16 unit buffer
    flat = torch.empty(D * S, dtype=torch.bfloat16, device=dev)
    zs.zs_gather_unit(sh_b, flat)
    check_bits(to_np(flat), O.gather_unit(want), "bfloat16 unit")
