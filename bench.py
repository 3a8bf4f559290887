#!/usr/bin/env python3
"""Benchmark of the ZeRO-3 shard step on one MI355X.

Workload (default): rank 0's shard of a LLaMA-70B-shaped model at D = 8
simulated ranks -- 80 decoder-block units (d = 8192, GQA k/v 1024 wide,
FFN 28672) plus the root unit (embedding, final norm, LM head), one bucket
per unit: 81 buckets, 8,622,081,024 shard parameters with fp32 master, m
and v (103.5 GB) and a bf16 working shard (17.2 GB), all resident in HBM.

One step = for each unit, in order:
  1. zs_adamw_step: the fused reduce-scatter arithmetic + AdamW on the
     unit's shard, from 8 bf16 gradient contributions (what the
     reduce-scatter delivers; a pool of 4 distinct contribution sets is
     cycled over the buckets, generated before timing);
  2. zs_gather_unit: the all-gather's local rebuild of the unit's full bf16
     parameters (855.7M for a block) into the transient unit buffer, from
     this rank's fresh shard and the 7 peer shards.
The flat layout and pack of a unit happen once, at wrap time; they are
timed separately (one block unit, fp32) and reported under "wrap".

Prints one JSON line. `value` is shard params/s over the whole step;
`roofline` is the fused AdamW kernel's achieved HBM bandwidth from HIP
events on its stream; `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload: one more step of five of the timed buckets,
recomputed from host copies of the very inputs the GPU consumed, whose
results `parity` compares with the GPU's bit for bit (the run exits with
status 3 if any differ). The other workloads' shards get the same check and
oracle timing (`cpu_baseline.per_workload`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "params/s and achieved HBM GB/s (% of peak) for fused reduce+AdamW shard step"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
CONTRIB_POOL = 4
PMC_FILE = os.path.join(ROOT, "profiles", "adamw_fused_llama70b_hbm_counters.md")
_CSRC = os.path.join(ROOT, "fsdp_sharded_optimizer_zs_amd", "csrc")
# what decides the fused kernel's code: its source, the headers it includes
# (launch shape, geometry) and the compiler flags
KERNEL_SRCS = tuple(os.path.join(_CSRC, f) for f in ("zs_step.hip", "zs_internal.h", "zs_grid.h"))


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """Hash of what decides the step kernels' code -- their source and the
    headers it includes, with comments and whitespace removed, and the
    compiler flags -- so that the stored counters stay tied to the code, not
    to its comments."""
    import re
    from fsdp_sharded_optimizer_zs_amd import build as zs_build
    parts = []
    for path in KERNEL_SRCS:
        with open(path) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        parts.append(re.sub(r"\s+", " ", src).strip())
    parts.append(" ".join(zs_build.FLAGS))
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()[:16]


def traffic_from_profiles():
    """Measured HBM bytes per launch of the fused kernel, from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source;
    else None. The summary holds `key: value` lines in a fenced block."""
    try:
        with open(PMC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    rec = {}
    for line in text.splitlines():
        k, sep, val = line.partition(":")
        if sep and k.strip() in ("kernel_src_sha256_16", "hbm_bytes_per_launch"):
            rec[k.strip()] = val.strip()
    if rec.get("kernel_src_sha256_16") != kernel_hash():
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ the oracle
# Only the CPU-baseline leg below runs the oracle: on host copies of exactly
# the inputs a timed GPU step consumed, it recomputes that step, times itself
# on one host core, and compares its results with the GPU's bit for bit.

def host_np(x):
    """Host numpy copy of a device tensor (bf16 / int16 bits as uint16)."""
    import numpy as np
    if x.dtype.is_floating_point and x.element_size() == 2:
        x = x.view(dtype=__import__("torch").int16)
    a = x.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def bf16_ulps(a, b):
    import numpy as np

    def order(h):
        h = h.astype(np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h)
    return int(np.abs(order(a) - order(b)).max(initial=0))


def oracle_check(snapshot, gpu_out, dtype: str, t: int, hp: dict):
    """Run the oracle's rank step on a host snapshot (p, m, v, contributions)
    and compare with the GPU's (p, m, v, w) for the same step. Returns
    (params, oracle seconds, record)."""
    import numpy as np
    from oracle import zs_oracle as O
    p0, m0, v0, cs = snapshot
    t0 = time.perf_counter()
    want = O.rank_step(p0, m0, v0, cs, O.BF16 if dtype == "bf16" else O.FP32,
                       O.AdamWHP(step=t, **hp))
    secs = time.perf_counter() - t0
    rec = {"bit_exact": True, "max_rel_err": 0.0, "max_w_ulps": 0}
    for name, g, w in zip(("p", "m", "v", "w"), gpu_out, want):
        g, w = np.ascontiguousarray(g), np.ascontiguousarray(w)
        if g.tobytes() != w.tobytes():
            rec["bit_exact"] = False
        if name == "w":
            rec["max_w_ulps"] = max(rec["max_w_ulps"], bf16_ulps(g, w))
        else:
            d = np.abs(g.astype(np.float64) - w.astype(np.float64))
            den = np.abs(w.astype(np.float64))
            rel = np.where(d == 0, 0.0, d / np.maximum(den, 1e-300))
            rec["max_rel_err"] = max(rec["max_rel_err"], float(rel.max(initial=0.0)))
    rec["within_tolerance"] = rec["max_rel_err"] <= 1e-6 and rec["max_w_ulps"] <= 1
    return p0.size, secs, rec


def snapshot_step(zs, sl_tensors, cs, h, n=None, keep_working_shard=False):
    """Host copies of (p, m, v, contributions), restricted to the first n
    elements, then one GPU step on the whole slice (the call the timed leg
    makes); returns (snapshot, GPU result restricted the same way)."""
    p, m, v, w = sl_tensors
    k = p.numel() if n is None else n
    snap = (host_np(p[:k]), host_np(m[:k]), host_np(v[:k]), [host_np(c[:k]) for c in cs])
    if keep_working_shard:
        zs.zs_adamw_step_ex(p, m, v, w, cs, h, keep_working_shard=True)
    else:
        zs.zs_adamw_step(p, m, v, w, cs, h)
    out = (host_np(p[:k]), host_np(m[:k]), host_np(v[:k]), host_np(w[:k]))
    return snap, out


def timed_calls(torch, fn, reps: int, warm: int = 3) -> float:
    """Average ms per call of `reps` back-to-back calls of fn, timed with
    events, after `warm` untimed calls queued just before them (no host
    synchronization in between). The warm calls keep the GPU busy while the
    host queues the timed ones, so that the events see only GPU time, and
    take the first touches of the buffers: on the ragged unit the first few
    packs after the inputs are made run about 10% slower than later ones."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for _ in range(warm):
        fn()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def pipeline_leg(zs, torch, p, m, v, wshard, buckets, pool, D, step_t, hp, reps: int = 3):
    """Per-bucket streamed step over all of the rank's buckets:
    contributions copied into two alternating staging slots on a transfer
    stream while the fused step of the previous bucket runs on the compute
    stream (zs_step_pipelined). The prefetch figure is the pinned-host form,
    where the transfer crosses PCIe as a collective's data would cross the
    network; the device-source form is reported as HBM contention (the copy
    and the step share the same HBM, so there is nothing to hide). Times the
    copies alone, the steps alone (sources already resident) and the
    pipelined form; overlap efficiency = (copy + step - pipelined) /
    min(copy, step), the fraction of the shorter phase hidden. Over PCIe the
    copies take about 40 times as long as the steps, so 1% of drift in the
    copy rate moves the efficiency by 0.4: the copies are run once untimed
    (first touches of the pinned pages), then copies alone and the pipelined
    form alternate `reps` times and the medians are used."""
    import statistics
    dev = p.device
    bmax = pool.shape[2]
    staging = (torch.empty((D, bmax), dtype=torch.int16, device=dev),
               torch.empty((D, bmax), dtype=torch.int16, device=dev))
    compute = torch.cuda.Stream(device=dev)
    transfer = torch.cuda.Stream(device=dev)
    res = {}
    nb = len(buckets)

    def timed(stream, fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    for kind in ("pinned_host_sources", "device_sources_hbm_contention"):
        if kind.startswith("device_sources"):
            srcs = [[pool[b % pool.shape[0], k, :sz] for k in range(D)]
                    for b, (_, sz, _, _, _) in enumerate(buckets[:nb])]
        else:
            hpool = torch.empty((2, D, bmax), dtype=torch.int16, pin_memory=True)
            hpool.copy_(pool[:2])
            srcs = [[hpool[b % 2, k, :sz] for k in range(D)]
                    for b, (_, sz, _, _, _) in enumerate(buckets[:nb])]
        bl = [(p[sl], m[sl], v[sl], wshard[sl], srcs[b])
              for b, (sl, sz, _, _, _) in enumerate(buckets[:nb])]
        h = dict(step=step_t, **hp)

        def copies():
            for b, (_, sz, _, _, _) in enumerate(buckets[:nb]):
                for k in range(D):
                    staging[b & 1][k, :sz].copy_(srcs[b][k], non_blocking=True)

        def steps():                                # sources resident
            for b, (sl, sz, cs, _, _) in enumerate(buckets[:nb]):
                zs.zs_adamw_step(p[sl], m[sl], v[sl], wshard[sl], cs, zs.AdamWHP(**h))

        def piped():
            zs.zs_step_pipelined(bl, staging, h, compute, transfer)

        timed(transfer, copies)                     # untimed: first touches
        tcs, tps = [], []
        for _ in range(reps):
            tcs.append(timed(transfer, copies))
            tps.append(timed(compute, piped))
        tk = timed(compute, steps)
        tc, tp = statistics.median(tcs), statistics.median(tps)
        moved = sum(D * 2 * sz for (_, sz, _, _, _) in buckets[:nb])
        res[kind] = {"buckets": nb, "copy_ms": tc, "copy_GB_s": moved / (tc / 1e3) / 1e9,
                     "step_ms": tk, "pipelined_ms": tp,
                     "serial_ms": tc + tk,
                     "overlap_efficiency": (tc + tk - tp) / min(tc, tk),
                     "copy_ms_each": tcs, "pipelined_ms_each": tps}
        del srcs, bl
    return res


def hybrid_leg(zs, torch, W, dev, hp, steps: int, arenas):
    """HYBRID_SHARD shard step on the full LLaMA-7B rank shard of a 4-node x
    8-GPU job (D = 8 per node, 4 replica groups, bf16 collectives): one
    zs_adamw_step_ex per unit bucket (33), 32 bf16 contributions each. The
    same buckets are also stepped with the flat 32-contribution reduce
    (zs_adamw_step), which moves the same 26 + 32 * 2 = 90 B/param. The
    shard's p, m, v and w are placed at the start of the 70B run's state
    arrays (`arenas`, re-initialized here), tens of GB apart as a rank's own
    state arrays are."""
    w = W.get("llama7b_hybrid")
    R, D = w.replicas, w.D
    sizes = [zs.zs_unit_layout(u.numels, D)[3] for u in w.units]
    S = int(sum(sizes))
    bmax = max(sizes)
    P, M, V, WS = arenas
    p, m, v, ws = P[:S], M[:S], V[:S], WS[:S]
    p.copy_(W.master_init(S, 6000, dev))
    m.zero_()
    v.zero_()
    pool = torch.empty((2, R * D, bmax), dtype=torch.int16, device=dev)
    for s_ in range(2):
        for k in range(R * D):
            pool[s_, k].copy_(W.contribution(w, bmax, 1, s_, k, dev))
    off = 0
    bl = []
    for b, sz in enumerate(sizes):
        bl.append((slice(off, off + sz), [pool[b % 2, k, :sz] for k in range(R * D)]))
        off += sz
    torch.cuda.synchronize()

    def run(t, hybrid):
        h = dict(step=t, **hp)
        for sl, cs in bl:
            if hybrid:
                zs.zs_adamw_step_ex(p[sl], m[sl], v[sl], ws[sl], cs, h, replicas=R,
                                    round_to_reduce_dtype=w.round_reduce)
            else:
                zs.zs_adamw_step(p[sl], m[sl], v[sl], ws[sl], cs, h)

    res = {"workload": w.description, "shard_params": S, "buckets": len(sizes),
           "replicas": R, "D": D, "algorithmic_bytes_per_param": 26 + R * D * 2}
    for name, hybrid in (("hybrid", True), ("flat32", False)):
        run(1, hybrid)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for t in range(2, 2 + steps):
            run(t, hybrid)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"ms_per_step": ms, "params_per_s": S / (ms / 1e3),
                     "GB_s": (26 + R * D * 2) * S / (ms / 1e3) / 1e9}
    del pool
    torch.cuda.empty_cache()
    return res


def hbm_directions(zs, torch, dev, read_bytes: int, write_bytes: int):
    """HBM's own rates for one direction at a time (zs_hbm_probe: reads,
    writes and a copy over a 4 GiB buffer, and a triad of two 4 GiB read
    streams and one write stream -- the step's 2:1 ratio in three streams --,
    the best of a grid that covers the buffers and persistent grids of 1-4
    workgroups per CU)
    and the rate the step's mix of read_bytes and write_bytes per param would
    reach if reads and writes overlapped perfectly at those rates."""
    n = 4 << 30
    a2 = torch.empty(2 * n, dtype=torch.uint8, device=dev)   # the triad's two read streams
    a = a2[:n]
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    zs.zs_hbm_probe(zs.ZS_PROBE_WRITE, a2)
    torch.cuda.synchronize()
    best = {}
    for name, kind, moved in (("read", zs.ZS_PROBE_READ, n), ("write", zs.ZS_PROBE_WRITE, n),
                              ("copy", zs.ZS_PROBE_COPY, 2 * n),
                              ("triad", zs.ZS_PROBE_TRIAD, 3 * n)):
        for per_cu in (0, 1, 2, 3, 4):
            dst = b[:16] if kind == zs.ZS_PROBE_READ else (None if kind == zs.ZS_PROBE_WRITE
                                                           else b)
            src = a2 if kind == zs.ZS_PROBE_TRIAD else a
            ms = []
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                zs.zs_hbm_probe(kind, src, dst, blocks_per_cu=per_cu)
                e1.record()
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            rate = moved / (min(ms) / 1e3) / 1e9
            if rate > best.get(name, (0.0, 0))[0]:
                best[name] = (rate, per_cu)
    del a, a2, b
    torch.cuda.empty_cache()
    rd, wr = best["read"][0], best["write"][0]
    bound = (read_bytes + write_bytes) / (read_bytes / rd + write_bytes / wr)
    return {"read_GB_s": rd, "read_blocks_per_cu": best["read"][1],
            "write_GB_s": wr, "write_blocks_per_cu": best["write"][1],
            "copy_GB_s": best["copy"][0], "copy_blocks_per_cu": best["copy"][1],
            "triad_GB_s": best["triad"][0], "triad_blocks_per_cu": best["triad"][1],
            "step_mix": f"{read_bytes} B read + {write_bytes} B written per param",
            "ideal_overlap_bound_GB_s": bound}


def configs_leg(zs, torch, W, dev, hp, launches: int, arenas, oracle: bool):
    """The fused reduce + AdamW kernel alone on the rank shards of the other
    workloads (one launch over each whole shard, contributions resident):
    3.3M GPT at D=4, one LLaMA-7B block at D=8, the full LLaMA-7B at D=32
    (Student-t gradients) and the 10,000-tensor ragged unit at D=16 with fp32
    contributions. Reports the average launch time and HBM GB/s at the
    algorithmic 26 + D * es bytes per param. Each shard's p, m, v (and w) are
    placed at the start of the 70B run's own four state arrays (`arenas`,
    re-initialized here), so that they sit tens of GB apart in HBM as a
    rank's separately allocated state arrays do; allocated back to back they
    run 10-15% slower.

    With `oracle`, the first (untimed) step of each shard is also recomputed
    by the CPU oracle from host copies of its inputs and compared bit for bit:
    the whole shard for the 3.3M GPT, the 7B block and the ragged unit, the
    first 2^24 params for the full 7B shard (its 32 contributions of 210M
    params make the whole shard about a minute of oracle time)."""
    res = {}
    oracle_n = {"gpt3m": None, "llama7b_block": None, "llama7b_full": 1 << 24, "ragged": None}
    P, M, V, WS = arenas
    busy = torch.empty(1 << 30, device=dev)        # 4 GiB: a fill of about 0.6 ms
    for name in ("gpt3m", "llama7b_block", "llama7b_full", "ragged"):
        w = W.get(name)
        S = int(sum(zs.zs_unit_layout(u.numels, w.D)[3] for u in w.units))
        es = 2 if w.reduce_dtype == "bf16" else 4
        p, m, v, ws = P[:S], M[:S], V[:S], WS[:S]
        p.copy_(W.master_init(S, 7000 + w.index, dev))
        m.zero_()
        v.zero_()
        mask = W.step_mask(w, S, 1, 0, dev)
        cs = [W.contribution(w, S, 1, 0, k, dev, mask) for k in range(w.D)]
        del mask
        check = None
        if oracle:                                  # first step, checked by the oracle
            snap, got = snapshot_step(zs, (p, m, v, ws), cs, zs.AdamWHP(step=1, **hp),
                                      oracle_n[name])
            n, secs, rec = oracle_check(snap, got, w.reduce_dtype, 1, hp)
            del snap, got
            bpp_ = 26 + w.D * es
            check = dict(rec, params=n, oracle_s=secs, oracle_params_per_s=n / secs,
                         oracle_GB_s=bpp_ * n / secs / 1e9, cores=1,
                         sample="whole shard" if oracle_n[name] is None
                         else f"first {n} params of the shard")
        else:
            zs.zs_adamw_step(p, m, v, ws, cs, dict(step=1, **hp))      # warm
        hps = [zs.AdamWHP(step=t, **hp) for t in range(2, 2 + launches)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # Two untimed launches, then a long fill ahead of the timed ones keeps
        # the GPU busy while the host queues them, so that small shards are
        # timed back to back on the GPU rather than at the rate the host can
        # issue calls.
        for h in hps[:2]:
            zs.zs_adamw_step(p, m, v, ws, cs, h)
        busy.fill_(1.0)
        e0.record()
        for h in hps:
            zs.zs_adamw_step(p, m, v, ws, cs, h)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        bpp = 26 + w.D * es
        res[name] = {"shard_params": S, "D": w.D, "reduce_dtype": w.reduce_dtype,
                     "bytes_per_param": bpp, "launch_ms": ms,
                     "params_per_s": S / (ms / 1e3), "GB_s": bpp * S / (ms / 1e3) / 1e9}
        if check is not None:
            res[name]["oracle"] = check
        del cs
        torch.cuda.empty_cache()
    del busy
    torch.cuda.empty_cache()
    return res


def ragged_move_leg(zs, torch, W, dev, reps: int = 5):
    """Pack and gather of the ragged 10,000-tensor unit (about 3.78e9
    elements, D = 16), fp32 and bf16: the unit's tensors are separate
    allocations, so most pieces land at another offset within 16 bytes than
    their source. Kernel time only: the tensor table is built once and
    reused (zs_pack_flat's `table`). Algorithmic bytes: pack es * N read +
    es * N_pad written; gather es * N_pad read and written. Afterwards every
    tensor is compared with its view of the gathered unit (gather(pack(x))
    == x) and the pad must be +0."""
    w = W.get("ragged")
    unit = w.units[0]
    D = w.D
    res = {}
    for dtype in ("f32", "bf16"):
        ts = [t.reshape(-1) for t in W.tensor_values(unit, dtype, 5, dev)]
        _, N, N_pad, S = zs.zs_unit_layout(unit.numels, D)
        es = ts[0].element_size()
        shards = [torch.empty(S, dtype=ts[0].dtype, device=dev) for _ in range(D)]
        flat = torch.empty(N_pad, dtype=ts[0].dtype, device=dev)
        table = zs.zs_pack_flat(ts, D, shards)               # builds the table
        pack_ms = timed_calls(torch, lambda: zs.zs_pack_flat(ts, D, shards, table=table), reps)
        gather_ms = timed_calls(torch, lambda: zs.zs_gather_unit(shards, flat), reps)
        pos, exact = 0, True
        for t in ts:
            exact = exact and bool(torch.equal(flat[pos:pos + t.numel()], t))
            pos += t.numel()
        exact = exact and not bool(flat[N:].view(torch.int16 if es == 2 else torch.int32).any())
        res[dtype] = {"tensors": len(ts), "N": N, "N_pad": N_pad, "D": D,
                      "pack_ms": pack_ms, "pack_GB_s": es * (N + N_pad) / (pack_ms / 1e3) / 1e9,
                      "gather_ms": gather_ms,
                      "gather_GB_s": 2 * es * N_pad / (gather_ms / 1e3) / 1e9,
                      "gather_of_pack_exact": exact}
        if not exact:
            raise SystemExit(f"ragged {dtype}: gather(pack(x)) != x")
        del ts, shards, flat, table
        torch.cuda.empty_cache()
    return res


def reshard_ckpt_leg(zs, torch, W, dev, p, m, v, wshard, sl, D):
    """Re-shard and shard checkpoint rates: zs_reshard of one 70B block
    unit's fp32 master (855,654,400 elements) from D=8 to 6 shards (HBM
    bytes = 2 x 4 B per element) and of its bf16 working shards (2 x 2 B),
    then zs_shard_save / zs_shard_load of one block bucket's rank state (p,
    m, v, w: 14 B per param) through a file in the system temp directory."""
    import tempfile
    unit = W.get("llama70b").units[0]
    N = unit.numel
    S, S2 = -(-N // D), -(-N // 6)
    src = [p[sl][:S] for _ in range(1)] + [torch.empty(S, device=dev) for _ in range(D - 1)]
    dst = [torch.empty(S2, device=dev) for _ in range(6)]
    ms = timed_calls(torch, lambda: zs.zs_reshard(src, N, dst), 5)
    res = {"reshard_block_unit_f32_8_to_6": {"elements": N, "ms": ms,
                                              "GB_s": 8 * N / (ms / 1e3) / 1e9}}
    del src, dst
    torch.cuda.empty_cache()
    # the same in bf16: odd S2 puts every other new shard at an odd element
    # offset from its sources (the shifted-load path)
    src = [wshard[sl][:S]] + [torch.empty(S, dtype=torch.int16, device=dev) for _ in range(D - 1)]
    dst = [torch.empty(S2, dtype=torch.int16, device=dev) for _ in range(6)]
    ms = timed_calls(torch, lambda: zs.zs_reshard(src, N, dst), 5)
    res["reshard_block_unit_bf16_8_to_6"] = {"elements": N, "ms": ms,
                                             "GB_s": 4 * N / (ms / 1e3) / 1e9}
    del src, dst
    torch.cuda.empty_cache()
    Sb = sl.stop - sl.start
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "rank0.zss")
        t0 = time.perf_counter()
        zs.zs_shard_save(path, 0, D, Sb * D, 1, p[sl], m[sl], v[sl], wshard[sl])
        t_save = time.perf_counter() - t0
        t0 = time.perf_counter()
        zs.zs_shard_load(path, p[sl], m[sl], v[sl], wshard[sl])
        t_load = time.perf_counter() - t0
    res["checkpoint_one_bucket"] = {"bytes": 14 * Sb, "save_s": t_save, "load_s": t_load,
                                    "save_GB_s": 14 * Sb / t_save / 1e9,
                                    "load_GB_s": 14 * Sb / t_load / 1e9}
    return res


def offload_leg(zs, torch, W, dev, hp, threads: int):
    """ZeRO-Offload on the full LLaMA-7B rank shard at D=32 (the CPU-offload
    example of the 7.10 page: ~100 ms/step extra over ~50 GB/s PCIe): p, m, v
    in pinned host memory, 32 bf16 contributions on the device. Times one
    zs_offload_step (device reduce, gradient down, host AdamW, working shard
    up) and, apart, the host AdamW alone and the two transfers alone."""
    w = W.get("llama7b_full")
    D = w.D
    S = int(sum(zs.zs_unit_layout(u.numels, D)[3] for u in w.units))
    cs = [W.contribution(w, S, 1, 0, k, dev) for k in range(D)]
    pin = dict(pin_memory=True)
    ph = torch.empty(S, dtype=torch.float32, **pin)
    ph.copy_(W.master_init(S, 7100, dev))
    mh = torch.zeros(S, dtype=torch.float32, **pin)
    vh = torch.zeros(S, dtype=torch.float32, **pin)
    gh = torch.empty(S, dtype=torch.float32, **pin)
    wh = torch.empty(S, dtype=torch.int16, **pin)
    gdev = torch.empty(S, device=dev)
    wdev = torch.empty(S, dtype=torch.int16, device=dev)
    stream, h2d = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()

    def step(t):
        zs.zs_offload_step(cs, gdev, gh, ph, mh, vh, wh, wdev, dict(step=t, **hp),
                           threads=threads, chunk=1 << 24, stream=stream, h2d_stream=h2d)
        h2d.synchronize()
        stream.synchronize()

    step(1)
    t0 = time.perf_counter()
    for t in range(2, 5):
        step(t)
    t_step = (time.perf_counter() - t0) / 3
    t0 = time.perf_counter()
    for t in range(5, 8):
        zs.zs_adamw_step_host(ph, mh, vh, wh, gh, dict(step=t, **hp), threads=threads)
    t_host = (time.perf_counter() - t0) / 3
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    with torch.cuda.stream(stream):
        e[0].record()
        gh.copy_(gdev, non_blocking=True)
        e[1].record()
        e[2].record()
        wdev.copy_(wh, non_blocking=True)
        e[3].record()
    torch.cuda.synchronize()
    d2h, h2d_ms = e[0].elapsed_time(e[1]), e[2].elapsed_time(e[3])
    res = {"workload": "full LLaMA-7B, rank-0 shard at D=32 (32 bf16 contributions)",
           "shard_params": S, "threads": threads,
           "offload_step_ms": t_step * 1e3,
           "host_adamw_ms": t_host * 1e3, "host_adamw_params_per_s": S / t_host,
           "host_adamw_GB_s": 30 * S / t_host / 1e9,
           "grad_d2h_ms": d2h, "grad_d2h_GB_s": 4 * S / (d2h / 1e3) / 1e9,
           "weights_h2d_ms": h2d_ms, "weights_h2d_GB_s": 2 * S / (h2d_ms / 1e3) / 1e9}
    del cs, ph, mh, vh, gh, wh, gdev, wdev
    torch.cuda.empty_cache()
    return res


def unfused_leg(zs, torch, p, m, v, wshard, buckets, D, step_t, hp):
    """The unfused form of the step on the same 70B buckets: zs_reduce_shard
    writes the fp32 gradient (A3: D * 2 + 4 B/param), then zs_adamw_step
    reads it as its single contribution (A4: 30 B/param); 50 B/param in all
    against the fused kernel's 42. Results are bit-identical to the fused
    step; this leg shows what the fusion saves."""
    dev = p.device
    bmax = max(sz for _, sz, _, _, _ in buckets)
    g = torch.empty(bmax, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in buckets]
    h = dict(step=step_t, **hp)
    for rep in range(2):
        for i, (sl, sz, cs, _, _) in enumerate(buckets):
            if rep:
                ev[i][0].record()
            zs.zs_reduce_shard(cs, g[:sz])
            if rep:
                ev[i][1].record()
            zs.zs_adamw_step(p[sl], m[sl], v[sl], wshard[sl], [g[:sz]], h)
            if rep:
                ev[i][2].record()
    torch.cuda.synchronize()
    S = sum(sz for _, sz, _, _, _ in buckets)
    red = sum(e[0].elapsed_time(e[1]) for e in ev)
    ada = sum(e[1].elapsed_time(e[2]) for e in ev)
    return {"reduce_ms_per_step": red, "reduce_GB_s": (D * 2 + 4) * S / (red / 1e3) / 1e9,
            "adamw_one_f32_contribution_ms_per_step": ada,
            "adamw_one_f32_contribution_GB_s": 30 * S / (ada / 1e3) / 1e9,
            "unfused_ms_per_step": red + ada, "bytes_per_param": 2 * D + 4 + 30}


def in_place_leg(zs, torch, p, m, v, buckets, step_t, hp, steps: int = 3):
    """The step with an in-place all-gather, as FSDP lays a unit out: the
    rank's bf16 working shard is written by the step straight into its own
    slot of the unit buffer (slot 0 for rank 0), and zs_gather_unit then
    copies only the D - 1 peer shards. Wall time per step over the same 81
    buckets, beside the main leg's out-of-place form."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for rep in range(2):
        if rep:
            torch.cuda.synchronize()
            ev[0].record()
        for t in range(steps if rep else 1):
            h = zs.AdamWHP(step=step_t + t, **hp)
            for sl, sz, cs, shards, ubuf in buckets:
                slot = ubuf[:sz]
                zs.zs_adamw_step(p[sl], m[sl], v[sl], slot, cs, h)
                zs.zs_gather_unit([slot] + shards[1:], ubuf)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    S = sum(sz for _, sz, _, _, _ in buckets)
    return {"ms_per_step": ms, "params_per_s": S / (ms / 1e3)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the unfused (reduce, then AdamW) form of the step")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the no-arithmetic stream ceiling on the same buckets")
    ap.add_argument("--no-in-place", action="store_true",
                    help="skip the step with an in-place all-gather")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the ZeRO-Offload (host-core AdamW) leg")
    ap.add_argument("--host-threads", type=int, default=16,
                    help="host threads for the offload leg (default 16)")
    ap.add_argument("--no-ckpt", action="store_true",
                    help="skip the re-shard and shard checkpoint leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the fused-kernel rates on the other workloads' shards")
    ap.add_argument("--no-hybrid", action="store_true",
                    help="skip the HYBRID_SHARD (4 nodes x 8 GPUs, LLaMA-7B) step leg")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="skip the per-bucket streamed (overlapped) step leg")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged 10,000-tensor unit's pack and gather leg")
    ap.add_argument("--no-copy", action="store_true",
                    help="skip the plain 4 GiB device copy (the copy ceiling and the HBM "
                         "counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the shard step is measured on one GPU only (asked for --gpus {args.gpus}); the "
              "multi-GPU form of the shard step is a design, not a measured path.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import fsdp_sharded_optimizer_zs_amd as zs
    import workloads as W

    zs.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.get("llama70b")
    D = w.D
    sizes = [zs.zs_unit_layout(u.numels, D)[3] for u in w.units]
    S = int(sum(sizes))
    starts = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    bmax = max(sizes)
    hp = dict(W.ADAMW_HP)

    log(f"allocating rank shard: S={S} ({S * 14 / 1e9:.1f} GB of p, m, v, w)")
    # The rank's state is one arena, p | m | v | w: each fp32 array is 34.6 GB,
    # so the three streams the step rewrites sit tens of GB apart in HBM
    # (arrays a few GB apart run the same kernel 10-15% slower).
    arena = torch.empty(14 * S, dtype=torch.uint8, device=dev)
    p = arena[:4 * S].view(torch.float32)
    m = arena[4 * S:8 * S].view(torch.float32)
    v = arena[8 * S:12 * S].view(torch.float32)
    wshard = arena[12 * S:].view(torch.int16)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4000)
    for a in range(0, S, 1 << 30):
        b = min(S, a + (1 << 30))
        torch.randn(b - a, generator=gen, device=dev, out=p[a:b]).mul_(W.PARAM_STD)
    m.zero_()
    v.zero_()
    log(f"generating {CONTRIB_POOL} contribution sets of {D} x {bmax} bf16")
    pool = torch.empty((CONTRIB_POOL, D, bmax), dtype=torch.int16, device=dev)
    for s in range(CONTRIB_POOL):
        for k in range(D):
            pool[s, k].copy_(W.contribution(w, bmax, 1, s, k, dev))
    peers = torch.empty((D - 1, bmax), dtype=torch.int16, device=dev)
    peers.copy_(pool[0, 1:])                  # stand-in for the other ranks' shards
    unit_buf = torch.empty(D * bmax, dtype=torch.int16, device=dev)
    torch.cuda.synchronize()

    # wrap time: layout + pack of one block unit's fp32 master (timed apart)
    blk = w.units[0]
    ts = [t.reshape(-1) for t in W.tensor_values(blk, "f32", 1, dev)]
    bshards = [torch.empty(sizes[0], device=dev) for _ in range(D)]
    table = zs.zs_pack_flat(ts, D, bshards)
    pack_ms = timed_calls(torch, lambda: zs.zs_pack_flat(ts, D, bshards, table=table), 5)
    pack_bytes = 2 * 4 * blk.numel
    del ts, bshards, table
    torch.cuda.empty_cache()

    buckets = []
    for b, sz in enumerate(sizes):
        sl = slice(int(starts[b]), int(starts[b + 1]))
        cs = [pool[b % CONTRIB_POOL, k, :sz] for k in range(D)]
        shards = [wshard[sl]] + [peers[r, :sz] for r in range(D - 1)]
        buckets.append((sl, sz, cs, shards, unit_buf[:D * sz]))

    n_launch = len(buckets)
    K = args.steps
    # Per (timed step, bucket), two events that the fused kernel's launch
    # itself records at the kernel's start and end (zs_adamw_step_timed: the
    # kernel's own execution time, with no marker packets enqueued between the
    # kernels), and per timed step one event after its last gather; all read
    # only after the timed region. Recording each once here creates it.
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_launch)]
          for _ in range(K)]
    ev_end = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for e in [x for evs in ev for pair in evs for x in pair] + ev_end:
        e.record()
    torch.cuda.synchronize()

    # Each unit's fused step is followed at once by its all-gather, which reads
    # the rank's fresh working shard: the step stores that shard with
    # cache-allocating stores (ZS_W_KEEP), so the gather reads it from the
    # Infinity Cache and it crosses HBM once (written back later) instead of
    # twice. Every other stream stays non-temporal; the bits are the same.
    def step(t: int, evs, end):
        h = zs.AdamWHP(step=t, **hp)
        for i, (sl, sz, cs, shards, ubuf) in enumerate(buckets):
            if evs:
                zs.zs_adamw_step_timed(p[sl], m[sl], v[sl], wshard[sl], cs, h, evs[i][0],
                                       evs[i][1], keep_working_shard=True)
            else:
                zs.zs_adamw_step_ex(p[sl], m[sl], v[sl], wshard[sl], cs, h,
                                    keep_working_shard=True)
            zs.zs_gather_unit(shards, ubuf)
        if end is not None:
            end.record()

    log(f"warmup {args.warmup} step(s)")
    for t in range(1, args.warmup + 1):
        step(t, None, None)
    torch.cuda.synchronize()
    log(f"timing {K} step(s) of {n_launch} units")
    t0 = time.perf_counter()
    for j in range(K):
        step(args.warmup + 1 + j, ev[j], ev_end[j])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    adam_ms = sum(e[0].elapsed_time(e[1]) for evs in ev for e in evs)
    # each gather: from its unit's fused kernel's end to the next one's start
    # (after the last unit, to the step's end event)
    gather_ms = sum(evs[i][1].elapsed_time(evs[i + 1][0] if i + 1 < n_launch else ev_end[j])
                    for j, evs in enumerate(ev) for i in range(n_launch))
    ms_per_step = elapsed * 1e3 / K
    log(f"{ms_per_step:.2f} ms/step")

    # CPU baseline and in-run parity: the oracle recomputes one more step of
    # five of the timed buckets (blocks 0, 1, 39, 79 and the root) from host
    # copies of the state and contributions those GPU steps consumed, on one
    # host core, and the results are compared bit for bit.
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline + parity: oracle on five of the timed buckets (host copies)")
        t_chk = args.warmup + K + 1
        h = zs.AdamWHP(step=t_chk, **hp)
        tot_n, tot_s, recs = 0, 0.0, []
        for b in (0, 1, 39, 79, n_launch - 1):
            sl, sz, cs, _, _ = buckets[b]
            snap, got = snapshot_step(zs, (p[sl], m[sl], v[sl], wshard[sl]), cs, h,
                                      keep_working_shard=True)
            n, secs, rec = oracle_check(snap, got, "bf16", t_chk, hp)
            del snap, got
            tot_n, tot_s = tot_n + n, tot_s + secs
            recs.append(dict(rec, bucket=b, params=n))
        out_parity = {"workload": "llama70b", "buckets": [r["bucket"] for r in recs],
                      "params": tot_n, "step": t_chk,
                      "bit_exact": all(r["bit_exact"] for r in recs),
                      "max_rel_err": max(r["max_rel_err"] for r in recs),
                      "max_w_ulps": max(r["max_w_ulps"] for r in recs),
                      "tolerance": "p, m, v rel 1e-6; w 1 bf16 ulp (bit identity expected)"}
        rate = tot_n / tot_s
        cpu = {"value": rate, "unit": "params/s", "cores": 1, "kind": "oracle",
               "GB_s": (26 + 2 * D) * tot_n / tot_s / 1e9,
               "sample": f"one step of five of the timed 70B buckets (blocks 0, 1, 39, 79 and "
                         f"the root: {tot_n} params, D=8 bf16 contributions) from host copies "
                         f"of the GPU's inputs, {tot_s:.1f} s of single-threaded numpy"}
        log(f"oracle {rate / 1e6:.1f} M params/s; parity bit_exact={out_parity['bit_exact']}")

    # The same buckets and contributions through zs_stream_ceiling: the fused
    # kernel's streams without its arithmetic (it overwrites p, m, v, w, which
    # are re-initialized afterwards).
    if not args.no_ceiling:
        # the fused kernel alone over the same buckets (no gathers between,
        # the working shard stored non-temporally like every other stream):
        # the like-for-like partner of the stream ceiling
        # (both timed like the main leg: events tied to each kernel launch)
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_launch)]
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_launch)]
        for e in [x for pair in fev + cev for x in pair]:
            e.record()
        for rep in range(2):
            h = zs.AdamWHP(step=args.warmup + K + 2 + rep, **hp)
            for i, (sl, sz, cs, _, _) in enumerate(buckets):
                if rep:
                    zs.zs_adamw_step_timed(p[sl], m[sl], v[sl], wshard[sl], cs, h, fev[i][0],
                                           fev[i][1])
                else:
                    zs.zs_adamw_step(p[sl], m[sl], v[sl], wshard[sl], cs, h)
        torch.cuda.synchronize()
        alone_s = sum(a.elapsed_time(b) for a, b in fev) / 1e3 / n_launch
        for rep in range(2):
            for i, (sl, sz, cs, _, _) in enumerate(buckets):
                if rep:
                    zs.zs_stream_ceiling_timed(p[sl], m[sl], v[sl], wshard[sl], cs, cev[i][0],
                                               cev[i][1])
                else:
                    zs.zs_stream_ceiling(p[sl], m[sl], v[sl], wshard[sl], cs)
        torch.cuda.synchronize()
        ceiling_s = sum(a.elapsed_time(b) for a, b in cev) / 1e3 / n_launch
        for a in range(0, S, 1 << 30):
            b = min(S, a + (1 << 30))
            torch.randn(b - a, generator=gen, device=dev, out=p[a:b]).mul_(W.PARAM_STD)
        m.zero_()
        v.zero_()
        torch.cuda.synchronize()

    es = 2
    bpp = 26 + D * es                              # fused: 12 read + 14 written + D*es
    adam_launches = K * n_launch
    adam_avg_s = adam_ms / 1e3 / adam_launches
    # median per-launch rate over the timed launches
    bucket_rates = sorted(bpp * sz / (e[0].elapsed_time(e[1]) / 1e3) / 1e9
                          for evs in ev for e, (_, sz, _, _, _) in zip(evs, buckets))
    median_rate = bucket_rates[len(bucket_rates) // 2]
    bytes_per_launch = bpp * S / n_launch
    achieved = bytes_per_launch / adam_avg_s / 1e9
    gather_bytes = 4.0 * D * S                     # D*S bf16 read + written per step
    traffic = traffic_from_profiles()
    ceiling = None
    if not args.no_ceiling:
        ceiling_gbs = bytes_per_launch / ceiling_s / 1e9
        alone_gbs = bytes_per_launch / alone_s / 1e9
        ceiling = {"kernel": "zs_stream_ceiling: the same streams, launch shape and non-temporal "
                             "cache hints, no arithmetic, launches back to back",
                   "avg_launch_ms": ceiling_s * 1e3,
                   "GB_s": ceiling_gbs, "frac_of_peak": ceiling_gbs / PEAK_HBM_GBS,
                   "fused_alone": {"what": "the fused kernel over the same buckets back to back, "
                                           "no gathers between, working shard non-temporal",
                                   "avg_launch_ms": alone_s * 1e3, "GB_s": alone_gbs,
                                   "frac_of_peak": alone_gbs / PEAK_HBM_GBS},
                   "fused_alone_over_ceiling": alone_gbs / ceiling_gbs,
                   "fused_in_step_over_ceiling": achieved / ceiling_gbs}
    out = {
        "metric": METRIC,
        "value": S * K / elapsed,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "llama70b rank-0 shard, D=8, 81 unit buckets (80 blocks + root), "
                        "fused reduce+AdamW then unit all-gather rebuild per bucket",
            "shard_params": S, "D": D, "reduce_dtype": "bf16", "param_dtype": "bf16",
            "master_dtype": "f32", "buckets": n_launch,
        },
        "roofline": {
            "bound": "hbm", "kernel": "adamw_vec_kernel<bf16, FlatSum<bf16, 8>>",
            "working_shard_stores": "ZS_W_KEEP: cache-allocating, read by the unit gather right "
                                    "after (2 of the 42 algorithmic B/param go to the Infinity "
                                    "Cache and reach HBM when it writes them back); every other "
                                    "stream non-temporal",
            "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
            "traffic_source": ("committed counter summary profiles/" + os.path.basename(PMC_FILE)
                               + ", taken on this kernel code (hash " + kernel_hash() + "); "
                               "not measured in this run") if traffic else
                              "no counter summary for this kernel code",
            "traffic_over_algorithmic": (traffic / bytes_per_launch) if traffic else None,
            "algorithmic_bytes_per_param": bpp,
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "avg_launch_ms": adam_avg_s * 1e3,
            "launch_timing": "HIP events recorded by each fused kernel's launch at the kernel's "
                             "own start and end (zs_adamw_step_timed, hipExtLaunchKernel) on its "
                             "stream; the stream ceiling and fused_alone are timed the same way",
            "median_launch_GB_s": median_rate,
            "stream_ceiling": ceiling,
        },
        "adamw_fused": {"params_per_s": S * K / (adam_ms / 1e3),
                        "ms_per_step": adam_ms / K, "GB_s": achieved},
        "gather": {"ms_per_step": gather_ms / K,
                   "GB_s": gather_bytes * K / (gather_ms / 1e3) / 1e9},
        "wrap": {"pack_block_unit_f32_ms": pack_ms,
                 "pack_GB_s": pack_bytes / (pack_ms / 1e3) / 1e9},
    }
    if cpu is not None:
        out["parity"] = out_parity
    if not args.no_ceiling:
        log("HBM direction probes: reads, writes and a copy alone")
        dirs = hbm_directions(zs, torch, dev, read_bytes=28, write_bytes=14)
        dirs["fused_over_bound"] = achieved / dirs["ideal_overlap_bound_GB_s"]
        dirs["fused_over_triad"] = achieved / dirs["triad_GB_s"]
        out["roofline"]["hbm_directions"] = dirs
    if not args.no_copy:
        a = torch.empty(1 << 30, device=dev)          # 4 GiB fp32
        bb = torch.empty_like(a)
        a.fill_(1.0)
        copy_ms = timed_calls(torch, lambda: bb.copy_(a), 4, warm=2)
        out["copy_4GiB"] = {"ms": copy_ms, "GB_s": 2 * 4 * (1 << 30) / (copy_ms / 1e3) / 1e9}
        del a, bb
    if not args.no_unfused:
        log("unfused leg: zs_reduce_shard then zs_adamw_step on the same buckets")
        out["unfused"] = unfused_leg(zs, torch, p, m, v, wshard, buckets, D, args.warmup + K + 1, hp)
        out["unfused"]["fused_ms_per_step"] = adam_ms / K
    if not args.no_in_place:
        log("in-place leg: the working shard written into its slot of the unit buffer")
        out["in_place_gather"] = in_place_leg(zs, torch, p, m, v, buckets,
                                              args.warmup + K + 1, hp)
        out["in_place_gather"]["main_ms_per_step"] = ms_per_step
    if not args.no_pipeline:
        log("pipeline leg: contributions streamed per bucket, overlapped with the step")
        out["pipeline"] = pipeline_leg(zs, torch, p, m, v, wshard, buckets, pool, D,
                                       args.warmup + K + 1, hp)
    if not args.no_ragged:
        log("ragged leg: pack and gather of the 10,000-tensor unit, fp32 and bf16")
        out["ragged_pack_gather"] = ragged_move_leg(zs, torch, W, dev)
    if not args.no_ckpt:
        log("re-shard and checkpoint leg")
        out["reshard_checkpoint"] = reshard_ckpt_leg(zs, torch, W, dev, p, m, v, wshard,
                                                     buckets[0][0], D)
    if not args.no_offload:
        log("offload leg: LLaMA-7B D=32 rank shard, AdamW on host cores")
        out["offload"] = offload_leg(zs, torch, W, dev, hp, args.host_threads)
    if not args.no_hybrid:
        log("hybrid leg: LLaMA-7B rank shard under HYBRID_SHARD, 4 x 8 contributions")
        out["hybrid_shard"] = hybrid_leg(zs, torch, W, dev, hp, steps=3,
                                         arenas=(p, m, v, wshard))
    if not args.no_configs:
        log("configs leg: the fused kernel on the other workloads' rank shards")
        out["other_workloads"] = configs_leg(zs, torch, W, dev, hp, launches=10,
                                             arenas=(p, m, v, wshard),
                                             oracle=not args.no_cpu_baseline)
    if cpu is not None:
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
        except OSError:
            pass
        cpu["host"] = {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
                       "cpu_model": model}
        if "other_workloads" in out:
            cpu["per_workload"] = {k: v["oracle"] for k, v in out["other_workloads"].items()
                                   if "oracle" in v}
        out["cpu_baseline"] = cpu
        checks = [out["parity"]] + list(cpu.get("per_workload", {}).values())
        out["parity"]["all_bit_exact"] = all(c["bit_exact"] for c in checks)
    print(json.dumps(out), flush=True)
    if "parity" in out and not out["parity"]["all_bit_exact"]:
        log("PARITY FAILURE: a timed GPU step differs from the oracle")
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())
