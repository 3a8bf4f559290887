"""CPU oracle for one data-parallel rank's ZeRO-3 shard step.

TEST INFRASTRUCTURE ONLY. This module exists to check the HIP path; the
product never imports, links or runs it. Only the tests, the smoke check and
the benchmark's CPU-baseline leg may call it. It shares no code with the HIP
path: plain numpy, one rounding per elementwise operation, every constant
converted to numpy.float32 explicitly, slow and obviously in order.

Sources (web pages, cited by title and section):

* [ZT] "7.10 -- Fully-sharded data parallel (FSDP / ZeRO-3)", AI / ML Theory,
  chapter 7: section 2 (memory buckets), 3 (ZeRO-1 partition P_r and the
  rank-local optimizer step), 4 (reduce-scatter), 5 (ZeRO-3 unit loop, memory
  accounting), 6 (API, bf16 params over fp32 master and Adam state).
* [GPT8] "Building GPT from Scratch -- Part 8: FSDP -- When the Model Won't
  Fit": "AllGather vs AllReduce" (the two diagrams), "The Lifecycle of a
  Parameter", "Mixed Precision", TL;DR / "Key Takeaways" (same math as DDP).
* [RP] "Distributed LLM Fine-Tuning at Scale: FSDP, ZeRO-3, and Multi-GPU
  Orchestration": section 1 (tier table), section 2 (MixedPrecision policy
  with bf16 reduce dtype).

The pages name Adam/AdamW, an fp32 master copy, and the m and v moments,
but print no update equations, no flat-buffer rule and no rounding rules.
Where they are silent this oracle takes the plainest reading, stated at
each function. Precision: the pages fix fp32 for the master copy and the
moments and bf16 for the working weights, so the oracle computes in fp32
(fp64 only for the host-side scalar constants, rounded to fp32 once).

Parity pins: every function below is pinned in tests/ by closed forms, brute
force, library routines or the pages' printed numbers. Parity unpinned: the
choice of AdamW operation order among mathematically equal forms (see
adamw_step); no page fixes it, and its values are pinned only by closed
forms, exact special cases and an error bound against a float64 Adam.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Sequence, Tuple

import numpy as np

F32 = np.float32
U16 = np.uint16
U32 = np.uint32

BF16 = "bf16"
FP32 = "f32"


# ----------------------------------------------------------------- bf16 bits
# bf16 values travel as raw uint16 bit patterns: the upper half of an IEEE
# binary32 word.

def bf16_widen(h: np.ndarray) -> np.ndarray:
    """bf16 bits -> float32, exact: the bits become the high half of a word."""
    h = np.asarray(h).view(U16) if np.asarray(h).dtype == np.int16 else np.asarray(h, dtype=U16)
    return (h.astype(U32) << U32(16)).view(F32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, IEEE round-to-nearest, ties to even.

    Written from the definition on the bit pattern: keep the high 16 bits,
    and look at the 16 dropped bits r. r above half (0x8000) rounds the
    magnitude up, r below half truncates, r exactly half rounds to the even
    neighbour (the one whose kept low bit is 0). A carry out of the mantissa
    moves to the next binade, and past the largest finite value to infinity,
    as IEEE rounding does. A NaN keeps its sign and high payload and is made
    quiet (bit 6 of the bf16 pattern set).
    """
    u = np.ascontiguousarray(x, dtype=F32).view(U32)
    hi = (u >> U32(16)).astype(U32)
    r = u & U32(0xFFFF)
    up = (r > U32(0x8000)) | ((r == U32(0x8000)) & ((hi & U32(1)) == U32(1)))
    out = hi + up.astype(U32)
    is_nan = (u & U32(0x7FFFFFFF)) > U32(0x7F800000)
    out = np.where(is_nan, hi | U32(0x0040), out)
    return out.astype(U16)


# ------------------------------------------------------------- O1: layout
def unit_layout(numels: Sequence[int], D: int) -> Tuple[List[int], int, int, int]:
    """Flat layout of one FSDP unit.

    [ZT 3] gives each rank r a partition P_r of roughly 1/D of the
    parameters; [ZT 6] and [GPT8 "PyTorch FSDP Implementation"] make one
    transformer block one unit. Reading taken for the unspecified flat rule:
    the unit's tensors are laid end to end in registration order with no
    per-tensor alignment, and the flat length N is padded up to the next
    multiple of D so that every rank owns an equal contiguous shard of S
    elements.

    Returns (offsets, N, N_pad, S); offsets has T+1 entries, offsets[j] is
    where tensor j starts and offsets[T] == N.
    """
    if D < 1:
        raise ValueError("D must be >= 1")
    offsets = [0]
    for n in numels:
        if n < 0:
            raise ValueError("numel must be >= 0")
        offsets.append(offsets[-1] + int(n))
    N = offsets[-1]
    S = -(-N // D)          # ceil(N / D)
    N_pad = S * D
    return offsets, N, N_pad, S


# ------------------------------------------------------ O2: pack and split
def pack_flat(tensors: Sequence[np.ndarray], D: int) -> List[np.ndarray]:
    """Flatten a unit and split it into D shards (bit copy, +0 padding).

    The flat unit is the row-major ravel of each tensor, concatenated in
    order, followed by N_pad - N zero elements; shard r is flat[r*S:(r+1)*S],
    the rank-r block of the all-gather diagram in [GPT8 "AllGather vs
    AllReduce"] and the local_shard of the unit loop in [ZT 5.1]. Values are
    copied as bits: bf16 (uint16), fp32 or any other dtype.
    """
    arrs = [np.ascontiguousarray(t).ravel() for t in tensors]
    dtype = arrs[0].dtype if arrs else np.dtype(U16)
    _, N, N_pad, S = unit_layout([a.size for a in arrs], D)
    flat = np.zeros(N_pad, dtype=dtype)        # +0.0 bits in the pad
    pos = 0
    for a in arrs:
        flat[pos:pos + a.size] = a
        pos += a.size
    return [flat[r * S:(r + 1) * S].copy() for r in range(D)]


def flat_source(offsets: Sequence[int], flat_index: np.ndarray):
    """Where flat positions come from, by the definition of pack_flat: for
    each flat index i returns (j, e) with i = offsets[j] + e, or j = -1 for
    a pad position (i >= N). Empty tensors never own a position."""
    offs = np.asarray(offsets, dtype=np.int64)
    i = np.asarray(flat_index, dtype=np.int64)
    j = np.searchsorted(offs, i, side="right") - 1
    pad = i >= offs[-1]
    j = np.where(pad, -1, j)
    e = np.where(pad, 0, i - offs[np.maximum(j, 0)])
    return j, e


# --------------------------------------------------------------- O3: reduce
def reduce_shard(contribs: Sequence[np.ndarray], dtype: str, scale=None) -> np.ndarray:
    """Reduce-scatter arithmetic for one shard: the mean of D contributions.

    [GPT8 "AllGather vs AllReduce"]: rank r receives the sum over ranks k of
    g_k restricted to its shard; [ZT 4]: reduce-scatter is the all-reduce
    whose output is scattered, so rank r's piece equals the all-reduce result
    on P_r; DDP's all-reduce gives the averaged gradient ([GPT8 "AllGather vs
    AllReduce"], first line). Reading taken: contributions arrive in the
    reduce dtype (bf16 [RP 2] or fp32 [GPT8 "Mixed Precision"]), are widened
    to fp32, summed left to right in rank order starting from c_0, and the
    sum is multiplied once by float32(1/D). The result stays fp32.

    ``scale`` replaces 1/D as the one multiplier (rounded to float32 once):
    1 gives the plain sum of the reduce-scatter diagram, 1/D the average.
    """
    D = len(contribs)
    if D < 1:
        raise ValueError("need at least one contribution")

    def widen(c):
        if dtype == BF16:
            return bf16_widen(c)
        if dtype == FP32:
            return np.asarray(c, dtype=F32)
        raise ValueError(dtype)

    s = widen(contribs[0]).copy()
    for k in range(1, D):
        s = (s + widen(contribs[k])).astype(F32)
    mult = F32(1.0 / D) if scale is None else F32(scale)
    return (s * mult).astype(F32)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """The value a float32 result takes once stored in the reduce dtype:
    bf16 rounds to nearest even (bf16_round) and widens back exactly; fp32
    is unchanged."""
    x = np.asarray(x, dtype=F32)
    if dtype == BF16:
        return bf16_widen(bf16_round(x))
    if dtype == FP32:
        return x.copy()
    raise ValueError(dtype)


def reduce_shard_hybrid(contribs: Sequence[np.ndarray], dtype: str, replicas: int,
                        round_to_reduce_dtype: bool, scale=None) -> np.ndarray:
    """Reduce-scatter arithmetic under HYBRID_SHARD, optionally rounding
    each collective's output to the reduce dtype.

    [GPT8 "Sharding Strategies", "HYBRID_SHARD: The Multi-Node Strategy"]:
    parameters are fully sharded across the D GPUs of a node and replicated
    across the R nodes; a node reduce-scatters its gradients over its local
    ranks, and the nodes then combine their shards with one all-reduce per
    step. [RP 2] and [GPT8 "Mixed Precision"] name the dtype the collectives
    communicate in (bf16 or fp32). Reading taken: contributions are ordered
    replica-major (contribs[j*D + k] is local rank k of node j). Node j's
    partial sum s_j is the left fold of its D widened contributions in fp32;
    when the collectives' outputs are held in the reduce dtype, s_j is
    rounded to it. The nodes' partial sums are folded left in node order in
    fp32 and, again when rounding, rounded to the reduce dtype. The mean is
    one multiply by float32(1/(R*D)) (or by float32(scale) when given, as in
    reduce_shard); the result stays fp32. With R = 1 and no rounding this is
    reduce_shard exactly.
    """
    n = len(contribs)
    if replicas < 1 or n < 1 or n % replicas:
        raise ValueError("need R >= 1 groups of D >= 1 contributions")
    D = n // replicas

    def widen(c):
        if dtype == BF16:
            return bf16_widen(c)
        if dtype == FP32:
            return np.asarray(c, dtype=F32)
        raise ValueError(dtype)

    total = None
    for j in range(replicas):
        s = widen(contribs[j * D]).copy()
        for k in range(1, D):
            s = (s + widen(contribs[j * D + k])).astype(F32)
        if round_to_reduce_dtype:
            s = round_to_dtype(s, dtype)
        total = s if total is None else (total + s).astype(F32)
    if round_to_reduce_dtype:
        total = round_to_dtype(total, dtype)
    mult = F32(1.0 / n) if scale is None else F32(scale)
    return (total * mult).astype(F32)


# --------------------------------------------------------------- O4: AdamW
@dataclasses.dataclass(frozen=True)
class AdamWHP:
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    step: int            # t >= 1: the step being taken


def adamw_constants(hp: AdamWHP) -> dict:
    """Scalar constants of one AdamW step, in double, each rounded to fp32 once.

    beta^t is the product of t factors beta taken left to right in double
    starting from 1.0. The bias corrections are Adam's 1 - beta1^t and
    1 - beta2^t; the step size is lr / (1 - beta1^t); the second-moment
    correction is applied as sqrt(v) / sqrt(1 - beta2^t); decoupled weight
    decay multiplies the parameter by (1 - lr * wd).
    """
    if hp.step < 1:
        raise ValueError("step must be >= 1")
    b1t = 1.0
    b2t = 1.0
    for _ in range(hp.step):
        b1t = b1t * hp.beta1
        b2t = b2t * hp.beta2
    return dict(
        B1=F32(hp.beta1), B1c=F32(1.0 - hp.beta1),
        B2=F32(hp.beta2), B2c=F32(1.0 - hp.beta2),
        SS=F32(hp.lr / (1.0 - b1t)),
        BC2S=F32(math.sqrt(1.0 - b2t)),
        DEC=F32(1.0 - hp.lr * hp.weight_decay),
        EPS=F32(hp.eps),
    )


def adamw_step(p: np.ndarray, m: np.ndarray, v: np.ndarray, g: np.ndarray,
               hp: AdamWHP):
    """One AdamW step on a rank's shard; returns new (p, m, v, w).

    [ZT 3]: rank r updates only its partition with its fp32 master, m and v
    and its slice of the gradient; [ZT 6] and [GPT8 "Mixed Precision"]: the
    master copy and the moments stay fp32, the user-visible parameters are
    bf16. The pages print no equations; this is Adam with bias correction
    and decoupled weight decay, evaluated in fp32 in exactly this order, each
    operation rounded on its own (no fused multiply-add):

        p1  = p * DEC
        m1  = B1 * m + B1c * g
        v1  = B2 * v + B2c * (g * g)
        den = sqrt(v1) / BC2S + EPS
        p2  = p1 - SS * (m1 / den)
        w   = bf16_round(p2)

    Mathematically equal orderings round differently near cancellation, so
    this order is the spec; its choice among equal forms is parity unpinned
    (no page fixes it), while its values are pinned by closed forms.
    """
    k = adamw_constants(hp)
    p = np.asarray(p, dtype=F32)
    m = np.asarray(m, dtype=F32)
    v = np.asarray(v, dtype=F32)
    g = np.asarray(g, dtype=F32)
    p1 = (p * k["DEC"]).astype(F32)
    m1 = ((k["B1"] * m).astype(F32) + (k["B1c"] * g).astype(F32)).astype(F32)
    gg = (g * g).astype(F32)
    v1 = ((k["B2"] * v).astype(F32) + (k["B2c"] * gg).astype(F32)).astype(F32)
    den = ((np.sqrt(v1).astype(F32) / k["BC2S"]).astype(F32) + k["EPS"]).astype(F32)
    upd = (k["SS"] * (m1 / den).astype(F32)).astype(F32)
    p2 = (p1 - upd).astype(F32)
    return p2, m1, v1, bf16_round(p2)


def rank_step(p, m, v, contribs: Sequence[np.ndarray], dtype: str, hp: AdamWHP, scale=None):
    """The rank's shard step: reduce (O3), then AdamW (O4) on its result.

    This is steps 6-7 of [GPT8 "The Lifecycle of a Parameter"]: the reduce-
    scatter gives the rank its gradient shard, the optimizer updates only
    the local shard. Returns (p, m, v, w).
    """
    g = reduce_shard(contribs, dtype, scale)
    return adamw_step(p, m, v, g, hp)


def rank_step_hybrid(p, m, v, contribs: Sequence[np.ndarray], dtype: str, hp: AdamWHP,
                     replicas: int, round_to_reduce_dtype: bool, scale=None):
    """The rank's shard step with the HYBRID_SHARD / reduce-dtype reduce of
    reduce_shard_hybrid, then AdamW (O4). Returns (p, m, v, w)."""
    g = reduce_shard_hybrid(contribs, dtype, replicas, round_to_reduce_dtype, scale)
    return adamw_step(p, m, v, g, hp)


# --------------------------------------------------------------- O5: gather
def gather_unit(shards: Sequence[np.ndarray]) -> np.ndarray:
    """All-gather's local result: flat[r*S + j] = shard_r[j] for every r, j.

    [GPT8 "AllGather vs AllReduce"]: after the all-gather every GPU holds
    [A, B, C, D], rank r's block at position r; [ZT 5.1] gathers a block's
    local shards into its full parameters before each forward and backward.
    All N_pad elements are written, padding included.
    """
    return np.concatenate([np.asarray(s) for s in shards]) if shards else np.zeros(0, U16)


def reshard(shards: Sequence[np.ndarray], N: int, D_new: int) -> List[np.ndarray]:
    """Re-shard a unit of N elements from its D shards to D_new shards.

    [GPT8 "Checkpointing with FSDP"]: a sharded state dict resumes only on
    the same GPU count, while the full state dict (gathered) loads on any
    count. Re-sharding is that full state dict's gather followed by the
    split of a fresh wrap: gather_unit, cut to the N real elements, then
    pack_flat at D_new (its pad is +0 again). Bits are copied unchanged.
    """
    flat = gather_unit(shards)[:N]
    return pack_flat([flat], D_new)


def unit_views(flat: np.ndarray, shapes: Sequence[Tuple[int, ...]]) -> List[np.ndarray]:
    """Per-tensor views of a gathered flat unit at the layout's offsets."""
    offsets, _, _, _ = unit_layout([int(np.prod(s, dtype=np.int64)) for s in shapes], 1)
    return [flat[offsets[j]:offsets[j + 1]].reshape(shapes[j]) for j in range(len(shapes))]


# ----------------------------------------------------------- accounting
def bytes_per_device(N: float, D: int, stage: int) -> float:
    """Per-device non-activation bytes under bf16 mixed precision with Adam.

    [ZT 2]: 2 bytes of bf16 working weights, about 6 of gradients (bf16 plus
    an fp32 accumulator) and 12 of fp32 master, m and v per parameter: 20 in
    all. Stage 0 is pure DP; ZeRO-1 shards the 12 ([ZT 2], [ZT 3]), ZeRO-2
    also the 6 ([ZT 4]), ZeRO-3 all 20 ([ZT 5.2]).
    """
    if stage == 0:
        return 20.0 * N
    if stage == 1:
        return 12.0 * N / D + 2.0 * N + 6.0 * N
    if stage == 2:
        return (12.0 + 6.0) * N / D + 2.0 * N
    if stage == 3:
        return 20.0 * N / D
    raise ValueError(stage)


def bucket_bytes(N: float) -> dict:
    """[ZT 2]'s three buckets of pure DP, per device, for N parameters."""
    return dict(weights=2.0 * N, grads=6.0 * N, optimizer=12.0 * N, total=20.0 * N)


def transient_block_bytes(block_params: float, buffers: int = 1) -> float:
    """[ZT 5.2]: the gathered bf16 block takes |theta_block| * 2 bytes; the
    forward/backward overlap keeps two such buffers."""
    return 2.0 * block_params * buffers


def zero3_steady_bytes(N: float, D: int, block_params: float) -> float:
    """[ZT 5.2]: sharded 20N/D plus the two transient block buffers."""
    return bytes_per_device(N, D, 3) + transient_block_bytes(block_params, 2)
