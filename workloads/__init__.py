"""Seeded synthetic inputs for the ZeRO-3 shard step.

This module is shared by the tests, the benchmark and the smoke check. It
holds the model shapes and value distributions of the workloads and the
seeded generators that draw their inputs. It holds none of the shard step's
own arithmetic: no flat layout, no padding rule, no reduction and no
optimizer. It imports neither the oracle nor the HIP binding.

Workloads (shapes from the pages; sizes are exact element counts):

* ``gpt3m``      -- the 3.3M-parameter GPT of "Building GPT from Scratch --
  Part 8: FSDP" ("The Problem"): 4 blocks, d_model 256, ff 1024, vocab 512,
  tied 512x256 embedding, one FSDP unit, D = 4, bf16 gradients ~N(0, 1e-3).
* ``llama7b_block`` -- one LLaMA-7B decoder block (d = 4096, FFN 11008) as one
  unit ("7.10 -- Fully-sharded data parallel (FSDP / ZeRO-3)", section 5.2
  sizes a block at 12 d^2), D = 8.
* ``llama7b_full`` -- 32 such blocks plus the root unit (embedding, final norm,
  LM head), rank 0's shard at D = 32, Student-t (nu = 3) gradients.
* ``llama70b``   -- the 70B shape of the multi-node section of the Part 8 page
  (80 blocks, d = 8192, GQA k/v 1024 wide, FFN 28672, vocab 32000), rank 0's
  shard at D = 8, one bucket per unit.
* ``llama7b_hybrid`` -- the full LLaMA-7B under HYBRID_SHARD as in the Part 8
  page's multi-node profile (4 nodes x 8 GPUs): rank 0's shard at D = 8 with
  4 replica groups of 8 bf16 contributions, collectives held in bf16.
* ``ragged``     -- 10,000 one-dimensional tensors with log-uniform sizes in
  [64, 2^22], D = 16, fp32 gradients with a shared 1% exact-zero mask (the
  fp32 reduce dtype of the Part 8 page's "Mixed Precision" section).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Sequence, Tuple

import numpy as np

# AdamW hyperparameters shared by every workload (lr, betas, eps, wd).
ADAMW_HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)

PARAM_STD = 0.02      # fp32 master init ~N(0, 0.02)
GRAD_SCALE = 1e-3     # gradient contributions ~N(0, 1e-3) (or t_3 x 1e-3)

Shape = Tuple[int, ...]


@dataclasses.dataclass(frozen=True)
class Tensor:
    name: str
    shape: Shape

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= int(s)
        return n


@dataclasses.dataclass(frozen=True)
class Unit:
    """One FSDP unit: an ordered list of tensors (registration order)."""
    name: str
    tensors: Tuple[Tensor, ...]

    @property
    def numels(self) -> List[int]:
        return [t.numel for t in self.tensors]

    @property
    def numel(self) -> int:
        return sum(self.numels)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # numeric id used in seeds
    D: int                     # simulated data-parallel ranks
    reduce_dtype: str          # "bf16" or "f32"
    steps: int
    grad_dist: str             # "normal" or "student_t3"
    zero_frac: float           # fraction of entries forced to exactly 0
    units: Tuple[Unit, ...]
    ranks: Tuple[int, ...]     # ranks whose shard is stepped and checked
    description: str
    replicas: int = 1          # HYBRID_SHARD replica groups (nodes); 1 = FULL_SHARD
    round_reduce: bool = False  # collectives' outputs held in the reduce dtype


def _gpt3m_unit() -> Unit:
    d, ff, vocab, blocks = 256, 1024, 512, 4
    ts = [Tensor("tok_emb", (vocab, d))]
    for b in range(blocks):
        ts += [
            Tensor(f"h{b}.ln1.w", (d,)), Tensor(f"h{b}.ln1.b", (d,)),
            Tensor(f"h{b}.attn.wq", (d, d)), Tensor(f"h{b}.attn.wk", (d, d)),
            Tensor(f"h{b}.attn.wv", (d, d)), Tensor(f"h{b}.attn.wo", (d, d)),
            Tensor(f"h{b}.ln2.w", (d,)), Tensor(f"h{b}.ln2.b", (d,)),
            Tensor(f"h{b}.ff.w1", (ff, d)), Tensor(f"h{b}.ff.w2", (d, ff)),
        ]
    ts += [Tensor("ln_f.w", (d,)), Tensor("ln_f.b", (d,))]
    return Unit("gpt3m", tuple(ts))


def llama_block_unit(name: str, d: int, ffn: int, kv: int) -> Unit:
    """Decoder block in registration order q, k, v, o, gate, up, down, norms."""
    return Unit(name, (
        Tensor("wq", (d, d)), Tensor("wk", (kv, d)), Tensor("wv", (kv, d)),
        Tensor("wo", (d, d)), Tensor("w_gate", (ffn, d)), Tensor("w_up", (ffn, d)),
        Tensor("w_down", (d, ffn)), Tensor("input_norm", (d,)),
        Tensor("post_attn_norm", (d,)),
    ))


def llama_root_unit(name: str, d: int, vocab: int) -> Unit:
    return Unit(name, (
        Tensor("embed", (vocab, d)), Tensor("final_norm", (d,)),
        Tensor("lm_head", (vocab, d)),
    ))


def ragged_numels(seed: int = 5, count: int = 10_000,
                  lo: int = 64, hi: int = 1 << 22) -> List[int]:
    """numel = floor(exp(U[ln lo, ln hi])), drawn from a seeded generator."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(lo), math.log(hi), size=count)
    return [int(x) for x in np.floor(np.exp(u)).astype(np.int64)]


def _ragged_unit(seed: int = 5) -> Unit:
    kinds = ("norm", "bias", "matrix")
    ns = ragged_numels(seed)
    return Unit("ragged", tuple(Tensor(f"t{i}.{kinds[i % 3]}", (n,))
                                for i, n in enumerate(ns)))


def get(name: str) -> Workload:
    """Workload by name (built on demand: the ragged unit draws 10,000 sizes)."""
    if name == "gpt3m":
        return Workload("gpt3m", 1, 4, "bf16", 10, "normal", 0.0,
                        (_gpt3m_unit(),), (0, 1, 2, 3),
                        "3.3M-param GPT, one unit, D=4, bf16 grads, 10 steps")
    if name == "llama7b_block":
        return Workload("llama7b_block", 2, 8, "bf16", 20, "normal", 0.0,
                        (llama_block_unit("block", 4096, 11008, 4096),), (0,),
                        "one LLaMA-7B decoder block as one unit, D=8, 20 steps")
    if name == "llama7b_full":
        units = tuple(llama_block_unit(f"block{i}", 4096, 11008, 4096)
                      for i in range(32)) + (llama_root_unit("root", 4096, 32000),)
        return Workload("llama7b_full", 3, 32, "bf16", 10, "student_t3", 0.0,
                        units, (0,),
                        "full LLaMA-7B (32 blocks + root), rank-0 shard, D=32")
    if name == "llama70b":
        units = tuple(llama_block_unit(f"block{i}", 8192, 28672, 1024)
                      for i in range(80)) + (llama_root_unit("root", 8192, 32000),)
        return Workload("llama70b", 4, 8, "bf16", 3, "normal", 0.0, units, (0,),
                        "LLaMA-70B shape (80 GQA blocks + root), rank-0 shard, "
                        "D=8, one bucket per unit")
    if name == "llama7b_hybrid":
        units = tuple(llama_block_unit(f"block{i}", 4096, 11008, 4096)
                      for i in range(32)) + (llama_root_unit("root", 4096, 32000),)
        return Workload("llama7b_hybrid", 6, 8, "bf16", 3, "normal", 0.0, units, (0,),
                        "full LLaMA-7B under HYBRID_SHARD on 4 nodes x 8 GPUs: rank-0 "
                        "shard at D=8, 4 replica groups, bf16 collectives, one bucket "
                        "per unit", replicas=4, round_reduce=True)
    if name == "ragged":
        return Workload("ragged", 5, 16, "f32", 5, "normal", 0.01,
                        (_ragged_unit(),), (0, 15),
                        "10,000 ragged tensors, D=16, fp32 grads, 1% zeros")
    raise KeyError(name)


NAMES = ("gpt3m", "llama7b_block", "llama7b_full", "llama70b", "ragged", "llama7b_hybrid")


def seed_for(workload_index: int, step: int, bucket: int, k: int) -> int:
    """Seed of contribution k of a bucket at a step (disjoint per field)."""
    return ((workload_index * 4096 + step) * 4096 + bucket) * 256 + k


# ---------------------------------------------------------------- generators
# torch is imported lazily so that CPU-only users of the shapes need not pay
# for it. Generators run on any torch device; values depend on the device's
# generator, so a test always copies the drawn tensor, never re-draws it.

def _torch():
    import torch
    return torch


def normal_f32(n: int, std: float, seed: int, device="cpu"):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    return x.mul_(std)


def student_t3_f32(n: int, scale: float, seed: int, device="cpu"):
    """t_3 variate z / sqrt(chi2_3 / 3), chi2_3 the sum of 3 squared normals."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros(n, device=device, dtype=torch.float32)
    for _ in range(3):
        e = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        chi.addcmul_(e, e)
    return z.div_(chi.div_(3.0).sqrt_()).mul_(scale)


def as_bf16_bits(x_f32):
    """torch's own fp32 -> bf16 cast, returned as raw int16 bit patterns."""
    torch = _torch()
    return x_f32.to(torch.bfloat16).view(torch.int16)


def zero_mask(n: int, frac: float, seed: int, device="cpu"):
    """Boolean mask with each entry True with probability frac (seeded)."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.rand(n, generator=g, device=device) < frac


def contribution(w: Workload, n: int, step: int, bucket: int, k: int,
                 device="cpu", mask=None):
    """One gradient contribution of length n in the workload's reduce dtype.

    bf16 contributions come back as int16 bit patterns, fp32 ones as float32.
    ``mask`` (True = force exact zero) is shared by all contributions of a
    step when the workload asks for exact zeros.
    """
    seed = seed_for(w.index, step, bucket, k)
    if w.grad_dist == "student_t3":
        x = student_t3_f32(n, GRAD_SCALE, seed, device)
    else:
        x = normal_f32(n, GRAD_SCALE, seed, device)
    if mask is not None:
        x.masked_fill_(mask, 0.0)
    if w.reduce_dtype == "bf16":
        return as_bf16_bits(x)
    return x


def step_mask(w: Workload, n: int, step: int, bucket: int, device="cpu"):
    if w.zero_frac <= 0.0:
        return None
    return zero_mask(n, w.zero_frac, seed_for(w.index, step, bucket, 255), device)


def master_init(n: int, seed: int, device="cpu"):
    """fp32 master parameters ~N(0, 0.02)."""
    return normal_f32(n, PARAM_STD, seed, device)


def tensor_values(unit: Unit, dtype: str, seed: int, device="cpu") -> list:
    """Per-tensor parameter values of a unit (fp32 ~N(0, 0.02), or its bf16
    cast as int16 bits), one seeded draw per tensor."""
    out = []
    for j, t in enumerate(unit.tensors):
        x = normal_f32(t.numel, PARAM_STD, seed * 1_000_003 + j, device)
        x = x.view(t.shape) if t.shape else x
        out.append(as_bf16_bits(x) if dtype == "bf16" else x)
    return out


def small_random_unit(rng: np.random.Generator, max_tensors: int = 12,
                      max_numel: int = 5000) -> Unit:
    """A small ragged unit for parity tests: sizes include 0, 1 and odd."""
    T = int(rng.integers(1, max_tensors + 1))
    special = [0, 1, 2, 3, 7, 8, 9, 15, 17, 63, 64, 65, 255, 257]
    ts = []
    for j in range(T):
        if rng.random() < 0.4:
            n = int(rng.choice(special))
        else:
            n = int(rng.integers(0, max_numel))
        ts.append(Tensor(f"t{j}", (n,)))
    return Unit("small", tuple(ts))


def total_numel(units: Sequence[Unit]) -> int:
    return sum(u.numel for u in units)
