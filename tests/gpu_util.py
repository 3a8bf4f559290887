"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import zs_oracle as O

REL_TOL = 1e-6     # p, m, v: |a - b| <= 1e-6 |b| per element
BF16_ULPS = 1      # w: at most 1 bf16 ulp (ordered-bit distance)


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_np(t) -> np.ndarray:
    """Copy a device tensor to host; bf16/int16 bits come back as uint16."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def bf16_order(h: np.ndarray) -> np.ndarray:
    h = h.astype(np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h)


def check_f32(got: np.ndarray, want: np.ndarray, what: str, exact: bool = False):
    """Tolerance of the step (rel 1e-6 per element; NaN matches NaN)."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, what
    both_nan = np.isnan(got) & np.isnan(want)
    same = (got == want) | both_nan
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    ok = same | (diff <= REL_TOL * np.abs(want.astype(np.float64)))
    bad = np.flatnonzero(~ok)
    assert bad.size == 0, (f"{what}: {bad.size} elements beyond rel {REL_TOL}, first at "
                           f"{bad[0]}: got {got[bad[0]]!r} want {want[bad[0]]!r}")
    if exact:
        ne = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
        ne = ne[~both_nan[ne]]
        assert ne.size == 0, (f"{what}: {ne.size} elements not bit-identical, first at "
                              f"{ne[0]}: {got[ne[0]]!r} vs {want[ne[0]]!r}")


def check_bf16(got: np.ndarray, want: np.ndarray, what: str, exact: bool = False):
    got = np.asarray(got).view(np.uint16)
    want = np.asarray(want).view(np.uint16)
    assert got.shape == want.shape, what
    nan_g = (got & 0x7FFF) > 0x7F80
    nan_w = (want & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_g, nan_w), f"{what}: NaN positions differ"
    d = np.abs(bf16_order(got) - bf16_order(want))
    d[nan_g] = 0
    assert d.max(initial=0) <= BF16_ULPS, f"{what}: {int((d > BF16_ULPS).sum())} beyond 1 ulp"
    if exact:
        ne = np.flatnonzero((got != want) & ~nan_g)
        assert ne.size == 0, f"{what}: {ne.size} bf16 values not bit-identical (first {ne[:4]})"


def check_bits(got: np.ndarray, want: np.ndarray, what: str):
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.dtype.itemsize == want.dtype.itemsize and got.size == want.size, what
    if got.tobytes() != want.tobytes():
        g = got.view(np.uint8 if got.dtype.itemsize == 1 else f"u{got.dtype.itemsize}")
        w = want.view(g.dtype)
        bad = np.flatnonzero(g != w)
        raise AssertionError(f"{what}: {bad.size} elements differ, first at {bad[0]}")


class SampledRank:
    """The oracle's copy of one rank's shard state, on a fixed index sample.

    The step is elementwise, so the oracle run on the sampled elements gives
    the exact expected values there, at any shard size."""

    def __init__(self, idx: torch.Tensor, p: torch.Tensor, m: torch.Tensor, v: torch.Tensor):
        self.idx = idx
        self.p = to_np(p[idx])
        self.m = to_np(m[idx])
        self.v = to_np(v[idx])
        self.w = None

    def step(self, contribs, dtype: str, hp: O.AdamWHP):
        cs = [to_np(c[self.idx]) for c in contribs]
        self.p, self.m, self.v, self.w = O.rank_step(self.p, self.m, self.v, cs, dtype, hp)

    def check(self, p, m, v, w, what: str, exact: bool = True):
        check_f32(to_np(p[self.idx]), self.p, what + " p", exact)
        check_f32(to_np(m[self.idx]), self.m, what + " m", exact)
        check_f32(to_np(v[self.idx]), self.v, what + " v", exact)
        check_bf16(to_np(w[self.idx]), self.w, what + " w", exact)


def sample_indices(S: int, n: int, seed: int, dev) -> torch.Tensor:
    """n random positions plus both ends (first and last 4096 elements)."""
    if S == 0:
        return torch.zeros(0, dtype=torch.int64, device=dev)
    g = np.random.default_rng(seed)
    parts = [np.arange(min(S, 4096)), np.arange(max(0, S - 4096), S),
             g.integers(0, S, size=min(n, S))]
    return torch.from_numpy(np.unique(np.concatenate(parts))).to(dev)
