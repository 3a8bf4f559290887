"""Pins of the oracle's bf16 conversions against torch's CPU cast (a library
routine), over every bf16 pattern and every fp32 pattern (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import zs_oracle as O


def torch_round(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_widen_every_bf16_pattern():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_widen(h).view(np.uint32)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy().view(np.uint32)
    nan = (h & 0x7FFF) > 0x7F80
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(ours[nan].view(np.float32)))


def test_round_trip_every_bf16_pattern():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    back = O.bf16_round(O.bf16_widen(h))
    nan = (h & 0x7FFF) > 0x7F80
    assert np.array_equal(back[~nan], h[~nan])
    assert np.array_equal(back[nan] | 0x0040, back[nan])          # quiet
    assert np.array_equal(back[nan] & 0x8000, h[nan] & 0x8000)    # sign kept


@pytest.mark.slow
def test_round_every_fp32_pattern():
    """All 2^32 fp32 bit patterns, in chunks; NaNs compared by class only.
    Chunks of 2^21 keep every temporary below the allocator's mmap threshold,
    so memory is reused instead of faulted in afresh (4-5x faster than 2^26)."""
    step = 1 << 21
    for start in range(0, 1 << 32, step):
        u = np.arange(start, start + step, dtype=np.uint32)
        x = u.view(np.float32)
        a = O.bf16_round(x)
        b = torch_round(x)
        nan = (u & 0x7FFFFFFF) > 0x7F800000
        assert not np.any((a != b) & ~nan), hex(start)
        assert np.all((a[nan] & 0x7FFF) > 0x7F80)


def test_round_structured_patterns():
    """Every high half with low halves around the rounding thresholds (fast
    subset of the exhaustive test): ties both ways, just above and below."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000], np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    x = u.view(np.float32)
    a = O.bf16_round(x)
    b = torch_round(x)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    assert np.array_equal(a[~nan], b[~nan])


def test_round_named_cases():
    cases = [
        (0x3F800000, 0x3F80),   # 1.0
        (0x80000000, 0x8000),   # -0.0 keeps its sign
        (0x7F800000, 0x7F80),   # inf
        (0x7F7FFFFF, 0x7F80),   # largest finite rounds up to inf
        (0x3F808000, 0x3F80),   # tie, kept bit even: stays
        (0x3F818000, 0x3F82),   # tie, kept bit odd: rounds up to even
        (0x00008001, 0x0001),   # denormal above half rounds up
        (0x00008000, 0x0000),   # denormal tie rounds to even (zero)
    ]
    for bits, want in cases:
        x = np.array([bits], np.uint32).view(np.float32)
        assert int(O.bf16_round(x)[0]) == want, hex(bits)
