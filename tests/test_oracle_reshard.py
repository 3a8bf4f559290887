"""Pins of the oracle's D -> D' re-shard (CPU only): brute force against
plain-list code on every small case, numpy.split where both shard counts
divide N, the identity and round-trip properties, and bit preservation."""
import itertools

import numpy as np
import pytest

from oracle import zs_oracle as O


def naive_reshard(shards, N, D2):
    """Element by element from the definition: flat position i lives in old
    shard i // S at i % S; new shard r holds positions r*S2 .. r*S2+S2-1, and
    positions at or past N are +0."""
    S = len(shards[0]) if shards else 0
    S2 = -(-N // D2)
    out = []
    for r in range(D2):
        row = []
        for j in range(S2):
            i = r * S2 + j
            row.append(int(shards[i // S][i % S]) if i < N else 0)
        out.append(row)
    return out


def test_brute_force_small():
    for N in range(0, 23):
        for D in range(1, 7):
            flat = np.arange(1, N + 1, dtype=np.uint16)
            shards = O.pack_flat([flat], D)
            for D2 in range(1, 7):
                got = O.reshard(shards, N, D2)
                want = naive_reshard(shards, N, D2)
                assert [list(map(int, g)) for g in got] == want, (N, D, D2)


@pytest.mark.parametrize("N,D,D2", [(240, 8, 4), (240, 4, 8), (960, 32, 12), (600, 3, 5)])
def test_matches_numpy_split_when_divisible(N, D, D2):
    rng = np.random.default_rng(N + D + D2)
    flat = rng.standard_normal(N).astype(np.float32)
    new = O.reshard(O.pack_flat([flat], D), N, D2)
    for a, b in zip(new, np.split(flat, D2)):
        assert a.tobytes() == b.tobytes()


def test_identity_and_round_trip():
    rng = np.random.default_rng(1)
    for N, D, D2 in itertools.product([1, 17, 1000, 4099], [1, 3, 8, 16], [1, 2, 5, 8, 64]):
        flat = rng.integers(0, 1 << 16, size=N).astype(np.uint16)
        shards = O.pack_flat([flat], D)
        same = O.reshard(shards, N, D)
        assert all(a.tobytes() == b.tobytes() for a, b in zip(same, shards))
        back = O.reshard(O.reshard(shards, N, D2), N, D)
        assert all(a.tobytes() == b.tobytes() for a, b in zip(back, shards))
        assert O.gather_unit(O.reshard(shards, N, D2))[:N].tobytes() == flat.tobytes()


def test_bits_preserved_and_pad_zero():
    x = np.array([np.nan, -0.0, np.inf, -np.inf, 1e-45, -3.0, 7.0], np.float32)
    x[0] = np.frombuffer(np.uint32(0x7FC12345).tobytes(), np.float32)[0]
    shards = O.pack_flat([x], 3)
    new = O.reshard(shards, x.size, 4)
    flat = O.gather_unit(new)
    assert flat[:x.size].tobytes() == x.tobytes()
    assert flat[x.size:].view(np.uint32).tolist() == [0] * (flat.size - x.size)
