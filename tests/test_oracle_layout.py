"""Pins of the oracle's layout, pack/split and gather (CPU only).

Pinned against naive list code (brute force over tiny units), numpy.split
(a library routine) where no padding is needed, and the round-trip identity
of the all-gather diagram of "Building GPT from Scratch -- Part 8: FSDP".
"""
import itertools

import numpy as np
import pytest

from conftest import read_golden
from oracle import zs_oracle as O
import workloads as W


def naive_shards(numels, D):
    """Plain-list layout: element e of tensor j gets label (j, e); pad None."""
    flat = [(j, e) for j, n in enumerate(numels) for e in range(n)]
    S = 0
    while S * D < len(flat):
        S += 1
    flat += [None] * (S * D - len(flat))
    return [flat[r * S:(r + 1) * S] for r in range(D)], S


def labelled_tensors(numels):
    # value 1 + 16*j + e: unique, never 0 (0 marks the pad), fits uint16
    return [np.arange(n, dtype=np.uint16) + np.uint16(1 + 16 * j) for j, n in enumerate(numels)]


def test_layout_bruteforce_small_units():
    cases = 0
    for T in range(0, 4):
        for numels in itertools.product(range(10), repeat=T):
            for D in range(1, 9):
                ref, S_ref = naive_shards(numels, D)
                offsets, N, N_pad, S = O.unit_layout(numels, D)
                assert S == S_ref and N == sum(numels) and N_pad == S * D
                assert 0 <= N_pad - N < D
                assert offsets[0] == 0 and offsets[-1] == N
                if T == 0:
                    continue
                shards = O.pack_flat(labelled_tensors(numels), D)
                assert len(shards) == D
                for r in range(D):
                    want = [0 if lab is None else 1 + 16 * lab[0] + lab[1] for lab in ref[r]]
                    assert shards[r].tolist() == want
                cases += 1
    assert cases > 8000


def test_every_source_element_once_and_pad_zero():
    rng = np.random.default_rng(1)
    for _ in range(50):
        numels = [int(x) for x in rng.integers(0, 300, size=rng.integers(1, 9))]
        D = int(rng.integers(1, 17))
        ts = [rng.integers(1, 2**31, size=n, dtype=np.int64).astype(np.uint32) for n in numels]
        vals = np.concatenate(ts) if ts else np.zeros(0, np.uint32)
        shards = O.pack_flat(ts, D)
        flat = np.concatenate(shards)
        _, N, N_pad, S = O.unit_layout(numels, D)
        assert flat.size == N_pad and all(s.size == S for s in shards)
        assert np.array_equal(np.sort(flat[:N]), np.sort(vals))
        assert not flat[N:].any()


def test_no_pad_matches_numpy_split():
    rng = np.random.default_rng(2)
    for D in (1, 2, 4, 8, 16):
        numels = [int(x) for x in rng.integers(1, 50, size=7)]
        numels[-1] += (-sum(numels)) % D   # make N a multiple of D
        ts = [rng.standard_normal(n).astype(np.float32) for n in numels]
        shards = O.pack_flat(ts, D)
        for a, b in zip(shards, np.split(np.concatenate(ts), D)):
            assert a.tobytes() == b.tobytes()


def test_gather_of_pack_is_identity_bitwise():
    rng = np.random.default_rng(3)
    for dt in (np.uint16, np.float32):
        for _ in range(20):
            shapes = [tuple(int(x) for x in rng.integers(1, 9, size=rng.integers(1, 3)))
                      for _ in range(int(rng.integers(1, 6)))]
            ts = [rng.integers(0, 65535, size=s).astype(dt) if dt is np.uint16
                  else rng.standard_normal(s).astype(dt) for s in shapes]
            D = int(rng.integers(1, 11))
            flat = O.gather_unit(O.pack_flat(ts, D))
            views = O.unit_views(flat, shapes)
            for a, b in zip(views, ts):
                assert a.tobytes() == b.tobytes()


def test_bits_preserved_for_nan_and_negative_zero():
    x = np.array([0x7FC1, 0xFFFF, 0x8000, 0x0001, 0x7F80], dtype=np.uint16)
    sh = O.pack_flat([x], 2)
    assert np.concatenate(sh)[:5].tobytes() == x.tobytes()
    f = np.array([-0.0, np.nan, 1e-45], dtype=np.float32)
    assert np.concatenate(O.pack_flat([f], 4))[:3].tobytes() == f.tobytes()


def test_allgather_diagram():
    """All-gather diagram: rank r holds block r; afterwards all hold A B C D."""
    rows = read_golden("collective_diagrams.txt")
    before = {int(r[1]): r[2].split() for r in rows if r[0] == "allgather.before"}
    after = [r[2].split() for r in rows if r[0] == "allgather.after"][0]
    D = len(before)
    S = 3
    blocks = {sym: np.arange(S, dtype=np.uint16) + np.uint16(10 * (i + 1))
              for i, sym in enumerate("ABCD")}
    shards = []
    for r in range(D):
        held = [s for s in before[r] if s != "-"]
        assert held == [before[r][r]]          # rank r holds only block r
        shards.append(blocks[held[0]])
    flat = O.gather_unit(shards)
    assert flat.tolist() == np.concatenate([blocks[s] for s in after]).tolist()


def test_workload_sizes_match_pages():
    """Unit sizes follow from the shapes; the pages round them."""
    gpt = W.get("gpt3m")
    assert gpt.units[0].numel == 3_281_408
    assert round(gpt.units[0].numel / 1e6, 1) == 3.3          # "3.3M-parameter GPT"
    blk = W.get("llama7b_block").units[0].numel
    assert blk == 202_383_360
    # the 12 d^2 estimate of the 7.10 page, section 5.2, is within 1%
    assert abs(blk - 12 * 4096 ** 2) / blk < 0.01
    full = W.total_numel(W.get("llama7b_full").units)
    assert full == 6_738_415_616 and round(full / 1e9) == 7
    u70 = W.get("llama70b").units
    assert u70[0].numel == 855_654_400 and u70[-1].numel == 524_296_192
    assert round(W.total_numel(u70) / 1e9) == 69                # "70B"-class


@pytest.mark.parametrize("name,D,S", [
    ("gpt3m", 4, 820_352), ("llama7b_block", 8, 25_297_920)])
def test_shard_lengths(name, D, S):
    w = W.get(name)
    _, N, N_pad, s = O.unit_layout(w.units[0].numels, D)
    assert s == S and N_pad == N


def test_rank_shard_lengths_multi_unit():
    w = W.get("llama70b")
    S = [O.unit_layout(u.numels, w.D)[3] for u in w.units]
    assert S[0] == 106_956_800 and S[-1] == 65_537_024
    assert sum(S) == 8_622_081_024
    w = W.get("llama7b_full")
    assert sum(O.unit_layout(u.numels, w.D)[3] for u in w.units) == 210_575_488


def test_flat_source_against_pack():
    rng = np.random.default_rng(9)
    for _ in range(30):
        numels = [int(x) for x in rng.integers(0, 40, size=rng.integers(1, 8))]
        D = int(rng.integers(1, 9))
        offsets, N, N_pad, S = O.unit_layout(numels, D)
        ts = labelled_tensors(numels)
        flat = np.concatenate(O.pack_flat(ts, D)) if N_pad else np.zeros(0, np.uint16)
        j, e = O.flat_source(offsets, np.arange(N_pad))
        for i in range(N_pad):
            want = 0 if j[i] < 0 else int(ts[j[i]][e[i]])
            assert int(flat[i]) == want
