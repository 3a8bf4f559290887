"""The oracle's memory accounting against the figures the pages print
(tests/golden/memory_accounting.txt, each row with its page and section)."""
import pytest

from conftest import read_golden
from oracle import zs_oracle as O

GB, MB = 1e9, 1e6
N7, N70 = 7e9, 70e9


def computed(key):
    if key == "dp7b_weights":
        return O.bucket_bytes(N7)["weights"] / GB
    if key == "dp7b_grads":
        return O.bucket_bytes(N7)["grads"] / GB
    if key == "dp7b_optimizer":
        return O.bucket_bytes(N7)["optimizer"] / GB
    if key == "dp7b_total":
        return O.bytes_per_device(N7, 1, 0) / GB
    if key == "zero1_optimizer_d32":
        # what ZeRO-1 saves over pure DP leaves 12N/D of the 12N bucket
        saved = O.bytes_per_device(N7, 32, 0) - O.bytes_per_device(N7, 32, 1)
        return (O.bucket_bytes(N7)["optimizer"] - saved) / GB
    if key == "zero2_grads_d32":
        # what ZeRO-2 saves over ZeRO-1 leaves 6N/D of the 6N bucket
        saved = O.bytes_per_device(N7, 32, 1) - O.bytes_per_device(N7, 32, 2)
        return (O.bucket_bytes(N7)["grads"] - saved) / GB
    if key == "block_buffer_d4096":
        return O.transient_block_bytes(12 * 4096 ** 2) / MB
    if key == "two_block_buffers":
        return O.transient_block_bytes(12 * 4096 ** 2, 2) / MB
    if key == "zero3_7b_d32":
        return O.zero3_steady_bytes(N7, 32, 12 * 4096 ** 2) / GB
    if key == "dp70b_total":
        return O.bytes_per_device(N70, 8, 0) / GB
    if key == "zero2_70b_d8":
        return O.bytes_per_device(N70, 8, 2) / GB
    if key == "fp32_copy_7b":
        return 4 * N7 / GB
    if key == "bf16_copy_7b":
        return O.bucket_bytes(N7)["weights"] / GB
    if key == "bf16_copy_7b_d4":
        return O.bucket_bytes(N7)["weights"] / 4 / GB
    raise KeyError(key)


ROWS = read_golden("memory_accounting.txt")


@pytest.mark.parametrize("row", ROWS, ids=[r[0] for r in ROWS])
def test_page_figure(row):
    key, value, _unit, tol, _cite = row
    got = computed(key)
    want = float(value)
    assert abs(got - want) <= float(tol) * want + 1e-12, (key, got, want)


def test_stage_ordering_and_limits():
    """Each stage shards one more bucket, so memory falls monotonically, and
    ZeRO-3 is exactly the DP total over D."""
    for D in (2, 8, 32, 128):
        b = [O.bytes_per_device(N7, D, s) for s in range(4)]
        assert b[0] > b[1] > b[2] > b[3]
        assert b[3] == b[0] / D
    for s in range(4):
        assert O.bytes_per_device(N7, 1, s) == pytest.approx(20 * N7)
