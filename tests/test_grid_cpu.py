"""Launch geometry of every kernel (zs_grid.h), checked on the host.

The header is compiled with the host C++ compiler into a small driver that
evaluates each launcher's grid for given sizes; the test checks that every
grid is a legal launch (1 .. 2^24 - 1 workgroups of 256 threads, so that the
thread count fits in 32 bits) and that an uncapped grid covers its work (the
kernels loop in grid-stride order past a capped one).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "fsdp_sharded_optimizer_zs_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cstring>
#include "zs_grid.h"
using namespace zs;
int main() {
    char fn[32];
    long long a, b, c;
    while (std::scanf("%31s %lld %lld %lld", fn, &a, &b, &c) == 4) {
        long long r = -1;
        if (!std::strcmp(fn, "tiled")) r = step_tiled_grid(a, int(b));
        else if (!std::strcmp(fn, "scalar")) r = step_scalar_grid(a);
        else if (!std::strcmp(fn, "gflat")) r = gather_flat_grid(a);
        else if (!std::strcmp(fn, "gcopy")) r = gather_copy_grid(a, int(b));
        else if (!std::strcmp(fn, "item")) r = item_grid(a, int(b), int(c));
        else if (!std::strcmp(fn, "streams")) r = streams_grid(a, int(b));
        else if (!std::strcmp(fn, "probe_r")) r = probe_grid(true, a, int(b), int(c));
        else if (!std::strcmp(fn, "probe_w")) r = probe_grid(false, a, int(b), int(c));
        std::printf("%lld\n", r);
    }
    std::printf("max %lld\n", (long long)kMaxGrid);
    return 0;
}
"""

MAXG = (2**32 - 1) // 256
SIZES = [0, 1, 255, 256, 257, 1023, 1024, 1025, 2**24, 2**31 - 1, 2**31, 2**32 - 256,
         2**32 - 255, 2**32 - 1, 2**32, 2**32 + 1, 2**36, 2**40, 2**50, (2**63 - 1) // 64]


@pytest.fixture(scope="module")
def grid_driver(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("grid")
    src, exe = d / "drv.cpp", d / "drv"
    src.write_text(DRIVER)
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)

    def run(cases):
        inp = "".join(f"{f} {a} {b} {c}\n" for f, a, b, c in cases)
        out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True,
                             check=True).stdout.split("\n")
        assert out[len(cases)] == f"max {MAXG}"
        return [int(x) for x in out[:len(cases)]]
    return run


def check(blocks, units, per_block):
    assert 1 <= blocks <= MAXG
    assert blocks * 256 <= 2**32 - 1          # the launch's thread count fits in 32 bits
    if blocks < MAXG:                          # uncapped: the grid covers the work
        assert blocks * per_block >= units


def test_cap_is_largest_legal_grid(grid_driver):
    assert MAXG == 2**24 - 1
    (b,) = grid_driver([("scalar", 2**40, 0, 0)])
    assert b == MAXG


@pytest.mark.parametrize("S", SIZES)
def test_step_grids(grid_driver, S):
    cases = [("tiled", S, t, 0) for t in (1, 2, 4)] + [("scalar", S, 0, 0), ("streams", S, 2, 0)]
    got = grid_driver(cases)
    for (_, _, t, _), b in zip(cases[:3], got[:3]):
        check(b, S // (t * 512), 4)            # one wavefront per tile group, 4 per workgroup
    check(got[3], S, 256)                      # one lane per element
    check(got[4], S // 1024, 4)


@pytest.mark.parametrize("S", SIZES)
def test_move_grids(grid_driver, S):
    cases, want = [], []
    for es in (2, 4):
        if S > (2**63 - 1) // 16 // es:
            continue
        cases.append(("gcopy", S, es, 0))
        want.append(((S * es + 15) // 16 + 1, 256))
        for D in (1, 8, 64):
            if S * D > (2**63 - 1) // 16:
                continue
            per = 8192 // es
            cases.append(("item", S, es, D))
            want.append((-(-S // per) * D, 1))   # one workgroup per 8 KiB work item
            cases.append(("gflat", S * es // 16 * D, 0, 0))
            want.append((S * es // 16 * D, 256))
    for b, (units, per) in zip(grid_driver(cases), want):
        check(b, units, per)


@pytest.mark.parametrize("nvec", [0, 1, 2, 511, 512, 513, 2**28, 2**32, 2**40])
def test_probe_grids(grid_driver, nvec):
    cases = [(f, nvec, pc, 256) for f in ("probe_r", "probe_w") for pc in (0, 1, 4, 16)]
    for (f, _, pc, cu), b in zip(cases, grid_driver(cases)):
        lanes = (nvec + 1) // 2 if f == "probe_r" else nvec
        if pc == 0:
            check(b, lanes, 256)
        else:
            assert 1 <= b <= min(MAXG, pc * cu)
