"""Properties of the gfx950 code the library's HIP sources compile to, read
from hipcc's assembly output with the library's own flags (CPU only: hipcc
cross-compiles).

- No packed fp32 VALU instruction anywhere (v_pk_add/mul/fma_f32): the build
  turns the feature off, and a flag that silently stopped working would let
  the compiler emit them again.
- No step kernel spills to scratch.
- The fused step for 8 bf16 contributions issues a whole tile pair's loads
  (16 contribution vectors and 12 state vectors per lane) before it first
  waits on any of them: the schedule that sets its HBM rate. Without the
  kernel's occupancy attribute the compiler interleaves loads and waits.
- The long bf16 folds (16 and 32 contributions and run-time group sizes, flat
  and two-level, fused and reduce-only) issue their contribution loads in
  batches before waiting: an unrolled 16-way fold once issued them one at a
  time behind waits (5.1 against 6.2 TB/s).
- Every kernel reads device memory with global (or scalar) loads, never flat
  ones, and the sources compile without an alignment-mismatch warning (a
  4-byte aligned source vector once reached the copy loop typed as 16-byte
  aligned).
"""
import os
import re
import shutil
import subprocess

import pytest

from fsdp_sharded_optimizer_zs_amd import build as B

pytestmark = pytest.mark.slow

HIPCC = next((c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc"))
              if c and os.path.exists(c)), None)


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if HIPCC is None:
        pytest.skip("hipcc not available")
    out = {}
    warnings = {}
    d = tmp_path_factory.mktemp("isa")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    for src in ("zs_step.hip", "zs_move.hip", "zs_diag.hip"):
        dst = d / (src + ".s")
        cmd = [HIPCC] + flags + ["--cuda-device-only", "-S", "-x", "hip",
                                 os.path.join(B.CSRC, src), "-o", str(dst)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out[src] = dst.read_text()
        warnings[src] = r.stderr
    out["warnings"] = warnings
    return out


def functions(text):
    """(name, body) of every kernel in an assembly listing."""
    res = []
    for m in re.finditer(r"^(_Z\S+):\s*(?:;.*)?$", text, re.M):
        end = text.find("s_endpgm", m.end())
        res.append((m.group(1), text[m.end():end]))
    return res


def test_no_packed_fp32_instructions(asm):
    for src, text in asm.items():
        if src == "warnings":
            continue
        hits = re.findall(r"^\s*(v_pk_(?:add|mul|fma)_f32)\b", text, re.M)
        assert not hits, f"{src}: {sorted(set(hits))}"


def test_step_kernels_do_not_spill(asm):
    text = asm["zs_step.hip"]
    sizes = re.findall(r"\.private_segment_fixed_size:\s*(\d+)", text)
    assert sizes and all(int(x) == 0 for x in sizes)


def test_fused_step_issues_a_tile_pair_of_loads_before_waiting(asm):
    kern = [(n, b) for n, b in functions(asm["zs_step.hip"])
            if re.search(r"adamw_vec_kernelILi1ENS0_7FlatSumILi1ELi8EEELi2E", n)]
    assert len(kern) == 1, [n for n, _ in kern]
    ops = re.findall(r"^\s*(global_load_dwordx4|s_waitcnt\s+vmcnt)", kern[0][1], re.M)
    longest = run = 0
    for op in ops:
        run = run + 1 if op == "global_load_dwordx4" else 0
        longest = max(longest, run)
    assert longest >= 28, f"longest run of loads before a wait: {longest}"


def load_runs(body):
    """Lengths of the runs of dwordx4 loads between two vmcnt waits."""
    ops = re.findall(r"^\s*(global_load_dwordx4|s_waitcnt\s+vmcnt)", body, re.M)
    out, run = [], 0
    for op in ops:
        if op == "global_load_dwordx4":
            run += 1
        else:
            if run:
                out.append(run)
            run = 0
    if run:
        out.append(run)
    return out


def test_long_bf16_folds_issue_loads_in_batches(asm):
    # flat and two-level, fused and reduce-only, at 16 and 32 contributions
    # and at run-time group sizes (a loop of batches of 8, then one batch of
    # the remainder): loads issued one at a time behind a wait stay rare
    # (the unrolled 16-way fold that was 5.1 TB/s had 28 of its 44 such)
    pat = (r"(adamw|reduce)_vec_kernelILi1ENS0_(7FlatSum|9HybridSum)ILi1ELi(0|16|32)EEELi2E")
    kern = [(n, b) for n, b in functions(asm["zs_step.hip"]) if re.search(pat, n)]
    assert len(kern) == 12, [n for n, _ in kern]
    for n, b in kern:
        runs = load_runs(b)
        singles = sum(1 for r in runs if r == 1)
        assert 10 * singles <= sum(runs), f"{n}: load runs {runs}"


def test_kernels_use_global_loads_and_true_alignment(asm):
    for src in ("zs_step.hip", "zs_move.hip", "zs_diag.hip"):
        for n, b in functions(asm[src]):
            flat = re.findall(r"^\s*(flat_(?:load|store)\w*)", b, re.M)
            assert not flat, f"{src} {n}: {sorted(set(flat))}"
        assert "align-mismatch" not in asm["warnings"][src], asm["warnings"][src][-2000:]
