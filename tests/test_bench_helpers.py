"""Host-side helpers of bench.py (no GPU): the stored-counter lookup is tied
to the step kernels' code, not to their comments or layout whitespace."""
import os

import bench


def test_committed_counters_match_the_current_kernel_source():
    # the committed summary was taken on the current step kernels
    t = bench.traffic_from_profiles()
    assert t is not None and 4.4e9 < t < 4.6e9


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    src, hdr = tmp_path / "k.hip", tmp_path / "k.h"
    src.write_text("int f(int x) { return x + 1; }  // one\n/* two */\n")
    hdr.write_text("#define TILES 2\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", (str(src), str(hdr)))
    h0 = bench.kernel_hash()
    src.write_text("// a new comment\nint f(int x)   {\n  return x + 1; /* c */ }\n")
    assert bench.kernel_hash() == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_hash() != h0


def test_kernel_hash_covers_headers_and_flags(tmp_path, monkeypatch):
    from fsdp_sharded_optimizer_zs_amd import build as zs_build
    src, hdr = tmp_path / "k.hip", tmp_path / "k.h"
    src.write_text("int f(int x) { return x + 1; }\n")
    hdr.write_text("#define TILES 2\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", (str(src), str(hdr)))
    h0 = bench.kernel_hash()
    hdr.write_text("#define TILES 4\n")
    h1 = bench.kernel_hash()
    assert h1 != h0
    monkeypatch.setattr(zs_build, "FLAGS", zs_build.FLAGS + ["-DZS_EXTRA=1"])
    assert bench.kernel_hash() != h1


def test_traffic_is_null_when_the_kernel_changed(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int g() { return 0; }\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", (str(src),))
    assert bench.traffic_from_profiles() is None


def test_gpus_above_one_exit_with_a_message(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err
