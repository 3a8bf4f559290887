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


def test_oracle_check_reports_bit_identity_and_planted_differences():
    """The bench's in-run parity check on host arrays (no GPU): the oracle's
    own result passes as bit-exact; a result with one bit flipped in p or
    one bf16 ulp added to w is reported, with its size."""
    import numpy as np
    from oracle import zs_oracle as O
    rng = np.random.default_rng(0)
    S, D = 4099, 8
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    cs = [O.bf16_round((rng.standard_normal(S) * 1e-3).astype(np.float32)) for _ in range(D)]
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    want = O.rank_step(p, m, v, cs, O.BF16, O.AdamWHP(step=1, **hp))
    n, secs, rec = bench.oracle_check((p, m, v, cs), want, "bf16", 1, hp)
    assert n == S and secs >= 0
    assert rec["bit_exact"] and rec["within_tolerance"] and rec["max_w_ulps"] == 0
    bad_p = want[0].copy()
    bad_p.view(np.uint32)[17] ^= 1                      # one ulp in one fp32 element
    _, _, rec = bench.oracle_check((p, m, v, cs), (bad_p,) + tuple(want[1:]), "bf16", 1, hp)
    assert not rec["bit_exact"] and 0 < rec["max_rel_err"] < 1e-6 and rec["within_tolerance"]
    bad_w = want[3].copy()
    bad_w[5] = bad_w[5] + 2 if bad_w[5] & 0x8000 == 0 else bad_w[5] - 2
    _, _, rec = bench.oracle_check((p, m, v, cs), tuple(want[:3]) + (bad_w,), "bf16", 1, hp)
    assert not rec["bit_exact"] and rec["max_w_ulps"] == 2 and not rec["within_tolerance"]
