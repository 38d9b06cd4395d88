"""bench.py's host-side contract, checked without a GPU: the one-GPU refusal,
the byte model behind the roofline line, and the committed counter summary
being tied to the kernel source it was measured on."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_bytes_per_owned_element():
    # Reduce: N bf16 chunks read + the fp32 mean written; AdamW: mean, master,
    # m, v read and master, m, v, bf16 written; gather: N - 1 bf16 shards read
    # and written.  78 B at N = 8: 9.75 bytes per arena element.
    b = bench.bytes_per_owned(8)
    assert b == {"reduce": 20, "adamw": 30, "gather": 28}
    assert sum(b.values()) * 842_301_952 == 65_699_552_256
    assert bench.bytes_per_owned(4)["gather"] == 12


def test_traffic_is_reported_only_for_the_measured_source(monkeypatch):
    # The committed counters carry the digest of the kernel source they were
    # measured on; bench.py reports their traffic only while it matches.
    text = open(bench.COUNTERS).read()
    digest = [l.split("=")[1].strip() for l in text.splitlines()
              if l.startswith("kernel_code_digest")][0]
    monkeypatch.setattr(bench, "kernel_digest", lambda: digest)
    for kernel in ("reduce", "adamw", "gather"):
        assert bench.measured_traffic(kernel) > 0
    monkeypatch.setattr(bench, "kernel_digest", lambda: "0" * 64)
    assert bench.measured_traffic("adamw") is None


def test_digest_ignores_comments_and_white_space(tmp_path, monkeypatch):
    src = open(bench.KERNEL_SRC).read()
    base = bench.kernel_digest()
    alt = tmp_path / "grz.hip"
    alt.write_text("// a comment\n" + src.replace("\n", "\n  ") + "\n/* another */\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(alt))
    assert bench.kernel_digest() == base
    alt.write_text(src.replace("kThreads = 256", "kThreads = 128"))
    assert bench.kernel_digest() != base


def test_multi_process_oracle_timing_runs_on_disjoint_tiles():
    # The baseline's second line: the same oracle step over forked workers.
    r = bench.cpu_baseline_parallel(count=20_001, n=8, rank=0, chunk=1, workers=2)
    assert r["cores"] == 2 and r["kind"] == "oracle" and r["value"] > 0
    assert "20001 owned parameters in 2 tiles" in r["sample"]


def test_all_ranks_oracle_timing_whole_arena_and_prefix():
    import torch

    from gradient_reduce_zero_amd.plan import Hyper
    from workloads import rank_grad

    p, n = 8 * 4096 * 3, 8
    grads = [rank_grad(p, 1e-3, "bf16", 11 + r) for r in range(n)]
    whole = bench.cpu_baseline_all_ranks(grads, [(0, p // 2), (p // 2, p // 2)], n, Hyper(), p)
    assert whole["value"] > 0 and whole["sample"].startswith("the whole arena, 2 bucket(s)")
    part = bench.cpu_baseline_all_ranks(grads, [(0, p)], n, Hyper(), 10_007)
    assert part["sample"].startswith(f"the first 10000 of {p} parameters")
    assert grads[0].dtype == torch.bfloat16


def test_ddp_byte_model():
    # sP + 4P/N (reduce) + 2 * 4P(N-1)/N (peer means read and written) + 30P:
    # 39.5 P at N = 8 with bf16 gradients, 4P(N-1)/N of it simulation-only.
    p = 8 * 1000
    b = bench.ddp_bytes(p, 8)
    assert b == {"reduce": 2 * p + p // 2, "gather": 7 * p, "adamw": 30 * p}
    assert sum(b.values()) == 39.5 * p


def test_ddp_oracle_timing_runs():
    from gradient_reduce_zero_amd.plan import Hyper
    from workloads import rank_grad

    inc = [rank_grad(5000, 1e-3, "bf16", 21 + j) for j in range(8)]
    r = bench.cpu_baseline_ddp(inc, 8, Hyper(), 4099)
    assert r["value"] > 0 and "an arena of 4096 parameters" in r["sample"]


def test_multi_process_oracle_timing_reports_a_failed_worker_promptly():
    # A worker that raises (here: an unknown wire precision) ends the run with
    # an error naming it, instead of leaving the others waiting.
    import time

    import pytest

    t0 = time.monotonic()
    with pytest.raises(RuntimeError, match="unknown wire precision"):
        bench.cpu_baseline_parallel(1000, 8, 0, 1, 2, wire="fp8")
    assert time.monotonic() - t0 < 60
