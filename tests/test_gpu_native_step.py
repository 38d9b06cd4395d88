"""The library from plain C on the GPU, against the oracle.

tests/cabi/gpu_step.c (built by ``__graft_entry__.build()``) runs one ZeRO-1
step of N simulated ranks through include/grz.h with its own hipMalloc'd
memory -- no Python binding and no torch in that process.  This test writes
its inputs (seeded, synthetic), runs it as a child process and compares what
it wrote with the oracle's zero1_step, bit for bit.
"""

import math
import os
import subprocess

import numpy as np
import pytest

import gradient_reduce_zero_amd as grz
from oracle.step import Hyper as OHyper
from oracle.step import zero1_step
from parity_util import assert_bits, oracle_states
from workloads import grad_seed, master_init, rank_grad, to_bits

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "cabi", "gpu_step")


@pytest.mark.parametrize("n", [3, 8])
def test_plain_c_step_matches_the_oracle(tmp_path, n):
    if not os.path.exists(EXE):
        pytest.fail("tests/cabi/gpu_step is not built: run __graft_entry__.build()")
    a, b = n * (2 * 4096 + 40), n * (4096 + 8)
    buckets = [(a, b), (0, a)]
    p = a + b
    hg = [to_bits(rank_grad(p, 1e-2, "bf16", grad_seed(2, r))) for r in range(n)]
    master = to_bits(master_init(p))
    states = oracle_states(master, buckets, n)
    hyper = grz.Hyper(max_norm=0.05)
    s = grz.step_scalars(hyper, 1)
    args = np.array([s["lr"], s["beta1"], s["beta2"], s["eps"], s["weight_decay"],
                     s["bias_corr1"], s["bias_corr2"]], np.float32)
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(np.array([n, len(buckets)], np.int32).tobytes())
        f.write(np.array([p], np.int64).tobytes())
        f.write(np.array(buckets, np.int64).tobytes())
        f.write(args.tobytes())
        f.write(np.array([hyper.max_norm], np.float64).tobytes())
        for g in hg:
            f.write(g.tobytes())
        for w, _, _ in states:
            f.write(np.array([w.size], np.int64).tobytes())
            f.write(w.astype(np.float32).tobytes())
    res = subprocess.run([EXE, str(tmp_path / "in.bin"), str(tmp_path / "out.bin")],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    raw = open(tmp_path / "out.bin", "rb").read()
    sqnorm = np.frombuffer(raw, np.float64, 1, 0)[0]
    scale = np.frombuffer(raw, np.float32, 1, 8)[0]
    same = np.frombuffer(raw, np.int32, 1, 12)[0]
    pos = 16
    ref = zero1_step(hg, "bf16", buckets, states, OHyper(max_norm=0.05), 1)
    assert math.isclose(sqnorm, ref["sqnorm"], rel_tol=1e-13)
    assert_bits(np.array([scale]), np.array([ref["scale"]], np.float32), "clip factor")
    assert ref["scale"] < 1 and same == 1
    for r in range(n):
        k = states[r][0].size
        got = [np.frombuffer(raw, np.float32, k, pos + 4 * k * i) for i in range(4)]
        pos += 16 * k
        assert_bits(got[0], ref["means"][r], f"rank {r} mean")
        for i in range(3):
            assert_bits(got[1 + i], ref["states"][r][i], f"rank {r} state {i}")
    assert_bits(np.frombuffer(raw, np.uint16, p, pos), ref["arena"], "replica 0")
    assert pos + 2 * p == len(raw)
