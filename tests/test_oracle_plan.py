"""Bucket plan and memory model of the oracle against hand-worked cases and the
numbers the pages print."""

import pytest

from oracle.memory import zero_memory_bytes
from oracle.plan import plan_buckets
from workloads import arena


def test_plan_hand_worked():
    # Tensors of 4, 3, 5, 2, 9 elements at 1 byte each, cap 7 bytes, walked
    # from the last: [9] alone (over the cap), then 2 + 5 = 7, then 3 + 4 = 7.
    assert plan_buckets([4, 3, 5, 2, 9], 7, 1) == [(14, 9), (7, 7), (0, 7)]
    # Cap 6: 9 alone; 2 + 5 > 6 so 2 alone; 5 alone (5 + 3 > 6); 3; 4 + ... none left.
    assert plan_buckets([4, 3, 5, 2, 9], 6, 1) == [(14, 9), (12, 2), (7, 5), (4, 3), (0, 4)]
    assert plan_buckets([4, 3, 5, 2, 9], 100, 1) == [(0, 23)]
    assert plan_buckets([], 10, 1) == []
    assert plan_buckets([0, 5, 0], 10, 2) == [(0, 5)]


@pytest.mark.parametrize("name", ["char_gpt", "gpt2_124m", "gpt2_1p5b"])
def test_plan_invariants_at_model_sizes(name):
    a = arena(name)
    cap = 25 * 2 ** 20
    buckets = plan_buckets(a.numels, cap, 2)
    # Buckets tile the arena, from its end to its start.
    pos = a.numel
    for off, length in buckets:
        assert off + length == pos
        pos = off
    assert pos == 0
    starts = {o for o, _, _ in a.spans()}
    sizes = {o: n for o, n, _ in a.spans()}
    for i, (off, length) in enumerate(buckets):
        assert off in starts
        if length * 2 > cap:
            assert sizes[off] == length  # only one tensor may exceed the cap
        if i + 1 < len(buckets):
            nxt_off, _ = buckets[i + 1]
            # The next tensor in backward order did not fit.
            prev_tensor = max(o for o in starts if o < off)
            assert (off + length - prev_tensor) * 2 > cap


def test_gpt2_124m_plan_shape():
    a = arena("gpt2_124m")
    buckets = plan_buckets(a.numels, 25 * 2 ** 20, 2)
    assert len(buckets) == 9
    assert buckets[-1] == (0, 50257 * 768)  # wte alone, reduced last
    assert all(length % 64 == 0 for _, length in buckets)


def test_zero_memory_table(golden):
    for n_params, n_gpus, stage, gb, dec in golden("zero_memory.txt"):
        got = zero_memory_bytes(float(n_params), int(n_gpus), int(stage)) / 1e9
        assert round(got, int(dec)) == float(gb)
    assert zero_memory_bytes(7.5e9, 64, 1) / 1e9 == 31.40625
    assert zero_memory_bytes(7.5e9, 64, 2) / 1e9 == 16.640625


def test_char_gpt_arena_matches_printed_memory(golden):
    mb, per, dec = golden("char_gpt_memory.txt")[0]
    assert round(arena("char_gpt").numel * int(per) / 1e6, int(dec)) == float(mb)
