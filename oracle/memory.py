"""ZeRO model-state bytes per GPU (oracle; test infrastructure).

"Lab 09 -- Parallelism, simulated", s.4 "ZeRO: where 16 bytes per parameter
go": mixed-precision Adam holds 2 bytes of bf16 weights, 2 of bf16 gradients
and k bytes of optimizer state per parameter (k = 12 for fp32 master, m and
v); stage 1 divides the optimizer term by N, stage 2 also the gradient term,
stage 3 also the weight term ("What to implement", item 5, and its tip).

Pins (tests/test_oracle_plan.py, test_zero_memory_table and
test_char_gpt_arena_matches_printed_memory): the page's table, 7.5e9
parameters on 64 GPUs: 120 / 31.4 / 16.6 / 1.875 GB, and 7e9 on 8 GPUs: 112 /
38.5 / 26.25 / 14 GB (1 GB = 1e9 bytes).
"""


def zero_memory_bytes(n_params, n_gpus, stage, k=12):
    """Model-state bytes one GPU holds at ZeRO ``stage`` (0 to 3)."""
    w, g, o = 2.0 * n_params, 2.0 * n_params, float(k) * n_params
    if stage >= 1:
        o /= n_gpus
    if stage >= 2:
        g /= n_gpus
    if stage >= 3:
        w /= n_gpus
    return w + g + o
