"""Bucket plan in reverse layer order (oracle; test infrastructure).

"Distributed training" (noeira), "Overlap and graphs": plan_buckets turns the
gradient-ready marks into buckets in backward order, merged up to a size
target.  "Lab 09 -- Parallelism, simulated", s.2: PyTorch DDP's buckets are
25 MB by default and each is all-reduced as soon as backward has produced it.
"A4 -- Multi-GPU with NCCL and ZeRO-1", "Part 4": the backward pass produces
layer L-1 first and layer 0 last, then the embeddings.

Reading: tensors sit in the arena in forward (layer-major) order; the plan
walks them from the last to the first and merges neighbours while the merged
bucket stays within the cap in bytes; a tensor that alone exceeds the cap is a
bucket of its own.  Buckets are returned in processing (backward) order as
``(offset, length)`` in elements, so each one is a contiguous arena range.

Pins (tests/test_oracle_plan.py): hand-worked small plans, and invariants at
the model sizes (the buckets tile the arena, none exceeds the cap unless it is
one tensor, merging the next tensor would exceed it).
"""


def plan_buckets(numels, cap_bytes, elem_bytes):
    """Buckets ``[(offset, length)]`` for tensors of ``numels`` (arena order)."""
    offsets = []
    pos = 0
    for n in numels:
        offsets.append(pos)
        pos += int(n)
    buckets = []
    lo = hi = None
    for i in range(len(numels) - 1, -1, -1):
        n = int(numels[i])
        if n == 0:
            continue
        t_lo, t_hi = offsets[i], offsets[i] + n
        if lo is None:
            lo, hi = t_lo, t_hi
        elif (hi - t_lo) * elem_bytes <= cap_bytes:
            lo = t_lo
        else:
            buckets.append((lo, hi - lo))
            lo, hi = t_lo, t_hi
    if lo is not None:
        buckets.append((lo, hi - lo))
    return buckets
