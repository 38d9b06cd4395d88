"""Host-side planning: bucket plan, shard geometry and per-step scalars.

* ``plan_buckets``: walk the arena's tensors from the last to the first (the
  order backward produces them: "A4 -- Multi-GPU with NCCL and ZeRO-1",
  "Part 4") and merge neighbours up to a byte cap ("Distributed training"
  (noeira), "Overlap and graphs", plan_buckets; "Lab 09 -- Parallelism,
  simulated", s.2: 25 MB DDP buckets).  A tensor larger than the cap is a
  bucket of its own.  Buckets are contiguous arena ranges, returned in
  processing order.
* ``zero_stage``: ZeRO-1 only when every bucket splits evenly over N, else
  stage 0 with the message the pages print ("A4", "Part 2 -- Tensor
  Sharding", set_zero_configs).
* ``step_scalars``: learning rate with linear warmup and the AdamW bias
  corrections 1 - beta^t (t from 1), computed in double precision and
  rounded to fp32 for the kernel.
"""

import sys
from dataclasses import dataclass

import numpy as np

DEFAULT_BUCKET_BYTES = 25 * 2 ** 20


def plan_buckets(numels, cap_bytes=DEFAULT_BUCKET_BYTES, elem_bytes=2):
    """``[(offset, length)]`` buckets for tensors of ``numels`` in arena order."""
    starts, pos = [], 0
    for n in numels:
        starts.append(pos)
        pos += int(n)
    plan, cur = [], None  # cur = [lo, hi)
    for i in reversed(range(len(numels))):
        n = int(numels[i])
        if n <= 0:
            continue
        lo = starts[i]
        if cur is not None and (cur[1] - lo) * elem_bytes <= cap_bytes:
            cur[0] = lo
            continue
        if cur is not None:
            plan.append((cur[0], cur[1] - cur[0]))
        cur = [lo, lo + n]
    if cur is not None:
        plan.append((cur[0], cur[1] - cur[0]))
    return plan


def whole_arena(numel):
    return [(0, int(numel))]


def owned_chunk(rank, nranks):
    """Chunk rank ``rank`` holds reduced after the ring reduce-scatter."""
    return (rank + 1) % nranks


def zero_stage(buckets, nranks, requested=1, log=sys.stderr):
    """Stage actually used: 1 if requested and every bucket divides by N, else 0
    ("A4", "Part 2 -- Tensor Sharding": an uneven split falls back to stage 0
    and says so)."""
    if requested == 1 and any(length % nranks for _, length in buckets):
        print(f"ZeRO-1 needs every bucket to split evenly over {nranks} ranks; "
              "running ZeRO stage 0 (plain data parallelism) instead", file=log)
        return 0
    return 0 if requested != 1 else 1


@dataclass
class Hyper:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    max_norm: float = 1.0
    warmup: int = 0


def step_scalars(hyper, t):
    """fp32 scalars of step ``t`` (t >= 1) as a dict for ``adamw_args``."""
    if t < 1:
        raise ValueError("steps count from 1")
    lr = hyper.lr * t / hyper.warmup if 0 < hyper.warmup and t <= hyper.warmup else hyper.lr
    f = np.float32
    return dict(lr=float(f(lr)), beta1=float(f(hyper.beta1)), beta2=float(f(hyper.beta2)),
                eps=float(f(hyper.eps)), weight_decay=float(f(hyper.weight_decay)),
                bias_corr1=float(f(1.0 - hyper.beta1 ** t)),
                bias_corr2=float(f(1.0 - hyper.beta2 ** t)))


def resident_bytes(numel, nranks, stage, grad_bytes=2, longest_bucket=0, shard_bytes=4):
    """Bytes one rank of this pipeline keeps resident for the model state.

    bf16 weights (2 per parameter); the gradient arena (``grad_bytes`` per
    parameter) below stage 2, or two staging buffers of the longest bucket at
    stage 2; the reduced gradient it holds for the optimizer (``shard_bytes``
    per parameter, sharded from stage 1: 4 for the fp32 mean, 2 with the
    gradient shard held in bf16); fp32 master, m and v (12 per parameter,
    sharded from stage 1).  Compare "Lab 09 -- Parallelism, simulated", s.4
    (2 + 2 + 12 bytes per parameter, stage 2 keeping bf16 gradient shards):
    with ``shard_bytes=2`` and the staging left out, stage 2 is the page's
    2 + 14/N bytes per parameter; the fp32 shard holds 2 bytes more per owned
    parameter.
    """
    if shard_bytes not in (2, 4):
        raise ValueError("the gradient shard is held in fp32 (4) or bf16 (2)")
    p, n = float(numel), float(nranks)
    shard = p / n if stage >= 1 else p
    grads = grad_bytes * p if stage < 2 else 2.0 * grad_bytes * longest_bucket
    return 2.0 * p + grads + float(shard_bytes) * shard + 12.0 * shard
