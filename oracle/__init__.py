"""Plain CPU oracle for the data-parallel / ZeRO-1 gradient pipeline.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
``gradient_reduce_zero_amd`` (no kernels, helpers, tables or constants) and
imports nothing from it.  It is slow on purpose: every function follows the
definition written on the source pages in plain NumPy, so that a reader can
check it against them line by line.

Sources (cited by page title and section):

* "Lab 09 -- Parallelism, simulated", s.1 "Ring all-reduce" (the N = 3
  schedule table, the byte count 2(N-1)/N * S), s.2 "Data parallelism: why
  averaging is exact", s.4 "ZeRO: where 16 bytes per parameter go",
  "Tips" (index bookkeeping) and "Common bugs".
* "A4 -- Multi-GPU with NCCL and ZeRO-1", "System Model", "Part 2 -- Tensor
  Sharding", "Part 3 -- Gradient Reduction" (ncclAvg), "Part 4 -- Multi-GPU
  Backward and Update" (reduce, then AdamW on the shard, then AllGather).
* "13.5 Multi-GPU from First Principles", s.13.5.3 and Eq. (13.5.1).
* "Distributed training" (noeira), "Four strategies, one interface"
  (set_lr / clip_grads_device / step), "Overlap and graphs" (plan_buckets).

Modules:

* ``ring``    -- message-passing ring all-reduce simulator with a byte count.
* ``reduce``  -- chunks, owners and the ring-order fold (reduce-scatter-mean).
* ``step``    -- grad norm, clip, AdamW, bf16 rounding, all-gather, full steps.
* ``plan``    -- bucket plan in reverse layer order.
* ``memory``  -- ZeRO model-state bytes per GPU.
* ``lsq``     -- least-squares gradients for the equal-shard identity.

Pinning status (what fixes each function other than itself) is listed in the
module docstrings.  Every function is pinned; none is "parity unpinned".
"""
