"""MI355X-native data-parallel / ZeRO-1 gradient pipeline.

Ring-order reduce-scatter-mean of N ranks' gradient arenas, global norm and
clip, AdamW on the owned shard and the bf16 all-gather, as hand-written HIP
kernels for gfx950 behind a C ABI (``include/grz.h``, ``libgrz.so``).  This
package is the thin Python side: the binding (same names as the C entry
points), host planning and the step drivers.  There is no CPU fallback: a
call fails if the library is not built.
"""

from ._native import (GRZ_ARGS_DEVICE, GRZ_BF16, GRZ_BF16_WIRE, GRZ_COOPERATIVE, GRZ_F32,
                      GRZ_F64, GRZ_IN_COMPACT,
                      GRZ_IN_RANGE, GRZ_IN_TILED, GRZ_MAX_RANKS, GRZ_MEAN_BF16,
                      GRZ_NOALLOC_SCRATCH_BYTES, GRZ_OUT_GLOBAL, GRZ_PIECE, GRZ_SUM, GRZ_UNEVEN,
                      GrzError, lib)
from .binding import (StepScalars, Tiled, adamw_args, dp_all_gather, dp_chunk_range,
                      dp_grad_sqnorm,
                      dp_grad_sqnorm_noalloc, dp_grad_sqnorm_of,
                      dp_grad_sqnorm_of_workspace, dp_grad_sqnorm_workspace,
                      dp_piece_count, dp_piece_offset, dp_reduce_scatter_mean,
                      dp_ring_chunk_owner, dp_ring_owned_chunk, dp_shard_numel, dp_tiled_numel,
                      fused_clear, fused_set_spin_limit, fused_timed_out,
                      grz_set_max_blocks,
                      grz_step_args_next, zero1_adamw_gather, zero1_adamw_step,
                      zero1_all_gather, zero1_fused_capacity, zero1_fused_step,
                      zero1_fused_workspace)
from .plan import (Hyper, owned_chunk, plan_buckets, resident_bytes, step_scalars, whole_arena,
                   zero_stage)
from .step import (CapturedStep, DDPOneRank, DDPStep, OverlappedZero1, Zero1AllRanks,
                   Zero1OneRank, Zero2AllRanks, one_rank_step, placed_zeros, state_phase,
                   tiled_receive)

__all__ = [n for n in dir() if not n.startswith("_")]
