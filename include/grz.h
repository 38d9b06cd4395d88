/*
 * grz.h -- C ABI of libgrz, the data-parallel / ZeRO-1 gradient pipeline on
 * one AMD Instinct MI355X (gfx950).
 *
 * One step of the pipeline, for N ranks whose gradients sit in N flat arenas:
 *
 *   dp_reduce_scatter_mean   ring-order average of the ranks' gradients
 *   dp_grad_sqnorm           global squared norm and clip factor
 *   dp_grad_sqnorm_of        the same, straight from an fp32 gradient array
 *   zero1_adamw_step         clipped AdamW on the owned shard (+ bf16 copy,
 *                            optionally written straight into the replicas)
 *   zero1_all_gather         owned bf16 shards into every replica arena
 *   dp_all_gather            the same for fp32 / fp64 / bf16 shards (the
 *                            second half of a plain all-reduce)
 *   zero1_fused_step         the four above for one shard in one launch
 *
 * Sources: "Lab 09 -- Parallelism, simulated" s.1 "Ring all-reduce" (the
 * N = 3 schedule table; "Tips": in reduce-scatter step t rank r sends chunk
 * (r - t) mod N and ends owning chunk (r + 1) mod N) and s.2 (sum, then
 * divide by N); "A4 -- Multi-GPU with NCCL and ZeRO-1", "Part 2 -- Tensor
 * Sharding", "Part 3 -- Gradient Reduction" (reduce-scatter with ncclAvg),
 * "Part 4 -- Multi-GPU Backward and Update" (AdamW only on the shard, then
 * all-gather); "Distributed training" (noeira), "Four strategies, one
 * interface" (clip_grads_device, step; one flat arena per replica) and "The
 * process group" (every rank simulated on one device).
 *
 * Conventions shared by every entry point:
 *
 *  - Memory.  Every pointer named "device" is HIP device memory owned by the
 *    caller; the library allocates nothing and keeps no state between calls
 *    (apart from the per-thread grid cap of grz_set_max_blocks, which never
 *    changes a result, and the static per-device scratch of
 *    dp_grad_sqnorm_noalloc), so concurrent calls on different streams are
 *    safe when they touch disjoint buffers.  Buffers must stay alive until
 *    the stream has run the enqueued work.  Host arrays (pointer tables, bucket lists, argument
 *    structs) are read during the call only.
 *  - Streams.  Work is enqueued on `stream` (0 = the null stream).  No entry
 *    point synchronises the host: results are ready when the stream is.
 *  - Errors.  Arguments are checked before anything is enqueued; on a bad
 *    argument nothing is launched and a GRZ_E* code is returned (see
 *    grz_strerror).  A launch failure reported by HIP returns GRZ_EHIP.
 *  - Buckets.  A bucket is a contiguous element range [offset, offset +
 *    length) of the arena; buckets are listed in processing order (reverse
 *    layer order: "Distributed training", "Overlap and graphs", plan_buckets;
 *    "A4", "Part 4": the backward pass produces the last layer first).
 *    Chunk c of a bucket is its c-th piece under the numpy.array_split rule
 *    (the first length % N chunks are one element longer).
 *  - Shards.  The ZeRO-1 shard of chunk c is chunk c of every bucket,
 *    concatenated in processing order ("shard-compact" layout).  Rank r owns
 *    chunk (r + 1) mod N.  Unless GRZ_UNEVEN is given, every bucket length
 *    must be divisible by N (an uneven count is an error in "Part 2 --
 *    Tensor Sharding"), else GRZ_EINDIVISIBLE.
 *  - Pieces.  The norm is summed over pieces of GRZ_PIECE consecutive
 *    elements of one chunk (the last piece of a chunk may be shorter).  The
 *    pieces of a plan are numbered bucket by bucket, chunk 0..N-1 within a
 *    bucket, piece by piece within a chunk; dp_piece_count gives their
 *    number and dp_piece_offset where a (bucket, chunk) starts.  The same
 *    pieces, hence the same norm bits, come out of a ZeRO-1 and a plain
 *    data-parallel run of the same plan.
 *  - Arithmetic.  bf16 and fp32 gradients are summed in fp32, fp64 ones in
 *    fp64, one rounding per addition, in ring order; the mean is one IEEE
 *    division by N.  AdamW runs in fp32 with every operation rounded on its
 *    own (no fused multiply-add) and correctly rounded division and square
 *    root.  bf16 outputs are round-to-nearest-even of the fp32 master.
 */
#ifndef GRZ_H
#define GRZ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  GRZ_OK = 0,
  GRZ_EINVAL = 1,        /* null pointer, bad count, bad dtype, bad flag, ... */
  GRZ_EINDIVISIBLE = 2,  /* a bucket length is not divisible by N            */
  GRZ_EALIGN = 3,        /* a device pointer is not aligned to its element   */
  GRZ_EHIP = 4,          /* HIP reported an error when launching             */
  GRZ_ERANGE = 5         /* a bucket leaves the arena or a size is too large */
};

/* Gradient element types. */
enum { GRZ_F32 = 0, GRZ_BF16 = 1, GRZ_F64 = 2 };

/* Flags.  An entry point returns GRZ_EINVAL for a flag it does not take:
 * the reduce (dp_reduce_scatter_mean and its _range form) takes all but
 * GRZ_ARGS_DEVICE and GRZ_COOPERATIVE, the _weighted form all but those and
 * GRZ_SUM; zero1_adamw_gather takes GRZ_UNEVEN, GRZ_ARGS_DEVICE and
 * GRZ_MEAN_BF16; the
 * all-gathers take GRZ_UNEVEN; zero1_fused_step GRZ_UNEVEN, GRZ_IN_COMPACT,
 * GRZ_ARGS_DEVICE and GRZ_COOPERATIVE.  Their meaning is in each entry
 * point's comment. */
enum {
  GRZ_SUM = 1,        /* keep the sum: skip the division by N            */
  GRZ_UNEVEN = 2,     /* allow bucket lengths not divisible by N         */
  GRZ_IN_COMPACT = 4, /* rank inputs hold only the reduced chunk, compact */
  GRZ_BF16_WIRE = 8,  /* bf16 gradients: round every partial sum to bf16  */
  GRZ_IN_RANGE = 16,  /* rank inputs hold only the reduced bucket range     */
  GRZ_ARGS_DEVICE = 32, /* zero1_adamw_gather: `args` is a device pointer   */
  GRZ_OUT_GLOBAL = 64,  /* reduce, chunk >= 0: mean_out indexed like the arena */
  GRZ_IN_TILED = 128,   /* with GRZ_IN_COMPACT: one receive buffer, the N ranks'
                           values of each piece side by side               */
  GRZ_MEAN_BF16 = 256,  /* the mean (gradient shard) is held in bf16         */
  GRZ_COOPERATIVE = 512 /* zero1_fused_step: a cooperative launch            */
};

#define GRZ_MAX_RANKS 16    /* N and the number of replicas per call       */
#define GRZ_PIECE 4096      /* elements per norm piece                      */

typedef struct {
  int64_t offset; /* first element of the bucket in the arena */
  int64_t length; /* elements in the bucket                   */
} grz_bucket;

/* Per-step AdamW scalars, all fp32.  bias_corr1/2 are 1 - beta1^t and
 * 1 - beta2^t for the step t (starting at 1), evaluated by the caller. */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
  float bias_corr1;
  float bias_corr2;
} grz_adamw_args;

/* Version of the ABI (major * 100 + minor). */
int grz_version(void);

/* Launch-width knob: the largest grid (workgroups) the grid-stride kernels
 * use; the default, 2^30, means one workgroup per tile (4096 elements and
 * 256 threads for the reduce, 512 and 64 for the all-gather, 256 and 64 for
 * the optimizer).
 * It changes speed only; the piece layout, the fold order and the norm tree,
 * hence every result bit, do not depend on it.  It applies to the calls the
 * calling host thread makes afterwards (each thread has its own value,
 * starting at 2^30), so callers on other threads never see it.  GRZ_EINVAL
 * outside 1..2^30. */
int grz_set_max_blocks(int blocks);

/* Static description of a status code; never NULL. */
const char* grz_strerror(int status);

/* Chunk rank `rank` owns after the ring reduce-scatter: (rank + 1) mod N
 * ("Lab 09", s.1, the "owns" row; "Tips").  -1 on a bad argument. */
int dp_ring_owned_chunk(int rank, int nranks);

/* Rank that owns chunk `chunk`: (chunk - 1) mod N.  -1 on a bad argument. */
int dp_ring_chunk_owner(int chunk, int nranks);

/* Range of chunk `chunk` of a bucket of `length` elements split over N
 * (array_split rule): *offset within the bucket and *count elements. */
int dp_chunk_range(int64_t length, int nranks, int chunk, int64_t* offset, int64_t* count);

/* Number of norm pieces of a plan over all N chunks of every bucket, or a
 * negative GRZ_E* code. */
int64_t dp_piece_count(const grz_bucket* buckets, int nbuckets, int nranks, int flags);

/* Index of the first piece of chunk `chunk` of bucket `bucket`, or a
 * negative GRZ_E* code. */
int64_t dp_piece_offset(const grz_bucket* buckets, int nbuckets, int nranks, int flags,
                        int bucket, int chunk);

/* Elements of the ZeRO-1 shard of chunk `chunk` (sum over buckets of the
 * chunk's length), or a negative GRZ_E* code. */
int64_t dp_shard_numel(const grz_bucket* buckets, int nbuckets, int nranks, int chunk,
                       int flags);

/* Elements of the GRZ_IN_TILED receive buffer of chunk `chunk`: the chunk's
 * pieces (GRZ_PIECE elements each, the last piece of each bucket's chunk
 * possibly shorter) times N times GRZ_PIECE, or a negative GRZ_E* code. */
int64_t dp_tiled_numel(const grz_bucket* buckets, int nbuckets, int nranks, int chunk,
                       int flags);

/*
 * Ring-order reduce-scatter-mean ("Lab 09", s.1 and "Tips"; "A4", "Part 3",
 * ncclReduceScatter / ncclAllReduce with ncclAvg).
 *
 * rank_grads  host array of N device pointers: rank j's flat gradient arena
 *             of `dtype` elements.  With GRZ_IN_COMPACT, rank j's values of
 *             chunk `chunk` only, in shard-compact layout (what arrives over
 *             the wire for one owner).  With GRZ_IN_COMPACT | GRZ_IN_TILED,
 *             the N ranks' values arrive in one receive buffer of
 *             dp_tiled_numel elements: number the chunk's pieces k = 0, 1, ...
 *             in plan order (bucket by bucket, GRZ_PIECE elements each, the
 *             last piece of each bucket's chunk possibly shorter); rank j's
 *             values of piece k start at element (k * N + j) * GRZ_PIECE
 *             (the rest of a short piece's slot is not read).  rank_grads[j]
 *             must then be the buffer + j * GRZ_PIECE elements (GRZ_EINVAL
 *             otherwise).  A tile's loads are then one contiguous run instead
 *             of N runs in N buffers, which MI355X's HBM streams faster (the
 *             7B share's reduce 2.62-2.65 ms against 2.76-2.77 ms); the
 *             results are the same bits.
 * nranks      N, 1..GRZ_MAX_RANKS.
 * dtype       GRZ_F32, GRZ_BF16 (uint16 bit patterns) or GRZ_F64.
 * buckets     host array of `nbuckets` (1..) buckets in processing order.
 * chunk       0..N-1: reduce that chunk of every bucket (ZeRO-1; mean_out is
 *             shard-compact, dp_shard_numel elements).  -1: reduce every
 *             chunk (plain data parallelism; mean_out is indexed like the
 *             arena and only bucket ranges are written).
 * flags       GRZ_SUM, GRZ_UNEVEN, GRZ_IN_COMPACT (needs chunk >= 0),
 *             GRZ_IN_TILED (needs GRZ_IN_COMPACT),
 *             GRZ_OUT_GLOBAL (chunk >= 0: mean_out is indexed like the arena
 *             and only the chunk's ranges are written -- the reduce-scatter
 *             half of a plain all-reduce, whose all-gather half, dp_all_gather,
 *             brings the other chunks; no effect with chunk -1),
 *             GRZ_BF16_WIRE (needs GRZ_BF16): the ring's wire format is bf16,
 *             so every partial sum of the fold -- the last one included -- is
 *             rounded to bf16 (nearest even) before the next rank adds to it
 *             ("13.5 Multi-GPU from First Principles", exercise 8); the mean
 *             is that bf16 sum divided by N in fp32.
 *             GRZ_MEAN_BF16 (F32 or BF16 input): the owner holds its gradient
 *             shard in bf16, as "Lab 09", s.4 counts a ZeRO-2 rank's bytes
 *             (2 per parameter, divided by N): the fp32 mean is rounded once
 *             to bf16 (nearest even) and written as uint16 bit patterns.
 * mean_out    device; fp32 for F32/BF16 input (uint16 bf16 patterns with
 *             GRZ_MEAN_BF16), fp64 for F64 input.
 * piece_sqnorm device fp64 array of dp_piece_count elements, or NULL.  The
 *             slots of the reduced chunks receive the sum of squares of the
 *             piece's output values (with GRZ_MEAN_BF16, of the rounded
 *             values); other slots are left untouched.
 *
 * Element c-th chunk value = (((g_c + g_{c+1}) + g_{c+2}) + ... + g_{c-1}) / N
 * with rank indices mod N: the sum starts at rank c and travels the ring.
 */
int dp_reduce_scatter_mean(const void* const* rank_grads, int nranks, int dtype,
                           const grz_bucket* buckets, int nbuckets, int chunk, int flags,
                           void* mean_out, double* piece_sqnorm, hipStream_t stream);

/*
 * dp_reduce_scatter_mean restricted to buckets [bucket_first, bucket_first +
 * bucket_count) of the plan: the call a bucket-overlapped backward issues as
 * each bucket's gradients become ready ("A4", "Part 3": the reduction runs
 * on its own stream, ordered after the compute stream by an event; "Lab 09",
 * s.2, and "Distributed training", "Overlap and graphs": each bucket is
 * reduced as soon as backward has produced it).  Shard-compact offsets,
 * arena offsets, piece numbers and GRZ_IN_TILED slots are those of the whole
 * plan (only the range's slots are read), so reducing
 * the buckets one call at a time, in any order, leaves exactly the bytes one
 * call over the whole plan leaves.  GRZ_EINVAL if the range leaves the plan.
 *
 * With GRZ_IN_RANGE (not with GRZ_IN_COMPACT), rank_grads[j] holds only the
 * range: arena element i is at index i - lo, lo the lowest offset of the
 * range's buckets.  This is how a ZeRO-2 backward feeds the reduction from a
 * staging buffer the size of one bucket instead of a full gradient arena
 * ("Lab 09", s.4, stage 2 shards the gradients too; "Distributed training",
 * "Four strategies, one interface", ZeroSharded[2]).
 */
int dp_reduce_scatter_mean_range(const void* const* rank_grads, int nranks, int dtype,
                                 const grz_bucket* buckets, int nbuckets, int bucket_first,
                                 int bucket_count, int chunk, int flags, void* mean_out,
                                 double* piece_sqnorm, hipStream_t stream);

/*
 * Token-weighted reduce-scatter for shards of unequal size ("Lab 09", s.2:
 * with variable-length sequences, sum the per-token losses and divide by the
 * global token count; "13.5 Multi-GPU from First Principles", exercise 2:
 * averaging the shards' means weights a token by the size of its shard, and
 * the exact recipe needs the token counts exchanged before the update).
 *
 * rank_grads[j] holds rank j's gradient SUMMED over its own tokens (not
 * divided); token_counts (host, N entries >= 0) are the ranks' token counts.
 * The library adds the counts (the one extra scalar all-reduce) and computes
 * (ring-order sum) / total, one IEEE division, total <= 2^24 (GRZ_ERANGE
 * above, so that it is an exact fp32).  Everything else is
 * dp_reduce_scatter_mean_range; GRZ_SUM is refused.
 */
int dp_reduce_scatter_weighted(const void* const* rank_grads, const int64_t* token_counts,
                               int nranks, int dtype, const grz_bucket* buckets, int nbuckets,
                               int bucket_first, int bucket_count, int chunk, int flags,
                               void* mean_out, double* piece_sqnorm, hipStream_t stream);

/* Bytes of workspace dp_grad_sqnorm needs for `npieces` pieces (may be 0). */
size_t dp_grad_sqnorm_workspace(int64_t npieces);

/*
 * Global squared norm and clip factor ("Distributed training",
 * clip_grads_device(max_norm): clipping stays on the device).
 *
 * piece_sqnorm  device fp64, `npieces` partial sums in piece order.
 * max_norm      clip threshold; <= 0 disables clipping (factor 1).
 * workspace     device, dp_grad_sqnorm_workspace(npieces) bytes (NULL if 0).
 * sqnorm_out    device fp64 scalar: the pieces summed in a fixed tree order
 *               that depends only on npieces.
 * clip_scale_out device fp32 scalar: fp32(max_norm / sqrt(sqnorm)) when
 *               sqrt(sqnorm) > max_norm, else 1.
 */
int dp_grad_sqnorm(const double* piece_sqnorm, int64_t npieces, double max_norm,
                   void* workspace, double* sqnorm_out, float* clip_scale_out,
                   hipStream_t stream);

/*
 * dp_grad_sqnorm without a workspace argument and without allocating, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The tree's middle
 * levels go to a static array of GRZ_NOALLOC_SCRATCH_BYTES per device, which
 * the library holds until the process ends; its device address is looked up
 * on the first call on each device (the device current when the call is made,
 * which must be the stream's).  Same arguments, results (bit for bit) and
 * errors as dp_grad_sqnorm, plus GRZ_ERANGE when
 * dp_grad_sqnorm_workspace(npieces) exceeds GRZ_NOALLOC_SCRATCH_BYTES (more
 * than 33,546,240 pieces, about 1.4e11 gradient elements) and GRZ_EINVAL when
 * a non-null stream belongs to another device than the current one.  Nothing
 * needs clearing between calls: each call writes every scratch value it
 * reads.  All calls on one device share the array, so calls that overlap on
 * one device (different streams, or different host threads) race: order them.
 */
#define GRZ_NOALLOC_SCRATCH_BYTES 65536
int dp_grad_sqnorm_noalloc(const double* piece_sqnorm, int64_t npieces, double max_norm,
                           double* sqnorm_out, float* clip_scale_out, hipStream_t stream);

/*
 * dp_grad_sqnorm, and in its last launch the work of grz_step_args_next:
 * *current = table[min(*counter, count - 1)]; *counter += 1 (all device
 * memory).  A captured step ("Distributed training", "Overlap and graphs": one
 * graph per GPU, replayed) needs both before its optimizer runs; done by the
 * norm's single-workgroup launch they cost one launch fewer per replay.
 * Arguments and errors as dp_grad_sqnorm and grz_step_args_next.
 */
int dp_grad_sqnorm_step_args(const double* piece_sqnorm, int64_t npieces, double max_norm,
                             void* workspace, double* sqnorm_out, float* clip_scale_out,
                             const grz_adamw_args* table, int64_t count, int64_t* counter,
                             grz_adamw_args* current, hipStream_t stream);

/* Bytes of workspace dp_grad_sqnorm_of needs for `n` gradient elements. */
size_t dp_grad_sqnorm_of_workspace(int64_t n);

/*
 * dp_grad_sqnorm over a plain fp32 gradient array that is already reduced
 * (one chunk of one bucket): the library forms the piece sums itself, pieces
 * of GRZ_PIECE consecutive elements summed exactly as dp_reduce_scatter_mean
 * sums them, then combines them in the same tree.  So the result equals, bit
 * for bit, dp_reduce_scatter_mean of a single rank (N = 1, one bucket of `n`
 * elements) followed by dp_grad_sqnorm ("Distributed training",
 * clip_grads_device(max_norm) on a flat fp32 arena).
 *
 * grad          device fp32, `n` elements (any 4-byte alignment).
 * workspace     device, dp_grad_sqnorm_of_workspace(n) bytes, 8-byte aligned;
 *               on return it holds the ceil(n / GRZ_PIECE) piece sums first.
 * sqnorm_out, clip_scale_out, max_norm  as for dp_grad_sqnorm (either output
 *               may be NULL, not both).
 * Errors: GRZ_EINVAL for a NULL grad/workspace with n > 0, both outputs NULL
 * or n < 0; GRZ_EALIGN; GRZ_ERANGE beyond 4096^3 pieces.
 */
int dp_grad_sqnorm_of(const float* grad, int64_t n, double max_norm, void* workspace,
                      double* sqnorm_out, float* clip_scale_out, hipStream_t stream);

/*
 * Clipped AdamW on one rank's shard ("A4", "Part 4": adamw_update only for
 * this rank's shard; "Distributed training", step()).
 *
 * master, m, v  device fp32, `n` elements each, updated in place.
 * mean_grad     device fp32, `n` elements (dp_reduce_scatter_mean output).
 * clip_scale    device fp32 scalar (dp_grad_sqnorm output) or NULL for 1.
 * args          host, the step's scalars.
 * bf16_out      device uint16, `n` elements of RNE_bf16(new master), or NULL.
 *
 * Per element: g = mean*scale; m = b1*m + (1-b1)*g; v = b2*v + (1-b2)*(g*g);
 * master -= lr*((m/bc1) / (sqrt(v/bc2) + eps) + wd*master).
 */
int zero1_adamw_step(float* master, float* m, float* v, const float* mean_grad, int64_t n,
                     const float* clip_scale, const grz_adamw_args* args, uint16_t* bf16_out,
                     hipStream_t stream);

/*
 * zero1_adamw_step with the all-gather fused into its epilogue: the new bf16
 * weights of the shard of chunk `chunk` go straight to their arena offsets in
 * every replica (no shard-compact bf16 round trip).  The shard geometry is
 * (buckets, nbuckets, nranks, chunk, flags) as in dp_reduce_scatter_mean;
 * chunk -1 means the whole plan in arena indexing (plain data parallelism:
 * master, m, v and mean_grad are then indexed like the arena).
 *
 * mean_grad  device; fp32 values, or with GRZ_MEAN_BF16 the bf16 patterns
 *            the reduce wrote with that flag (each widened exactly to fp32
 *            before the clip factor multiplies it).
 * replicas   host array of `nreplicas` (0..GRZ_MAX_RANKS) device uint16
 *            arenas.
 * flags      GRZ_UNEVEN; GRZ_MEAN_BF16; GRZ_ARGS_DEVICE: `args` points to
 *            device memory and is read by the kernel when it runs, so that a
 *            captured step (HIP graph) can be replayed with each step's
 *            scalars ("Distributed training", "Overlap and graphs": one graph
 *            per GPU, replayed).
 */
int zero1_adamw_gather(float* master, float* m, float* v, const void* mean_grad,
                       const grz_bucket* buckets, int nbuckets, int nranks, int chunk,
                       int flags, const float* clip_scale, const grz_adamw_args* args,
                       uint16_t* const* replicas, int nreplicas, hipStream_t stream);

/*
 * Enqueue: *current = table[min(*counter, count - 1)]; *counter += 1.  All
 * three are device pointers; `table` holds the per-step scalars of steps
 * 1..count (row t-1 for step t) and `*counter` the next row.  Placed in front
 * of a zero1_adamw_gather(..., GRZ_ARGS_DEVICE, current, ...) inside a
 * captured step, it advances the step scalars on every replay.
 */
int grz_step_args_next(const grz_adamw_args* table, int64_t count, int64_t* counter,
                       grz_adamw_args* current, hipStream_t stream);

/*
 * All-gather of bf16 shards ("Lab 09", s.1, all-gather rows of the N = 3
 * table; "A4", "Part 4", ncclAllGather after the update).
 *
 * shards     host array of N entries: shards[r] is rank r's shard-compact
 *            bf16 shard (chunk (r + 1) mod N of every bucket) on the device,
 *            or NULL for a rank whose shard is already in place.
 * replicas   host array of `nreplicas` device uint16 arenas; every non-NULL
 *            shard is copied into each of them at its arena offsets.
 */
int zero1_all_gather(const uint16_t* const* shards, int nranks, const grz_bucket* buckets,
                     int nbuckets, int flags, uint16_t* const* replicas, int nreplicas,
                     hipStream_t stream);

/*
 * zero1_all_gather for shards of any element type: GRZ_BF16 (2 bytes),
 * GRZ_F32 (4) or GRZ_F64 (8).  With fp32 shards it is the all-gather half of
 * a plain all-reduce of the mean ("Lab 09", s.1: an all-reduce is a
 * reduce-scatter followed by an all-gather; "A4", "Part 3", ncclAllReduce):
 * rank r's mean of chunk (r + 1) mod N, from dp_reduce_scatter_mean, lands at
 * its arena offsets in every replica.  The copy is of bytes: the values
 * arrive unchanged.  shards[r] is shard-compact (dp_shard_numel elements) or
 * NULL; replicas are arenas of `dtype` elements.  Errors as zero1_all_gather,
 * plus GRZ_EINVAL for another dtype and GRZ_EALIGN for a pointer not aligned
 * to its element.
 */
int dp_all_gather(const void* const* shards, int nranks, int dtype, const grz_bucket* buckets,
                  int nbuckets, int flags, void* const* replicas, int nreplicas,
                  hipStream_t stream);

/* Bytes of workspace zero1_fused_step needs for a plan of `npieces` pieces. */
size_t zero1_fused_workspace(int64_t npieces);

/*
 * Pieces (GRZ_PIECE-element tiles of the reduced chunks) that one
 * zero1_fused_step launch can hold for N ranks of `dtype` gradients on the
 * current device: 4 per workgroup that can be resident at once, less one
 * workgroup that folds the norm (1024 resident on a 256-CU MI355X, so 4092
 * pieces, 16.76 M elements).  A plan of more than 4096 pieces in all (the
 * peers' included) takes one more folding workgroup per 4096 pieces, so 4
 * pieces less each.  A negative value is minus a GRZ_E* code.
 */
int64_t zero1_fused_capacity(int nranks, int dtype);

/*
 * The whole step of one shard in one launch: reduce-scatter-mean, global
 * norm, clip, AdamW and the bf16 write ("A4", "Part 4": reduce, update the
 * shard, all-gather; "Distributed training", "Four strategies, one
 * interface": clip_grads_device then step), for a shard small enough that
 * its mean stays in registers.  Every result is bit-identical to
 *   dp_reduce_scatter_mean -> dp_grad_sqnorm -> zero1_adamw_gather
 * on the same inputs; the mean itself is never stored unless `mean_out` is
 * given, which saves 8 bytes of memory traffic per owned element.  The grid
 * synchronises internally (all pieces summed before the norm is read: each
 * piece sum is published in a workspace slot that carries the launch's
 * parity, and the readers poll it), so its workgroups must be resident at
 * once.  The grid is sized to what the occupancy allows resident, so on a
 * device that runs nothing else at the same time they are; with
 * GRZ_COOPERATIVE the launch is cooperative and HIP guarantees it (or
 * refuses the launch), at about 17 us more per call on MI355X.  Without it,
 * kernels of other streams that hold compute units for longer than the
 * poll limit make the waits give up (see `workspace`): the call then
 * reports it and no tile holds anything but its old state or its update.
 *
 * rank_grads, nranks, dtype, buckets, nbuckets, chunk
 *            as for dp_reduce_scatter_mean; dtype GRZ_BF16 or GRZ_F32.
 *            chunk >= 0: one rank's ZeRO-1 shard (master/m/v and mean_out
 *            shard-compact); chunk = -1: every chunk (plain data parallelism,
 *            master/m/v indexed like the arena).
 * flags      GRZ_UNEVEN, GRZ_IN_COMPACT (as for the reduce), GRZ_ARGS_DEVICE
 *            (as for zero1_adamw_gather), GRZ_COOPERATIVE (above).
 *            GRZ_BF16_WIRE, GRZ_SUM, GRZ_IN_TILED and GRZ_MEAN_BF16 are not
 *            taken (GRZ_EINVAL): use the separate entry points.
 * master, m, v  device fp32 state, updated in place.
 * args       the step's scalars (host, or device with GRZ_ARGS_DEVICE).
 * max_norm   clip threshold (<= 0: no clipping).
 * replicas   host array of `nreplicas` device bf16 arenas (0..16); each gets
 *            the new weights of the processed chunks at their arena offsets.
 * piece_sqnorm device fp64, dp_piece_count entries.  The kernel writes the
 *            pieces of the processed chunks; the other entries (the peers'
 *            pieces, when chunk >= 0) must hold their values already.
 * workspace  device, zero1_fused_workspace(npieces) bytes, 8-byte aligned,
 *            ZEROED before its first use.  Its first 256 bytes are control
 *            words: the 32-bit word at byte 8 is the time-out flag, the word
 *            at byte 12 the number of polls a wait makes before it gives up
 *            (0, as zeroed: 2^22, a few seconds; the caller may set it
 *            before the launch), the words at bytes 16 and 20 a launch
 *            counter and the piece count of the last launch.  The rest holds
 *            the published piece sums.  A completed call leaves the workspace
 *            ready for the next call of a plan with the same piece count; a
 *            call with another piece count raises the flag and writes
 *            nothing.  A non-zero flag means a wait gave up (or the piece
 *            count changed): a workgroup whose wait gave up writes nothing
 *            after it (its tiles of master, m, v, the replicas and the mean
 *            keep their previous values, and it stores no norm), so each tile
 *            holds either its previous state or its correct update; the
 *            call's result as a whole is then incomplete, and while the flag
 *            is up every further call on the workspace returns at once
 *            without writing anything.  Zero the workspace (the poll limit
 *            word may be kept) before the next call.  Calls that share a
 *            workspace must not overlap.  The peers' entries of piece_sqnorm
 *            are sums of squares: non-negative (a NaN is carried as NaN).
 * sqnorm_out, clip_scale_out  device scalars as for dp_grad_sqnorm, or NULL.
 * mean_out   device fp32 copy of the mean (as dp_reduce_scatter_mean writes
 *            it), or NULL.
 * Errors: as dp_reduce_scatter_mean and zero1_adamw_gather; GRZ_ERANGE when
 * the plan has more pieces than zero1_fused_capacity (less its folding
 * workgroups), more than 32 (bucket, chunk) segments, or more than 2^20
 * pieces in all; GRZ_EHIP when the launch fails (with GRZ_COOPERATIVE, also
 * when the device cannot launch cooperatively).
 */
int zero1_fused_step(const void* const* rank_grads, int nranks, int dtype,
                     const grz_bucket* buckets, int nbuckets, int chunk, int flags,
                     float* master, float* m, float* v, const grz_adamw_args* args,
                     double max_norm, uint16_t* const* replicas, int nreplicas,
                     double* piece_sqnorm, void* workspace, double* sqnorm_out,
                     float* clip_scale_out, float* mean_out, hipStream_t stream);

/*
 * zero1_fused_step whose step scalars come from a table and advance in the
 * same launch, for a captured step replayed once per step ("Distributed
 * training", "Overlap and graphs": one graph per GPU, replayed): the launch
 * uses row min(*counter, count - 1) of `table` (rows as for
 * grz_step_args_next), copies it to *current and adds one to *counter, as
 * grz_step_args_next followed by zero1_fused_step with GRZ_ARGS_DEVICE would,
 * without the extra launch.  table, counter and current are device pointers;
 * GRZ_ARGS_DEVICE is implied (passing it: GRZ_EINVAL).  A call refused at its
 * start (the workspace's flag up, or another piece count; see
 * zero1_fused_step) leaves the counter as it was; after a wait gave up it
 * may have advanced (workgroup 0 advances it once it has the norm).
 * Everything else is zero1_fused_step.
 */
int zero1_fused_step_args(const void* const* rank_grads, int nranks, int dtype,
                          const grz_bucket* buckets, int nbuckets, int chunk, int flags,
                          float* master, float* m, float* v, const grz_adamw_args* table,
                          int64_t count, int64_t* counter, grz_adamw_args* current,
                          double max_norm, uint16_t* const* replicas, int nreplicas,
                          double* piece_sqnorm, void* workspace, double* sqnorm_out,
                          float* clip_scale_out, float* mean_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GRZ_H */
