/*
 * Host-side checks of libgrz, built and run by tests/test_native_host.py,
 * once against the regular library and once against a build whose host code
 * carries AddressSanitizer.  Only host logic runs: plan helpers on
 * pseudo-random plans, and argument errors that every entry point must
 * report before it enqueues anything (no call here reaches a kernel launch;
 * the pointers passed are never dereferenced).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "grz.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {  /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}
static int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1)); }

static int failures = 0;
#define CHECK(cond, ...)                              \
  do {                                                \
    if (!(cond)) {                                    \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                   \
      fprintf(stderr, "\n");                          \
      if (++failures > 20) exit(1);                   \
    }                                                 \
  } while (0)

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static void random_plans(int rounds) {
  grz_bucket b[16];
  for (int it = 0; it < rounds; ++it) {
    const int n = (int)pick(1, GRZ_MAX_RANKS);
    const int nb = (int)pick(0, 12);
    int64_t pos = 0, lens[16];
    for (int i = 0; i < nb; ++i) {
      int64_t len = pick(0, 3) == 0 ? pick(0, 70) : pick(0, 200000);
      if (pick(0, 1)) len -= len % n; /* half the buckets divide evenly */
      lens[i] = len;
    }
    for (int i = nb - 1; i >= 0; --i) { /* reverse layer order: the last bucket is first in the arena */
      b[i].offset = pos;
      b[i].length = lens[i];
      pos += lens[i];
    }
    int divisible = 1;
    for (int i = 0; i < nb; ++i) divisible &= (lens[i] % n == 0);
    int64_t pieces = 0, shard_total = 0;
    for (int i = 0; i < nb; ++i) {
      int64_t expect_off = 0;
      for (int c = 0; c < n; ++c) {
        int64_t off = -1, cnt = -1;
        CHECK(dp_chunk_range(lens[i], n, c, &off, &cnt) == GRZ_OK, "chunk_range");
        CHECK(off == expect_off, "chunks tile the bucket");
        CHECK(cnt == lens[i] / n || cnt == lens[i] / n + 1, "array_split sizes");
        CHECK(dp_piece_offset(b, nb, n, 0, i, c) == pieces, "piece offset %d %d", i, c);
        expect_off += cnt;
        pieces += ceil_div(cnt, GRZ_PIECE);
      }
      CHECK(expect_off == lens[i], "chunks cover the bucket");
    }
    CHECK(dp_piece_count(b, nb, n, 0) == pieces, "piece count");
    int64_t tiled_pieces = 0;
    for (int c = 0; c < n; ++c) {
      const int64_t s = dp_shard_numel(b, nb, n, c, 0);
      const int64_t su = dp_shard_numel(b, nb, n, c, GRZ_UNEVEN);
      /* the tiled receive buffer: one N-piece slot per piece of the chunk */
      const int64_t tu = dp_tiled_numel(b, nb, n, c, GRZ_UNEVEN);
      CHECK(tu >= 0 && tu % ((int64_t)n * GRZ_PIECE) == 0, "tiled receive size");
      CHECK(tu / n >= su, "a slot holds every value of its piece");
      tiled_pieces += tu / ((int64_t)n * GRZ_PIECE);
      if (divisible) CHECK(s == su, "shard size");
      else CHECK(s == -GRZ_EINDIVISIBLE, "indivisible shard must fail");
      shard_total += su;
      CHECK(dp_ring_chunk_owner(dp_ring_owned_chunk(c, n), n) == c, "owner of owned chunk");
    }
    CHECK(shard_total == pos, "shards partition the arena");
    CHECK(tiled_pieces == pieces, "the chunks' tiled slots are the plan's pieces");
    CHECK(dp_piece_offset(b, nb, n, 0, nb, 0) < 0, "bucket out of range");
    CHECK(dp_piece_count(b, nb, GRZ_MAX_RANKS + 1, 0) < 0, "too many ranks");
  }
}

static void argument_errors(void) {
  const grz_bucket ok[1] = {{0, 1024}};
  const grz_bucket odd[1] = {{0, 1023}};
  const grz_bucket neg[1] = {{-8, 64}};
  void* fake[2] = {(void*)0x100000, (void*)0x200000};
  void* odd_ptr[2] = {(void*)0x100001, (void*)0x200000};
  void* out = (void*)0x300000;
  const void* const* r = (const void* const*)fake;
  CHECK(dp_reduce_scatter_mean(r, 0, GRZ_F32, ok, 1, 0, 0, out, NULL, NULL) == GRZ_EINVAL, "N=0");
  CHECK(dp_reduce_scatter_mean(r, 17, GRZ_F32, ok, 1, 0, 0, out, NULL, NULL) == GRZ_EINVAL, "N=17");
  CHECK(dp_reduce_scatter_mean(r, 2, 9, ok, 1, 0, 0, out, NULL, NULL) == GRZ_EINVAL, "dtype");
  CHECK(dp_reduce_scatter_mean(r, 2, GRZ_F32, ok, 1, 2, 0, out, NULL, NULL) == GRZ_EINVAL, "chunk");
  CHECK(dp_reduce_scatter_mean(r, 2, GRZ_F32, ok, 1, -2, 0, out, NULL, NULL) == GRZ_EINVAL, "chunk");
  CHECK(dp_reduce_scatter_mean(r, 2, GRZ_F32, ok, 1, 0, 1 << 9, out, NULL, NULL) == GRZ_EINVAL, "flag");
  CHECK(dp_reduce_scatter_mean(r, 2, GRZ_F32, odd, 1, 0, 0, out, NULL, NULL) == GRZ_EINDIVISIBLE,
        "indivisible");
  CHECK(dp_reduce_scatter_mean(r, 2, GRZ_F32, neg, 1, 0, 0, out, NULL, NULL) == GRZ_ERANGE, "range");
  CHECK(dp_reduce_scatter_mean(r, 2, GRZ_F32, ok, 1, 0, 0, NULL, NULL, NULL) == GRZ_EINVAL, "null out");
  CHECK(dp_reduce_scatter_mean(NULL, 2, GRZ_F32, ok, 1, 0, 0, out, NULL, NULL) == GRZ_EINVAL, "null in");
  CHECK(dp_reduce_scatter_mean((const void* const*)odd_ptr, 2, GRZ_F32, ok, 1, 0, 0, out, NULL,
                               NULL) == GRZ_EALIGN, "alignment");
  CHECK(dp_reduce_scatter_mean(r, 2, GRZ_F32, ok, 1, 0, 0, out, (double*)0x400004, NULL) ==
        GRZ_EALIGN, "piece alignment");
  CHECK(dp_reduce_scatter_mean(r, 2, GRZ_F32, ok, 1, 0, GRZ_BF16_WIRE, out, NULL, NULL) ==
        GRZ_EINVAL, "wire on fp32");
  CHECK(dp_reduce_scatter_mean(r, 2, GRZ_F32, ok, 1, 0, GRZ_IN_RANGE | GRZ_IN_COMPACT, out, NULL,
                               NULL) == GRZ_EINVAL, "range + compact");
  CHECK(dp_reduce_scatter_mean_range(r, 2, GRZ_F32, ok, 1, 1, 1, 0, 0, out, NULL, NULL) ==
        GRZ_EINVAL, "range past the plan");
  const int64_t counts[2] = {3, 4}, zero[2] = {0, 0}, big[2] = {1 << 24, 1};
  CHECK(dp_reduce_scatter_weighted(r, NULL, 2, GRZ_F32, ok, 1, 0, 1, 0, 0, out, NULL, NULL) ==
        GRZ_EINVAL, "no counts");
  CHECK(dp_reduce_scatter_weighted(r, zero, 2, GRZ_F32, ok, 1, 0, 1, 0, 0, out, NULL, NULL) ==
        GRZ_EINVAL, "zero tokens");
  CHECK(dp_reduce_scatter_weighted(r, big, 2, GRZ_F32, ok, 1, 0, 1, 0, 0, out, NULL, NULL) ==
        GRZ_ERANGE, "too many tokens");
  CHECK(dp_reduce_scatter_weighted(r, counts, 2, GRZ_F32, ok, 1, 0, 1, 0, GRZ_SUM, out, NULL,
                                   NULL) == GRZ_EINVAL, "sum with weights");
  double* ws = (double*)0x500000;
  CHECK(dp_grad_sqnorm(NULL, 5, 1.0, ws, (double*)0x600000, NULL, NULL) == GRZ_EINVAL, "null pieces");
  CHECK(dp_grad_sqnorm((double*)0x700000, -1, 1.0, ws, (double*)0x600000, NULL, NULL) ==
        GRZ_EINVAL, "negative count");
  CHECK(dp_grad_sqnorm((double*)0x700000, 5000, 1.0, NULL, (double*)0x600000, NULL, NULL) ==
        GRZ_EINVAL, "missing workspace");
  CHECK(dp_grad_sqnorm((double*)0x700000, 5, 1.0, NULL, NULL, NULL, NULL) == GRZ_EINVAL, "no outputs");
  CHECK(dp_grad_sqnorm((double*)0x700004, 5, 1.0, NULL, (double*)0x600000, NULL, NULL) ==
        GRZ_EALIGN, "piece alignment");
  grz_adamw_args args = {1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 0.1f, 0.05f};
  float* f = (float*)0x800000;
  CHECK(zero1_adamw_step(NULL, f, f, f, 16, NULL, &args, NULL, NULL) == GRZ_EINVAL, "null master");
  CHECK(zero1_adamw_step(f, f, f, f, -1, NULL, &args, NULL, NULL) == GRZ_EINVAL, "negative n");
  CHECK(zero1_adamw_step(f, f, f, f, 16, NULL, NULL, NULL, NULL) == GRZ_EINVAL, "null args");
  CHECK(zero1_adamw_step((float*)0x800002, f, f, f, 16, NULL, &args, NULL, NULL) == GRZ_EALIGN,
        "misaligned master");
  uint16_t* reps[1] = {(uint16_t*)0x900000};
  CHECK(zero1_adamw_gather(f, f, f, f, odd, 1, 2, 0, 0, NULL, &args, reps, 1, NULL) ==
        GRZ_EINDIVISIBLE, "indivisible gather");
  CHECK(zero1_adamw_gather(f, f, f, f, ok, 1, 2, 0, GRZ_SUM, NULL, &args, reps, 1, NULL) ==
        GRZ_EINVAL, "sum flag on the optimizer");
  CHECK(zero1_adamw_gather(f, f, f, f, ok, 1, 2, 0, 0, NULL, &args, reps, GRZ_MAX_RANKS + 1,
                           NULL) == GRZ_EINVAL, "too many replicas");
  const uint16_t* shards[2] = {(uint16_t*)0xA00000, (uint16_t*)0xB00000};
  CHECK(zero1_all_gather(NULL, 2, ok, 1, 0, reps, 1, NULL) == GRZ_EINVAL, "null shards");
  CHECK(zero1_all_gather(shards, 2, odd, 1, 0, reps, 1, NULL) == GRZ_EINDIVISIBLE, "indivisible");
  CHECK(zero1_all_gather(shards, 2, ok, 1, GRZ_SUM, reps, 1, NULL) == GRZ_EINVAL, "flag");
  CHECK(zero1_all_gather(shards, 0, ok, 1, 0, reps, 1, NULL) == GRZ_EINVAL, "N=0");
  const void* vshards[2] = {(void*)0xA00000, (void*)0xB00000};
  void* vreps[1] = {(void*)0x900000};
  void* vodd[1] = {(void*)0x900002};
  CHECK(dp_all_gather(vshards, 2, 7, ok, 1, 0, vreps, 1, NULL) == GRZ_EINVAL, "gather dtype");
  CHECK(dp_all_gather(vshards, 2, GRZ_F32, odd, 1, 0, vreps, 1, NULL) == GRZ_EINDIVISIBLE,
        "indivisible fp32 gather");
  CHECK(dp_all_gather(vshards, 2, GRZ_F32, ok, 1, 0, vodd, 1, NULL) == GRZ_EALIGN,
        "fp32 replica off its alignment");
  CHECK(zero1_adamw_gather(f, f, f, f, ok, 1, 2, 0, GRZ_OUT_GLOBAL, NULL, &args, reps, 1,
                           NULL) == GRZ_EINVAL, "reduce-only flag on the optimizer");
  CHECK(grz_set_max_blocks(0) == GRZ_EINVAL, "blocks");
  /* The norm straight from an fp32 array. */
  CHECK(dp_grad_sqnorm_of_workspace(0) == 0, "empty workspace");
  CHECK(dp_grad_sqnorm_of_workspace(4097) == 2 * sizeof(double), "two pieces");
  CHECK(dp_grad_sqnorm_of(NULL, 8, 1.0, ws, (double*)0x600000, NULL, NULL) == GRZ_EINVAL,
        "null gradient");
  CHECK(dp_grad_sqnorm_of(f, 8, 1.0, NULL, (double*)0x600000, NULL, NULL) == GRZ_EINVAL,
        "null workspace");
  CHECK(dp_grad_sqnorm_of(f, -1, 1.0, ws, (double*)0x600000, NULL, NULL) == GRZ_EINVAL,
        "negative count");
  CHECK(dp_grad_sqnorm_of(f, 8, 1.0, ws, NULL, NULL, NULL) == GRZ_EINVAL, "no outputs");
  CHECK(dp_grad_sqnorm_of((float*)0x800002, 8, 1.0, ws, (double*)0x600000, NULL, NULL) ==
        GRZ_EALIGN, "misaligned gradient");
  /* The one-launch step refuses before it looks for a device. */
  double* parts = (double*)0xC00000;
  void* fws = (void*)0xD00000;
  CHECK(zero1_fused_step(r, 2, GRZ_BF16, ok, 1, 0, GRZ_SUM, f, f, f, &args, 1.0, reps, 1, parts,
                         fws, NULL, NULL, NULL, NULL) == GRZ_EINVAL, "sum mode");
  CHECK(zero1_fused_step(r, 2, GRZ_BF16, ok, 1, 0, GRZ_BF16_WIRE, f, f, f, &args, 1.0, reps, 1,
                         parts, fws, NULL, NULL, NULL, NULL) == GRZ_EINVAL, "wire mode");
  CHECK(zero1_fused_step(r, 2, GRZ_F64, ok, 1, 0, 0, f, f, f, &args, 1.0, reps, 1, parts, fws,
                         NULL, NULL, NULL, NULL) == GRZ_EINVAL, "fp64 gradients");
  CHECK(zero1_fused_step(r, 2, GRZ_BF16, odd, 1, 0, 0, f, f, f, &args, 1.0, reps, 1, parts, fws,
                         NULL, NULL, NULL, NULL) == GRZ_EINDIVISIBLE, "indivisible");
  CHECK(zero1_fused_step(r, 2, GRZ_BF16, ok, 1, -1, GRZ_IN_COMPACT, f, f, f, &args, 1.0, reps, 1,
                         parts, fws, NULL, NULL, NULL, NULL) == GRZ_EINVAL, "compact without chunk");
  CHECK(zero1_fused_step(r, 2, GRZ_BF16, ok, 1, 0, 0, f, f, f, &args, 1.0, reps, 1, NULL, fws,
                         NULL, NULL, NULL, NULL) == GRZ_EINVAL, "no pieces");
  CHECK(zero1_fused_step(r, 2, GRZ_BF16, ok, 1, 0, 0, f, f, f, &args, 1.0, reps, 1, parts, NULL,
                         NULL, NULL, NULL, NULL) == GRZ_EINVAL, "no workspace");
  CHECK(zero1_fused_step(r, 2, GRZ_BF16, ok, 1, 0, 0, (float*)0x800002, f, f, &args, 1.0, reps, 1,
                         parts, fws, NULL, NULL, NULL, NULL) == GRZ_EALIGN, "misaligned master");
  CHECK(zero1_fused_workspace(4097) > zero1_fused_workspace(4096), "level sums");
  CHECK(zero1_fused_capacity(0, GRZ_BF16) == -GRZ_EINVAL, "capacity N=0");
  /* Signatures that differ from a bare "void" helper or a workspace-free
   * norm: dp_chunk_range reports bad arguments, dp_grad_sqnorm takes a
   * workspace sized by dp_grad_sqnorm_workspace, and its no-allocation form
   * refuses a tree beyond its static scratch before touching a device. */
  int64_t o = 0, c = 0;
  CHECK(dp_chunk_range(64, 3, 3, &o, &c) == GRZ_EINVAL, "chunk index N");
  CHECK(dp_chunk_range(-1, 3, 0, &o, &c) == GRZ_EINVAL, "negative length");
  CHECK(dp_chunk_range(64, 3, 0, NULL, &c) == GRZ_EINVAL, "null offset");
  CHECK(dp_grad_sqnorm_workspace(4096) == 0, "one block needs no workspace");
  CHECK(dp_grad_sqnorm_workspace(4097) == 2 * sizeof(double), "two level sums");
  CHECK(dp_grad_sqnorm_workspace((int64_t)8190 * 4096) == GRZ_NOALLOC_SCRATCH_BYTES,
        "largest tree the static scratch holds");
  CHECK(dp_grad_sqnorm_noalloc((double*)0x700000, (int64_t)8190 * 4096 + 1, 1.0,
                               (double*)0x600000, NULL, NULL) == GRZ_ERANGE, "noalloc range");
  CHECK(dp_grad_sqnorm_noalloc((double*)0x700000, -1, 1.0, (double*)0x600000, NULL, NULL) ==
        GRZ_EINVAL, "noalloc count");
  CHECK(dp_grad_sqnorm_step_args((double*)0x700000, 5, 1.0, NULL, (double*)0x600000, NULL,
                                 NULL, 4, (int64_t*)0xC00000, (grz_adamw_args*)0xD00000,
                                 NULL) == GRZ_EINVAL, "step-args norm without a table");
  CHECK(dp_grad_sqnorm_step_args((double*)0x700000, 5, 1.0, NULL, (double*)0x600000, NULL,
                                 (grz_adamw_args*)0xD00000, 4, (int64_t*)0xC00004,
                                 (grz_adamw_args*)0xD00000, NULL) == GRZ_EALIGN,
        "step-args norm, counter off its alignment");
  int64_t* ctr = (int64_t*)0xC00000;
  grz_adamw_args* table = (grz_adamw_args*)0xD00000;
  CHECK(grz_step_args_next(NULL, 4, ctr, table, NULL) == GRZ_EINVAL, "null table");
  CHECK(grz_step_args_next(table, 0, ctr, table, NULL) == GRZ_EINVAL, "empty table");
  CHECK(grz_step_args_next(table, 4, (int64_t*)0xC00004, table, NULL) == GRZ_EALIGN, "counter");
  CHECK(zero1_adamw_gather(f, f, f, f, ok, 1, 2, 0, GRZ_ARGS_DEVICE, NULL,
                           (const grz_adamw_args*)0xE00002, reps, 1, NULL) == GRZ_EALIGN,
        "device args alignment");
}

int main(void) {
  random_plans(3000);
  argument_errors();
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
