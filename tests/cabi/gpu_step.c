/*
 * The library from plain C on the GPU: one ZeRO-1 step of N simulated ranks
 * through include/grz.h, with device memory from hipMalloc -- no Python and
 * no torch.  Per rank r (chunk c = (r + 1) mod N): dp_reduce_scatter_mean,
 * then one dp_grad_sqnorm over every rank's pieces, then per rank
 * zero1_adamw_gather writing the new bf16 weights into all N replicas.
 *
 * usage: gpu_step <input file> <output file>
 *
 * Input (little-endian): int32 N, int32 nbuckets, int64 P; nbuckets x
 * (int64 offset, int64 length); grz_adamw_args (7 float32); float64 max_norm;
 * N x P uint16 gradient arenas (bf16 bits); then per rank r: int64 shard
 * length and that many float32 master values (shard-compact, chunk
 * (r + 1) mod N).
 * Output: float64 sqnorm, float32 clip factor, int32 1 if all N replicas are
 * byte-equal; per rank: mean, master, m, v (shard length float32 each); then
 * replica 0 (P uint16).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "grz.h"

#define MAXR GRZ_MAX_RANKS

static void die(const char* what, const char* why) {
  fprintf(stderr, "gpu_step: %s: %s\n", what, why);
  exit(1);
}

static void hip(hipError_t e, const char* what) {
  if (e != hipSuccess) die(what, hipGetErrorString(e));
}

static void grz(int st, const char* what) {
  if (st != GRZ_OK) die(what, grz_strerror(st));
}

static void rd(void* p, size_t size, size_t n, FILE* f) {
  if (fread(p, size, n, f) != n) die("input", "short read");
}

static void wr(const void* p, size_t size, size_t n, FILE* f) {
  if (fwrite(p, size, n, f) != n) die("output", "short write");
}

static void* dalloc(size_t bytes) {
  void* p = NULL;
  hip(hipMalloc(&p, bytes ? bytes : 16), "hipMalloc");
  return p;
}

int main(int argc, char** argv) {
  if (argc != 3) die("usage", "gpu_step <input> <output>");
  FILE* in = fopen(argv[1], "rb");
  if (!in) die("input", "cannot open");
  int32_t n = 0, nb = 0;
  int64_t p = 0;
  rd(&n, 4, 1, in);
  rd(&nb, 4, 1, in);
  rd(&p, 8, 1, in);
  if (n < 1 || n > MAXR || nb < 1 || nb > 64 || p < 1) die("input", "bad sizes");
  grz_bucket* buckets = malloc(sizeof(grz_bucket) * (size_t)nb);
  for (int b = 0; b < nb; ++b) {
    rd(&buckets[b].offset, 8, 1, in);
    rd(&buckets[b].length, 8, 1, in);
  }
  grz_adamw_args args;
  double max_norm;
  rd(&args, sizeof(float), 7, in);
  rd(&max_norm, 8, 1, in);

  uint16_t* host_g = malloc((size_t)p * 2);
  const void* grads[MAXR];
  for (int r = 0; r < n; ++r) {
    rd(host_g, 2, (size_t)p, in);
    void* d = dalloc((size_t)p * 2);
    hip(hipMemcpy(d, host_g, (size_t)p * 2, hipMemcpyHostToDevice), "upload gradient");
    grads[r] = d;
  }
  int64_t shard[MAXR];
  float *w[MAXR], *m[MAXR], *v[MAXR], *mean[MAXR];
  for (int r = 0; r < n; ++r) {
    rd(&shard[r], 8, 1, in);
    const int c = dp_ring_owned_chunk(r, n);
    if (shard[r] != dp_shard_numel(buckets, nb, n, c, 0)) die("input", "shard length");
    const size_t bytes = (size_t)shard[r] * 4;
    float* hw = malloc(bytes ? bytes : 4);
    rd(hw, 4, (size_t)shard[r], in);
    w[r] = dalloc(bytes);
    m[r] = dalloc(bytes);
    v[r] = dalloc(bytes);
    mean[r] = dalloc(bytes);
    hip(hipMemcpy(w[r], hw, bytes, hipMemcpyHostToDevice), "upload master");
    hip(hipMemset(m[r], 0, bytes), "clear m");
    hip(hipMemset(v[r], 0, bytes), "clear v");
    free(hw);
  }
  fclose(in);

  const int64_t npieces = dp_piece_count(buckets, nb, n, 0);
  if (npieces < 0) grz((int)-npieces, "dp_piece_count");
  double* partials = dalloc((size_t)npieces * 8);
  void* ws = dalloc(dp_grad_sqnorm_workspace(npieces));
  double* sqnorm = dalloc(8);
  float* scale = dalloc(4);
  uint16_t* reps[MAXR];
  for (int r = 0; r < n; ++r) {
    reps[r] = dalloc((size_t)p * 2);
    hip(hipMemset(reps[r], 0, (size_t)p * 2), "clear replica");
  }

  for (int r = 0; r < n; ++r)
    grz(dp_reduce_scatter_mean(grads, n, GRZ_BF16, buckets, nb, dp_ring_owned_chunk(r, n), 0,
                               mean[r], partials, 0),
        "dp_reduce_scatter_mean");
  grz(dp_grad_sqnorm(partials, npieces, max_norm, ws, sqnorm, scale, 0), "dp_grad_sqnorm");
  for (int r = 0; r < n; ++r)
    grz(zero1_adamw_gather(w[r], m[r], v[r], mean[r], buckets, nb, n, dp_ring_owned_chunk(r, n),
                           0, scale, &args, reps, n, 0),
        "zero1_adamw_gather");
  hip(hipDeviceSynchronize(), "synchronize");

  FILE* out = fopen(argv[2], "wb");
  if (!out) die("output", "cannot open");
  double hs;
  float hc;
  hip(hipMemcpy(&hs, sqnorm, 8, hipMemcpyDeviceToHost), "sqnorm");
  hip(hipMemcpy(&hc, scale, 4, hipMemcpyDeviceToHost), "scale");
  wr(&hs, 8, 1, out);
  wr(&hc, 4, 1, out);
  uint16_t* r0 = malloc((size_t)p * 2);
  uint16_t* rk = malloc((size_t)p * 2);
  hip(hipMemcpy(r0, reps[0], (size_t)p * 2, hipMemcpyDeviceToHost), "replica 0");
  int32_t same = 1;
  for (int r = 1; r < n; ++r) {
    hip(hipMemcpy(rk, reps[r], (size_t)p * 2, hipMemcpyDeviceToHost), "replica");
    if (memcmp(r0, rk, (size_t)p * 2) != 0) same = 0;
  }
  wr(&same, 4, 1, out);
  for (int r = 0; r < n; ++r) {
    const size_t bytes = (size_t)shard[r] * 4;
    float* h = malloc(bytes ? bytes : 4);
    float* src[4] = {mean[r], w[r], m[r], v[r]};
    for (int k = 0; k < 4; ++k) {
      hip(hipMemcpy(h, src[k], bytes, hipMemcpyDeviceToHost), "state");
      wr(h, 4, (size_t)shard[r], out);
    }
    free(h);
  }
  wr(r0, 2, (size_t)p, out);
  fclose(out);
  printf("gpu_step: %d ranks, %lld parameters, sqnorm %.9e, clip factor %.9g\n", n,
         (long long)p, hs, (double)hc);
  return 0;
}
