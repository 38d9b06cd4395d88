// grz.hip -- HIP kernels and C ABI of the data-parallel / ZeRO-1 gradient
// pipeline for AMD Instinct MI355X (gfx950, CDNA4, wave64).
//
// Kernels (all HBM-bandwidth bound; nothing here is a contraction, so no MFMA;
// one workgroup per tile -- 256 threads for the reduce, one wave for the
// optimizer and the copy -- lane-contiguous 8/16-byte accesses, non-temporal
// hints, workgroup and tile sizes and occupancy caps chosen by measurement):
//   rs_mean_kernel   ring-order N-way fold of 64/128-bit loads (from N
//                    buffers, or one tiled receive buffer that holds each
//                    piece's N contributions side by side), fp32 (fp64)
//                    mean, fp64 sum of squares per GRZ_PIECE-element piece
//   sqnorm_level_kernel / sqnorm_final_kernel
//                    fixed-shape fp64 tree over the piece sums -> norm, clip
//   piece_sqnorm_kernel
//                    the piece sums of an already reduced fp32 array
//   adamw_kernel     clip + AdamW on fp32 master/m/v, bf16 round-to-nearest-
//                    even written to any number of replica arenas
//   gather_kernel    shard copies into replica arenas (all-gather), in
//                    16-bit words: bf16 elements, or fp32 / fp64 ones as 2 / 4
//   fused_step_kernel
//                    the reduce, the norm and clip + AdamW of one shard in one
//                    cooperative launch, the mean held in registers
//
// The ring order of the fold and the chunk ownership follow "Lab 09 --
// Parallelism, simulated", s.1 "Ring all-reduce" (the N = 3 schedule table)
// and its "Tips" (reduce-scatter step t: rank r sends chunk (r - t) mod N, so
// chunk c's partial sum starts at rank c and ends at rank c - 1, its owner).
// The step order (reduce, clip, AdamW on the shard, all-gather) follows
// "A4 -- Multi-GPU with NCCL and ZeRO-1", "Part 4 -- Multi-GPU Backward and
// Update", and "Distributed training" (noeira), "Four strategies, one
// interface".
//
// Build flags this file relies on: -ffp-contract=off (every a*b+c rounds
// twice, as the fp32 reference does) and -fhip-fp32-correctly-rounded-divide-
// sqrt (IEEE division and square root).

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>
#include <vector>

#include "grz.h"

namespace {

constexpr int kThreads = 256;          // 4 waves of 64
constexpr int kMaxSegs = 64;           // segments per launch (kernel-argument budget)
constexpr int kReduceFan = 4096;       // values one block folds in the norm tree

static_assert(GRZ_PIECE % (kThreads * 8) == 0, "piece shape");

// Grid width cap of the grid-stride kernels, per calling host thread (so that
// callers on different threads never see each other's setting).  Measured on
// MI355X: one workgroup per tile (no cap in practice) streams fastest.
thread_local int g_max_blocks = 1 << 30;

// Polls of a wait of the fused step before it gives up, when the workspace
// does not set its own limit.  Each poll is a device-scope load (about a
// microsecond) and a short sleep, so this bounds a wait at a few seconds.
constexpr unsigned kDefaultSpinLimit = 1u << 22;

// One contiguous run of work: `len` elements read at `src` and written at
// `dst`, whose first tile is `tile0` of the launch and first norm piece is
// `piece0` of the plan.  `chunk` is the ring chunk (fold start) for the
// reduce kernel and the source shard for the gather kernel.  `vec` is 1 when
// every pointer + offset of the run is aligned for the kernel's vector
// accesses (8 or 16 bytes); otherwise the run goes element by element, in the
// same lane order.
struct Seg {
  int64_t src;
  int64_t dst;
  int64_t len;
  int64_t piece0;
  int64_t tile0;
  int32_t chunk;
  int32_t vec;
};

// The segment of a launch that holds `tile`: the last of the first nsegs
// whose tile0 <= tile.  tile0 does not decrease, so those segments are a
// prefix: count them, first by groups of 8, then inside the group, with all
// loads of a round issued before the first comparison (two dependent rounds
// of kernel-argument reads where a binary search over 64 takes six).
// Measured on MI355X at the 7B one-rank share, two runs alternating with the
// binary search: the optimizer 3.75-3.97 ms against 3.96-4.04 ms, the
// all-gather copy 3.51-3.55 against 3.58-3.62, the step 9.94-10.21 against
// 10.30-10.39; with 291 reverse-layer buckets the step 10.28-10.30 against
// 10.65-10.76 ms.
template <typename S, int M>
__device__ __forceinline__ int find_seg(const S (&seg)[M], int nsegs, int64_t tile) {
  static_assert(M % 8 == 0, "segment groups of 8");
  if (nsegs <= 1) return 0;
  int g = 0;
#pragma unroll
  for (int i = 1; i < M / 8; ++i) {
    const int64_t t0 = seg[i * 8].tile0;
    g += static_cast<int>(i * 8 < nsegs) & static_cast<int>(t0 <= tile);
  }
  int64_t t[7];
#pragma unroll
  for (int i = 1; i < 8; ++i) t[i - 1] = seg[g * 8 + i].tile0;
  int idx = g * 8;
#pragma unroll
  for (int i = 1; i < 8; ++i)
    idx += static_cast<int>(g * 8 + i < nsegs) & static_cast<int>(t[i - 1] <= tile);
  return idx;
}

// ---------------------------------------------------------------------------
// Element access.  bf16 values are uint16 bit patterns; widening puts them in
// the top half of a binary32, which is exact.

template <typename T> struct AccOf { using type = float; };
template <> struct AccOf<double> { using type = double; };

__device__ __forceinline__ float widen1(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
__device__ __forceinline__ float widen1(const float* p) { return *p; }
__device__ __forceinline__ double widen1(const double* p) { return *p; }

// Global accesses.  Every access instruction of a wave covers one contiguous
// run: lane l touches bytes [w*l, w*(l+1)) of it, w = 8 or 16.  (Measured on
// MI355X: non-temporal 16-byte stores that leave 16-byte holes between lanes,
// to be filled by a second instruction, stream at well under half the rate
// of contiguous ones.)  So a lane owns G consecutive fp32 (G = 4) or fp64
// (G = 2) values of an fp32/fp64 stream per access, and the matching G bf16
// values of a bf16 stream (8 bytes).
//
// Every stream is touched once per step and is far larger than the caches.
// Each kernel picks a cache policy for its loads and stores (bit 0:
// non-temporal loads, bit 1: non-temporal stores), chosen by measurement; it
// changes speed only, never a result bit.
#ifndef GRZ_RS_POLICY
#define GRZ_RS_POLICY 3
#endif
#ifndef GRZ_ADAM_POLICY
#define GRZ_ADAM_POLICY 3
#endif
#ifndef GRZ_AG_POLICY
#define GRZ_AG_POLICY 3
#endif
constexpr int kNtLoad = 1, kNtStore = 2;

// Full tiles of the reduce take a path that issues all K * N loads of the
// tile before the first addition (the per-access path waits for each
// access's N loads in turn).  Measured on MI355X at the 7B one-rank share:
// the reduce 2.60-2.75 ms against 2.73-2.82 ms.  The same for the optimizer
// (16 loads) and the all-gather copy (2 loads) measured slower, so they keep
// the per-access path.  Speed only, never a result bit.
#ifndef GRZ_RS_BATCH
#define GRZ_RS_BATCH 1
#endif

// Workgroup sizes and tiles (elements per workgroup) of the optimizer and
// the all-gather: one wave each, one 16-byte access per lane per stream.
// Measured on MI355X at the 7B one-rank share, three repetitions each: the
// optimizer with 64-thread workgroups and 256-element tiles at 3 waves per
// SIMD 3.92-3.95 ms, against 3.99-4.07 ms with 256 threads and 1024-element
// tiles (128 threads, 512 to 4096 elements and 2 to 8 waves measured in
// between or slower); the all-gather copy with 64 threads and 512-element
// tiles, uncapped, 3.57-3.62 ms, against 3.70-3.72 ms with 256 threads and
// 4096 elements at 5 waves (it needs 8 or more waves per SIMD at this tile:
// 4.13 ms at 5, 5.81 ms at 3).  Smaller workgroups finish and refill one by
// one, which keeps more of each CU's memory requests in flight.  Speed
// only, never a result bit.
#ifndef GRZ_ADAM_THREADS
#define GRZ_ADAM_THREADS 64
#endif
#ifndef GRZ_ADAM_TILE
#define GRZ_ADAM_TILE 256
#endif
#ifndef GRZ_AG_THREADS
#define GRZ_AG_THREADS 64
#endif
#ifndef GRZ_AG_TILE
#define GRZ_AG_TILE 512
#endif
static_assert(GRZ_ADAM_TILE % (GRZ_ADAM_THREADS * 4) == 0, "optimizer tile shape");
static_assert(GRZ_AG_TILE % (GRZ_AG_THREADS * 8) == 0, "all-gather tile shape");

// Occupancy caps, in waves per SIMD (0 = no cap).  Measured on MI355X: the
// reduce at 2 waves per SIMD for 5 to 16 input streams (7B one-rank share,
// N = 8: 2.75 ms against 2.90 ms uncapped; N = 16: 2.47 ms against 2.63 at 3
// and 3.81 at 6) and at 3 for up to four (N = 2: 4.37 ms against 5.16 at 2;
// a 134 M-element shard at N = 3: 5.8 TB/s against 4.95 at 2, at N = 4: 6.5
// against 6.1, and the 7B share at N = 4 the same either way); the
// optimizer at 3 waves (4.2 ms at 5 or more, 4.7 ms at 2, with the
// workgroups above); the all-gather copy of one 16-byte access per lane runs
// best uncapped.  Speed only, never a result bit.
//
// A small launch of the reduce runs better at 3 waves for every N: with few
// tiles per CU, more of them resident shortens the ramp and the tail.  At
// N = 8 (3 against 2 waves): GPT-2 124M one-rank share (3,802 tiles) 0.056
// against 0.062 ms; the 124M ranks' reduces of all 8 ranks 0.446 against
// 0.483 ms, the char GPT's 0.115 against 0.124 ms; one launch of 30,416
// tiles the same either way; the 1.5B share at N = 8 (47,534 tiles) 0.638
// against 0.618 ms and the 7B share (205,641 tiles) 2.85 against 2.79 ms.
// So launches of at most kRsSmallTiles tiles take the small-launch cap.
#ifndef GRZ_RS_WAVES
#define GRZ_RS_WAVES 2
#endif
#ifndef GRZ_RS_WAVES_FEW
#define GRZ_RS_WAVES_FEW 3
#endif
#ifndef GRZ_RS_WAVES_SMALL
#define GRZ_RS_WAVES_SMALL 3
#endif
static_assert(GRZ_RS_WAVES > 0 && GRZ_RS_WAVES_FEW > 0 && GRZ_RS_WAVES_SMALL > 0,
              "the reduce's caps are per N");
constexpr int64_t kRsSmallTiles = 16384;
// The reduce's cap for N ranks (every N from 1 to 16 has its own kernel),
// for a large launch or a small one.  Up to four ranks it is the same cap
// either way (so the same kernel).
template <int NR, bool SMALL> struct RsWaves {
  static constexpr int value = (NR >= 1 && NR <= 4) ? GRZ_RS_WAVES_FEW
                               : SMALL               ? GRZ_RS_WAVES_SMALL
                                                     : GRZ_RS_WAVES;
};
#ifndef GRZ_ADAM_WAVES
#define GRZ_ADAM_WAVES 3
#endif
#ifndef GRZ_AG_WAVES
#define GRZ_AG_WAVES 0
#endif
#if GRZ_AG_WAVES > 0
#define GRZ_AG_ATTR __attribute__((amdgpu_waves_per_eu(GRZ_AG_WAVES, GRZ_AG_WAVES)))
#else
#define GRZ_AG_ATTR
#endif
#if GRZ_ADAM_WAVES > 0
#define GRZ_ADAM_ATTR __attribute__((amdgpu_waves_per_eu(GRZ_ADAM_WAVES, GRZ_ADAM_WAVES)))
#else
#define GRZ_ADAM_ATTR
#endif

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int P, typename V>
__device__ __forceinline__ V ldv(const void* p) {
  if constexpr ((P & kNtLoad) != 0)
    return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else
    return *reinterpret_cast<const V*>(p);
}

template <int P, typename V>
__device__ __forceinline__ void stv(void* p, V v) {
  if constexpr ((P & kNtStore) != 0)
    __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
  else
    *reinterpret_cast<V*>(p) = v;
}

// Elements per lane per access for an accumulation type.
template <typename Acc> struct Geo {
  static constexpr int G = 16 / static_cast<int>(sizeof(Acc));
  static constexpr int K = GRZ_PIECE / (kThreads * G);  // accesses per lane per tile
};

template <int P>
__device__ __forceinline__ void loadg(const uint16_t* p, float (&x)[4]) {
  const u32x2 u = ldv<P, u32x2>(p);
  x[0] = __uint_as_float(u[0] << 16);
  x[1] = __uint_as_float(u[0] & 0xffff0000u);
  x[2] = __uint_as_float(u[1] << 16);
  x[3] = __uint_as_float(u[1] & 0xffff0000u);
}
template <int P>
__device__ __forceinline__ void loadg(const float* p, float (&x)[4]) {
  const u32x4 u = ldv<P, u32x4>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(u[i]);
}
template <int P>
__device__ __forceinline__ void loadg(const double* p, double (&x)[2]) {
  const u32x4 u = ldv<P, u32x4>(p);
  x[0] = __hiloint2double(static_cast<int>(u[1]), static_cast<int>(u[0]));
  x[1] = __hiloint2double(static_cast<int>(u[3]), static_cast<int>(u[2]));
}
template <int P>
__device__ __forceinline__ void storeg(float* p, const float (&x)[4]) {
  u32x4 u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = __float_as_uint(x[i]);
  stv<P>(p, u);
}
template <int P>
__device__ __forceinline__ void storeg(double* p, const double (&x)[2]) {
  u32x4 u;
  u[0] = static_cast<uint32_t>(__double2loint(x[0]));
  u[1] = static_cast<uint32_t>(__double2hiint(x[0]));
  u[2] = static_cast<uint32_t>(__double2loint(x[1]));
  u[3] = static_cast<uint32_t>(__double2hiint(x[1]));
  stv<P>(p, u);
}

// Round-to-nearest-even of a binary32 to bf16: add half an ulp of the kept
// part (minus one when the kept part is even, so that exact ties go to the
// even neighbour) and drop the low half.  NaN keeps its sign and becomes the
// quiet NaN pattern; values that round past the largest finite bf16 carry
// into the exponent and become infinities.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The value a bf16 wire carries: x rounded to bf16 (nearest even), widened back.
__device__ __forceinline__ float bf16_wire(float x) {
  return __uint_as_float(bf16_rne(x) << 16);
}

// Stores 4 values that are bf16 values already (their low halves are zero) as
// 4 bf16 patterns, one 8-byte access.
template <int P>
__device__ __forceinline__ void store_bf16(uint16_t* p, const float (&x)[4]) {
  u32x2 u;
  u[0] = (__float_as_uint(x[0]) >> 16) | (__float_as_uint(x[1]) & 0xffff0000u);
  u[1] = (__float_as_uint(x[2]) >> 16) | (__float_as_uint(x[3]) & 0xffff0000u);
  stv<P>(p, u);
}

// Sum of one double per thread over the 256-thread block, in a fixed tree:
// a xor butterfly inside each wave (every lane ends with the same balanced
// tree sum of its wave) then (w0 + w1) + (w2 + w3).  The shape depends on
// nothing but the thread index, so the result is reproducible bit for bit.
__device__ __forceinline__ double block_sum_fixed(double s, double* lds) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s += __shfl_xor(s, m, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = s;
  __syncthreads();
  const double r = (lds[0] + lds[1]) + (lds[2] + lds[3]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// K1: reduce-scatter-mean.  One tile = one norm piece of GRZ_PIECE elements
// of one chunk, one workgroup.  Access k (0 <= k < K) of lane l covers the G
// elements at k*256*G + l*G of the tile, so each wave instruction reads one
// contiguous run per rank and writes one contiguous run of the mean.

template <typename TIn>
struct RsArgs {
  const TIn* rank[GRZ_MAX_RANKS];
  // 0: rank j's values of a segment start at rank[j] + src.  Otherwise
  // (GRZ_IN_TILED) piece k of a segment sits at rank[j] + src + k * tstride:
  // one receive buffer holding, piece by piece, the N ranks' values of each
  // piece side by side (rank[j] = buffer + j * GRZ_PIECE, tstride = N *
  // GRZ_PIECE), so that a tile's loads are one contiguous run.
  int64_t tstride;
  typename AccOf<TIn>::type* out;
  // GRZ_MEAN_BF16: the mean rounded to bf16 (nearest even) goes here instead
  // of `out`, and the piece sums are those of the rounded values.
  uint16_t* outb;
  double* partials;
  int64_t ntiles;
  int nsegs;
  int nranks;
  int average;   // divide the sum by `divisor`
  int pow2;      // divisor is a power of two: x / d == x * (1 / d) exactly
  double divisor;  // N, or the global token count of a token-weighted mean
  Seg seg[kMaxSegs];
};

// Fold one access's G elements over the ranks in ring order starting at rank
// c; NR > 0 fixes N at compile time so that every rank's load is in flight
// before the first add.
template <typename TIn, int NR, bool WIRE, typename Acc = typename AccOf<TIn>::type,
          int G = Geo<Acc>::G>
__device__ __forceinline__ void fold_vec(const TIn* const* rank, int nranks, int c, int64_t off,
                                         Acc (&acc)[G]) {
  if constexpr (NR > 0) {
    Acc x[NR][G];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      int r = c + j;
      r = r >= NR ? r - NR : r;
      loadg<GRZ_RS_POLICY>(rank[r] + off, x[j]);
    }
#pragma unroll
    for (int k = 0; k < G; ++k) acc[k] = x[0][k];
#pragma unroll
    for (int j = 1; j < NR; ++j)
#pragma unroll
      for (int k = 0; k < G; ++k) {
        acc[k] = x[j][k] + acc[k];
        if constexpr (WIRE) acc[k] = bf16_wire(acc[k]);
      }
  } else {
    const int n = nranks;
    loadg<GRZ_RS_POLICY>(rank[c] + off, acc);
    for (int j = 1; j < n; ++j) {
      int r = c + j;
      r = r >= n ? r - n : r;
      Acc x[G];
      loadg<GRZ_RS_POLICY>(rank[r] + off, x);
#pragma unroll
      for (int k = 0; k < G; ++k) {
        acc[k] = x[k] + acc[k];
        if constexpr (WIRE) acc[k] = bf16_wire(acc[k]);
      }
    }
  }
}

template <typename TIn, int NR, bool WIRE>
__device__ __forceinline__ typename AccOf<TIn>::type fold_one(const TIn* const* rank, int nranks,
                                                              int c, int64_t off) {
  using Acc = typename AccOf<TIn>::type;
  const int n = NR > 0 ? NR : nranks;
  Acc acc = widen1(rank[c] + off);
  for (int j = 1; j < n; ++j) {
    int r = c + j;
    r = r >= n ? r - n : r;
    acc = widen1(rank[r] + off) + acc;
    if constexpr (WIRE) acc = bf16_wire(acc);
  }
  return acc;
}

// fold_vec over accesses k0 .. k0 + KB - 1 of a full tile at once: all
// KB * NR loads are issued before the first addition.  `off` is the lane's
// first element; the fold of each element is the same sequence of additions
// as fold_vec's.
template <typename TIn, int NR, bool WIRE, int KB, typename Acc = typename AccOf<TIn>::type,
          int G = Geo<Acc>::G>
__device__ __forceinline__ void fold_tile(const TIn* const* rank, int c, int64_t off, int k0,
                                          Acc (&acc)[KB][G]) {
  Acc x[KB][NR][G];
#pragma unroll
  for (int k = 0; k < KB; ++k)
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      int r = c + j;
      r = r >= NR ? r - NR : r;
      loadg<GRZ_RS_POLICY>(rank[r] + off + static_cast<int64_t>(k0 + k) * kThreads * G,
                           x[k][j]);
    }
#pragma unroll
  for (int k = 0; k < KB; ++k)
#pragma unroll
    for (int i = 0; i < G; ++i) {
      acc[k][i] = x[k][0][i];
#pragma unroll
      for (int j = 1; j < NR; ++j) {
        acc[k][i] = x[k][j][i] + acc[k][i];
        if constexpr (WIRE) acc[k][i] = bf16_wire(acc[k][i]);
      }
    }
}

// WIRE (bf16 gradients only) rounds every partial sum of the fold to bf16, as a
// ring whose wire format is bf16 does once per hop ("13.5 Multi-GPU from
// First Principles", exercise 8).
template <typename TIn, int NR, bool WIRE, int WAVES, bool OB>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(WAVES, WAVES))) void rs_mean_kernel(const RsArgs<TIn> a) {
  using Acc = typename AccOf<TIn>::type;
  static_assert(!OB || sizeof(Acc) == 4, "a bf16 mean is the rounding of an fp32 one");
  constexpr int G = Geo<Acc>::G;
  constexpr int K = Geo<Acc>::K;
  __shared__ double lds[kThreads / 64];
  const Acc nf = static_cast<Acc>(a.divisor);  // exact: an integer below 2^24
  const Acc inv = static_cast<Acc>(1) / nf;
  const int lane = threadIdx.x;

  for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const Seg& s = a.seg[find_seg(a.seg, a.nsegs, tile)];
    const int64_t piece = tile - s.tile0;
    const int64_t e0 = piece * GRZ_PIECE;
    const int64_t left = s.len - e0;  // > 0
    const int c = s.chunk;
    const int64_t ib = a.tstride ? s.src + piece * a.tstride : s.src + e0;  // tile's input
    double sq = 0.0;
    bool done = false;
    if constexpr (GRZ_RS_BATCH && NR > 0 && sizeof(TIn) < 8) {
      if (s.vec && left >= GRZ_PIECE) {
        // At most 64 registers of loads in flight per lane (32 bf16 loads of
        // 8 bytes, 16 fp32 loads of 16 bytes): for bf16 the whole tile for
        // N <= 8 and two accesses at a time for N = 9..16, for fp32 the whole
        // tile for N <= 4 and two accesses for N = 5..8.  Beyond that the
        // three-wave shape of small launches spilled.  The squares are added
        // in the same order either way.
        constexpr int LW = static_cast<int>(sizeof(TIn)) * G / 4;  // registers per load
        constexpr int KB = NR * K * LW <= 64 ? K : (NR * (K / 2) * LW <= 64 ? K / 2 : 1);
        static_assert(K % KB == 0, "batch shape");
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += KB) {
          Acc acc[KB][G];
          fold_tile<TIn, NR, WIRE, KB>(a.rank, c, ib + lane * G, k0, acc);
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) {
            const int k = k0 + kk;
#pragma unroll
            for (int i = 0; i < G; ++i) {
              if (a.average) acc[kk][i] = a.pow2 ? acc[kk][i] * inv : acc[kk][i] / nf;
              if constexpr (OB) acc[kk][i] = bf16_wire(acc[kk][i]);
              sq = __fma_rn(static_cast<double>(acc[kk][i]), static_cast<double>(acc[kk][i]),
                            sq);
            }
            const int64_t o = s.dst + e0 + (k * kThreads + lane) * G;
            if constexpr (OB)
              store_bf16<GRZ_RS_POLICY>(a.outb + o, acc[kk]);
            else
              storeg<GRZ_RS_POLICY>(a.out + o, acc[kk]);
          }
        }
        done = true;
      }
    }
    if (!done) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t rel = static_cast<int64_t>(k * kThreads + lane) * G;
        const int64_t e = e0 + rel;
        if (s.vec && rel + G <= left) {
          Acc acc[G];
          fold_vec<TIn, NR, WIRE>(a.rank, a.nranks, c, ib + rel, acc);
#pragma unroll
          for (int i = 0; i < G; ++i) {
            if (a.average) acc[i] = a.pow2 ? acc[i] * inv : acc[i] / nf;
            if constexpr (OB) acc[i] = bf16_wire(acc[i]);
            sq = __fma_rn(static_cast<double>(acc[i]), static_cast<double>(acc[i]), sq);
          }
          if constexpr (OB)
            store_bf16<GRZ_RS_POLICY>(a.outb + s.dst + e, acc);
          else
            storeg<GRZ_RS_POLICY>(a.out + s.dst + e, acc);
        } else {
          for (int i = 0; i < G; ++i) {
            if (rel + i >= left) break;
            Acc v = fold_one<TIn, NR, WIRE>(a.rank, a.nranks, c, ib + rel + i);
            if (a.average) v = a.pow2 ? v * inv : v / nf;
            if constexpr (OB) v = bf16_wire(v);
            sq = __fma_rn(static_cast<double>(v), static_cast<double>(v), sq);
            if constexpr (OB)
              a.outb[s.dst + e + i] = static_cast<uint16_t>(__float_as_uint(v) >> 16);
            else
              a.out[s.dst + e + i] = v;
          }
        }
      }
    }
    const double tot = block_sum_fixed(sq, lds);
    if (a.partials != nullptr && lane == 0) a.partials[s.piece0 + piece] = tot;
  }
}

// ---------------------------------------------------------------------------
// K2: the fixed-order fp64 tree over piece sums.  Block j of a level folds
// values [j*4096, (j+1)*4096): lane l adds values l, l+256, ..., l+3840 in
// that order, then block_sum_fixed.  The tree depends only on the count.

// Block fold of values [base, base + 4096) of x (those below n): lane l adds
// values base + l, base + l + 256, ..., base + l + 3840 in that order, then
// block_sum_fixed.
__device__ __forceinline__ double fan_block_sum(const double* __restrict__ x, int64_t n,
                                                int64_t base, double* lds) {
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kReduceFan / kThreads; ++k) {
    const int64_t i = base + k * kThreads + threadIdx.x;
    if (i < n) s += x[i];
  }
  return block_sum_fixed(s, lds);
}

// The clip factor: fp32(max_norm / norm) when norm = sqrt(sqnorm) exceeds
// max_norm, else 1 (also when max_norm <= 0, and for a NaN norm, where the
// comparison is false).
__device__ __forceinline__ float clip_factor(double sqnorm, double max_norm) {
  float scale = 1.0f;
  if (max_norm > 0.0) {
    const double norm = sqrt(sqnorm);
    if (norm > max_norm) scale = static_cast<float>(max_norm / norm);
  }
  return scale;
}

__global__ __launch_bounds__(kThreads) void sqnorm_level_kernel(const double* __restrict__ x,
                                                                int64_t n, int64_t nblocks,
                                                                double* __restrict__ y) {
  __shared__ double lds[kThreads / 64];
  for (int64_t j = blockIdx.x; j < nblocks; j += gridDim.x) {
    const double tot = fan_block_sum(x, n, j * kReduceFan, lds);
    if (threadIdx.x == 0) y[j] = tot;
  }
}

// The step scalars of a captured step, advanced by the norm's last launch
// (see dp_grad_sqnorm_step_args): current = table[min(counter, count - 1)],
// then counter += 1.  `table` null: nothing to advance.
struct StepArgsNext {
  const grz_adamw_args* table;
  int64_t count;
  int64_t* counter;
  grz_adamw_args* current;
};

__device__ __forceinline__ void step_args_next(const StepArgsNext& a) {
  const int64_t c = *a.counter;
  const int64_t i = c < 0 ? 0 : (c >= a.count ? a.count - 1 : c);
  *a.current = a.table[i];
  *a.counter = c + 1;
}

__global__ __launch_bounds__(kThreads) void sqnorm_final_kernel(const double* __restrict__ x,
                                                                int64_t n, double max_norm,
                                                                double* __restrict__ sqnorm_out,
                                                                float* __restrict__ scale_out,
                                                                const StepArgsNext next) {
  __shared__ double lds[kThreads / 64];
  const double tot = fan_block_sum(x, n, 0, lds);
  if (threadIdx.x == 0) {
    if (sqnorm_out != nullptr) *sqnorm_out = tot;
    if (scale_out != nullptr) *scale_out = clip_factor(tot, max_norm);
    if (next.table != nullptr) step_args_next(next);
  }
}

// Piece sums of one fp32 array: piece p is [p*4096, (p+1)*4096), one
// workgroup, the same lane mapping and accumulation order as the reduce
// kernel's (access k of lane l: the 4 elements at k*1024 + 4*l, squares
// accumulated in fp64 with one rounding each, then block_sum_fixed).
__global__ __launch_bounds__(kThreads) void piece_sqnorm_kernel(const float* __restrict__ g,
                                                                int64_t n, int64_t npieces,
                                                                int vec,
                                                                double* __restrict__ partials) {
  constexpr int G = 4;
  constexpr int K = GRZ_PIECE / (kThreads * G);
  __shared__ double lds[kThreads / 64];
  for (int64_t piece = blockIdx.x; piece < npieces; piece += gridDim.x) {
    const int64_t e0 = piece * GRZ_PIECE;
    const int64_t left = n - e0;
    double sq = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t rel = static_cast<int64_t>(k * kThreads + threadIdx.x) * G;
      if (vec && rel + G <= left) {
        float x[G];
        loadg<kNtLoad>(g + e0 + rel, x);
#pragma unroll
        for (int i = 0; i < G; ++i)
          sq = __fma_rn(static_cast<double>(x[i]), static_cast<double>(x[i]), sq);
      } else {
        for (int i = 0; i < G; ++i) {
          if (rel + i >= left) break;
          const double x = g[e0 + rel + i];
          sq = __fma_rn(x, x, sq);
        }
      }
    }
    const double tot = block_sum_fixed(sq, lds);
    if (threadIdx.x == 0) partials[piece] = tot;
  }
}

// ---------------------------------------------------------------------------
// K3: clip + AdamW over shard-compact fp32 state; the new master is rounded
// to bf16 and written to every replica at the arena offset of its segment.

struct AdamArgs {
  float* master;
  float* m;
  float* v;
  const float* grad;
  const uint16_t* gradb;  // GRZ_MEAN_BF16: the mean as bf16 patterns (`grad` unused)
  const float* scale;   // device scalar or null (1)
  const grz_adamw_args* dargs;  // step scalars in device memory, or null (use the fields below)
  uint16_t* rep[GRZ_MAX_RANKS];
  int nrep;
  int nsegs;
  int64_t ntiles;
  float lr, b1, b2, eps, wd, bc1, bc2;
  Seg seg[kMaxSegs];
};

typedef const __attribute__((address_space(4))) grz_adamw_args ConstArgs;

// One element, every operation rounded on its own (the file is built with
// -ffp-contract=off; '/' and sqrtf are the IEEE ones).
__device__ __forceinline__ void adamw1(float& w, float& m, float& v, float g, float lr,
                                       float b1, float omb1, float b2, float omb2,
                                       float eps, float wd, float bc1, float bc2) {
  m = b1 * m + omb1 * g;
  v = b2 * v + omb2 * (g * g);
  const float mh = m / bc1;
  const float vh = v / bc2;
  const float u = mh / (__builtin_sqrtf(vh) + eps);
  w = w - lr * (u + wd * w);
}

// Access k (0 <= k < K) of lane l covers the 4 elements at k*T*4 + 4*l of
// the tile (T = GRZ_ADAM_THREADS): 16-byte accesses of the fp32 streams,
// 8-byte bf16 stores (and loads of a bf16 mean, GB), each wave instruction
// one contiguous run.
template <bool GB>
__global__ __launch_bounds__(GRZ_ADAM_THREADS) GRZ_ADAM_ATTR void adamw_kernel(
    const AdamArgs a) {
  constexpr int G = 4;
  constexpr int K = GRZ_ADAM_TILE / (GRZ_ADAM_THREADS * G);
  const float scale = a.scale != nullptr ? *a.scale : 1.0f;
  float lr = a.lr, b1 = a.b1, b2 = a.b2, eps = a.eps, wd = a.wd, bc1 = a.bc1, bc2 = a.bc2;
  if (a.dargs != nullptr) {
    // Read as constant memory (the scalars do not change while the kernel
    // runs), so that they arrive through uniform loads rather than a vector
    // load that every workgroup waits for before its first tile.
    const ConstArgs* d = (const ConstArgs*)(a.dargs);  // an address-space cast
    lr = d->lr; b1 = d->beta1; b2 = d->beta2; eps = d->eps; wd = d->weight_decay;
    bc1 = d->bias_corr1; bc2 = d->bias_corr2;
  }
  const float omb1 = 1.0f - b1;  // exact: 1/2 <= b1 <= 1 (Sterbenz)
  const float omb2 = 1.0f - b2;
  const int lane = threadIdx.x;

  for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const Seg& s = a.seg[find_seg(a.seg, a.nsegs, tile)];
    const int64_t e0 = (tile - s.tile0) * GRZ_ADAM_TILE;
    const int64_t left = s.len - e0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t rel = static_cast<int64_t>(k * GRZ_ADAM_THREADS + lane) * G;
      const int64_t e = e0 + rel;
      if (s.vec && rel + G <= left) {
        const int64_t i = s.src + e;
        float g[G], w[G], m[G], v[G];
        if constexpr (GB)
          loadg<GRZ_ADAM_POLICY>(a.gradb + i, g);
        else
          loadg<GRZ_ADAM_POLICY>(a.grad + i, g);
        loadg<GRZ_ADAM_POLICY>(a.master + i, w);
        loadg<GRZ_ADAM_POLICY>(a.m + i, m);
        loadg<GRZ_ADAM_POLICY>(a.v + i, v);
        uint32_t b[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
          adamw1(w[j], m[j], v[j], g[j] * scale, lr, b1, omb1, b2, omb2, eps, wd, bc1, bc2);
          b[j] = bf16_rne(w[j]);
        }
        storeg<GRZ_ADAM_POLICY>(a.master + i, w);
        storeg<GRZ_ADAM_POLICY>(a.m + i, m);
        storeg<GRZ_ADAM_POLICY>(a.v + i, v);
        u32x2 packed;
        packed[0] = b[0] | (b[1] << 16);
        packed[1] = b[2] | (b[3] << 16);
        for (int r = 0; r < a.nrep; ++r) stv<GRZ_ADAM_POLICY>(a.rep[r] + s.dst + e, packed);
      } else {
        for (int j = 0; j < G; ++j) {
          if (rel + j >= left) break;
          const int64_t i = s.src + e + j;
          float w = a.master[i], m = a.m[i], v = a.v[i];
          const float g = GB ? widen1(a.gradb + i) : a.grad[i];
          adamw1(w, m, v, g * scale, lr, b1, omb1, b2, omb2, eps, wd, bc1, bc2);
          a.master[i] = w;
          a.m[i] = m;
          a.v[i] = v;
          const uint16_t b = static_cast<uint16_t>(bf16_rne(w));
          for (int r = 0; r < a.nrep; ++r) a.rep[r][s.dst + e + j] = b;
        }
      }
    }
  }
}

// The next step's scalars for a captured (replayed) step: current =
// table[min(counter, count - 1)], then counter += 1.  One thread.
__global__ void args_next_kernel(const StepArgsNext next) {
  if (threadIdx.x == 0 && blockIdx.x == 0) step_args_next(next);
}

// ---------------------------------------------------------------------------
// All-gather: copy shard segments (source shard = Seg::chunk) into replicas.

struct GatherArgs {
  const uint16_t* shard[GRZ_MAX_RANKS];
  uint16_t* rep[GRZ_MAX_RANKS];
  int nrep;
  int nsegs;
  int64_t ntiles;
  Seg seg[kMaxSegs];
};

// Access k (0 <= k < K) of lane l copies the 8 elements (16 bytes) at
// k*T*8 + 8*l of the tile (T = GRZ_AG_THREADS).
__global__ __launch_bounds__(GRZ_AG_THREADS) GRZ_AG_ATTR void gather_kernel(
    const GatherArgs a) {
  constexpr int G = 8;
  constexpr int K = GRZ_AG_TILE / (GRZ_AG_THREADS * G);
  const int lane = threadIdx.x;
  for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const Seg& s = a.seg[find_seg(a.seg, a.nsegs, tile)];
    const int64_t e0 = (tile - s.tile0) * GRZ_AG_TILE;
    const int64_t left = s.len - e0;
    const uint16_t* src = a.shard[s.chunk];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t rel = static_cast<int64_t>(k * GRZ_AG_THREADS + lane) * G;
      const int64_t e = e0 + rel;
      if (s.vec && rel + G <= left) {
        const u32x4 u = ldv<GRZ_AG_POLICY, u32x4>(src + s.src + e);
        for (int r = 0; r < a.nrep; ++r) stv<GRZ_AG_POLICY>(a.rep[r] + s.dst + e, u);
      } else {
        for (int j = 0; j < G; ++j) {
          if (rel + j >= left) break;
          const uint16_t u = src[s.src + e + j];
          for (int r = 0; r < a.nrep; ++r) a.rep[r][s.dst + e + j] = u;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// K1 + K2 + K3 in one launch, for a shard whose mean fits in the registers of
// the co-resident grid: the reduce keeps every mean value in registers, the
// piece sums go through self-flagging workspace slots (below) to the
// workgroups that fold the norm in the same tree as dp_grad_sqnorm, and the
// same registers feed AdamW once the norm is known.  The
// mean never goes to memory (unless asked for), which saves 8 bytes per owned
// element against the three-kernel path.  The arithmetic of every value is
// that of rs_mean_kernel, sqnorm_*_kernel and adamw_kernel, so the results are
// the same bits.  The grid is sized to be resident at once, and every wait is
// bounded.

constexpr int kFusedPieces = 4;   // pieces (tiles) a workgroup holds in registers
constexpr int kFusedSegs = 32;    // segments per launch

// A segment of the fused launch: offsets of one chunk of one bucket in the
// rank inputs (`in`), in master/m/v and the optional mean (`st`) and in the
// replica arenas (`glob`).  vec bit 0: the reduce accesses are 16/8-byte
// aligned; bit 1: the state and replica accesses are.
struct FSeg {
  int64_t in;
  int64_t st;
  int64_t glob;
  int64_t len;
  int64_t piece0;
  int64_t tile0;
  int32_t chunk;
  int32_t vec;
};

template <typename TIn>
struct FusedArgs {
  const TIn* rank[GRZ_MAX_RANKS];
  uint16_t* rep[GRZ_MAX_RANKS];
  float* master;
  float* m;
  float* v;
  float* mean_out;                // optional copy of the mean
  double* partials;               // piece sums of the whole plan (peers' filled in)
  unsigned* ctl;                  // control words of the workspace (see kCtlBytes)
  uint64_t* slots;                // published piece sums, one per piece of the plan
  uint64_t* lslots;               // published first-level sums of the norm tree
  uint64_t* total;                // the published norm
  double* sqnorm_out;
  float* scale_out;
  const grz_adamw_args* dargs;    // step scalars in device memory, or null
  StepArgsNext next;              // or the launch takes them from a table and advances it
  double max_norm;
  double divisor;
  int64_t ntiles;                 // pieces this launch reduces
  int64_t npieces;                // pieces of the plan
  int nred;                       // workgroups that reduce; the others fold the norm
  int nranks;
  int nrep;
  int nsegs;
  int pow2;
  float lr, b1, b2, eps, wd, bc1, bc2;
  FSeg seg[kFusedSegs];
};

// The norm of the one-launch step needs every piece sum of the plan before
// any workgroup may clip, and no grid-wide barrier: each sum is published in
// a slot of the workspace that says by itself whether it belongs to this
// launch.  A sum of squares is never negative, so bit 63 of its fp64 pattern
// is free; a launch stores its sums with bit 63 set to its parity (one plus
// the low bit of the launch counter in the workspace), and a reader polls
// the slot with device-scope loads until the bit matches.  The value is its
// own flag, so nothing else has to be ordered: no counter, no fence, and none
// of the L2 write-back and invalidation that a device-scope release and
// acquire cost on this chip (with a two-level barrier the launch took 0.24 ms
// at the GPT-2 124M one-rank share).  The tree is dp_grad_sqnorm's, folded by
// workgroups after the reducing ones, which hold no mean: with more than 4096
// pieces, folder j folds level block j and publishes it in its own slot and
// every reducing workgroup folds the level slots itself; with fewer, the one
// folder folds the pieces and publishes the norm, which every reducing
// workgroup waits for.  Workgroup 0 advances the launch counter once it has
// the norm.  A NaN sum is published as the one quiet NaN.
//
// Control words (32-bit, the first kCtlBytes of the workspace): word 2 the
// time-out flag, word 3 the poll limit (0 means kDefaultSpinLimit), word 4
// the launch counter, word 5 the piece count of the last launch plus one.
// Every launch rewrites every slot of its plan, so a slot holds the last
// launch's parity as long as the piece count stays the same; a launch with
// another piece count raises the flag instead of reading slots that older
// launches may have left at its parity.  A wait that reaches the limit
// raises the flag and its workgroup stops; a launch that finds the flag
// raised does nothing at all, so a workspace whose last call gave up stays
// stopped until it is cleared (zeroed, which also makes every slot stale).
constexpr size_t kCtlBytes = 256;
constexpr uint64_t kSignBit = 1ull << 63;

__device__ __forceinline__ void publish(uint64_t* slot, double x, uint64_t parity) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(x)) & ~kSignBit;
  if (u > 0x7ff0000000000000ull) u = 0x7ff8000000000000ull;
  __hip_atomic_store(slot, u | (parity << 63), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls `slot` until it holds this launch's value (true) or `limit` polls
// have passed (false).
__device__ __forceinline__ bool collect(uint64_t* slot, uint64_t parity, unsigned limit,
                                        double* x) {
  for (unsigned polls = 0;;) {
    const uint64_t u = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((u >> 63) == parity) {
      *x = __longlong_as_double(static_cast<long long>(u & ~kSignBit));
      return true;
    }
    if (++polls >= limit) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// fan_block_sum over published slots [base, base + 4096) (those below n): the
// same additions in the same order, each value taken once it is published.
// A lane loads its 16 slots kBatch at a time (all at once: the folders hold
// no mean, so the registers are there) and polls again only those that were
// not published yet.  False (in every thread) when a wait of any thread gave
// up.
__device__ __forceinline__ bool fan_block_collect(uint64_t* slots, int64_t n, int64_t base,
                                                  uint64_t parity, unsigned limit,
                                                  double* lds, double* out) {
  constexpr int kPer = kReduceFan / kThreads;
  constexpr int kBatch = kPer;
  double s = 0.0;
  bool ok = true;
#pragma unroll
  for (int k0 = 0; k0 < kPer; k0 += kBatch) {
    uint64_t u[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t i = base + (k0 + k) * kThreads + threadIdx.x;
      u[k] = i < n ? __hip_atomic_load(slots + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : parity << 63;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t i = base + (k0 + k) * kThreads + threadIdx.x;
      if (i < n && ok) {
        double x;
        if ((u[k] >> 63) == parity)
          x = __longlong_as_double(static_cast<long long>(u[k] & ~kSignBit));
        else
          ok = collect(slots + i, parity, limit, &x);
        if (ok) s += x;
      }
    }
  }
  const bool all_ok = __syncthreads_and(ok) != 0;
  *out = block_sum_fixed(s, lds);
  return all_ok;
}

// fan_block_sum of n <= 256 published values (value l in lane l alone), as
// fan_block_collect computes it, with one load per lane.
__device__ __forceinline__ bool small_collect(uint64_t* slots, int64_t n, uint64_t parity,
                                              unsigned limit, double* lds, double* out) {
  double s = 0.0;
  bool ok = true;
  if (threadIdx.x < n) {
    double x;
    ok = collect(slots + threadIdx.x, parity, limit, &x);
    if (ok) s += x;
  }
  const bool all_ok = __syncthreads_and(ok) != 0;
  *out = block_sum_fixed(s, lds);
  return all_ok;
}

// At most 128 VGPRs, so that 4 waves per SIMD (4 workgroups per CU) fit: the
// mean registers per lane (16 per piece held) plus the fold's and AdamW's
// working set.  PIECES: the pieces a workgroup can hold (kFusedPieces, or 1
// for a launch whose pieces fit one per reducing workgroup).  The update
// takes B accesses at a time and the first B accesses' state is loaded
// before the norm is known: two with four pieces held, the whole piece
// (12 loads) with one, which the registers then have room for.
template <typename TIn, int NR, bool WIRE, int PIECES>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void fused_step_kernel(const FusedArgs<TIn> a) {
  constexpr int G = 4;
  constexpr int K = GRZ_PIECE / (kThreads * G);
  constexpr int B = PIECES == 1 ? K : 2;
  static_assert(K % B == 0, "the update's batches");
  __shared__ double lds[kThreads / 64];
  __shared__ double norm_lds;
  const float nf = static_cast<float>(a.divisor);
  const float inv = 1.0f / nf;
  const int lane = threadIdx.x;
  float mean[PIECES][K][G];

  // The control words, read once per workgroup.  A workspace whose last call
  // gave up, or that served a plan of another piece count (whose slots would
  // not all have been rewritten by the last launch), does nothing until it is
  // cleared; a plan of another piece count also raises the flag.
  __shared__ unsigned ctl_lds[2];
  __shared__ int64_t step_lds;  // the step counter, with a table of step scalars
  if (lane == 0) {
    if (a.next.table != nullptr)
      step_lds = __hip_atomic_load(a.next.counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned flag = __hip_atomic_load(a.ctl + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned plan = __hip_atomic_load(a.ctl + 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool other_plan = plan != 0 && plan != static_cast<unsigned>(a.npieces + 1);
    if (other_plan && flag == 0)
      __hip_atomic_store(a.ctl + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ctl_lds[0] = (flag != 0 || other_plan) ? 1u : 0u;
    ctl_lds[1] = __hip_atomic_load(a.ctl + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (ctl_lds[0] != 0) return;
  const unsigned launch_no = ctl_lds[1];
  const uint64_t parity = (launch_no + 1u) & 1u;
  const unsigned set = a.ctl[3];
  const unsigned limit = set != 0 ? set : kDefaultSpinLimit;

  // Publish the pieces this launch does not reduce (the peers'), as given.
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + lane; i < a.npieces;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    bool own = false;
    for (int j = 0; j < a.nsegs; ++j) {
      const FSeg& s = a.seg[j];
      own = own || (i >= s.piece0 && i < s.piece0 + (s.len + GRZ_PIECE - 1) / GRZ_PIECE);
    }
    if (!own) publish(a.slots + i, a.partials[i], parity);
  }

  // The workgroups after the first nred fold the norm and hold no mean: with
  // a level below the final fold, workgroup nred + j folds level block j;
  // without, workgroup nred folds the pieces into the norm.  Each publishes
  // its sum.  (Workgroup 0 is a folder only when the launch reduces nothing;
  // it then goes on to take the norm like the others.)
  const int64_t nl = a.npieces > kReduceFan ? (a.npieces + kReduceFan - 1) / kReduceFan : 0;
  if (static_cast<int>(blockIdx.x) >= a.nred) {
    const int64_t f = blockIdx.x - a.nred;
    double t;
    const bool ok = fan_block_collect(a.slots, a.npieces, nl > 0 ? f * kReduceFan : 0, parity,
                                      limit, lds, &t);
    if (!ok) {
      if (lane == 0) __hip_atomic_store(a.ctl + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (lane == 0) publish(nl > 0 ? a.lslots + f : a.total, t, parity);
    if (blockIdx.x != 0) return;
  }

  // Reduce: the pieces blockIdx.x, blockIdx.x + nred, ... of the launch.
#pragma unroll
  for (int p = 0; p < PIECES; ++p) {
    const int64_t tile = blockIdx.x + static_cast<int64_t>(p) * a.nred;
    if (tile < a.ntiles) {
      const FSeg& s = a.seg[find_seg(a.seg, a.nsegs, tile)];
      const int64_t piece = tile - s.tile0;
      const int64_t e0 = piece * GRZ_PIECE;
      const int64_t left = s.len - e0;
      double sq = 0.0;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t rel = static_cast<int64_t>(k * kThreads + lane) * G;
        const int64_t e = e0 + rel;
        if ((s.vec & 1) && rel + G <= left) {
          fold_vec<TIn, NR, WIRE>(a.rank, a.nranks, s.chunk, s.in + e, mean[p][k]);
#pragma unroll
          for (int i = 0; i < G; ++i) {
            mean[p][k][i] = a.pow2 ? mean[p][k][i] * inv : mean[p][k][i] / nf;
            sq = __fma_rn(static_cast<double>(mean[p][k][i]),
                          static_cast<double>(mean[p][k][i]), sq);
          }
          if (a.mean_out != nullptr) storeg<GRZ_RS_POLICY>(a.mean_out + s.st + e, mean[p][k]);
        } else {
#pragma unroll
          for (int i = 0; i < G; ++i) {
            float x = 0.0f;
            if (rel + i < left) {
              x = fold_one<TIn, NR, WIRE>(a.rank, a.nranks, s.chunk, s.in + e + i);
              x = a.pow2 ? x * inv : x / nf;
              sq = __fma_rn(static_cast<double>(x), static_cast<double>(x), sq);
              if (a.mean_out != nullptr) a.mean_out[s.st + e + i] = x;
            }
            mean[p][k][i] = x;
          }
        }
      }
      const double tot = block_sum_fixed(sq, lds);
      if (lane == 0) {
        a.partials[s.piece0 + piece] = tot;
        publish(a.slots + s.piece0 + piece, tot, parity);
      }
    }
  }

  // The first B accesses of the first piece's state, loaded before the
  // norm is known (the state is this workgroup's alone), so that they are in
  // flight while it waits.
  float pw[B][G], pm[B][G], pv[B][G];
  bool pre = false;
  if (blockIdx.x < a.ntiles) {
    const FSeg& s = a.seg[find_seg(a.seg, a.nsegs, blockIdx.x)];
    const int64_t e0 = (blockIdx.x - s.tile0) * GRZ_PIECE;
    if ((s.vec & 2) && static_cast<int64_t>((B - 1) * kThreads + lane) * G + G <= s.len - e0) {
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int64_t i = s.st + e0 + static_cast<int64_t>(j * kThreads + lane) * G;
        loadg<GRZ_ADAM_POLICY>(a.master + i, pw[j]);
        loadg<GRZ_ADAM_POLICY>(a.m + i, pm[j]);
        loadg<GRZ_ADAM_POLICY>(a.v + i, pv[j]);
      }
      pre = true;
    }
  }

  // Norm: the tree of dp_grad_sqnorm (at most one level below the final
  // fold), from the folders' published sums.  With a level, every workgroup
  // folds the level sums itself (the same tree, so the same bits
  // everywhere); without, it takes the norm the folder published.  A
  // workgroup whose wait gives up has not seen every piece sum, so it writes
  // nothing more (its tiles keep their old state) and raises the flag.
  bool ok = true;
  {
    double t = 0.0;
    if (nl > 0)
      ok = small_collect(a.lslots, nl, parity, limit, lds, &t);
    else if (lane == 0)
      ok = collect(a.total, parity, limit, &t);
    if (lane == 0) norm_lds = t;
  }
  if (__syncthreads_or(!ok) != 0) {
    if (lane == 0) __hip_atomic_store(a.ctl + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const double sqnorm = norm_lds;
  const float scale = clip_factor(sqnorm, a.max_norm);
  if (blockIdx.x == 0 && lane == 0) {
    if (a.sqnorm_out != nullptr) *a.sqnorm_out = sqnorm;
    if (a.scale_out != nullptr) *a.scale_out = scale;
    // Every workgroup has read the launch counter and the step counter (each
    // published a piece after reading them), so both can advance.
    __hip_atomic_store(a.ctl + 4, launch_no + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.ctl + 5, static_cast<unsigned>(a.npieces + 1), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (a.next.table != nullptr) {
      const int64_t c = step_lds;
      *a.next.current = a.next.table[c < 0 ? 0 : (c >= a.next.count ? a.next.count - 1 : c)];
      __hip_atomic_store(a.next.counter, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // Clip + AdamW from the registers; bf16 weights into every replica.
  float lr = a.lr, b1 = a.b1, b2 = a.b2, eps = a.eps, wd = a.wd, bc1 = a.bc1, bc2 = a.bc2;
  if (a.next.table != nullptr) {
    // Row min(counter, count - 1) of the table: the step scalars
    // grz_step_args_next would have copied to `current`.
    const int64_t c = step_lds;
    const ConstArgs* d = (const ConstArgs*)(a.next.table +
                                            (c < 0 ? 0 : (c >= a.next.count ? a.next.count - 1 : c)));
    lr = d->lr; b1 = d->beta1; b2 = d->beta2; eps = d->eps; wd = d->weight_decay;
    bc1 = d->bias_corr1; bc2 = d->bias_corr2;
  } else if (a.dargs != nullptr) {
    // Read as constant memory (the scalars do not change while the kernel
    // runs), so that they arrive through uniform loads rather than a vector
    // load that every workgroup waits for before its first tile.
    const ConstArgs* d = (const ConstArgs*)(a.dargs);  // an address-space cast
    lr = d->lr; b1 = d->beta1; b2 = d->beta2; eps = d->eps; wd = d->weight_decay;
    bc1 = d->bias_corr1; bc2 = d->bias_corr2;
  }
  const float omb1 = 1.0f - b1;
  const float omb2 = 1.0f - b2;
#pragma unroll
  for (int p = 0; p < PIECES; ++p) {
    const int64_t tile = blockIdx.x + static_cast<int64_t>(p) * a.nred;
    if (tile < a.ntiles) {
      const FSeg& s = a.seg[find_seg(a.seg, a.nsegs, tile)];
      const int64_t e0 = (tile - s.tile0) * GRZ_PIECE;
      const int64_t left = s.len - e0;
      // B accesses at a time: all their loads are in flight before the
      // first update.
#pragma unroll
      for (int kb = 0; kb < K; kb += B) {
        float w[B][G], m[B][G], v[B][G];
        bool vec[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
          const int64_t rel = static_cast<int64_t>((kb + j) * kThreads + lane) * G;
          vec[j] = (s.vec & 2) && rel + G <= left;
          if (p == 0 && kb == 0 && pre) {
#pragma unroll
            for (int q = 0; q < G; ++q) {
              w[j][q] = pw[j][q];
              m[j][q] = pm[j][q];
              v[j][q] = pv[j][q];
            }
          } else if (vec[j]) {
            const int64_t i = s.st + e0 + rel;
            loadg<GRZ_ADAM_POLICY>(a.master + i, w[j]);
            loadg<GRZ_ADAM_POLICY>(a.m + i, m[j]);
            loadg<GRZ_ADAM_POLICY>(a.v + i, v[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
          const int k = kb + j;
          const int64_t rel = static_cast<int64_t>(k * kThreads + lane) * G;
          const int64_t e = e0 + rel;
          if (vec[j]) {
            const int64_t i = s.st + e;
            uint32_t b[G];
#pragma unroll
            for (int q = 0; q < G; ++q) {
              adamw1(w[j][q], m[j][q], v[j][q], mean[p][k][q] * scale, lr, b1, omb1, b2,
                     omb2, eps, wd, bc1, bc2);
              b[q] = bf16_rne(w[j][q]);
            }
            storeg<GRZ_ADAM_POLICY>(a.master + i, w[j]);
            storeg<GRZ_ADAM_POLICY>(a.m + i, m[j]);
            storeg<GRZ_ADAM_POLICY>(a.v + i, v[j]);
            u32x2 packed;
            packed[0] = b[0] | (b[1] << 16);
            packed[1] = b[2] | (b[3] << 16);
            for (int r = 0; r < a.nrep; ++r) stv<GRZ_ADAM_POLICY>(a.rep[r] + s.glob + e, packed);
          } else {
#pragma unroll
            for (int q = 0; q < G; ++q) {
              if (rel + q < left) {
                const int64_t i = s.st + e + q;
                float ws = a.master[i], ms = a.m[i], vs = a.v[i];
                adamw1(ws, ms, vs, mean[p][k][q] * scale, lr, b1, omb1, b2, omb2, eps, wd, bc1,
                       bc2);
                a.master[i] = ws;
                a.m[i] = ms;
                a.v[i] = vs;
                const uint16_t bb = static_cast<uint16_t>(bf16_rne(ws));
                for (int r = 0; r < a.nrep; ++r) a.rep[r][s.glob + e + q] = bb;
              }
            }
          }
        }
      }
    }
  }
}

// Every kernel takes its arguments by value: keep each struct within the 4 KB
// a launch may pass.
static_assert(sizeof(RsArgs<double>) <= 4096 && sizeof(RsArgs<uint16_t>) <= 4096,
              "reduce arguments exceed 4 KB");
static_assert(sizeof(AdamArgs) <= 4096, "optimizer arguments exceed 4 KB");
static_assert(sizeof(GatherArgs) <= 4096, "all-gather arguments exceed 4 KB");
static_assert(sizeof(FusedArgs<float>) <= 4096, "fused-step arguments exceed 4 KB");

// ---------------------------------------------------------------------------
// Host side: plan geometry, argument checks and launches.

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline void chunk_of(int64_t length, int n, int c, int64_t* off, int64_t* cnt) {
  const int64_t q = length / n, rem = length % n;
  *off = c * q + (c < rem ? c : rem);
  *cnt = q + (c < rem ? 1 : 0);
}

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

int check_plan(const grz_bucket* buckets, int nbuckets, int nranks, int chunk, int flags) {
  if (nranks < 1 || nranks > GRZ_MAX_RANKS) return GRZ_EINVAL;
  if (nbuckets < 0 || (nbuckets > 0 && buckets == nullptr)) return GRZ_EINVAL;
  if (chunk < -1 || chunk >= nranks) return GRZ_EINVAL;
  if (flags & ~(GRZ_SUM | GRZ_UNEVEN | GRZ_IN_COMPACT | GRZ_BF16_WIRE | GRZ_IN_RANGE |
                GRZ_OUT_GLOBAL | GRZ_IN_TILED | GRZ_MEAN_BF16))
    return GRZ_EINVAL;
  for (int b = 0; b < nbuckets; ++b) {
    if (buckets[b].offset < 0 || buckets[b].length < 0) return GRZ_ERANGE;
    if (buckets[b].length > (INT64_MAX >> 4) - buckets[b].offset) return GRZ_ERANGE;
    if (chunk >= 0 && !(flags & GRZ_UNEVEN) && buckets[b].length % nranks != 0)
      return GRZ_EINDIVISIBLE;
  }
  return GRZ_OK;
}

// Segments of a plan: one per (bucket, chunk) processed, in plan order.
// src/dst are filled for the reduce kernel's view; callers remap them.
struct PlanSeg {
  int64_t global;   // arena offset of the chunk
  int64_t compact;  // shard-compact offset (chunk >= 0) or arena offset
  int64_t len;
  int64_t piece0;
  int chunk;
  int bucket;
  int64_t input;    // offset in the rank inputs when they hold a bucket range only
  int64_t lpiece0;  // (chunk >= 0) pieces of the chunk in the buckets before this one
};

// The segments of buckets [first, first + count) of the plan; offsets and
// piece numbers are those of the whole plan.
std::vector<PlanSeg> plan_segments(const grz_bucket* buckets, int nbuckets, int n, int chunk,
                                   int first = 0, int count = -1) {
  if (count < 0) count = nbuckets - first;
  std::vector<PlanSeg> out;
  int64_t piece = 0, compact = 0, lpiece = 0;
  for (int b = 0; b < nbuckets; ++b) {
    const bool take = b >= first && b < first + count;
    for (int c = 0; c < n; ++c) {
      int64_t off, cnt;
      chunk_of(buckets[b].length, n, c, &off, &cnt);
      if (chunk < 0 || c == chunk) {
        if (cnt > 0 && take) {
          const int64_t g = buckets[b].offset + off;
          out.push_back({g, chunk < 0 ? g : compact, cnt, piece, c, b, g, lpiece});
        }
        if (chunk >= 0) {
          compact += cnt;
          lpiece += ceil_div(cnt, GRZ_PIECE);
        }
      }
      piece += ceil_div(cnt, GRZ_PIECE);
    }
  }
  return out;
}

// Workgroups of a grid-stride launch over `units` tiles: at most the knob and
// at most what a dispatch can express (its grid counts work-items in 32
// bits).  Every such kernel loops over its tiles, so any width gives the same
// results.
int64_t grid_for(int64_t units, int block) {
  const int64_t cap = g_max_blocks;
  const int64_t hw = static_cast<int64_t>(UINT32_MAX) / block;
  int64_t grid = units < cap ? units : cap;
  return grid < hw ? grid : hw;
}

template <typename T> struct NoDeduce { using type = T; };

// Launches `kernel` and returns the status of this launch alone (the return
// value of hipLaunchKernel): an error the caller has not collected yet stays
// in the runtime's last-error slot, neither cleared nor taken for ours.  The
// argument types are the kernel's own, so each params entry points at an
// object of exactly its parameter's type.
template <typename... A>
int launch(void (*kernel)(A...), dim3 grid, dim3 block, hipStream_t stream,
           typename NoDeduce<A>::type... a) {
  void* params[] = {static_cast<void*>(&a)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, params, 0,
                         stream) == hipSuccess ? GRZ_OK : GRZ_EHIP;
}

template <typename Args>
int launch_batches(std::vector<Seg>& segs, Args& args,
                   void (*kernel)(const Args), hipStream_t stream,
                   int64_t tile_elems = GRZ_PIECE, int block = kThreads) {
  for (size_t first = 0; first < segs.size(); first += kMaxSegs) {
    const size_t cnt = segs.size() - first < static_cast<size_t>(kMaxSegs)
                           ? segs.size() - first : static_cast<size_t>(kMaxSegs);
    int64_t tiles = 0;
    for (size_t i = 0; i < cnt; ++i) {
      args.seg[i] = segs[first + i];
      args.seg[i].tile0 = tiles;
      tiles += ceil_div(segs[first + i].len, tile_elems);
    }
    if (tiles == 0) continue;
    args.nsegs = static_cast<int>(cnt);
    args.ntiles = tiles;
    const int64_t grid = grid_for(tiles, block);
    const int st = launch(kernel, dim3(static_cast<unsigned>(grid)), dim3(block), stream, args);
    if (st != GRZ_OK) return st;
  }
  return GRZ_OK;
}

template <typename TIn, int NR, bool WIRE, bool OB>
int rs_launch_shape(std::vector<Seg>& segs, RsArgs<TIn>& args, bool small,
                    hipStream_t stream) {
  constexpr int WL = RsWaves<NR, false>::value, WS = RsWaves<NR, true>::value;
  return small ? launch_batches(segs, args, rs_mean_kernel<TIn, NR, WIRE, WS, OB>, stream)
               : launch_batches(segs, args, rs_mean_kernel<TIn, NR, WIRE, WL, OB>, stream);
}

template <typename TIn, int NR>
int rs_launch(std::vector<Seg>& segs, RsArgs<TIn>& args, bool wire, hipStream_t stream) {
  int64_t tiles = 0;
  for (const Seg& s : segs) tiles += ceil_div(s.len, GRZ_PIECE);
  const bool small = tiles <= kRsSmallTiles;
  const bool ob = args.outb != nullptr;
  if constexpr (sizeof(TIn) == 2) {
    if (wire)
      return ob ? rs_launch_shape<TIn, NR, true, true>(segs, args, small, stream)
                : rs_launch_shape<TIn, NR, true, false>(segs, args, small, stream);
  }
  if constexpr (sizeof(TIn) < 8) {
    if (ob) return rs_launch_shape<TIn, NR, false, true>(segs, args, small, stream);
  }
  return rs_launch_shape<TIn, NR, false, false>(segs, args, small, stream);
}

template <typename TIn>
int rs_dispatch(const void* const* rank_grads, int n, const std::vector<PlanSeg>& ps,
                int flags, int64_t divisor, void* mean_out, double* partials,
                hipStream_t stream) {
  using Acc = typename AccOf<TIn>::type;
  static RsArgs<TIn> proto;  // zero-initialised template
  RsArgs<TIn> args = proto;
  // One access moves G elements: G * out_esz bytes of the mean (16, or 8 for a
  // bf16 mean), G * sizeof(TIn) of each input.
  constexpr size_t in_bytes = Geo<Acc>::G * sizeof(TIn);
  const bool ob = (flags & GRZ_MEAN_BF16) != 0;
  const size_t out_esz = ob ? 2 : sizeof(Acc);
  const size_t out_bytes = Geo<Acc>::G * out_esz;
  bool vec_base = aligned(mean_out, out_bytes);
  for (int j = 0; j < n; ++j) {
    if (!aligned(rank_grads[j], sizeof(TIn))) return GRZ_EALIGN;
    vec_base = vec_base && aligned(rank_grads[j], in_bytes);
    args.rank[j] = static_cast<const TIn*>(rank_grads[j]);
  }
  args.out = ob ? nullptr : static_cast<Acc*>(mean_out);
  args.outb = ob ? static_cast<uint16_t*>(mean_out) : nullptr;
  args.partials = partials;
  args.nranks = n;
  args.average = (flags & GRZ_SUM) ? 0 : 1;
  args.divisor = static_cast<double>(divisor);
  args.pow2 = (divisor & (divisor - 1)) == 0;
  const bool compact_in = (flags & GRZ_IN_COMPACT) != 0;
  const bool out_global = (flags & GRZ_OUT_GLOBAL) != 0;
  args.tstride = (flags & GRZ_IN_TILED) ? static_cast<int64_t>(n) * GRZ_PIECE : 0;
  std::vector<Seg> segs;
  segs.reserve(ps.size());
  for (const PlanSeg& p : ps) {
    Seg s{};
    s.src = args.tstride ? p.lpiece0 * args.tstride : compact_in ? p.compact : p.input;
    s.dst = out_global ? p.global : p.compact;
    s.len = p.len;
    s.piece0 = p.piece0;
    s.chunk = p.chunk;
    s.vec = vec_base && (s.src * sizeof(TIn)) % in_bytes == 0 &&
            (s.dst * out_esz) % out_bytes == 0;
    segs.push_back(s);
  }
  const bool wire = (flags & GRZ_BF16_WIRE) != 0;
  // Every N the library takes has its own unrolled fold.
  static_assert(GRZ_MAX_RANKS == 16, "one case per N below");
  switch (n) {
    case 1: return rs_launch<TIn, 1>(segs, args, wire, stream);
    case 2: return rs_launch<TIn, 2>(segs, args, wire, stream);
    case 3: return rs_launch<TIn, 3>(segs, args, wire, stream);
    case 4: return rs_launch<TIn, 4>(segs, args, wire, stream);
    case 5: return rs_launch<TIn, 5>(segs, args, wire, stream);
    case 6: return rs_launch<TIn, 6>(segs, args, wire, stream);
    case 7: return rs_launch<TIn, 7>(segs, args, wire, stream);
    case 8: return rs_launch<TIn, 8>(segs, args, wire, stream);
    case 9: return rs_launch<TIn, 9>(segs, args, wire, stream);
    case 10: return rs_launch<TIn, 10>(segs, args, wire, stream);
    case 11: return rs_launch<TIn, 11>(segs, args, wire, stream);
    case 12: return rs_launch<TIn, 12>(segs, args, wire, stream);
    case 13: return rs_launch<TIn, 13>(segs, args, wire, stream);
    case 14: return rs_launch<TIn, 14>(segs, args, wire, stream);
    case 15: return rs_launch<TIn, 15>(segs, args, wire, stream);
    case 16: return rs_launch<TIn, 16>(segs, args, wire, stream);
    default: return GRZ_EINVAL;
  }
}

int sqnorm_levels(int64_t n, int64_t* sizes, int max_levels) {
  int levels = 0;
  while (n > kReduceFan && levels < max_levels) {
    n = ceil_div(n, kReduceFan);
    sizes[levels++] = n;
  }
  return levels;
}

int reduce_entry(const void* const* rank_grads, int nranks, int64_t divisor, int dtype,
                 const grz_bucket* buckets, int nbuckets, int bucket_first, int bucket_count,
                 int chunk, int flags, void* mean_out, double* piece_sqnorm,
                 hipStream_t stream);

// Appends segment `s`, split so that the part after a short head writes
// whole 64-byte blocks of its destination (`dst0` = byte address of the
// destination of element 0 of the segment, `elem` = destination element
// bytes, `g` = elements per vector access): a store run that starts inside a
// block turns every block it covers into two partial writes at the memory
// side.  `keep` (the byte addresses, at the segment's element 0, of the
// `nkeep` other streams the kernel writes, `keep_elem` bytes per element)
// refuses a head that would move one of them off its blocks.  Measured on
// MI355X, GPT-2 1.5B: the optimizer's bf16 writes into a chunk 32 bytes off a
// block boundary ran 2.8 ms against 2.2 ms on one (at N = 4); a head that
// moved its fp32 master, m and v 32 bytes off instead ran 1.07 ms against
// 0.94 (at N = 8), hence `keep`.  For the optimizer and the copy only, whose
// tiles carry no meaning; every element's result is the same.
void push_block_aligned(std::vector<Seg>& segs, Seg s, uintptr_t dst0, int elem, int g,
                        const uintptr_t* keep, int nkeep, int keep_elem) {
  const int64_t mis = static_cast<int64_t>(dst0 % 64);
  if (s.vec && mis % (elem * g) == 0 && mis != 0) {
    const int64_t head = (64 - mis) / elem;  // a multiple of g
    bool ok = head < s.len;
    for (int k = 0; k < nkeep && ok; ++k)
      ok = keep[k] % 64 != 0 || (keep[k] + head * keep_elem) % 64 == 0;
    if (ok) {
      Seg h = s;
      h.len = head;
      segs.push_back(h);
      s.src += head;
      s.dst += head;
      s.len -= head;
    }
  }
  segs.push_back(s);
}

// All-gather of shards whose elements are `units` 16-bit words (1 bf16, 2
// fp32, 4 fp64): the plan's segments in elements, copied as words by the
// bf16 copy kernel.
int gather_entry(const void* const* shards, int nranks, int units, const grz_bucket* buckets,
                 int nbuckets, int flags, void* const* replicas, int nreplicas,
                 hipStream_t stream) {
  if (flags & ~GRZ_UNEVEN) return GRZ_EINVAL;
  if (shards == nullptr) return GRZ_EINVAL;
  if (nreplicas < 0 || nreplicas > GRZ_MAX_RANKS) return GRZ_EINVAL;
  if (nreplicas > 0 && replicas == nullptr) return GRZ_EINVAL;
  for (int r = 0; r < nranks && r < GRZ_MAX_RANKS; ++r) {
    const int st = check_plan(buckets, nbuckets, nranks, (r + 1) % nranks, flags);
    if (st != GRZ_OK) return st;
  }
  const int st = check_plan(buckets, nbuckets, nranks, -1, flags);
  if (st != GRZ_OK) return st;
  const size_t elem = 2 * static_cast<size_t>(units);
  for (int b = 0; b < nbuckets; ++b)  // word offsets must stay below 2^59
    if (buckets[b].offset + buckets[b].length > (INT64_MAX >> 4) / units) return GRZ_ERANGE;
  static GatherArgs proto;
  GatherArgs a = proto;
  bool vec_base = true;
  for (int r = 0; r < nreplicas; ++r) {
    if (replicas[r] == nullptr) return GRZ_EINVAL;
    if (!aligned(replicas[r], elem)) return GRZ_EALIGN;
    vec_base = vec_base && aligned(replicas[r], 16);
    a.rep[r] = static_cast<uint16_t*>(replicas[r]);
  }
  a.nrep = nreplicas;
  if (nreplicas == 0) return GRZ_OK;
  std::vector<Seg> segs;
  for (int r = 0; r < nranks; ++r) {
    a.shard[r] = static_cast<const uint16_t*>(shards[r]);
    if (shards[r] == nullptr) continue;
    if (!aligned(shards[r], elem)) return GRZ_EALIGN;
    const bool vr = vec_base && aligned(shards[r], 16);
    for (const PlanSeg& p : plan_segments(buckets, nbuckets, nranks, (r + 1) % nranks)) {
      Seg s{};
      s.src = p.compact * units;
      s.dst = p.global * units;
      s.len = p.len * units;
      s.chunk = r;
      s.vec = vr && s.src % 8 == 0 && s.dst % 8 == 0;
      push_block_aligned(segs, s, reinterpret_cast<uintptr_t>(a.rep[0] + s.dst), 2, 8, nullptr,
                         0, 0);
    }
  }
  return launch_batches(segs, a, gather_kernel, stream, GRZ_AG_TILE, GRZ_AG_THREADS);
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI

extern "C" {

int grz_version(void) { return 103; }

const char* grz_strerror(int status) {
  switch (status) {
    case GRZ_OK: return "ok";
    case GRZ_EINVAL: return "invalid argument";
    case GRZ_EINDIVISIBLE: return "bucket length not divisible by N: no even shard split";
    case GRZ_EALIGN: return "device pointer not aligned to its element size";
    case GRZ_EHIP: return "HIP launch error";
    case GRZ_ERANGE: return "bucket or size out of range";
    default: return "unknown status";
  }
}

int grz_set_max_blocks(int blocks) {
  if (blocks < 1 || blocks > (1 << 30)) return GRZ_EINVAL;
  g_max_blocks = blocks;
  return GRZ_OK;
}

int dp_ring_owned_chunk(int rank, int nranks) {
  if (nranks < 1 || rank < 0 || rank >= nranks) return -1;
  return (rank + 1) % nranks;
}

int dp_ring_chunk_owner(int chunk, int nranks) {
  if (nranks < 1 || chunk < 0 || chunk >= nranks) return -1;
  return (chunk + nranks - 1) % nranks;
}

int dp_chunk_range(int64_t length, int nranks, int chunk, int64_t* offset, int64_t* count) {
  if (length < 0 || nranks < 1 || chunk < 0 || chunk >= nranks || !offset || !count)
    return GRZ_EINVAL;
  chunk_of(length, nranks, chunk, offset, count);
  return GRZ_OK;
}

int64_t dp_piece_count(const grz_bucket* buckets, int nbuckets, int nranks, int flags) {
  const int st = check_plan(buckets, nbuckets, nranks, -1, flags);
  if (st != GRZ_OK) return -st;
  int64_t pieces = 0;
  for (int b = 0; b < nbuckets; ++b)
    for (int c = 0; c < nranks; ++c) {
      int64_t off, cnt;
      chunk_of(buckets[b].length, nranks, c, &off, &cnt);
      pieces += ceil_div(cnt, GRZ_PIECE);
    }
  return pieces;
}

int64_t dp_piece_offset(const grz_bucket* buckets, int nbuckets, int nranks, int flags,
                        int bucket, int chunk) {
  const int st = check_plan(buckets, nbuckets, nranks, -1, flags);
  if (st != GRZ_OK) return -st;
  if (bucket < 0 || bucket >= nbuckets || chunk < 0 || chunk >= nranks) return -GRZ_EINVAL;
  int64_t pieces = 0;
  for (int b = 0; b < nbuckets; ++b)
    for (int c = 0; c < nranks; ++c) {
      if (b == bucket && c == chunk) return pieces;
      int64_t off, cnt;
      chunk_of(buckets[b].length, nranks, c, &off, &cnt);
      pieces += ceil_div(cnt, GRZ_PIECE);
    }
  return -GRZ_EINVAL;
}

int64_t dp_shard_numel(const grz_bucket* buckets, int nbuckets, int nranks, int chunk,
                       int flags) {
  if (chunk < 0) return -GRZ_EINVAL;
  const int st = check_plan(buckets, nbuckets, nranks, chunk, flags);
  if (st != GRZ_OK) return -st;
  int64_t total = 0;
  for (int b = 0; b < nbuckets; ++b) {
    int64_t off, cnt;
    chunk_of(buckets[b].length, nranks, chunk, &off, &cnt);
    total += cnt;
  }
  return total;
}

int64_t dp_tiled_numel(const grz_bucket* buckets, int nbuckets, int nranks, int chunk,
                       int flags) {
  if (chunk < 0) return -GRZ_EINVAL;
  const int st = check_plan(buckets, nbuckets, nranks, chunk, flags);
  if (st != GRZ_OK) return -st;
  int64_t pieces = 0;
  for (int b = 0; b < nbuckets; ++b) {
    int64_t off, cnt;
    chunk_of(buckets[b].length, nranks, chunk, &off, &cnt);
    pieces += ceil_div(cnt, GRZ_PIECE);
  }
  if (pieces > (INT64_MAX >> 4) / (static_cast<int64_t>(nranks) * GRZ_PIECE)) return -GRZ_ERANGE;
  return pieces * nranks * GRZ_PIECE;
}

int dp_reduce_scatter_mean(const void* const* rank_grads, int nranks, int dtype,
                           const grz_bucket* buckets, int nbuckets, int chunk, int flags,
                           void* mean_out, double* piece_sqnorm, hipStream_t stream) {
  return dp_reduce_scatter_mean_range(rank_grads, nranks, dtype, buckets, nbuckets, 0, nbuckets,
                                      chunk, flags, mean_out, piece_sqnorm, stream);
}

int dp_reduce_scatter_mean_range(const void* const* rank_grads, int nranks, int dtype,
                                 const grz_bucket* buckets, int nbuckets, int bucket_first,
                                 int bucket_count, int chunk, int flags, void* mean_out,
                                 double* piece_sqnorm, hipStream_t stream) {
  return reduce_entry(rank_grads, nranks, nranks, dtype, buckets, nbuckets, bucket_first,
                      bucket_count, chunk, flags, mean_out, piece_sqnorm, stream);
}

int dp_reduce_scatter_weighted(const void* const* rank_grads, const int64_t* token_counts,
                               int nranks, int dtype, const grz_bucket* buckets, int nbuckets,
                               int bucket_first, int bucket_count, int chunk, int flags,
                               void* mean_out, double* piece_sqnorm, hipStream_t stream) {
  if (token_counts == nullptr || nranks < 1 || nranks > GRZ_MAX_RANKS) return GRZ_EINVAL;
  if (flags & GRZ_SUM) return GRZ_EINVAL;
  int64_t total = 0;  // the scalar all-reduce of the token counts
  for (int j = 0; j < nranks; ++j) {
    if (token_counts[j] < 0) return GRZ_EINVAL;
    total += token_counts[j];
    if (total > (int64_t(1) << 24)) return GRZ_ERANGE;
  }
  if (total == 0) return GRZ_EINVAL;
  return reduce_entry(rank_grads, nranks, total, dtype, buckets, nbuckets, bucket_first,
                      bucket_count, chunk, flags, mean_out, piece_sqnorm, stream);
}

}  // extern "C"

namespace {

int reduce_entry(const void* const* rank_grads, int nranks, int64_t divisor, int dtype,
                 const grz_bucket* buckets, int nbuckets, int bucket_first, int bucket_count,
                 int chunk, int flags, void* mean_out, double* piece_sqnorm,
                 hipStream_t stream) {
  int st = check_plan(buckets, nbuckets, nranks, chunk, flags);
  if (st != GRZ_OK) return st;
  if (bucket_first < 0 || bucket_count < 0 || bucket_first > nbuckets ||
      bucket_count > nbuckets - bucket_first)
    return GRZ_EINVAL;
  if (rank_grads == nullptr || mean_out == nullptr) return GRZ_EINVAL;
  if ((flags & GRZ_IN_COMPACT) && chunk < 0) return GRZ_EINVAL;
  if ((flags & GRZ_BF16_WIRE) && dtype != GRZ_BF16) return GRZ_EINVAL;
  if ((flags & GRZ_MEAN_BF16) && dtype != GRZ_BF16 && dtype != GRZ_F32) return GRZ_EINVAL;
  for (int j = 0; j < nranks; ++j)
    if (rank_grads[j] == nullptr) return GRZ_EINVAL;
  if (piece_sqnorm != nullptr && !aligned(piece_sqnorm, 8)) return GRZ_EALIGN;
  if ((flags & GRZ_IN_RANGE) && (flags & GRZ_IN_COMPACT)) return GRZ_EINVAL;
  if (flags & GRZ_IN_TILED) {
    // One receive buffer: rank j's pointer is the buffer + j pieces.
    if (!(flags & GRZ_IN_COMPACT)) return GRZ_EINVAL;
    const int64_t esz = dtype == GRZ_BF16 ? 2 : dtype == GRZ_F32 ? 4 : dtype == GRZ_F64 ? 8 : 0;
    if (esz == 0) return GRZ_EINVAL;
    const uintptr_t base = reinterpret_cast<uintptr_t>(rank_grads[0]);
    for (int j = 1; j < nranks; ++j)
      if (reinterpret_cast<uintptr_t>(rank_grads[j]) !=
          base + static_cast<uintptr_t>(j) * GRZ_PIECE * esz)
        return GRZ_EINVAL;
  }
  std::vector<PlanSeg> ps =
      plan_segments(buckets, nbuckets, nranks, chunk, bucket_first, bucket_count);
  if (flags & GRZ_IN_RANGE) {
    // Inputs hold only the range: arena index minus the range's lowest offset.
    int64_t base = INT64_MAX;
    for (int b = bucket_first; b < bucket_first + bucket_count; ++b)
      if (buckets[b].length > 0 && buckets[b].offset < base) base = buckets[b].offset;
    for (PlanSeg& p : ps) p.input = p.global - base;
  }
  switch (dtype) {
    case GRZ_BF16:
      if (!aligned(mean_out, (flags & GRZ_MEAN_BF16) ? 2 : 4)) return GRZ_EALIGN;
      return rs_dispatch<uint16_t>(rank_grads, nranks, ps, flags, divisor, mean_out,
                                   piece_sqnorm, stream);
    case GRZ_F32:
      if (!aligned(mean_out, (flags & GRZ_MEAN_BF16) ? 2 : 4)) return GRZ_EALIGN;
      return rs_dispatch<float>(rank_grads, nranks, ps, flags, divisor, mean_out, piece_sqnorm,
                                stream);
    case GRZ_F64:
      if (!aligned(mean_out, 8)) return GRZ_EALIGN;
      return rs_dispatch<double>(rank_grads, nranks, ps, flags, divisor, mean_out,
                                 piece_sqnorm, stream);
    default:
      return GRZ_EINVAL;
  }
}

}  // namespace

extern "C" {

size_t dp_grad_sqnorm_workspace(int64_t npieces) {
  if (npieces <= 0) return 0;
  int64_t sizes[8];
  const int levels = sqnorm_levels(npieces, sizes, 8);
  int64_t total = 0;
  for (int i = 0; i < levels; ++i) total += sizes[i];
  return static_cast<size_t>(total) * sizeof(double);
}

}  // extern "C"

namespace {

int check_step_args(const grz_adamw_args* table, int64_t count, const int64_t* counter,
                    const grz_adamw_args* current) {
  if (table == nullptr || counter == nullptr || current == nullptr || count < 1)
    return GRZ_EINVAL;
  if (!aligned(table, 4) || !aligned(counter, 8) || !aligned(current, 4)) return GRZ_EALIGN;
  return GRZ_OK;
}

int sqnorm_entry(const double* piece_sqnorm, int64_t npieces, double max_norm,
                 void* workspace, double* sqnorm_out, float* clip_scale_out,
                 const StepArgsNext& next, hipStream_t stream) {
  if (npieces < 0) return GRZ_EINVAL;
  if (npieces > 0 && piece_sqnorm == nullptr) return GRZ_EINVAL;
  if (sqnorm_out == nullptr && clip_scale_out == nullptr) return GRZ_EINVAL;
  if (!aligned(piece_sqnorm, 8) || !aligned(sqnorm_out, 8) || !aligned(clip_scale_out, 4) ||
      !aligned(workspace, 8))
    return GRZ_EALIGN;
  if (npieces > static_cast<int64_t>(kReduceFan) * kReduceFan * kReduceFan) return GRZ_ERANGE;
  int64_t sizes[8];
  const int levels = sqnorm_levels(npieces, sizes, 8);
  if (levels > 0 && workspace == nullptr) return GRZ_EINVAL;
  const double* in = piece_sqnorm;
  int64_t n = npieces;
  double* ws = static_cast<double*>(workspace);
  for (int i = 0; i < levels; ++i) {
    const unsigned grid = static_cast<unsigned>(grid_for(sizes[i], kThreads));
    const int st = launch(sqnorm_level_kernel, dim3(grid), dim3(kThreads), stream, in, n,
                          sizes[i], ws);
    if (st != GRZ_OK) return st;
    in = ws;
    n = sizes[i];
    ws += sizes[i];
  }
  return launch(sqnorm_final_kernel, dim3(1), dim3(kThreads), stream, in, n, max_norm,
                sqnorm_out, clip_scale_out, next);
}

}  // namespace

extern "C" {

int dp_grad_sqnorm(const double* piece_sqnorm, int64_t npieces, double max_norm,
                   void* workspace, double* sqnorm_out, float* clip_scale_out,
                   hipStream_t stream) {
  return sqnorm_entry(piece_sqnorm, npieces, max_norm, workspace, sqnorm_out, clip_scale_out,
                      StepArgsNext{}, stream);
}

int dp_grad_sqnorm_step_args(const double* piece_sqnorm, int64_t npieces, double max_norm,
                             void* workspace, double* sqnorm_out, float* clip_scale_out,
                             const grz_adamw_args* table, int64_t count, int64_t* counter,
                             grz_adamw_args* current, hipStream_t stream) {
  const int st = check_step_args(table, count, counter, current);
  if (st != GRZ_OK) return st;
  return sqnorm_entry(piece_sqnorm, npieces, max_norm, workspace, sqnorm_out, clip_scale_out,
                      StepArgsNext{table, count, counter, current}, stream);
}

}  // extern "C"

// The middle levels of the norm tree for callers that cannot allocate: one
// array per device, held until the process ends.  Host code never passes the
// array's own name to a kernel (on the host it is only a stand-in for the
// symbol); it looks the device address up once per device and uses that.
static __device__ __align__(256) double scratch[GRZ_NOALLOC_SCRATCH_BYTES / sizeof(double)];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];  // device address of `scratch`, per device

// The address of the current device's `scratch`, looked up on the first call
// on that device (with it current) and kept.
int scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GRZ_EHIP;
  if (dev < 0 || dev >= kScratchDevices) return GRZ_ERANGE;
  if (stream != nullptr) {  // another device's stream would get this device's address
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return GRZ_EHIP;
    if (sdev != dev) return GRZ_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return GRZ_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GRZ_OK;
}

}  // namespace

extern "C" {

int dp_grad_sqnorm_noalloc(const double* piece_sqnorm, int64_t npieces, double max_norm,
                           double* sqnorm_out, float* clip_scale_out, hipStream_t stream) {
  if (npieces < 0) return GRZ_EINVAL;
  if (dp_grad_sqnorm_workspace(npieces) > GRZ_NOALLOC_SCRATCH_BYTES) return GRZ_ERANGE;
  void* ws = nullptr;
  const int st = scratch_for_current_device(stream, &ws);
  if (st != GRZ_OK) return st;
  return dp_grad_sqnorm(piece_sqnorm, npieces, max_norm, ws, sqnorm_out, clip_scale_out,
                        stream);
}

size_t dp_grad_sqnorm_of_workspace(int64_t n) {
  if (n <= 0) return 0;
  const int64_t npieces = ceil_div(n, GRZ_PIECE);
  return static_cast<size_t>(npieces) * sizeof(double) + dp_grad_sqnorm_workspace(npieces);
}

int dp_grad_sqnorm_of(const float* grad, int64_t n, double max_norm, void* workspace,
                      double* sqnorm_out, float* clip_scale_out, hipStream_t stream) {
  if (n < 0 || (n > 0 && (grad == nullptr || workspace == nullptr))) return GRZ_EINVAL;
  if (sqnorm_out == nullptr && clip_scale_out == nullptr) return GRZ_EINVAL;
  if (!aligned(grad, 4) || !aligned(workspace, 8)) return GRZ_EALIGN;
  const int64_t npieces = ceil_div(n, GRZ_PIECE);
  if (npieces > static_cast<int64_t>(kReduceFan) * kReduceFan * kReduceFan) return GRZ_ERANGE;
  double* partials = static_cast<double*>(workspace);
  if (npieces > 0) {
    const unsigned grid = static_cast<unsigned>(grid_for(npieces, kThreads));
    const int st = launch(piece_sqnorm_kernel, dim3(grid), dim3(kThreads), stream, grad, n,
                          npieces, aligned(grad, 16) ? 1 : 0, partials);
    if (st != GRZ_OK) return st;
  }
  return dp_grad_sqnorm(partials, npieces, max_norm, partials + npieces, sqnorm_out,
                        clip_scale_out, stream);
}

// `mean_grad` holds fp32 values, or bf16 patterns when `grad_bf16`.
static int adamw_common(float* master, float* m, float* v, const void* mean_grad,
                        bool grad_bf16, const std::vector<PlanSeg>& ps, const float* clip_scale,
                        const grz_adamw_args* args, bool args_on_device,
                        uint16_t* const* replicas, int nreplicas, hipStream_t stream) {
  if (!master || !m || !v || !mean_grad || !args) return GRZ_EINVAL;
  if (args_on_device && !aligned(args, 4)) return GRZ_EALIGN;
  if (nreplicas < 0 || nreplicas > GRZ_MAX_RANKS) return GRZ_EINVAL;
  if (nreplicas > 0 && replicas == nullptr) return GRZ_EINVAL;
  const size_t gsz = grad_bf16 ? 2 : 4;
  if (!aligned(master, 4) || !aligned(m, 4) || !aligned(v, 4) || !aligned(mean_grad, gsz) ||
      !aligned(clip_scale, 4))
    return GRZ_EALIGN;
  static AdamArgs proto;
  AdamArgs a = proto;
  a.master = master;
  a.m = m;
  a.v = v;
  a.grad = grad_bf16 ? nullptr : static_cast<const float*>(mean_grad);
  a.gradb = grad_bf16 ? static_cast<const uint16_t*>(mean_grad) : nullptr;
  a.scale = clip_scale;
  bool vec_base = aligned(master, 16) && aligned(m, 16) && aligned(v, 16) &&
                  aligned(mean_grad, 4 * gsz);
  for (int r = 0; r < nreplicas; ++r) {
    if (replicas[r] == nullptr) return GRZ_EINVAL;
    if (!aligned(replicas[r], 2)) return GRZ_EALIGN;
    vec_base = vec_base && aligned(replicas[r], 8);
    a.rep[r] = replicas[r];
  }
  a.nrep = nreplicas;
  if (args_on_device) {
    a.dargs = args;
  } else {
    a.lr = args->lr;
    a.b1 = args->beta1;
    a.b2 = args->beta2;
    a.eps = args->eps;
    a.wd = args->weight_decay;
    a.bc1 = args->bias_corr1;
    a.bc2 = args->bias_corr2;
  }
  std::vector<Seg> segs;
  segs.reserve(ps.size());
  for (const PlanSeg& p : ps) {
    Seg s{};
    s.src = p.compact;
    s.dst = p.global;
    s.len = p.len;
    s.chunk = p.chunk;
    s.vec = vec_base && s.src % 4 == 0 && s.dst % 4 == 0;
    if (nreplicas > 0) {
      const uintptr_t keep[3] = {reinterpret_cast<uintptr_t>(master + s.src),
                                 reinterpret_cast<uintptr_t>(m + s.src),
                                 reinterpret_cast<uintptr_t>(v + s.src)};
      push_block_aligned(segs, s, reinterpret_cast<uintptr_t>(replicas[0] + s.dst), 2, 4, keep,
                         3, 4);
    } else
      segs.push_back(s);
  }
  return grad_bf16 ? launch_batches(segs, a, adamw_kernel<true>, stream, GRZ_ADAM_TILE,
                                    GRZ_ADAM_THREADS)
                   : launch_batches(segs, a, adamw_kernel<false>, stream, GRZ_ADAM_TILE,
                                    GRZ_ADAM_THREADS);
}

int zero1_adamw_step(float* master, float* m, float* v, const float* mean_grad, int64_t n,
                     const float* clip_scale, const grz_adamw_args* args, uint16_t* bf16_out,
                     hipStream_t stream) {
  if (n < 0) return GRZ_EINVAL;
  if (n == 0) return GRZ_OK;
  std::vector<PlanSeg> ps{{0, 0, n, 0, 0, 0, 0, 0}};
  uint16_t* reps[1] = {bf16_out};
  return adamw_common(master, m, v, mean_grad, false, ps, clip_scale, args, false, reps,
                      bf16_out ? 1 : 0, stream);
}

int zero1_adamw_gather(float* master, float* m, float* v, const void* mean_grad,
                       const grz_bucket* buckets, int nbuckets, int nranks, int chunk,
                       int flags, const float* clip_scale, const grz_adamw_args* args,
                       uint16_t* const* replicas, int nreplicas, hipStream_t stream) {
  const bool dev_args = (flags & GRZ_ARGS_DEVICE) != 0;
  const bool grad_bf16 = (flags & GRZ_MEAN_BF16) != 0;
  flags &= ~(GRZ_ARGS_DEVICE | GRZ_MEAN_BF16);
  const int st = check_plan(buckets, nbuckets, nranks, chunk, flags);
  if (st != GRZ_OK) return st;
  if (flags & (GRZ_SUM | GRZ_IN_COMPACT | GRZ_BF16_WIRE | GRZ_IN_RANGE | GRZ_OUT_GLOBAL |
               GRZ_IN_TILED))
    return GRZ_EINVAL;
  std::vector<PlanSeg> ps;
  if (chunk >= 0) {
    ps = plan_segments(buckets, nbuckets, nranks, chunk);
  } else {
    for (int b = 0; b < nbuckets; ++b)
      if (buckets[b].length > 0)
        ps.push_back({buckets[b].offset, buckets[b].offset, buckets[b].length, 0, 0, b,
                      buckets[b].offset, 0});
  }
  return adamw_common(master, m, v, mean_grad, grad_bf16, ps, clip_scale, args, dev_args,
                      replicas, nreplicas, stream);
}

int grz_step_args_next(const grz_adamw_args* table, int64_t count, int64_t* counter,
                       grz_adamw_args* current, hipStream_t stream) {
  const int st = check_step_args(table, count, counter, current);
  if (st != GRZ_OK) return st;
  return launch(args_next_kernel, dim3(1), dim3(64), stream,
                StepArgsNext{table, count, counter, current});
}

int zero1_all_gather(const uint16_t* const* shards, int nranks, const grz_bucket* buckets,
                     int nbuckets, int flags, uint16_t* const* replicas, int nreplicas,
                     hipStream_t stream) {
  return gather_entry(reinterpret_cast<const void* const*>(shards), nranks, 1, buckets,
                      nbuckets, flags, reinterpret_cast<void* const*>(replicas), nreplicas,
                      stream);
}

int dp_all_gather(const void* const* shards, int nranks, int dtype, const grz_bucket* buckets,
                  int nbuckets, int flags, void* const* replicas, int nreplicas,
                  hipStream_t stream) {
  const int units = dtype == GRZ_BF16 ? 1 : dtype == GRZ_F32 ? 2 : dtype == GRZ_F64 ? 4 : 0;
  if (units == 0) return GRZ_EINVAL;
  return gather_entry(shards, nranks, units, buckets, nbuckets, flags, replicas, nreplicas,
                      stream);
}

size_t zero1_fused_workspace(int64_t npieces) {
  if (npieces < 0) npieces = 0;
  const int64_t nl = npieces > kReduceFan ? ceil_div(npieces, kReduceFan) : 0;
  return kCtlBytes + static_cast<size_t>(npieces + nl + 1) * sizeof(uint64_t);
}

}  // extern "C"

namespace {

template <typename TIn, int NR, bool WIRE>
const void* fused_kernel_ptr(bool one_piece) {
  return one_piece ? reinterpret_cast<const void*>(&fused_step_kernel<TIn, NR, WIRE, 1>)
                   : reinterpret_cast<const void*>(&fused_step_kernel<TIn, NR, WIRE, kFusedPieces>);
}

// The fused kernel instance for (dtype, N) that holds kFusedPieces pieces
// per workgroup, or one, or null.  (The bf16-wire fold is not instantiated
// here: its per-hop rounding does not fit the register budget next to the
// held mean.)
const void* fused_kernel_for(int dtype, int nranks, bool one_piece = false) {
  if (dtype == GRZ_BF16) {
    switch (nranks) {
      case 1: return fused_kernel_ptr<uint16_t, 1, false>(one_piece);
      case 2: return fused_kernel_ptr<uint16_t, 2, false>(one_piece);
      case 4: return fused_kernel_ptr<uint16_t, 4, false>(one_piece);
      case 8: return fused_kernel_ptr<uint16_t, 8, false>(one_piece);
      default: return fused_kernel_ptr<uint16_t, 0, false>(one_piece);
    }
  }
  if (dtype == GRZ_F32) {
    switch (nranks) {
      case 1: return fused_kernel_ptr<float, 1, false>(one_piece);
      case 2: return fused_kernel_ptr<float, 2, false>(one_piece);
      case 4: return fused_kernel_ptr<float, 4, false>(one_piece);
      case 8: return fused_kernel_ptr<float, 8, false>(one_piece);
      default: return fused_kernel_ptr<float, 0, false>(one_piece);
    }
  }
  return nullptr;
}

// Workgroups of `kernel` that can be resident at once on the current device.
int fused_max_grid(const void* kernel, int* grid) {
  int dev = 0, cus = 0, coop = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GRZ_EHIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess)
    return GRZ_EHIP;
  if (!coop) return GRZ_EHIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess)
    return GRZ_EHIP;
  *grid = per_cu * cus;
  return *grid > 0 ? GRZ_OK : GRZ_EHIP;
}

template <typename TIn>
int fused_launch(const void* kernel, const void* kernel1, const void* const* rank_grads,
                 int nranks,
                 const std::vector<PlanSeg>& ps, int flags, float* master, float* m, float* v,
                 const grz_adamw_args* args, const StepArgsNext& next, double max_norm,
                 uint16_t* const* replicas,
                 int nreplicas, double* piece_sqnorm, int64_t npieces, void* workspace,
                 double* sqnorm_out, float* clip_scale_out, float* mean_out,
                 hipStream_t stream) {
  static FusedArgs<TIn> proto;
  FusedArgs<TIn> a = proto;
  constexpr size_t in_bytes = 4 * sizeof(TIn);
  bool vin = mean_out == nullptr || aligned(mean_out, 16);
  for (int j = 0; j < nranks; ++j) {
    if (!aligned(rank_grads[j], sizeof(TIn))) return GRZ_EALIGN;
    vin = vin && aligned(rank_grads[j], in_bytes);
    a.rank[j] = static_cast<const TIn*>(rank_grads[j]);
  }
  bool vst = aligned(master, 16) && aligned(m, 16) && aligned(v, 16);
  for (int r = 0; r < nreplicas; ++r) {
    vst = vst && aligned(replicas[r], 8);
    a.rep[r] = replicas[r];
  }
  const bool compact_in = (flags & GRZ_IN_COMPACT) != 0;
  int64_t tiles = 0;
  int nsegs = 0;
  for (const PlanSeg& p : ps) {
    FSeg& s = a.seg[nsegs++];
    s.in = compact_in ? p.compact : p.input;
    s.st = p.compact;
    s.glob = p.global;
    s.len = p.len;
    s.piece0 = p.piece0;
    s.tile0 = tiles;
    s.chunk = p.chunk;
    s.vec = ((vin && (s.in * sizeof(TIn)) % in_bytes == 0 && s.st % 4 == 0) ? 1 : 0) |
            ((vst && s.st % 4 == 0 && s.glob % 4 == 0) ? 2 : 0);
    tiles += ceil_div(p.len, GRZ_PIECE);
  }
  int max_grid = 0;
  const int st = fused_max_grid(kernel, &max_grid);
  if (st != GRZ_OK) return st;
  // One folding workgroup per level block of the norm tree (one without a
  // level); the rest of the resident grid reduces.
  const int64_t nl = npieces > kReduceFan ? ceil_div(npieces, kReduceFan) : 0;
  const int64_t nfold = nl > 0 ? nl : 1;
  if (nl > kThreads || nfold >= max_grid) return GRZ_ERANGE;
  const int64_t nred_max = max_grid - nfold;
  if (tiles > nred_max * kFusedPieces) return GRZ_ERANGE;
  const int64_t nred = tiles < nred_max ? tiles : nred_max;
  const int grid = static_cast<int>(nred + nfold);
  a.nred = static_cast<int>(nred);
  // When every reducing workgroup holds at most one piece, the instance that
  // holds one (the same arithmetic; room to load a whole piece's state while
  // the norm is pending), provided as many of its workgroups are resident.
  const void* run = kernel;
  if (tiles <= nred_max) {
    int max1 = 0;
    if (fused_max_grid(kernel1, &max1) == GRZ_OK && grid <= max1) run = kernel1;
  }
  a.master = master;
  a.m = m;
  a.v = v;
  a.mean_out = mean_out;
  a.partials = piece_sqnorm;
  a.ctl = static_cast<unsigned*>(workspace);
  a.slots = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kCtlBytes);
  a.lslots = a.slots + npieces;
  a.total = a.lslots + (npieces > kReduceFan ? ceil_div(npieces, kReduceFan) : 0);
  a.sqnorm_out = sqnorm_out;
  a.scale_out = clip_scale_out;
  a.max_norm = max_norm;
  a.divisor = static_cast<double>(nranks);
  a.pow2 = (nranks & (nranks - 1)) == 0;
  a.ntiles = tiles;
  a.npieces = npieces;
  a.nranks = nranks;
  a.nrep = nreplicas;
  a.nsegs = nsegs;
  if (next.table != nullptr) {
    a.next = next;
  } else if (flags & GRZ_ARGS_DEVICE) {
    a.dargs = args;
  } else {
    a.lr = args->lr;
    a.b1 = args->beta1;
    a.b2 = args->beta2;
    a.eps = args->eps;
    a.wd = args->weight_decay;
    a.bc1 = args->bias_corr1;
    a.bc2 = args->bias_corr2;
  }
  void* params[] = {&a};
  // The grid is what the occupancy allows resident at once, so on a device
  // that runs nothing else every workgroup is dispatched at once; the waits
  // are bounded besides, so a grid that is not resident ends with the flag
  // up rather than waiting for ever.  A cooperative launch has HIP guarantee
  // residency, at a cost (MI355X: 147 against 130 us per launch at the GPT-2
  // 124M one-rank share, 41 against 24 us at the char GPT).
  const hipError_t e =
      (flags & GRZ_COOPERATIVE)
          ? hipLaunchCooperativeKernel(run, dim3(grid), dim3(kThreads), params, 0, stream)
          : hipLaunchKernel(run, dim3(grid), dim3(kThreads), params, 0, stream);
  return e == hipSuccess ? GRZ_OK : GRZ_EHIP;
}

}  // namespace

extern "C" {

int64_t zero1_fused_capacity(int nranks, int dtype) {
  if (nranks < 1 || nranks > GRZ_MAX_RANKS) return -GRZ_EINVAL;
  const void* kernel = fused_kernel_for(dtype, nranks);
  if (kernel == nullptr) return -GRZ_EINVAL;
  int grid = 0;
  const int st = fused_max_grid(kernel, &grid);
  if (st != GRZ_OK) return -st;
  return static_cast<int64_t>(grid - 1) * kFusedPieces;  // one workgroup folds the norm
}

}  // extern "C"

namespace {

int fused_entry(const void* const* rank_grads, int nranks, int dtype,
                const grz_bucket* buckets, int nbuckets, int chunk, int flags, float* master,
                float* m, float* v, const grz_adamw_args* args, const StepArgsNext& next,
                double max_norm, uint16_t* const* replicas, int nreplicas,
                double* piece_sqnorm, void* workspace, double* sqnorm_out,
                float* clip_scale_out, float* mean_out, hipStream_t stream) {
  if (flags & ~(GRZ_UNEVEN | GRZ_IN_COMPACT | GRZ_ARGS_DEVICE | GRZ_COOPERATIVE))
    return GRZ_EINVAL;
  int st = check_plan(buckets, nbuckets, nranks, chunk,
                      flags & ~(GRZ_ARGS_DEVICE | GRZ_COOPERATIVE));
  if (st != GRZ_OK) return st;
  if ((flags & GRZ_IN_COMPACT) && chunk < 0) return GRZ_EINVAL;
  const void* kernel = fused_kernel_for(dtype, nranks);
  const void* kernel1 = fused_kernel_for(dtype, nranks, true);
  if (kernel == nullptr || kernel1 == nullptr) return GRZ_EINVAL;
  if (rank_grads == nullptr || master == nullptr || m == nullptr || v == nullptr ||
      args == nullptr || piece_sqnorm == nullptr || workspace == nullptr)
    return GRZ_EINVAL;
  for (int j = 0; j < nranks; ++j)
    if (rank_grads[j] == nullptr) return GRZ_EINVAL;
  if (nreplicas < 0 || nreplicas > GRZ_MAX_RANKS) return GRZ_EINVAL;
  if (nreplicas > 0 && replicas == nullptr) return GRZ_EINVAL;
  for (int r = 0; r < nreplicas; ++r) {
    if (replicas[r] == nullptr) return GRZ_EINVAL;
    if (!aligned(replicas[r], 2)) return GRZ_EALIGN;
  }
  if (!aligned(master, 4) || !aligned(m, 4) || !aligned(v, 4) || !aligned(mean_out, 4) ||
      !aligned(piece_sqnorm, 8) || !aligned(workspace, 8) || !aligned(sqnorm_out, 8) ||
      !aligned(clip_scale_out, 4) || !aligned(args, 4))
    return GRZ_EALIGN;
  const int64_t npieces = dp_piece_count(buckets, nbuckets, nranks, flags & GRZ_UNEVEN);
  if (npieces < 0) return static_cast<int>(-npieces);
  if (npieces > static_cast<int64_t>(kReduceFan) * kReduceFan) return GRZ_ERANGE;
  std::vector<PlanSeg> ps = plan_segments(buckets, nbuckets, nranks, chunk);
  if (ps.size() > static_cast<size_t>(kFusedSegs)) return GRZ_ERANGE;
  if (dtype == GRZ_BF16)
    return fused_launch<uint16_t>(kernel, kernel1, rank_grads, nranks, ps, flags, master, m, v,
                                  args, next, max_norm, replicas, nreplicas, piece_sqnorm,
                                  npieces, workspace, sqnorm_out, clip_scale_out, mean_out,
                                  stream);
  return fused_launch<float>(kernel, kernel1, rank_grads, nranks, ps, flags, master, m, v, args,
                             next, max_norm, replicas, nreplicas, piece_sqnorm, npieces,
                             workspace, sqnorm_out, clip_scale_out, mean_out, stream);
}

}  // namespace

extern "C" {

int zero1_fused_step(const void* const* rank_grads, int nranks, int dtype,
                     const grz_bucket* buckets, int nbuckets, int chunk, int flags,
                     float* master, float* m, float* v, const grz_adamw_args* args,
                     double max_norm, uint16_t* const* replicas, int nreplicas,
                     double* piece_sqnorm, void* workspace, double* sqnorm_out,
                     float* clip_scale_out, float* mean_out, hipStream_t stream) {
  return fused_entry(rank_grads, nranks, dtype, buckets, nbuckets, chunk, flags, master, m, v,
                     args, StepArgsNext{}, max_norm, replicas, nreplicas, piece_sqnorm,
                     workspace, sqnorm_out, clip_scale_out, mean_out, stream);
}

int zero1_fused_step_args(const void* const* rank_grads, int nranks, int dtype,
                          const grz_bucket* buckets, int nbuckets, int chunk, int flags,
                          float* master, float* m, float* v, const grz_adamw_args* table,
                          int64_t count, int64_t* counter, grz_adamw_args* current,
                          double max_norm, uint16_t* const* replicas, int nreplicas,
                          double* piece_sqnorm, void* workspace, double* sqnorm_out,
                          float* clip_scale_out, float* mean_out, hipStream_t stream) {
  if (flags & GRZ_ARGS_DEVICE) return GRZ_EINVAL;  // implied
  const int st = check_step_args(table, count, counter, current);
  if (st != GRZ_OK) return st;
  return fused_entry(rank_grads, nranks, dtype, buckets, nbuckets, chunk, flags, master, m, v,
                     table, StepArgsNext{table, count, counter, current}, max_norm, replicas,
                     nreplicas, piece_sqnorm, workspace, sqnorm_out, clip_scale_out, mean_out,
                     stream);
}

}  // extern "C"
