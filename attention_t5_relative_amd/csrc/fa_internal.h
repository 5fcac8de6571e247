// Internal launch descriptors shared by the C-ABI glue (api.cpp) and the
// kernel translation units.  Nothing here is part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace fa {

constexpr int kMaxThresholds = 128;   // (buckets per side) - (exact buckets) - 1 <= 127
constexpr int kMaxDistance = 1024;    // bounds the per-distance bias table in LDS
constexpr int kMaxSeqlen = 65536;
constexpr int kMaxDenseSeqlen = 16384; // a dense bias matrix (and its fp32 gradient) < 2^32 bytes

// T5 bucket boundaries for one (num_buckets, max_distance, bidirectional).
// For n >= me, bucket(n) = me + #{k : thr[k] <= n}; `sat` is the first n of
// the last bucket of a side (every n >= sat shares that bucket).
struct T5Geometry {
  int32_t nbp;        // buckets per side
  int32_t me;         // exact buckets per side (nbp / 2)
  int32_t sat;        // first saturated distance
  int32_t nthr;       // number of thresholds (nbp - me - 1)
  int32_t bidir;
  int32_t thr[kMaxThresholds];
};

enum BiasKind : int32_t {
  kBiasNone = 0,
  kBiasT5 = 1,
  kBiasAlibi = 2,
  kBiasDense = 3,
  kBiasFire = 4
};

// FIRE.  The bias b_h(x) = b2_h + sum_k w2_hk relu(w1_k x + b1_k) of the
// normalised distance x is piecewise linear in x: on each segment between
// consecutive kinks -b1_k / w1_k inside (0, 1) the set of active units is
// fixed and b_h = A_hs + B_hs x.  fire_setup_kernel (fire.hip) writes the
// segment table, fp32 words:
//   [0] m (kinks inside (0, 1), int bits), [2] c, [3] L
//   [kFireOffT + s]    t_s, s = 1 .. kFireTEnd - 1: the kinks t_1 <= .. <= t_m,
//                      then +inf
//   per head h at kFireShared + h * kFireHeadStride: A_hs * log2(e) at
//   [s], B_hs * log2(e) at [66 + s], s = 0 .. m
// The segment of x (the number of kinks <= x) comes from a branch-free binary
// search over t_1 .. t_127 (seven steps).
constexpr int kFireMaxHidden = 64;
constexpr int kFireSegs = kFireMaxHidden + 1;
constexpr int kFireOffT = 8;
constexpr int kFireTEnd = 128;                    // t_s stored for s < kFireTEnd
constexpr int kFireShared = 144;
constexpr int kFireHeadStride = 132;
constexpr int kFireOffA = kFireShared;            // in a workgroup's LDS copy
constexpr int kFireOffB = kFireShared + 66;
constexpr int kFireLds = kFireShared + kFireHeadStride;
constexpr int kFireTerms = 5;                     // gradient sums per (head, segment)
constexpr int kFireGradRows = kFireTerms * kFireSegs;
static_assert(kFireOffT + kFireTEnd <= kFireShared, "FIRE table layout");
// FIRE distance table (fire_dist_kernel): psi(d) = log2(c d + 1) at
// [kFireDistPad + d] and d / (c d + 1) at [n + kFireDistPad + d],
// n = maxlen + 2 kFireDistPad, for 0 <= d < maxlen + kFireDistPad and zero
// for d < 0: the kernels read a tile's distances, down to -127 (keys after
// the query near the diagonal) and up to maxlen + 126 (rows past a ragged
// end), with no range test.
constexpr int kFireDistPad = 128;
__host__ __device__ inline size_t fire_dist_floats(int maxlen) {
  return 2 * ((size_t)maxlen + 2 * kFireDistPad);
}
__host__ __device__ inline size_t fire_tab_floats(int heads) {
  return (size_t)kFireShared + (size_t)kFireHeadStride * heads;
}
__host__ __device__ inline int fire_theta_floats(int heads, int hidden) {
  return 2 * hidden + heads * hidden + heads + 2;
}

// One attention problem, dense or packed, as the kernels see it.
struct Problem {
  int32_t varlen;       // 0 dense [B,S,H,D], 1 packed [T,H,D]
  int32_t nbatch;       // dense B, packed nseq
  int32_t seqlen;       // dense S, packed max_seqlen
  int32_t total;        // packed T (dense: B*S)
  int32_t heads;
  int32_t head_dim;
  int32_t causal;
  float scale;
  float rope_base;      // 0: none
  int32_t bias;         // BiasKind
  const int32_t *cu_seqlens;
  const float *table;
  const float *slopes;
  const uint16_t *dense;  // bf16 [dense_batch, H, S, S] (kBiasDense)
  int32_t dense_batch;    // 1 (shared by the batch) or nbatch
  int32_t fire_hidden;    // kBiasFire: hidden units K (table = theta)
  T5Geometry t5;
};

struct FwdBuffers {
  const void *q, *k, *v;   // bf16; k already rotated when RoPE is on
  void *o;
  float *lse;
  const double2 *rope_cs;   // RoPE fp64 (cos, sin) table [seqlen, D/2] or nullptr
  const float *fire_tab;    // FIRE segment table or nullptr
  const float *fire_dist;   // FIRE distance table or nullptr
};

struct BwdBuffers {
  const void *q, *k, *v;   // bf16 (q, k rotated when RoPE is on)
  const void *o;           // bf16 forward output (centres the dq accumulation)
  const void *dout;
  const float *lse;
  const float *dlse;       // gradient with respect to lse (same layout) or nullptr
  void *dq, *dk, *dv;      // bf16 outputs
  const double2 *rope_cs;   // RoPE fp64 (cos, sin) table [seqlen, D/2] or nullptr
  float *delta;            // fp32, two lse-layout arrays: -D, then -lse / scale
  float *part;             // fp32 [num_buckets, parts] (T5 table gradient) or nullptr
  float *dtable;           // [num_buckets, H] or nullptr
  float *dbias;            // dense bias gradient fp32 [B, H, S, S] written per batch, or nullptr
  float *dbias_shared;     // dense bias gradient fp32 [1, H, S, S] summed over B > 1, or nullptr
  const float *fire_tab;   // FIRE segment table or nullptr
  const float *fire_dist;  // FIRE distance table or nullptr
  float *fire_g;           // FIRE: reduced gradient sums [kFireGradRows, H] or nullptr
};

// Launchers (return the first HIP error, hipSuccess otherwise).
int fwd_tile_rows(int head_dim);
hipError_t launch_fwd_impl(const Problem &p, const FwdBuffers &b, const int4 *sched, int nsched,
                           hipStream_t s);
// Packed-batch schedule: entries for `total` tokens in `nseq` sequences
// (a multiple of 8; see sched_kernel) and the int32 scratch it needs.
int sched_entries(int total, int nseq, int heads, int tile);
int sched_prefix_ints(int nseq);
hipError_t launch_sched(const int32_t *cu, int nseq, int heads, int tile, int nentries,
                        int32_t *prefix, int4 *sched, hipStream_t s);
// RoPE: cs[t][p] = (cos, sin) of t * base^(-2p/D) for t < p.seqlen (dense S,
// packed max_seqlen), fp64 [seqlen, D/2] pairs; and rotation of one or two
// bf16 [tokens, H, D] tensors (x1 / y1 may be nullptr).
hipError_t launch_rope_table(const Problem &p, double2 *cs, hipStream_t s);
hipError_t launch_rope_rotate(const Problem &p, const double2 *cs, const void *x0, void *y0,
                              const void *x1, void *y1, hipStream_t s);
int bwd_tile();
int64_t bwd_num_parts(const Problem &p, int nsched);
// dq, dkv, table-gradient reduction, FIRE gradient sums (between dkv and
// the reduction), the batch sum of a shared dense bias's gradient
enum BwdPhase { kBwdPre = 0, kBwdMain = 1, kBwdReduce = 2, kBwdFire = 3, kBwdDenseSum = 4 };
hipError_t launch_bwd_phase(const Problem &p, const BwdBuffers &b, const int4 *sched, int nsched,
                            int phase, hipStream_t s);
hipError_t launch_t5_buckets(const T5Geometry &g, int qlen, int klen, int32_t *out,
                             hipStream_t s);
hipError_t launch_fill_f32(float *p, size_t n, float v, hipStream_t s);
// FIRE (fire.hip): the segment table from theta, and d(theta) from the
// reduced per-(head, segment) gradient sums.
hipError_t launch_fire_setup(const Problem &p, float *tab, float *dist, hipStream_t s);
hipError_t launch_fire_grad(const Problem &p, const float *g, float *dtheta, hipStream_t s);
// MFMA throughput probe: kMfmaProbeBlocks x kMfmaProbeThreads lanes, each
// wave 4 chains x iters v_mfma_f32_32x32x16_bf16; sink holds one float per lane.
constexpr int kMfmaProbeBlocks = 2048;
constexpr int kMfmaProbeThreads = 256;
hipError_t launch_mfma_probe(float *sink, int iters, hipStream_t s);
// Dense bias gradient helper: zero the pairs with key > query of `count`
// [S, S] matrices (causal: the backward never visits most of them).
hipError_t launch_zero_upper(float *m, int count, int S, hipStream_t s);

// RMSNorm and cross-entropy (norm_loss.hip).  rmsnorm_bwd's dw partials are
// one fp32 row per workgroup: rmsnorm_bwd_grid(rows) * dim floats.
constexpr int kRmsMaxDim = 8192;
constexpr int kRmsBwdMaxGrid = 1024;
int rmsnorm_chunks_per_lane(int dim);
int rmsnorm_bwd_grid(int rows);
hipError_t launch_rmsnorm_fwd(const void *x, const void *w, void *y, float *rstd, int rows,
                              int dim, float eps, hipStream_t s);
hipError_t launch_rmsnorm_bwd(const void *x, const void *w, const float *rstd, const void *dy,
                              void *dx, float *dw, float *part, int rows, int dim,
                              hipStream_t s);
hipError_t launch_rmsnorm_dw(const float *part, float *dw, int rows, int dim, hipStream_t s);
hipError_t launch_ce_fwd(const void *z, const int32_t *labels, float *loss, float *lse, int rows,
                         int vocab, float z_loss, int ignore, hipStream_t s);
hipError_t launch_ce_bwd(const void *z, const int32_t *labels, const float *lse,
                         const float *dloss, void *dz, int rows, int vocab, float z_loss,
                         int ignore, hipStream_t s);



}  // namespace fa
