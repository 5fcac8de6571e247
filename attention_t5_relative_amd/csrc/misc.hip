// Small kernels around the attention kernels: the packed-batch tile schedule,
// the RoPE angle table and rotation of whole q / k tensors, the T5 bucket
// test hook, a fill kernel and an MFMA throughput probe.
#include "fa_device.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// Packed batches: map every workgroup id to {token0, length, head, tile} so
// the attention kernels need a single load to find their work.
//
// Workgroup ids are dispatched to the 8 XCDs in turn, and the kernels give
// XCD x the contiguous range of entries [x per, (x + 1) per), per = n / 8
// (xcd_remap).  A sequence's work grows with its length squared, so handing
// out whole sequences in order would load the XCDs very unevenly.  Instead
// the (sequence, head) pairs go round-robin over the XCDs: pair s H + h to
// XCD (s H + h) mod 8.  All tiles of a pair stay on one XCD, so its K and V
// are reused from that XCD's L2.  Sequences are taken longest first (by
// tile count, ties in index order; up to kSortMax sequences, beyond that in
// index order), so each XCD starts its heaviest pairs first and the short
// ones fill the end.  Within an XCD the entries follow the sequences in that
// order, then the pair's heads, then its tiles, longest causal rows first.
//
// One workgroup.  A bitonic sort in LDS ranks the sequences.  For each XCD
// x, an exclusive scan over the ranks of (tiles) * (pairs on x) goes into
// prefix[x][rank]; then every entry finds its rank by binary search.
// Entries past an XCD's work get length -1.  n must be a multiple of 8 and
// per at least every XCD's count (sched_entries gives such an n).  The
// order decides only which workgroup computes what, never a result.
// ---------------------------------------------------------------------------
constexpr int SCHED_NT = 256;
constexpr int kSortMax = 2048;     // sequences ranked by length
constexpr int kSortIdxBits = 19;   // sort key: (4095 - tiles) << 19 | index

// pairs of sequence s on XCD x: heads h = r, r + 8, ... below H with
// r = (x - s H) mod 8
__device__ __forceinline__ int xcd_first_head(int s, int heads, int x) {
  return ((x - (int)(((long long)s * heads) & 7)) + 8) & 7;
}
__device__ __forceinline__ int xcd_pairs(int s, int heads, int x) {
  const int r = xcd_first_head(s, heads, x);
  return r < heads ? (heads - 1 - r) / 8 + 1 : 0;
}

__global__ __launch_bounds__(SCHED_NT) void sched_kernel(const int32_t *cu, int nseq, int heads,
                                                          int tile, int nentries, int32_t *prefix,
                                                          int4 *sched) {
  __shared__ int scan[SCHED_NT];
  __shared__ int order[kSortMax];
  const int tid = threadIdx.x;
  const bool ranked = nseq <= kSortMax;
  if (ranked) {
    int n2 = 1;
    while (n2 < nseq) n2 <<= 1;
    for (int i = tid; i < n2; i += SCHED_NT) {
      int key = 0x7fffffff;
      if (i < nseq) {
        const int nt = (cu[i + 1] - cu[i] + tile - 1) / tile;
        key = ((4095 - min(nt, 4095)) << kSortIdxBits) | i;
      }
      order[i] = key;
    }
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n2; i += SCHED_NT) {
          const int l = i ^ j;
          if (l > i) {
            const int a = order[i], b = order[l];
            if (((i & k) == 0) == (a > b)) {
              order[i] = b;
              order[l] = a;
            }
          }
        }
        __syncthreads();
      }
  }
  // sequence of rank r
  auto seq_of = [&](int r) { return ranked ? (order[r] & ((1 << kSortIdxBits) - 1)) : r; };
  for (int x = 0; x < 8; ++x) {
    int32_t *px = prefix + (size_t)x * (nseq + 1);
    int carry = 0;
    for (int c0 = 0; c0 < nseq; c0 += SCHED_NT) {
      const int s = c0 + tid;
      int cnt = 0;
      if (s < nseq) {
        const int q = seq_of(s);
        const int len = cu[q + 1] - cu[q];
        cnt = ((len + tile - 1) / tile) * xcd_pairs(s, heads, x);
      }
      scan[tid] = cnt;
      __syncthreads();
      for (int off = 1; off < SCHED_NT; off <<= 1) {
        const int add = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += add;
        __syncthreads();
      }
      if (s < nseq) px[s] = carry + scan[tid] - cnt;
      carry += scan[SCHED_NT - 1];
      __syncthreads();
    }
    if (tid == 0) px[nseq] = carry;
  }
  __syncthreads();
  __threadfence_block();
  const int per = nentries >> 3;
  for (int gidx = tid; gidx < nentries; gidx += SCHED_NT) {
    int4 e = {0, -1, 0, 0};
    const int x = gidx / per, local = gidx - x * per;
    const int32_t *px = prefix + (size_t)x * (nseq + 1);
    if (x < 8 && local < px[nseq]) {
      int lo = 0, hi = nseq - 1;   // last s with px[s] <= local
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (px[mid] <= local) lo = mid; else hi = mid - 1;
      }
      const int s = lo, q = seq_of(s);
      const int t0 = cu[q], len = cu[q + 1] - t0;
      const int nt = (len + tile - 1) / tile;
      const int k = local - px[s];
      const int j = k / nt;
      const int hh = xcd_first_head(s, heads, x) + 8 * j;
      const int t = nt - 1 - (k - j * nt);   // longest causal rows first
      e = int4{t0, len, hh, t};
    }
    sched[gidx] = e;
  }
}

// ---------------------------------------------------------------------------
// RoPE.  The pair (2p, 2p + 1) at position t turns by t * base^(-2p/D).
//
// rope_table_kernel writes cs[t][p] = (cos, sin) of that angle for every
// position t < npos, in fp64 (positions reach 65535, where an fp32 angle
// would already be off by ~4e-3 rad; and an fp32 cos / sin would move about
// one rotated value in 10^4 to the neighbouring bf16).  The attention kernels
// read it to rotate Q rows in registers and to rotate dQ and dK back in
// their epilogues.
//
// rope_rotate_kernel rotates whole tensors that the kernels stream through
// LDS (K in the forward, Q and K in the backward), one 16-byte chunk (four
// pairs) of one row per thread with the table's angles: exact in fp64 and
// rounded once to bf16, as a full-bf16 pipeline hands rotated operands to
// the kernels.
// ---------------------------------------------------------------------------
constexpr int ROPE_NT = 256;

__device__ __forceinline__ int token_position(int token, int seqlen, const int32_t *cu, int nseq) {
  if (cu == nullptr) return token % seqlen;
  int lo = 0, hi = nseq - 1;   // last s with cu[s] <= token
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= token) lo = mid; else hi = mid - 1;
  }
  return token - cu[lo];
}

__device__ __forceinline__ void rope_angle_cs(int pos, int p, int D, double log2base, double &c,
                                              double &s) {
  const double theta = exp2(-(2.0 * p / D) * log2base);
  sincos((double)pos * theta, &s, &c);
}

__global__ __launch_bounds__(ROPE_NT) void rope_table_kernel(double2 *cs, int npos, int D,
                                                              double log2base) {
  const int half = D / 2;
  const long long idx = (long long)blockIdx.x * ROPE_NT + threadIdx.x;
  if (idx >= (long long)npos * half) return;
  const int t = (int)(idx / half), p = (int)(idx - (long long)t * half);
  double c, s;
  rope_angle_cs(t, p, D, log2base, c, s);
  cs[idx] = double2{c, s};
}

__global__ __launch_bounds__(ROPE_NT) void rope_rotate_kernel(const i32x4 *x0, i32x4 *y0,
                                                               const i32x4 *x1, i32x4 *y1,
                                                               const double2 *cs, int tokens,
                                                               int heads, int D, int seqlen,
                                                               const int32_t *cu, int nseq) {
  // one thread per 16-byte chunk (4 pairs) of one (token, head) row
  const int chunks = D / 8;
  const long long idx = (long long)blockIdx.x * ROPE_NT + threadIdx.x;
  if (idx >= (long long)tokens * heads * chunks) return;
  const long long row = idx / chunks;
  const int c = (int)(idx - row * chunks);
  const int token = (int)(row / heads);
  const double2 *e = cs + (size_t)token_position(token, seqlen, cu, nseq) * (D / 2) + 4 * c;
  const double2 a0 = e[0], a1 = e[1], a2 = e[2], a3 = e[3];
  auto turn = [&](i32x4 w) {
    w[0] = (int)rope_rotate_pair((uint32_t)w[0], a0.x, a0.y);
    w[1] = (int)rope_rotate_pair((uint32_t)w[1], a1.x, a1.y);
    w[2] = (int)rope_rotate_pair((uint32_t)w[2], a2.x, a2.y);
    w[3] = (int)rope_rotate_pair((uint32_t)w[3], a3.x, a3.y);
    return w;
  };
  y0[idx] = turn(x0[idx]);
  if (x1 != nullptr) y1[idx] = turn(x1[idx]);
}

// ---------------------------------------------------------------------------
// T5 bucket test hook: the same clamp-then-threshold path the attention
// kernels use to fill their per-distance bias table.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void t5_buckets_kernel(const T5Geometry g, int qlen, int klen,
                                                          int32_t *out) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)qlen * klen) return;
  const int i = (int)(idx / klen), j = (int)(idx - (long long)i * klen);
  const int r = min(max(j - i, -g.sat), g.sat);
  out[idx] = t5_bucket_dev(r, g);
}

__global__ __launch_bounds__(256) void fill_kernel(float *p, size_t n, float v) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < n) p[idx] = v;
}

// ---------------------------------------------------------------------------
// MFMA throughput probe: every wave issues only v_mfma_f32_32x32x16_bf16 in
// four independent accumulator chains (no loads in the loop), so the chip's
// sustained bf16 matrix rate can be measured under the same clock and power
// limits as the attention kernels.  Operands are distinct non-trivial bf16
// values per lane; each lane stores one sum so the work cannot be dropped.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMfmaProbeThreads) void mfma_probe_kernel(float *sink, int iters) {
  const int t = (int)(blockIdx.x * kMfmaProbeThreads + threadIdx.x);
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + (float)((t * 7 + i) & 15) * 0.0625f);
    b[i] = (__bf16)(0.5f - (float)((t * 5 + 3 * i) & 15) * 0.03125f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(b, a, c1);
    c2 = mfma32(a, a, c2);
    c3 = mfma32(b, b, c3);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[t] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float *sink, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(kMfmaProbeBlocks), dim3(kMfmaProbeThreads), 0, s,
                     sink, iters);
  return hipGetLastError();
}

int sched_entries(int total, int nseq, int heads, int tile) {
  // every XCD holds at most ceil(H / 8) pairs of each sequence, and a
  // sequence of length L has at most L / tile + 1 tiles
  const long long per = (long long)((heads + 7) / 8) * ((total + tile - 1) / tile + nseq);
  return (int)(8 * per);
}

int sched_prefix_ints(int nseq) { return 8 * (nseq + 1); }

hipError_t launch_sched(const int32_t *cu, int nseq, int heads, int tile, int nentries,
                        int32_t *prefix, int4 *sched, hipStream_t s) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(SCHED_NT), 0, s, cu, nseq, heads, tile,
                     nentries, prefix, sched);
  return hipGetLastError();
}

hipError_t launch_rope_table(const Problem &p, double2 *cs, hipStream_t s) {
  const int npos = p.seqlen;
  const long long n = (long long)npos * (p.head_dim / 2);
  if (n == 0) return hipSuccess;
  const int grid = (int)((n + ROPE_NT - 1) / ROPE_NT);
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid), dim3(ROPE_NT), 0, s, cs, npos, p.head_dim,
                     log2((double)p.rope_base));
  return hipGetLastError();
}

hipError_t launch_rope_rotate(const Problem &p, const double2 *cs, const void *x0, void *y0,
                              const void *x1, void *y1, hipStream_t s) {
  const int tokens = p.varlen ? p.total : p.nbatch * p.seqlen;
  const long long n = (long long)tokens * p.heads * (p.head_dim / 8);
  if (n == 0) return hipSuccess;
  const int grid = (int)((n + ROPE_NT - 1) / ROPE_NT);
  hipLaunchKernelGGL(rope_rotate_kernel, dim3(grid), dim3(ROPE_NT), 0, s,
                     static_cast<const i32x4 *>(x0), static_cast<i32x4 *>(y0),
                     static_cast<const i32x4 *>(x1), static_cast<i32x4 *>(y1), cs, tokens,
                     p.heads, p.head_dim, p.seqlen, p.varlen ? p.cu_seqlens : nullptr, p.nbatch);
  return hipGetLastError();
}

hipError_t launch_t5_buckets(const T5Geometry &g, int qlen, int klen, int32_t *out,
                             hipStream_t s) {
  const long long n = (long long)qlen * klen;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(t5_buckets_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g,
                     qlen, klen, out);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float *p, size_t n, float v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// One workgroup per matrix row (row r of matrix r / S): zero the entries
// with column > row.
__global__ __launch_bounds__(256) void zero_upper_kernel(float *m, int S) {
  const size_t row = blockIdx.x;
  const int i = (int)(row % (size_t)S);
  float *r = m + row * (size_t)S;
  for (int j = i + 1 + (int)threadIdx.x; j < S; j += 256) r[j] = 0.f;
}

hipError_t launch_zero_upper(float *m, int count, int S, hipStream_t s) {
  const size_t rows = (size_t)count * S;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_upper_kernel, dim3((unsigned)rows), dim3(256), 0, s, m, S);
  return hipGetLastError();
}

}  // namespace fa
