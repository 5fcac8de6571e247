// FIRE positional bias (functional interpolation for relative positions; the
// FAT5 report lists it among the encodings its kernels serve, note under
// "Noyau CUDA", and cites Li et al. for it).  For causal attention, query i
// and key j <= i:
//
//   x_ij = log(c (i - j) + 1) / log(c max(L, i) + 1)        in [0, 1]
//   b_hij = b2_h + sum_k w2_hk relu(w1_k x_ij + b1_k)
//
// theta = [w1 (K), b1 (K), w2 (H x K), b2 (H), c, L], fp32 on the device.
//
// A one-input ReLU network is piecewise linear: between consecutive kinks
// t_k = -b1_k / w1_k the active units are fixed, so b_h = A_hs + B_hs x on
// segment s.  The attention kernels therefore never evaluate the network:
// each element costs a table read (x), a segment lookup and one fma.  This
// file holds the small kernels around them:
//
//   fire_setup_kernel  theta -> the segment table (layout in fa_internal.h):
//                      sorted kinks and A, B per (head, segment);
//   fire_dist_kernel   psi(d) = log2(c d + 1) and d / (c d + 1) per distance:
//                      the kernels read x = psi(i - j) / log2(c max(L, i) + 1)
//                      from it, with no logarithm per element;
//   fire_grad_kernel   per-(head, segment) gradient sums -> d(theta).
//
// Gradient sums (accumulated by the dK/dV kernel over every visible pair of
// the segment, dS = dL/dS'):
//   G0 = sum dS            G1 = sum dS x           G2 = sum dS (d / e) / log2(E)
//   G3 = sum dS x w_i      G4 = sum over rows i < L of dS x
// with d = i - j, e = c d + 1, E = c max(L, i) + 1, w_i = max(L, i) / (E ln E).
// Then, with act(s, k) the units active on segment s:
//   db2_h   = sum_s G0_hs
//   dw2_hk  = sum_{s: act} (b1_k G0_hs + w1_k G1_hs)
//   db1_k   = sum_h w2_hk sum_{s: act} G0_hs,    dw1_k = sum_h w2_hk sum_{s: act} G1_hs
//   dc      = sum_hs B_hs (log2(e) G2_hs - G3_hs)          [dx/dc = (d/e - x m/E) / ln E]
//   dL      = -c / ((c L + 1) ln(c L + 1)) sum_hs B_hs G4_hs   [dx/dL on rows i < L]
#include "fa_device.h"

namespace fa {
namespace {

constexpr int FT = 256;

// theta up to b2 (w1, b1, w2, b2: 2K + HK + H floats) is copied to LDS once;
// every loop below reads it from there.
constexpr int kFireMaxHeadsLds = 256;   // heads whose w2 rows fit the LDS copy

// Kinks inside (0, 1), sorted ascending (ties by unit index), into
// tk[1 .. m] (fp64, LDS); returns m.  All threads of the workgroup call it.
// Each unit's kink is divided out once into tv (LDS; units without a kink
// in (0, 1) hold 2), then ranked against the others.
__device__ int fire_kinks(const float *w1, const float *b1, int K, double *tk, double *tv) {
  const int tid = threadIdx.x;
  bool valid = false;
  double t = 0.0;
  if (tid < K) {
    if (w1[tid] != 0.f) {
      t = -(double)b1[tid] / (double)w1[tid];
      valid = t > 0.0 && t < 1.0;
    }
    tv[tid] = valid ? t : 2.0;
  }
  const int m = __syncthreads_count(valid);
  if (valid) {
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const double tj = tv[j];
      rank += (tj < t || (tj == t && j < tid)) ? 1 : 0;
    }
    tk[rank + 1] = t;
  }
  __syncthreads();
  return m;
}

// A point inside segment s of [0, 1] cut at tk[1 .. m] (its midpoint).
__device__ __forceinline__ double fire_mid(const double *tk, int m, int s) {
  const double lo = s == 0 ? 0.0 : tk[s];
  const double hi = s == m ? 1.0 : tk[s + 1];
  return 0.5 * (lo + hi);
}

// Shared set-up of both kernels: theta's w1, b1 (and w2 when it fits) in
// LDS, the sorted kinks, and act[s] = the units active on segment s (bit k).
struct FireSmem {
  float w1[kFireMaxHidden], b1[kFireMaxHidden];
  float w2[kFireMaxHeadsLds * kFireMaxHidden];
  double tk[kFireSegs + 1];
  double tv[kFireMaxHidden];
  uint64_t act[kFireSegs];
};

__device__ int fire_prepare(const float *theta, int H, int K, FireSmem &sm) {
  const int tid = threadIdx.x;
  for (int i = tid; i < K; i += FT) {
    sm.w1[i] = theta[i];
    sm.b1[i] = theta[K + i];
  }
  if (H <= kFireMaxHeadsLds)
    for (int i = tid; i < H * K; i += FT) sm.w2[i] = theta[2 * K + i];
  __syncthreads();
  const int m = fire_kinks(sm.w1, sm.b1, K, sm.tk, sm.tv);
  for (int s = tid; s <= m; s += FT) {
    const double xs = fire_mid(sm.tk, m, s);
    uint64_t bits = 0;
    for (int k = 0; k < K; ++k)
      if ((double)sm.w1[k] * xs + (double)sm.b1[k] > 0.0) bits |= 1ull << k;
    sm.act[s] = bits;
  }
  __syncthreads();
  return m;
}

__device__ __forceinline__ float fire_w2(const FireSmem &sm, const float *theta, int H, int K,
                                         int h, int k) {
  return H <= kFireMaxHeadsLds ? sm.w2[h * K + k] : theta[2 * K + h * K + k];
}

__global__ __launch_bounds__(FT) void fire_setup_kernel(const float *theta, int H, int K,
                                                         float *tab) {
  __shared__ FireSmem sm;
  const int tid = threadIdx.x;
  const int m = fire_prepare(theta, H, K, sm);
  const int n = fire_theta_floats(H, K);
  for (int i = tid; i < kFireTEnd; i += FT)
    tab[kFireOffT + i] = i == 0 ? -INFINITY : (i <= m ? (float)sm.tk[i] : INFINITY);
  // A, B (log2 units) per (head, segment)
  const float *b2 = theta + 2 * K + H * K;
  for (int i = tid; i < H * kFireSegs; i += FT) {
    const int h = i / kFireSegs, s = i - h * kFireSegs;
    double A = 0.0, B = 0.0;
    if (s <= m) {
      A = b2[h];
      const uint64_t bits = sm.act[s];
      for (int k = 0; k < K; ++k)
        if ((bits >> k) & 1) {
          const double w = fire_w2(sm, theta, H, K, h, k);
          A += w * sm.b1[k];
          B += w * sm.w1[k];
        }
    }
    float *ph = tab + kFireShared + (size_t)h * kFireHeadStride;
    ph[s] = (float)(A * 1.4426950408889634);
    ph[66 + s] = (float)(B * 1.4426950408889634);
  }
  if (tid == 0) {
    tab[0] = __int_as_float(m);
    tab[1] = 0.f;
    tab[2] = theta[n - 2];
    tab[3] = theta[n - 1];
  }
}

// g: the reduced sums, row (s * kFireTerms + q) of [kFireGradRows, H].
__global__ __launch_bounds__(FT) void fire_grad_kernel(const float *theta, int H, int K,
                                                        const float *g, float *dtheta) {
  __shared__ FireSmem sm;
  __shared__ double red[2][FT];
  const int tid = threadIdx.x;
  const int m = fire_prepare(theta, H, K, sm);
  const int n = fire_theta_floats(H, K);
  const double c = theta[n - 2], L = theta[n - 1];
  auto G = [&](int s, int q, int h) { return (double)g[(size_t)(s * kFireTerms + q) * H + h]; };
  // dw2 [H, K]: b1_k G0 + w1_k G1 over the segments where unit k is active
  for (int i = tid; i < H * K; i += FT) {
    const int h = i / K, k = i - h * K;
    double t = 0.0;
    for (int s = 0; s <= m; ++s)
      if ((sm.act[s] >> k) & 1) t += (double)sm.b1[k] * G(s, 0, h) + (double)sm.w1[k] * G(s, 1, h);
    dtheta[2 * K + i] = (float)t;
  }
  // db2 [H]
  for (int h = tid; h < H; h += FT) {
    double t = 0.0;
    for (int s = 0; s <= m; ++s) t += G(s, 0, h);
    dtheta[2 * K + H * K + h] = (float)t;
  }
  // dw1, db1 [K]: sum over heads of w2_hk times the same segment sums.
  // Thread (g, k), g < NG = FT / K, takes the heads h = g (mod NG); the NG
  // partials of each unit are then added in g order (a fixed order).
  const int NG = FT / K;
  {
    const int k = tid % K, grp = tid / K;
    double t1 = 0.0, t0 = 0.0;
    if (grp < NG)
      for (int h = grp; h < H; h += NG) {
        double s1 = 0.0, s0 = 0.0;
        for (int s = 0; s <= m; ++s)
          if ((sm.act[s] >> k) & 1) {
            s1 += G(s, 1, h);
            s0 += G(s, 0, h);
          }
        const double w = fire_w2(sm, theta, H, K, h, k);
        t1 += w * s1;
        t0 += w * s0;
      }
    red[0][tid] = t1;
    red[1][tid] = t0;
  }
  __syncthreads();
  for (int k = tid; k < K; k += FT) {
    double t1 = 0.0, t0 = 0.0;
    for (int grp = 0; grp < NG; ++grp) {
      t1 += red[0][grp * K + k];
      t0 += red[1][grp * K + k];
    }
    dtheta[k] = (float)t1;
    dtheta[K + k] = (float)t0;
  }
  __syncthreads();   // red is reused below
  // dc, dL: one (head, segment) pair per thread and step, then a
  // fixed-order tree
  double pc = 0.0, pl = 0.0;
  for (int i = tid; i < H * (m + 1); i += FT) {
    const int h = i / (m + 1), s = i - h * (m + 1);
    double B = 0.0;
    const uint64_t bits = sm.act[s];
    for (int k = 0; k < K; ++k)
      if ((bits >> k) & 1) B += (double)fire_w2(sm, theta, H, K, h, k) * sm.w1[k];
    pc += B * (1.4426950408889634 * G(s, 2, h) - G(s, 3, h));
    pl += B * G(s, 4, h);
  }
  red[0][tid] = pc;
  red[1][tid] = pl;
  __syncthreads();
  for (int st = FT / 2; st > 0; st >>= 1) {
    if (tid < st) {
      red[0][tid] += red[0][tid + st];
      red[1][tid] += red[1][tid + st];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double EL = c * L + 1.0;
    dtheta[n - 2] = (float)red[0][0];
    dtheta[n - 1] = (float)(-c / (EL * log(EL)) * red[1][0]);
  }
}

// The distance table (layout in fa_internal.h), in fp64 and rounded once.
__global__ __launch_bounds__(FT) void fire_dist_kernel(const float *theta, int H, int K,
                                                        int maxlen, float *dist) {
  const int n = maxlen + 2 * kFireDistPad;
  const int idx = blockIdx.x * FT + threadIdx.x;
  if (idx >= 2 * n) return;
  const double c = theta[fire_theta_floats(H, K) - 2];
  const int half = idx >= n ? 1 : 0;
  const int d = idx - half * n - kFireDistPad;
  // d past the last distance (rows beyond a ragged end) keeps the formula,
  // so x stays monotone along a row of keys or a column of rows; d < 0
  // (keys after the query) reads 0
  double v = 0.0;
  if (d >= 0) v = half ? d / fma(c, (double)d, 1.0) : log2(fma(c, (double)d, 1.0));
  dist[idx] = (float)v;
}

}  // namespace

hipError_t launch_fire_setup(const Problem &p, float *tab, float *dist, hipStream_t s) {
  hipLaunchKernelGGL(fire_setup_kernel, dim3(1), dim3(FT), 0, s, p.table, p.heads, p.fire_hidden,
                     tab);
  const int n = 2 * (p.seqlen + 2 * kFireDistPad);
  hipLaunchKernelGGL(fire_dist_kernel, dim3((n + FT - 1) / FT), dim3(FT), 0, s, p.table, p.heads,
                     p.fire_hidden, p.seqlen, dist);
  return hipGetLastError();
}

hipError_t launch_fire_grad(const Problem &p, const float *g, float *dtheta, hipStream_t s) {
  hipLaunchKernelGGL(fire_grad_kernel, dim3(1), dim3(FT), 0, s, p.table, p.heads, p.fire_hidden,
                     g, dtheta);
  return hipGetLastError();
}

}  // namespace fa
