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
// each element costs a log2 (x), a segment lookup and one fma.  This file
// holds the two small single-workgroup kernels around them:
//
//   fire_setup_kernel  theta -> the segment table (layout in fa_internal.h):
//                      sorted kinks and A, B per (head, segment);
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

// Kinks inside (0, 1), sorted ascending (ties by unit index), into
// tk[1 .. m] (fp64, LDS); returns m.  All threads of the workgroup call it.
__device__ int fire_kinks(const float *theta, int K, double *tk) {
  const int tid = threadIdx.x;
  bool valid = false;
  double t = 0.0;
  if (tid < K) {
    const double w = theta[tid], b = theta[K + tid];
    if (w != 0.0) {
      t = -b / w;
      valid = t > 0.0 && t < 1.0;
    }
  }
  const int m = __syncthreads_count(valid);
  if (valid) {
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const double wj = theta[j], bj = theta[K + j];
      if (wj == 0.0) continue;
      const double tj = -bj / wj;
      if (!(tj > 0.0 && tj < 1.0)) continue;
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

__global__ __launch_bounds__(FT) void fire_setup_kernel(const float *theta, int H, int K,
                                                         float *tab) {
  __shared__ double tk[kFireSegs + 1];
  const int tid = threadIdx.x;
  const int m = fire_kinks(theta, K, tk);
  const int n = fire_theta_floats(H, K);
  for (int i = tid; i < kFireTEnd; i += FT)
    tab[kFireOffT + i] = i == 0 ? -INFINITY : (i <= m ? (float)tk[i] : INFINITY);
  // A, B (log2 units) per (head, segment)
  const float *w1 = theta, *b1 = theta + K, *w2 = theta + 2 * K, *b2 = theta + 2 * K + H * K;
  for (int i = tid; i < H * kFireSegs; i += FT) {
    const int h = i / kFireSegs, s = i - h * kFireSegs;
    double A = 0.0, B = 0.0;
    if (s <= m) {
      const double xs = fire_mid(tk, m, s);
      A = b2[h];
      for (int k = 0; k < K; ++k)
        if ((double)w1[k] * xs + (double)b1[k] > 0.0) {
          A += (double)w2[h * K + k] * b1[k];
          B += (double)w2[h * K + k] * w1[k];
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
  __shared__ double tk[kFireSegs + 1];
  __shared__ double xs[kFireSegs];
  __shared__ double red[2][FT];
  const int tid = threadIdx.x;
  const int m = fire_kinks(theta, K, tk);
  for (int s = tid; s <= m; s += FT) xs[s] = fire_mid(tk, m, s);
  __syncthreads();
  const float *w1 = theta, *b1 = theta + K, *w2 = theta + 2 * K;
  const int n = fire_theta_floats(H, K);
  const double c = theta[n - 2], L = theta[n - 1];
  auto G = [&](int s, int q, int h) { return (double)g[(size_t)(s * kFireTerms + q) * H + h]; };
  auto act = [&](int s, int k) { return (double)w1[k] * xs[s] + (double)b1[k] > 0.0; };
  // dw2 [H, K] and db2 [H]
  for (int i = tid; i < H * K; i += FT) {
    const int h = i / K, k = i - h * K;
    double t = 0.0;
    for (int s = 0; s <= m; ++s)
      if (act(s, k)) t += (double)b1[k] * G(s, 0, h) + (double)w1[k] * G(s, 1, h);
    dtheta[2 * K + i] = (float)t;
  }
  for (int h = tid; h < H; h += FT) {
    double t = 0.0;
    for (int s = 0; s <= m; ++s) t += G(s, 0, h);
    dtheta[2 * K + H * K + h] = (float)t;
  }
  // dw1, db1 [K]
  for (int k = tid; k < K; k += FT) {
    double t1 = 0.0, t0 = 0.0;
    for (int h = 0; h < H; ++h) {
      double s1 = 0.0, s0 = 0.0;
      for (int s = 0; s <= m; ++s)
        if (act(s, k)) {
          s1 += G(s, 1, h);
          s0 += G(s, 0, h);
        }
      t1 += (double)w2[h * K + k] * s1;
      t0 += (double)w2[h * K + k] * s0;
    }
    dtheta[k] = (float)t1;
    dtheta[K + k] = (float)t0;
  }
  // dc, dL: per-thread partials over heads, then a fixed-order tree
  double pc = 0.0, pl = 0.0;
  for (int h = tid; h < H; h += FT)
    for (int s = 0; s <= m; ++s) {
      double B = 0.0;
      for (int k = 0; k < K; ++k)
        if (act(s, k)) B += (double)w2[h * K + k] * w1[k];
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

}  // namespace

hipError_t launch_fire_setup(const Problem &p, float *tab, hipStream_t s) {
  hipLaunchKernelGGL(fire_setup_kernel, dim3(1), dim3(FT), 0, s, p.table, p.heads, p.fire_hidden,
                     tab);
  return hipGetLastError();
}

hipError_t launch_fire_grad(const Problem &p, const float *g, float *dtheta, hipStream_t s) {
  hipLaunchKernelGGL(fire_grad_kernel, dim3(1), dim3(FT), 0, s, p.table, p.heads, p.fire_hidden,
                     g, dtheta);
  return hipGetLastError();
}

}  // namespace fa
