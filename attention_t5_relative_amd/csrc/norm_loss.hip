// RMSNorm and cross-entropy with z-loss for gfx950: the report's two other
// fused kernels (FAT5 report, section on the Triton kernels: the RMSNorm
// layer of Zhang & Sennrich and the cross-entropy loss with the z-loss of de
// Brebisson & Vincent; benchmarks under "Torch vs Triton").  Both are bound
// by HBM bandwidth: one pass over the data forward, one backward, 16-byte
// loads and stores through range-checked buffer resources, fp32 arithmetic.
//
// RMSNorm: y = x / sqrt(mean x^2 + eps) * w per row; backward
//   r = rstd, g = dy w, dx = r (g - x r^2 sum(g x) / d), dw = sum_rows dy x r.
// Cross-entropy: lse = log sum exp z, loss = lse - z_y + c lse^2; backward
//   dz = dloss (softmax(z) (1 + 2 c lse) - onehot(y)); rows whose label is
//   the ignore index or outside the vocabulary carry no loss or gradient.
#include "fa_device.h"

namespace fa {
namespace {

constexpr int kNT = 256;   // 4 waves

__device__ __forceinline__ void unpack8(const i32x4 &v, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_lo((uint32_t)v[e]);
    f[2 * e + 1] = bf16_hi((uint32_t)v[e]);
  }
}

__device__ __forceinline__ i32x4 pack8(const float (&f)[8]) {
  return i32x4{(int)pack_bf16x2(f[0], f[1]), (int)pack_bf16x2(f[2], f[3]),
               (int)pack_bf16x2(f[4], f[5]), (int)pack_bf16x2(f[6], f[7])};
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ---------------------------------------------------------------------------
// RMSNorm forward: one wave per row.  Lane l holds 16-byte chunks l, l + 64,
// ... (K of them); chunks past the row read as 0 and their stores are
// dropped by the buffer range check.
// ---------------------------------------------------------------------------
template <int K>
__global__ __launch_bounds__(kNT) void rmsnorm_fwd_kernel(const uint16_t *x, const uint16_t *w,
                                                          uint16_t *y, float *rstd, int rows,
                                                          int dim, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kNT / 64) + (int)(threadIdx.x >> 6);
  if (row >= rows) return;   // the whole wave
  const uint32_t bytes = (uint32_t)dim * 2u;
  const rsrc_t rx = make_rsrc(x + (size_t)row * dim, bytes);
  const rsrc_t rw = make_rsrc(w, bytes);
  const rsrc_t ry = make_rsrc(y + (size_t)row * dim, bytes);
  i32x4 xv[K], wv[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    xv[k] = buf_load16(rx, (uint32_t)(lane + 64 * k) * 16u);
    wv[k] = buf_load16(rw, (uint32_t)(lane + 64 * k) * 16u);
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    float f[8];
    unpack8(xv[k], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)dim + eps);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    float f[8], g[8];
    unpack8(xv[k], f);
    unpack8(wv[k], g);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = f[e] * r * g[e];
    buf_store16(ry, (uint32_t)(lane + 64 * k) * 16u, pack8(f));
  }
  if (lane == 0) rstd[row] = r;
}

// ---------------------------------------------------------------------------
// RMSNorm backward: each wave takes rows wave_id, wave_id + waves, ...; dx is
// written per row, the dw partial stays in the lane's registers (columns of
// its chunks).  The workgroup's 4 partials are added in LDS (in wave order,
// 1024 columns at a time) into part[workgroup][dim]; rmsnorm_dw_kernel adds
// the workgroups in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kSlice = 1024;   // columns per LDS pass of the workgroup sum

template <int K>
__global__ __launch_bounds__(kNT) void rmsnorm_bwd_kernel(const uint16_t *x, const uint16_t *w,
                                                          const float *rstd, const uint16_t *dy,
                                                          uint16_t *dx, float *part, int rows,
                                                          int dim) {
  __shared__ float red[kNT / 64][kSlice];
  const int lane = threadIdx.x & 63, wave = (int)(threadIdx.x >> 6);
  const int waves = gridDim.x * (kNT / 64);
  const uint32_t bytes = (uint32_t)dim * 2u;
  const rsrc_t rw = make_rsrc(w, bytes);
  // Up to 4096 columns the weights stay unpacked in registers; wider rows
  // keep them as bf16 pairs (the float copy would not fit beside x, dy and
  // the dw partial) and unpack them where they are used.
  constexpr bool kPackW = K > 8;
  float wf[kPackW ? 1 : K][8], acc[K][8];
  i32x4 wp[kPackW ? K : 1];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const i32x4 v = buf_load16(rw, (uint32_t)(lane + 64 * k) * 16u);
    if constexpr (kPackW) wp[k] = v;
    else unpack8(v, wf[k]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
  }
  const auto weights = [&](int k, float (&g)[8]) {
    if constexpr (kPackW) unpack8(wp[k], g);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = wf[k][e];
  };
  const float inv_dim = 1.f / (float)dim;
  for (int row = blockIdx.x * (kNT / 64) + wave; row < rows; row += waves) {
    if constexpr (kPackW) {
      // keeps the unpacking inside the loop instead of hoisted out of it
#pragma unroll
      for (int k = 0; k < K; ++k) asm volatile("" : "+v"(wp[k]));
    }
    const rsrc_t rx = make_rsrc(x + (size_t)row * dim, bytes);
    const rsrc_t rdy = make_rsrc(dy + (size_t)row * dim, bytes);
    const rsrc_t rdx = make_rsrc(dx + (size_t)row * dim, bytes);
    i32x4 xv[K], dv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      xv[k] = buf_load16(rx, (uint32_t)(lane + 64 * k) * 16u);
      dv[k] = buf_load16(rdy, (uint32_t)(lane + 64 * k) * 16u);
    }
    const float r = rstd[row];
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float f[8], g[8], wk[8];
      unpack8(xv[k], f);
      unpack8(dv[k], g);
      weights(k, wk);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(g[e] * wk[e], f[e], dot);
    }
    const float cc = wave_sum(dot) * inv_dim * r * r;
    // unpack x and dy again below rather than keep both float copies live
#pragma unroll
    for (int k = 0; k < K; ++k) asm volatile("" : "+v"(xv[k]), "+v"(dv[k]));
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float f[8], g[8], o[8], wk[8];
      unpack8(xv[k], f);
      unpack8(dv[k], g);
      weights(k, wk);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = r * fmaf(-f[e], cc, g[e] * wk[e]);
        acc[k][e] = fmaf(g[e] * f[e], r, acc[k][e]);
      }
      buf_store16(rdx, (uint32_t)(lane + 64 * k) * 16u, pack8(o));
    }
  }
  // workgroup partial of dw, one slice of columns at a time (none without dw)
  if (part == nullptr) return;
  float *const out = part + (size_t)blockIdx.x * dim;
  for (int s0 = 0; s0 < dim; s0 += kSlice) {
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = 8 * (lane + 64 * k) + e - s0;
        if (col >= 0 && col < kSlice) red[wave][col] = acc[k][e];
      }
    __syncthreads();
    for (int col = threadIdx.x; col < kSlice && s0 + col < dim; col += kNT)
      out[s0 + col] = ((red[0][col] + red[1][col]) + red[2][col]) + red[3][col];
    __syncthreads();
  }
}

// dw[j] = sum over workgroup partials in a fixed order: one workgroup per
// block of 64 columns, 16 waves; wave v adds partials v, v + 16, ... with four
// interleaved accumulators (loads stay in flight), then the 16 wave sums are
// added in wave order.
constexpr int kDwWaves = 16;

__global__ __launch_bounds__(64 * kDwWaves) void rmsnorm_dw_kernel(const float *part, float *dw,
                                                                   int nparts, int dim) {
  __shared__ float red[kDwWaves][64];
  const int c = threadIdx.x & 63, v = (int)(threadIdx.x >> 6);
  const int col = blockIdx.x * 64 + c;
  float t0 = 0.f, t1 = 0.f, t2 = 0.f, t3 = 0.f;
  if (col < dim) {
    int p = v;
    for (; p + 3 * kDwWaves < nparts; p += 4 * kDwWaves) {
      t0 += part[(size_t)p * dim + col];
      t1 += part[(size_t)(p + kDwWaves) * dim + col];
      t2 += part[(size_t)(p + 2 * kDwWaves) * dim + col];
      t3 += part[(size_t)(p + 3 * kDwWaves) * dim + col];
    }
    for (; p < nparts; p += kDwWaves) t0 += part[(size_t)p * dim + col];
  }
  red[v][c] = (t0 + t1) + (t2 + t3);
  __syncthreads();
  if (v == 0 && col < dim) {
    float t = red[0][c];
#pragma unroll
    for (int u = 1; u < kDwWaves; ++u) t += red[u][c];
    dw[col] = t;
  }
}

// ---------------------------------------------------------------------------
// Cross-entropy with z-loss: one workgroup per row (vocab a multiple of 8).
// Forward: a running (max, sum of exp) per thread over its 16-byte chunks,
// merged across the workgroup; backward: softmax recomputed from the saved
// lse, written as bf16 (may overwrite the logits in place).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  s = s * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
  m = mn;
}

__device__ __forceinline__ bool label_ok(int y, int vocab, int ignore) {
  return y != ignore && y >= 0 && y < vocab;
}

__global__ __launch_bounds__(kNT) void ce_fwd_kernel(const uint16_t *z, const int32_t *labels,
                                                     float *loss, float *lse_out, int vocab,
                                                     float zl, int ignore) {
  __shared__ float rm[kNT / 64], rs[kNT / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  const rsrc_t rz = make_rsrc(z + (size_t)row * vocab, (uint32_t)vocab * 2u);
  const int nch = vocab / 8;
  float m = -INFINITY, s = 0.f;
#pragma unroll 4
  for (int c = tid; c < nch; c += kNT) {
    float f[8];
    unpack8(buf_load16(rz, (uint32_t)c * 16u), f);
    float cm = f[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, f[e]);
    const float mn = fmaxf(m, cm);
    const float off = -mn * kLog2e;
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) t += __builtin_amdgcn_exp2f(fmaf(f[e], kLog2e, off));
    s = fmaf(s, __builtin_amdgcn_exp2f(fmaf(m, kLog2e, off)), t);
    m = mn;
  }
  // threads that saw no chunk hold (-inf, 0): merge them as (m, 0) pairs
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    if (m2 > -INFINITY) {
      if (m > -INFINITY) lse_merge(m, s, m2, s2);
      else { m = m2; s = s2; }
    }
  }
  const int wave = tid >> 6;
  if ((tid & 63) == 0) {
    rm[wave] = m;
    rs[wave] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float M = rm[0], Ssum = rs[0];
#pragma unroll
    for (int v = 1; v < kNT / 64; ++v)
      if (rm[v] > -INFINITY) lse_merge(M, Ssum, rm[v], rs[v]);
    const float L = M + logf(Ssum);
    const int y = labels[row];
    float l = 0.f;
    if (label_ok(y, vocab, ignore)) {
      const float zy = bf16_bits(buf_load_u16(rz, (uint32_t)y * 2u));
      l = fmaf(zl * L, L, L - zy);
    }
    loss[row] = l;
    lse_out[row] = L;
  }
}

__global__ __launch_bounds__(kNT) void ce_bwd_kernel(const uint16_t *z, const int32_t *labels,
                                                     const float *lse, const float *dloss,
                                                     uint16_t *dz, int vocab, float zl,
                                                     int ignore) {
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint32_t bytes = (uint32_t)vocab * 2u;
  const rsrc_t rz = make_rsrc(z + (size_t)row * vocab, bytes);
  const rsrc_t rdz = make_rsrc(dz + (size_t)row * vocab, bytes);
  const int y = labels[row];
  const bool ok = label_ok(y, vocab, ignore);
  const float g = ok ? dloss[row] : 0.f;
  const float L = lse[row];
  const float sc = g * fmaf(2.f * zl, L, 1.f);
  const float off = -L * kLog2e;
  const int nch = vocab / 8;
#pragma unroll 4
  for (int c = tid; c < nch; c += kNT) {
    float f[8];
    unpack8(buf_load16(rz, (uint32_t)c * 16u), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[e] = sc * __builtin_amdgcn_exp2f(fmaf(f[e], kLog2e, off));
      if (ok && 8 * c + e == y) f[e] -= g;
    }
    buf_store16(rdz, (uint32_t)c * 16u, pack8(f));
  }
}

template <int K>
hipError_t launch_rms_fwd_k(const uint16_t *x, const uint16_t *w, uint16_t *y, float *rstd,
                            int rows, int dim, float eps, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_fwd_kernel<K>, dim3((rows + 3) / 4), dim3(kNT), 0, s, x, w, y, rstd,
                     rows, dim, eps);
  return hipGetLastError();
}

template <int K>
hipError_t launch_rms_bwd_k(const uint16_t *x, const uint16_t *w, const float *rstd,
                            const uint16_t *dy, uint16_t *dx, float *part, int rows, int dim,
                            int grid, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_bwd_kernel<K>, dim3(grid), dim3(kNT), 0, s, x, w, rstd, dy, dx, part,
                     rows, dim);
  return hipGetLastError();
}

}  // namespace

int rmsnorm_chunks_per_lane(int dim) {
  const int nch = (dim + 7) / 8;
  int k = 1;
  while (64 * k < nch) k *= 2;
  return k;
}

int rmsnorm_bwd_grid(int rows) {
  const int need = (rows + 3) / 4;
  return need < kRmsBwdMaxGrid ? need : kRmsBwdMaxGrid;
}

hipError_t launch_rmsnorm_fwd(const void *x, const void *w, void *y, float *rstd, int rows,
                              int dim, float eps, hipStream_t s) {
  const auto *xp = static_cast<const uint16_t *>(x);
  const auto *wp = static_cast<const uint16_t *>(w);
  auto *yp = static_cast<uint16_t *>(y);
  switch (rmsnorm_chunks_per_lane(dim)) {
    case 1: return launch_rms_fwd_k<1>(xp, wp, yp, rstd, rows, dim, eps, s);
    case 2: return launch_rms_fwd_k<2>(xp, wp, yp, rstd, rows, dim, eps, s);
    case 4: return launch_rms_fwd_k<4>(xp, wp, yp, rstd, rows, dim, eps, s);
    case 8: return launch_rms_fwd_k<8>(xp, wp, yp, rstd, rows, dim, eps, s);
    default: return launch_rms_fwd_k<16>(xp, wp, yp, rstd, rows, dim, eps, s);
  }
}

hipError_t launch_rmsnorm_bwd(const void *x, const void *w, const float *rstd, const void *dy,
                              void *dx, float *dw, float *part, int rows, int dim,
                              hipStream_t s) {
  const auto *xp = static_cast<const uint16_t *>(x);
  const auto *wp = static_cast<const uint16_t *>(w);
  const auto *dyp = static_cast<const uint16_t *>(dy);
  auto *dxp = static_cast<uint16_t *>(dx);
  const int grid = rmsnorm_bwd_grid(rows);
  hipError_t e;
  switch (rmsnorm_chunks_per_lane(dim)) {
    case 1: e = launch_rms_bwd_k<1>(xp, wp, rstd, dyp, dxp, part, rows, dim, grid, s); break;
    case 2: e = launch_rms_bwd_k<2>(xp, wp, rstd, dyp, dxp, part, rows, dim, grid, s); break;
    case 4: e = launch_rms_bwd_k<4>(xp, wp, rstd, dyp, dxp, part, rows, dim, grid, s); break;
    case 8: e = launch_rms_bwd_k<8>(xp, wp, rstd, dyp, dxp, part, rows, dim, grid, s); break;
    default: e = launch_rms_bwd_k<16>(xp, wp, rstd, dyp, dxp, part, rows, dim, grid, s); break;
  }
  if (e != hipSuccess || dw == nullptr) return e;
  return launch_rmsnorm_dw(part, dw, rows, dim, s);
}

hipError_t launch_rmsnorm_dw(const float *part, float *dw, int rows, int dim, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_dw_kernel, dim3((dim + 63) / 64), dim3(64 * kDwWaves), 0, s, part,
                     dw, rmsnorm_bwd_grid(rows), dim);
  return hipGetLastError();
}

hipError_t launch_ce_fwd(const void *z, const int32_t *labels, float *loss, float *lse, int rows,
                         int vocab, float z_loss, int ignore, hipStream_t s) {
  hipLaunchKernelGGL(ce_fwd_kernel, dim3(rows), dim3(kNT), 0, s,
                     static_cast<const uint16_t *>(z), labels, loss, lse, vocab, z_loss, ignore);
  return hipGetLastError();
}

hipError_t launch_ce_bwd(const void *z, const int32_t *labels, const float *lse,
                         const float *dloss, void *dz, int rows, int vocab, float z_loss,
                         int ignore, hipStream_t s) {
  hipLaunchKernelGGL(ce_bwd_kernel, dim3(rows), dim3(kNT), 0, s,
                     static_cast<const uint16_t *>(z), labels, lse, dloss,
                     static_cast<uint16_t *>(dz), vocab, z_loss, ignore);
  return hipGetLastError();
}

}  // namespace fa
