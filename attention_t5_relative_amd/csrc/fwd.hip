// Forward attention for gfx950 (FAT5 report, section "Noyau CUDA", second
// kernel): per (sequence, head, 128-query tile) one workgroup streams K and V
// through LDS in 64-key tiles, forms S' = scale * Q K^T + bias on the fly from
// the per-head table (or ALiBi), keeps a running softmax, accumulates O = P V,
// and writes O (bf16) and the row logsumexp (fp32).  The score matrix never
// leaves registers.
//
// Layout of the work inside a workgroup (4 waves, 32 query rows each):
//   S^T (keys x queries) = K Q^T on 32x32x16 bf16 MFMA, so each lane owns one
//   query row and 32 of the tile's keys: the row max and row sum are in-lane
//   reductions plus one exchange between the two half-waves.
//   O^T (dims x queries) = V^T P^T reuses P straight from the score
//   accumulators as the MFMA B operand; V is stored transposed in LDS with a
//   key order (key_perm16) that makes each lane's 8 keys contiguous.
#include "fa_device.h"

namespace fa {
namespace {

constexpr int BR = 128;   // query rows per workgroup
constexpr int BC = 64;    // keys per tile
constexpr int NT = 256;   // threads per workgroup
// A row's running max is only raised when a tile's max exceeds it by more
// than 2^8; until then exp2 values stay <= 256, exact enough in fp32 and bf16,
// and the O accumulator rescale is skipped.
constexpr float kRescaleLog2 = 8.0f;

struct FwdArgs {
  const uint16_t *q, *k, *v;
  uint16_t *o;
  float *lse;
  const int4 *sched;     // packed batches: {token0, length, head, q-tile}
  const float *table, *slopes;
  int32_t nbatch, seqlen, heads, total;
  int32_t nq, nwg;
  float scale_log2;      // scale * log2(e)
  T5Geometry t5;
};

template <int D, int BIAS, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NT, 2) void fwd_kernel(const FwdArgs a) {
  constexpr int NCH = D / 8;                  // 16-byte chunks per row
  constexpr int KLOADS = BC * NCH / NT;       // K chunks per thread per tile
  constexpr int VUNITS = (BC / 2) * NCH / NT; // (key pair, chunk) units per thread
  static_assert(KLOADS * NT == BC * NCH && VUNITS * NT == (BC / 2) * NCH, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][D * BC];
  __shared__ float lut[BIAS == kBiasT5 ? 2 * kMaxDistance + 1 : 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, il = lane & 31;
  const int g = xcd_remap(blockIdx.x, a.nwg);

  int h, qt, tok0, L, bidx = 0;
  if constexpr (VARLEN) {
    const int4 e = a.sched[g];
    tok0 = e.x;
    L = e.y;
    h = e.z;
    qt = e.w;
    if (L <= 0) return;
  } else {
    const int pair = g / a.nq;
    qt = a.nq - 1 - (g - pair * a.nq);        // longest causal rows first
    bidx = pair / a.heads;
    h = pair - bidx * a.heads;
    tok0 = bidx * a.seqlen;
    L = a.seqlen;
  }

  const int HD = a.heads * D;
  const size_t base = ((size_t)tok0 * a.heads + h) * D;
  const uint32_t nrec = ((uint32_t)(L - 1) * (uint32_t)HD + D) * 2u;
  const rsrc_t rq = make_rsrc(a.q + base, nrec);
  const rsrc_t rk = make_rsrc(a.k + base, nrec);
  const rsrc_t rv = make_rsrc(a.v + base, nrec);
  const rsrc_t ro = make_rsrc(a.o + base, nrec);

  const int q0 = qt * BR;
  const int wrow0 = q0 + 32 * wave;
  const int myrow = wrow0 + il;

  // Q as the B operand of S^T = K Q^T: lane (hl, il) holds row myrow,
  // dims 16s + 8hl .. +7 for k-step s.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = __builtin_bit_cast(
        bf16x8, buf_load16(rq, ((uint32_t)myrow * (uint32_t)HD + 16 * s + 8 * hl) * 2u));

  int sat = 0;
  if constexpr (BIAS == kBiasT5) {
    // bias (log2 units) by relative position r = j - i, clamped to [-sat, sat]
    sat = a.t5.sat;
    for (int x = tid; x <= 2 * sat; x += NT)
      lut[x] = a.table[t5_bucket_dev(x - sat, a.t5) * a.heads + h] * kLog2e;
  }
  float slope_l2 = 0.f;
  if constexpr (BIAS == kBiasAlibi) slope_l2 = -a.slopes[h] * kLog2e;

  const int kend = CAUSAL ? min(L, q0 + BR) : L;
  const int nkt = (kend + BC - 1) / BC;

  i32x4 kreg[KLOADS];
  i32x4 vreg[VUNITS][2];

  auto gload = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int c = tid + NT * u, row = c / NCH, col = c % NCH;
      kreg[u] = buf_load16(rk, ((uint32_t)(j0 + row) * (uint32_t)HD + col * 8) * 2u);
    }
#pragma unroll
    for (int u = 0; u < VUNITS; ++u) {
      const int unit = tid + NT * u, col = unit % NCH, kp = unit / NCH;
      vreg[u][0] = buf_load16(rv, ((uint32_t)(j0 + 2 * kp) * (uint32_t)HD + col * 8) * 2u);
      vreg[u][1] = buf_load16(rv, ((uint32_t)(j0 + 2 * kp + 1) * (uint32_t)HD + col * 8) * 2u);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int c = tid + NT * u, row = c / NCH, col = c % NCH;
      *reinterpret_cast<i32x4 *>(&ks[buf][row * D + ((col ^ (row & 7)) * 8)]) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < VUNITS; ++u) {
      const int unit = tid + NT * u, col = unit % NCH, kp = unit / NCH;
      const int kpr = key_perm16(2 * kp);
      const int kch = kpr >> 3, within = kpr & 7;
      const i32x4 x0 = vreg[u][0], x1 = vreg[u][1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = (uint32_t)x0[e >> 1], w1 = (uint32_t)x1[e >> 1];
        const uint32_t w = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                   : ((w0 & 0xffffu) | (w1 << 16));
        const int d = 8 * col + e;
        const int sw = kch ^ ((d ^ (d >> 3)) & 7);
        *reinterpret_cast<uint32_t *>(&vt[buf][d * BC + sw * 8 + within]) = w;
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;

  if (nkt > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int j0 = kt * BC;
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(j0 + BC);
    const bool active = !CAUSAL || (j0 <= wrow0 + 31);
    if (active) {
      const uint16_t *kb_s = ks[buf];
      const uint16_t *vt_s = vt[buf];
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        const int row = 32 * kb + il;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(
              &kb_s[row * D + (((2 * s + hl) ^ (row & 7)) * 8)]);
          sacc[kb] = mfma32(kf, qf[s], sacc[kb]);
        }
      }

      // Element (kb, r) of this lane: key j0 + 32kb + 8(r/4) + 4hl + r%4, query myrow.
      const int rmin = j0 - (wrow0 + 31), rmax = j0 + BC - 1 - wrow0;
      const bool mask_c = CAUSAL && rmax > 0;
      const bool mask_l = (j0 + BC > L);
      bool uniform = (BIAS == kBiasNone);
      float bconst = 0.f;
      if constexpr (BIAS == kBiasT5) {
        const int lo = min(max(rmin, -sat), sat), hi = min(max(rmax, -sat), sat);
        uniform = (lo == hi);
        bconst = lut[lo + sat];
      }

      float tmax;
      float nbias;   // added to fma(s, c, .) before exp2 on the uniform path
      if (uniform && !mask_c && !mask_l) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        mx = fmaxf(mx, xor32(mx));
        tmax = fmaf(mx, c, bconst);
        nbias = bconst;
      } else {
        const int rb = j0 - myrow + 4 * hl;
        const int jb = j0 + 4 * hl;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
            const int rr = rb + off;
            float t = sacc[kb][r] * c;
            if constexpr (BIAS == kBiasT5) t += lut[min(max(rr, -sat), sat) + sat];
            if constexpr (BIAS == kBiasAlibi) t = fmaf(fabsf((float)rr), slope_l2, t);
            if (mask_c && rr > 0) t = -INFINITY;
            if (mask_l && jb + off >= L) t = -INFINITY;
            sacc[kb][r] = t;
            mx = fmaxf(mx, t);
          }
        mx = fmaxf(mx, xor32(mx));
        tmax = mx;
        nbias = 0.f;
        // from here on sacc holds finished log2-domain scores: exp2(s*1 + 0 - m)
      }
      const float cc = (uniform && !mask_c && !mask_l) ? c : 1.f;

      const bool need = tmax > m_run + kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? exp2f(m_run - tmax) : 1.f;
        if (need) m_run = tmax;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      const float sub = nbias - m_use;

      bf16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * u + 2 * e], cc, sub));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * u + 2 * e + 1], cc, sub));
            l_run += p0 + p1;
            w[e] = pack_bf16x2(p0, p1);
          }
          i32x4 wv = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
          pb[kb][u] = __builtin_bit_cast(bf16x8, wv);
        }

#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = 32 * db + il;
        const int swz = (d ^ (d >> 3)) & 7;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int ch = 4 * kb + 2 * u + hl;
            const bf16x8 vf =
                *reinterpret_cast<const bf16x8 *>(&vt_s[d * BC + ((ch ^ swz) * 8)]);
            oacc[db] = mfma32(vf, pb[kb][u], oacc[db]);
          }
      }
    }
    if (kt + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      i32x2 w = {(int)pack_bf16x2(oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv),
                 (int)pack_bf16x2(oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv)};
      buf_store8(ro, ((uint32_t)myrow * (uint32_t)HD + 32 * db + 8 * rq + 4 * hl) * 2u, w);
    }
  if (hl == 0 && myrow < L) {
    const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    size_t idx;
    if constexpr (VARLEN)
      idx = (size_t)h * a.total + tok0 + myrow;
    else
      idx = ((size_t)bidx * a.heads + h) * a.seqlen + myrow;
    a.lse[idx] = lse;
  }
}

template <int D, int BIAS, bool CAUSAL, bool VARLEN>
hipError_t launch_t(const FwdArgs &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((fwd_kernel<D, BIAS, CAUSAL, VARLEN>), dim3(grid), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int D, int BIAS>
hipError_t launch_b(const FwdArgs &a, int grid, bool causal, bool varlen, hipStream_t s) {
  if (causal)
    return varlen ? launch_t<D, BIAS, true, true>(a, grid, s)
                  : launch_t<D, BIAS, true, false>(a, grid, s);
  return varlen ? launch_t<D, BIAS, false, true>(a, grid, s)
                : launch_t<D, BIAS, false, false>(a, grid, s);
}

template <int D>
hipError_t launch_d(const FwdArgs &a, int grid, int bias, bool causal, bool varlen,
                    hipStream_t s) {
  switch (bias) {
    case kBiasT5: return launch_b<D, kBiasT5>(a, grid, causal, varlen, s);
    case kBiasAlibi: return launch_b<D, kBiasAlibi>(a, grid, causal, varlen, s);
    default: return launch_b<D, kBiasNone>(a, grid, causal, varlen, s);
  }
}

}  // namespace

int fwd_tile_rows() { return BR; }

hipError_t launch_fwd_impl(const Problem &p, const FwdBuffers &b, const int4 *sched, int nsched,
                           hipStream_t s) {
  FwdArgs a;
  a.q = static_cast<const uint16_t *>(b.q);
  a.k = static_cast<const uint16_t *>(b.k);
  a.v = static_cast<const uint16_t *>(b.v);
  a.o = static_cast<uint16_t *>(b.o);
  a.lse = b.lse;
  a.sched = sched;
  a.table = p.table;
  a.slopes = p.slopes;
  a.nbatch = p.nbatch;
  a.seqlen = p.seqlen;
  a.heads = p.heads;
  a.total = p.total;
  a.scale_log2 = p.scale * kLog2e;
  a.t5 = p.t5;
  int grid;
  if (p.varlen) {
    a.nq = 0;
    grid = nsched;
  } else {
    a.nq = (p.seqlen + BR - 1) / BR;
    grid = p.nbatch * p.heads * a.nq;
  }
  a.nwg = grid;
  if (grid <= 0) return hipSuccess;
  if (p.head_dim == 64) return launch_d<64>(a, grid, p.bias, p.causal, p.varlen, s);
  return launch_d<128>(a, grid, p.bias, p.causal, p.varlen, s);
}

}  // namespace fa
