// Backward attention for gfx950.  The pages print no backward; this is the
// calculus of the forward they describe (FAT5 report, "Noyau CUDA"), with
// the bias table trained through the gradient of S':
//
//   dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K,
//   dTable[b, h] = sum over (i, j) with bucket b of dS_ij.
//
// Three kernels per call:
//   pre   row-parallel (128 queries per workgroup, forward-shaped): recomputes
//         P in fp32 and dP, writes D_i = sum_j P_ij dP_ij (consistent with the
//         P the main kernel recomputes, which D = rowsum(dO * O) from a bf16 O
//         is not), and zeroes the fp32 dQ accumulator rows it owns.
//   main  column-parallel (128 keys per workgroup, 32 per wave): loops over
//         query blocks; S = Q K^T puts each lane on one key, so P and dS feed
//         the dV and dK products straight from the accumulators; dS goes to
//         LDS transposed for dQ, which is added to the fp32 accumulator with
//         coalesced atomics; dS enters the dK and dQ products as a bf16 hi/lo
//         pair (16 significant bits); the table gradient is binned by relative
//         distance in per-wave LDS bins and reduced in a fixed order.
//   reduce (elsewhere) dQ fp32 -> bf16, bias partials -> dTable.
#include "fa_device.h"

namespace fa {
namespace {

constexpr int NT = 256;
constexpr int BR = 128;    // pre-pass: query rows per workgroup
constexpr int BC = 64;     // pre-pass: keys per tile
constexpr int BKV = 128;   // main: keys per workgroup
constexpr int NBINS = 2 * kMaxDistance + 1;

struct BwdArgs {
  const uint16_t *q, *k, *v, *dout;
  const float *lse;
  uint16_t *dk, *dv;
  float *dk_acc;           // fp32 dK in the rotated space (RoPE), else unused
  float *dq_acc;           // fp32 [tokens, H, D]
  float *delta;            // same layout as lse
  float *part;             // [nb, nwg] bias-gradient partials
  const int4 *sched;       // packed batches: {token0, length, head, tile}
  const float *table, *slopes;
  int32_t nbatch, seqlen, heads, total;
  int32_t ntile;           // dense: tiles of 128 per sequence
  int32_t nwg;
  int32_t nb;
  float scale, scale_log2;
  T5Geometry t5;
};

struct Work {
  int h, tile, tok0, L;
  size_t lse_base;         // index of row 0 in lse / delta
};

// Dense: logical id -> (batch, head, tile) with tile = g % ntile.
// Packed: the schedule entry.  Returns false for an empty entry.
template <bool VARLEN>
__device__ __forceinline__ bool locate(const BwdArgs &a, int g, Work &w) {
  if constexpr (VARLEN) {
    const int4 e = a.sched[g];
    if (e.y <= 0) return false;
    w.tok0 = e.x;
    w.L = e.y;
    w.h = e.z;
    w.tile = e.w;
    w.lse_base = (size_t)w.h * a.total + w.tok0;
  } else {
    const int pair = g / a.ntile;
    w.tile = g - pair * a.ntile;
    const int b = pair / a.heads;
    w.h = pair - b * a.heads;
    w.tok0 = b * a.seqlen;
    w.L = a.seqlen;
    w.lse_base = ((size_t)b * a.heads + w.h) * a.seqlen;
  }
  return true;
}

// ---------------------------------------------------------------------------
// Pre-pass
// ---------------------------------------------------------------------------
template <int D, int BIAS, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NT, 2) void bwd_pre_kernel(const BwdArgs a) {
  constexpr int NCH = D / 8;
  constexpr int KLOADS = BC * NCH / NT;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][BC * D];
  __shared__ float lut[BIAS == kBiasT5 ? NBINS : 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, il = lane & 31;
  const int g = xcd_remap(blockIdx.x, a.nwg);
  Work w;
  if (!locate<VARLEN>(a, g, w)) return;
  const int L = w.L, h = w.h;
  // longest causal rows first: packed entries count tiles down already
  const int qt = VARLEN ? w.tile : (a.ntile - 1 - w.tile);

  const int HD = a.heads * D;
  const size_t base = ((size_t)w.tok0 * a.heads + h) * D;
  const uint32_t nrec = ((uint32_t)(L - 1) * (uint32_t)HD + D) * 2u;
  const rsrc_t rq = make_rsrc(a.q + base, nrec);
  const rsrc_t rk = make_rsrc(a.k + base, nrec);
  const rsrc_t rv = make_rsrc(a.v + base, nrec);
  const rsrc_t rdo = make_rsrc(a.dout + base, nrec);
  const rsrc_t rdq = make_rsrc(a.dq_acc + base, nrec * 2u);

  const int q0 = qt * BR;
  const int wrow0 = q0 + 32 * wave;
  const int myrow = wrow0 + il;

  // zero the fp32 dQ rows of this tile (the main kernel adds into them)
  {
    constexpr int CH = BR * D / 4;   // 16-byte chunks
    const i32x4 z = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < CH / NT; ++u) {
      const int c = tid + NT * u, row = c / (D / 4), col = c % (D / 4);
      buf_store16(rdq, ((uint32_t)(q0 + row) * (uint32_t)HD + col * 4) * 4u, z);
    }
  }

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint32_t off = ((uint32_t)myrow * (uint32_t)HD + 16 * s + 8 * hl) * 2u;
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    df[s] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
  }
  const float lse2 = myrow < L ? a.lse[w.lse_base + myrow] * kLog2e : 0.f;

  int sat = 0;
  if constexpr (BIAS == kBiasT5) {
    sat = a.t5.sat;
    for (int x = tid; x <= 2 * sat; x += NT)
      lut[x] = a.table[t5_bucket_dev(x - sat, a.t5) * a.heads + h] * kLog2e;
  }
  float slope_l2 = 0.f;
  if constexpr (BIAS == kBiasAlibi) slope_l2 = -a.slopes[h] * kLog2e;

  const int kend = CAUSAL ? min(L, q0 + BR) : L;
  const int nkt = (kend + BC - 1) / BC;
  i32x4 kreg[KLOADS], vreg[KLOADS];
  auto gload = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int c = tid + NT * u, row = c / NCH, col = c % NCH;
      const uint32_t off = ((uint32_t)(j0 + row) * (uint32_t)HD + col * 8) * 2u;
      kreg[u] = buf_load16(rk, off);
      vreg[u] = buf_load16(rv, off);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int c = tid + NT * u, row = c / NCH, col = c % NCH;
      const int at = row * D + ((col ^ (row & 7)) * 8);
      *reinterpret_cast<i32x4 *>(&ks[buf][at]) = kreg[u];
      *reinterpret_cast<i32x4 *>(&vs[buf][at]) = vreg[u];
    }
  };

  const float c = a.scale_log2;
  float acc = 0.f;
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
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        pacc[kb] = f32x16{};
        const int row = 32 * kb + il;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const int at = row * D + (((2 * s + hl) ^ (row & 7)) * 8);
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&ks[buf][at]);
          const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&vs[buf][at]);
          sacc[kb] = mfma32(kf, qf[s], sacc[kb]);
          pacc[kb] = mfma32(vf, df[s], pacc[kb]);
        }
      }
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
      if (uniform && !mask_c && !mask_l) {
        const float sub = bconst - lse2;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc = fmaf(__builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c, sub)), pacc[kb][r], acc);
      } else {
        const int rb = j0 - myrow + 4 * hl;
        const int jb = j0 + 4 * hl;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
            const int rr = rb + off;
            float t = sacc[kb][r] * c;
            if constexpr (BIAS == kBiasT5) t += lut[min(max(rr, -sat), sat) + sat];
            if constexpr (BIAS == kBiasAlibi) t = fmaf(fabsf((float)rr), slope_l2, t);
            const bool dead = (mask_c && rr > 0) || (mask_l && jb + off >= L);
            const float p = dead ? 0.f : __builtin_amdgcn_exp2f(t - lse2);
            acc = fmaf(p, pacc[kb][r], acc);
          }
      }
    }
    if (kt + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }
  const float dsum = acc + xor32(acc);
  if (hl == 0 && myrow < L) a.delta[w.lse_base + myrow] = dsum;
}

// ---------------------------------------------------------------------------
// Main kernel
// ---------------------------------------------------------------------------
template <int D>
struct MainCfg {
  static constexpr int QB = (D == 64) ? 64 : 32;   // query rows per iteration
  static constexpr int PN = D + 8;                 // padded pitch, natural rows
  static constexpr int PQ = QB + 8;                // padded pitch, transposed rows
  static constexpr int PK = BKV + 8;               // padded pitch, K^T and dS rows
};

template <int D, int BIAS, bool CAUSAL, bool VARLEN, bool ROPE, bool DBIAS>
__global__ __launch_bounds__(NT, 1) void bwd_main_kernel(const BwdArgs a) {
  using C = MainCfg<D>;
  constexpr int QB = C::QB, PN = C::PN, PQ = C::PQ, PK = C::PK;
  constexpr int NCH = D / 8;
  constexpr int QUNITS = (QB / 2) * NCH / NT;     // (row pair, chunk) units per thread
  constexpr int KUNITS = (BKV / 2) * NCH / NT;
  static_assert(QUNITS == 1, "one q staging unit per thread");
  static_assert((QB / 32) * (D / 32) == 4, "one dQ block per wave");

  __shared__ __attribute__((aligned(16))) uint16_t qs[QB * PN];
  __shared__ __attribute__((aligned(16))) uint16_t dos[QB * PN];
  __shared__ __attribute__((aligned(16))) uint16_t qtr[D * PQ];
  __shared__ __attribute__((aligned(16))) uint16_t dotr[D * PQ];
  __shared__ __attribute__((aligned(16))) float lse2s[QB];
  __shared__ __attribute__((aligned(16))) float dls[QB];
  __shared__ __attribute__((aligned(16))) uint16_t dsh[QB * PK];
  __shared__ __attribute__((aligned(16))) uint16_t dsl[QB * PK];
  __shared__ __attribute__((aligned(16))) uint16_t ktr[D * PK];
  __shared__ float lut[BIAS == kBiasT5 ? NBINS : 1];
  __shared__ float bins[DBIAS ? 4 : 1][DBIAS ? NBINS : 1];
  __shared__ int16_t bkt[DBIAS ? NBINS : 1];
  __shared__ float ubin[4][2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, il = lane & 31;
  const int g = xcd_remap(blockIdx.x, a.nwg);
  Work w;
  if (!locate<VARLEN>(a, g, w)) return;
  const int L = w.L, h = w.h;
  // keys nearest the sequence start see the most queries under a causal
  // mask: packed entries count tiles down, so flip them
  const int ktile = VARLEN ? ((L + BKV - 1) / BKV - 1 - w.tile) : w.tile;
  const int kt0 = ktile * BKV;
  const int kw0 = kt0 + 32 * wave;
  const int myk = kw0 + il;

  const int HD = a.heads * D;
  const size_t base = ((size_t)w.tok0 * a.heads + h) * D;
  const uint32_t nrec = ((uint32_t)(L - 1) * (uint32_t)HD + D) * 2u;
  const rsrc_t rq = make_rsrc(a.q + base, nrec);
  const rsrc_t rk = make_rsrc(a.k + base, nrec);
  const rsrc_t rv = make_rsrc(a.v + base, nrec);
  const rsrc_t rdo = make_rsrc(a.dout + base, nrec);
  const rsrc_t rdk = make_rsrc(ROPE ? (const void *)(a.dk_acc + base) : (const void *)(a.dk + base),
                               ROPE ? nrec * 2u : nrec);
  const rsrc_t rdv = make_rsrc(a.dv + base, nrec);
  float *const dq_base = a.dq_acc + base;

  // this wave's 32 keys as the B operand of S = Q K^T and dP = dO V^T
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint32_t off = ((uint32_t)myk * (uint32_t)HD + 16 * s + 8 * hl) * 2u;
    kf[s] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
    vf[s] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
  }
  // K^T of the workgroup's 128 keys (natural key order) for dQ = dS K
#pragma unroll
  for (int u = 0; u < KUNITS; ++u) {
    const int unit = tid + NT * u, col = unit % NCH, kp = unit / NCH;
    const i32x4 x0 = buf_load16(rk, ((uint32_t)(kt0 + 2 * kp) * (uint32_t)HD + col * 8) * 2u);
    const i32x4 x1 = buf_load16(rk, ((uint32_t)(kt0 + 2 * kp + 1) * (uint32_t)HD + col * 8) * 2u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w0 = (uint32_t)x0[e >> 1], w1 = (uint32_t)x1[e >> 1];
      const uint32_t wd = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                  : ((w0 & 0xffffu) | (w1 << 16));
      *reinterpret_cast<uint32_t *>(&ktr[(8 * col + e) * PK + 2 * kp]) = wd;
    }
  }

  int sat = 0;
  if constexpr (BIAS == kBiasT5) {
    sat = a.t5.sat;
    for (int x = tid; x <= 2 * sat; x += NT) {
      const int b = t5_bucket_dev(x - sat, a.t5);
      lut[x] = a.table[b * a.heads + h] * kLog2e;
      if constexpr (DBIAS) {
        bkt[x] = (int16_t)b;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) bins[ww][x] = 0.f;
      }
    }
  }
  float slope_l2 = 0.f;
  if constexpr (BIAS == kBiasAlibi) slope_l2 = -a.slopes[h] * kLog2e;

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }
  float ub0 = 0.f, ub1 = 0.f;   // table-gradient sums of saturated tiles (low / high side)

  const float c = a.scale_log2;
  const float scale = a.scale;
  const int nqb = (L + QB - 1) / QB;
  const int qb_first = CAUSAL ? (kt0 / QB) : 0;

  // staging registers for one query block
  i32x4 qr0, qr1, dr0, dr1;
  float lsev = 0.f, dlv = 0.f;
  const int s_col = tid % NCH, s_ip = tid / NCH;
  auto gload = [&](int q0) {
    const uint32_t o0 = ((uint32_t)(q0 + 2 * s_ip) * (uint32_t)HD + s_col * 8) * 2u;
    const uint32_t o1 = o0 + (uint32_t)HD * 2u;
    qr0 = buf_load16(rq, o0);
    qr1 = buf_load16(rq, o1);
    dr0 = buf_load16(rdo, o0);
    dr1 = buf_load16(rdo, o1);
    if (tid < QB) {
      const int row = q0 + tid;
      lsev = row < L ? a.lse[w.lse_base + row] * kLog2e : 0.f;
      dlv = row < L ? a.delta[w.lse_base + row] : 0.f;
    }
  };
  auto lstore = [&]() {
    const int r0 = 2 * s_ip;
    *reinterpret_cast<i32x4 *>(&qs[r0 * PN + s_col * 8]) = qr0;
    *reinterpret_cast<i32x4 *>(&qs[(r0 + 1) * PN + s_col * 8]) = qr1;
    *reinterpret_cast<i32x4 *>(&dos[r0 * PN + s_col * 8]) = dr0;
    *reinterpret_cast<i32x4 *>(&dos[(r0 + 1) * PN + s_col * 8]) = dr1;
    const int ip = key_perm16(r0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * s_col + e;
      {
        const uint32_t w0 = (uint32_t)qr0[e >> 1], w1 = (uint32_t)qr1[e >> 1];
        const uint32_t wd = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                    : ((w0 & 0xffffu) | (w1 << 16));
        *reinterpret_cast<uint32_t *>(&qtr[d * PQ + ip]) = wd;
      }
      {
        const uint32_t w0 = (uint32_t)dr0[e >> 1], w1 = (uint32_t)dr1[e >> 1];
        const uint32_t wd = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                    : ((w0 & 0xffffu) | (w1 << 16));
        *reinterpret_cast<uint32_t *>(&dotr[d * PQ + ip]) = wd;
      }
    }
    if (tid < QB) {
      lse2s[tid] = lsev;
      dls[tid] = dlv;
    }
  };

  if (qb_first < nqb) gload(qb_first * QB);
  for (int qb = qb_first; qb < nqb; ++qb) {
    const int q0 = qb * QB;
    lstore();
    __syncthreads();
    if (qb + 1 < nqb) gload(q0 + QB);

#pragma unroll
    for (int rb = 0; rb < QB / 32; ++rb) {
      const int irow0 = q0 + 32 * rb;
      const bool active = !CAUSAL || (kw0 <= irow0 + 31);
      uint16_t *const dsh_blk = &dsh[(32 * rb + 4 * hl) * PK + 32 * wave + il];
      uint16_t *const dsl_blk = &dsl[(32 * rb + 4 * hl) * PK + 32 * wave + il];
      if (!active) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int roff = 8 * (r >> 2) + (r & 3);
          dsh_blk[roff * PK] = 0;
          dsl_blk[roff * PK] = 0;
        }
        continue;
      }
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const int at = (32 * rb + il) * PN + 16 * s + 8 * hl;
        const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(&qs[at]);
        const bf16x8 da = *reinterpret_cast<const bf16x8 *>(&dos[at]);
        sacc = mfma32(qa, kf[s], sacc);
        pacc = mfma32(da, vf[s], pacc);
      }
      // element r: row irow0 + 8(r/4) + 4hl + r%4, key myk
      float lv[16], dv[16];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&lse2s[32 * rb + 8 * qq + 4 * hl]);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&dls[32 * rb + 8 * qq + 4 * hl]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lv[4 * qq + e] = l4[e];
          dv[4 * qq + e] = d4[e];
        }
      }
      const int rmin = kw0 - (irow0 + 31), rmax = kw0 + 31 - irow0;
      const bool mask_c = CAUSAL && rmax > 0;
      const bool mask_r = irow0 + 32 > L;
      const bool mask_k = kw0 + 32 > L;
      bool uniform = (BIAS == kBiasNone);
      float bconst = 0.f;
      int ulo = 0;
      if constexpr (BIAS == kBiasT5) {
        ulo = min(max(rmin, -sat), sat);
        const int uhi = min(max(rmax, -sat), sat);
        uniform = (ulo == uhi);
        bconst = lut[ulo + sat];
      }
      float p[16], ds[16];
      if (uniform && !mask_c && !mask_r && !mask_k) {
        float tsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, bconst - lv[r]));
          ds[r] = p[r] * (pacc[r] - dv[r]);
          tsum += ds[r];
        }
        if constexpr (DBIAS) {
          if (ulo <= 0) ub0 += tsum; else ub1 += tsum;
        }
      } else {
        const int rbase = myk - irow0 - 4 * hl;
        const int rowb = irow0 + 4 * hl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int roff = 8 * (r >> 2) + (r & 3);
          const int rr = rbase - roff;
          float t = sacc[r] * c;
          int x = 0;
          if constexpr (BIAS == kBiasT5) {
            x = min(max(rr, -sat), sat) + sat;
            t += lut[x];
          }
          if constexpr (BIAS == kBiasAlibi) t = fmaf(fabsf((float)rr), slope_l2, t);
          const bool dead = (mask_c && rr > 0) || (mask_r && rowb + roff >= L) ||
                            (mask_k && myk >= L);
          p[r] = dead ? 0.f : __builtin_amdgcn_exp2f(t - lv[r]);
          ds[r] = p[r] * (pacc[r] - dv[r]);
          if constexpr (DBIAS) {
            if (!dead) atomicAdd(&bins[wave][x], ds[r]);
          }
        }
      }

      // dV += P^T dO and dK += scale dS^T Q; rows enter as the k dimension
      // in key_perm16 order, matching the transposed LDS tiles.
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint32_t pw[4], hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r0 = 8 * u + 2 * e;
          pw[e] = pack_bf16x2(p[r0], p[r0 + 1]);
          const float s0 = ds[r0] * scale, s1 = ds[r0 + 1] * scale;
          hw[e] = pack_bf16x2(s0, s1);
          lw[e] = pack_bf16x2(s0 - bf16_lo(hw[e]), s1 - bf16_hi(hw[e]));
        }
        const bf16x8 pa = __builtin_bit_cast(bf16x8, i32x4{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]});
        const bf16x8 ha = __builtin_bit_cast(bf16x8, i32x4{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3]});
        const bf16x8 la = __builtin_bit_cast(bf16x8, i32x4{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3]});
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int at = (32 * db + il) * PQ + 32 * rb + 16 * u + 8 * hl;
          const bf16x8 dob = *reinterpret_cast<const bf16x8 *>(&dotr[at]);
          const bf16x8 qb8 = *reinterpret_cast<const bf16x8 *>(&qtr[at]);
          dvacc[db] = mfma32(pa, dob, dvacc[db]);
          dkacc[db] = mfma32(ha, qb8, dkacc[db]);
          dkacc[db] = mfma32(la, qb8, dkacc[db]);
        }
        // dS (scaled, hi and lo) to LDS as [row][key] for dQ
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r0 = 8 * u + 2 * e;
          const int ro0 = 8 * (r0 >> 2) + (r0 & 3), ro1 = 8 * ((r0 + 1) >> 2) + ((r0 + 1) & 3);
          dsh_blk[ro0 * PK] = (uint16_t)(hw[e] & 0xffffu);
          dsh_blk[ro1 * PK] = (uint16_t)(hw[e] >> 16);
          dsl_blk[ro0 * PK] = (uint16_t)(lw[e] & 0xffffu);
          dsl_blk[ro1 * PK] = (uint16_t)(lw[e] >> 16);
        }
      }
    }
    __syncthreads();

    // dQ block of this wave: rows 32*rbq.., dims 32*dbq..; contraction over
    // the workgroup's 128 keys with dS as hi + lo.
    {
      const int rbq = wave / (D / 32), dbq = wave % (D / 32);
      f32x16 qacc = f32x16{};
#pragma unroll
      for (int s = 0; s < BKV / 16; ++s) {
        const int aa = (32 * rbq + il) * PK + 16 * s + 8 * hl;
        const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(&dsh[aa]);
        const bf16x8 al = *reinterpret_cast<const bf16x8 *>(&dsl[aa]);
        const bf16x8 kb8 =
            *reinterpret_cast<const bf16x8 *>(&ktr[(32 * dbq + il) * PK + 16 * s + 8 * hl]);
        qacc = mfma32(ah, kb8, qacc);
        qacc = mfma32(al, kb8, qacc);
      }
      const int rowq = q0 + 32 * rbq + 4 * hl;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rowq + 8 * (r >> 2) + (r & 3);
        if (row < L)
          __builtin_amdgcn_global_atomic_fadd_f32(
              dq_base + (size_t)row * HD + 32 * dbq + il, qacc[r]);
      }
    }
  }

  // dK, dV: lane holds dims 32*db + il of keys kw0 + 8(r/4) + 4hl + r%4
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * hl + (r & 3);
      const uint32_t el = (uint32_t)key * (uint32_t)HD + 32 * db + il;
      const uint32_t vb = pack_bf16x2(dvacc[db][r], 0.f);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(vb & 0xffffu), rdv, (int)(el * 2u), 0, 0);
      if constexpr (ROPE) {
        buf_store_f32(rdk, el * 4u, dkacc[db][r]);
      } else {
        const uint32_t kb = pack_bf16x2(dkacc[db][r], 0.f);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(kb & 0xffffu), rdk, (int)(el * 2u), 0, 0);
      }
    }

  if constexpr (DBIAS) {
    // saturated-tile sums: reduce over the wave, then fold into the end bins
    float s0 = ub0, s1 = ub1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      s0 += __shfl_xor(s0, off);
      s1 += __shfl_xor(s1, off);
    }
    if (lane == 0) {
      ubin[wave][0] = s0;
      ubin[wave][1] = s1;
    }
    __syncthreads();
    for (int x = tid; x <= 2 * sat; x += NT) {
      float t = bins[0][x] + bins[1][x] + bins[2][x] + bins[3][x];
      if (x == 0) t += ubin[0][0] + ubin[1][0] + ubin[2][0] + ubin[3][0];
      if (x == 2 * sat) t += ubin[0][1] + ubin[1][1] + ubin[2][1] + ubin[3][1];
      bins[0][x] = t;
    }
    __syncthreads();
    for (int b = tid; b < a.nb; b += NT) {
      float t = 0.f;
      for (int x = 0; x <= 2 * sat; ++x)
        if (bkt[x] == b) t += bins[0][x];
      a.part[(size_t)b * a.nwg + g] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// dQ conversion and table-gradient reduction
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float4 *x, uint2 *y, size_t n4) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 v = x[i];
  y[i] = uint2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}

// dtable[b, h] = sum of the partials of head h, one workgroup per (b, h):
// strided per-thread sums, then a tree in LDS, both in a fixed order.
// Partials are stored bucket-major, part[b * nwg + g].
__global__ __launch_bounds__(256) void dbias_reduce_kernel(const float *part, const int4 *sched,
                                                            int nwg, int nbatch, int heads,
                                                            int ntile, float *dtable) {
  __shared__ float red[256];
  const int idx = blockIdx.x, tid = threadIdx.x;
  const int b = idx / heads, h = idx - b * heads;
  const float *pb = part + (size_t)b * nwg;
  float t = 0.f;
  if (sched != nullptr) {
    for (int gg = tid; gg < nwg; gg += 256) {
      const int4 e = sched[gg];
      if (e.y > 0 && e.z == h) t += pb[gg];
    }
  } else {
    const int n = nbatch * ntile;
    for (int i = tid; i < n; i += 256) {
      const int bb = i / ntile, tt = i - bb * ntile;
      t += pb[(bb * heads + h) * ntile + tt];
    }
  }
  red[tid] = t;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) red[tid] += red[tid + st];
    __syncthreads();
  }
  if (tid == 0) dtable[idx] = red[0];
}

template <int D, int BIAS, bool CAUSAL, bool VARLEN>
hipError_t launch_pre_t(const BwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_pre_kernel<D, BIAS, CAUSAL, VARLEN>), dim3(a.nwg), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int D, int BIAS, bool CAUSAL, bool VARLEN, bool ROPE, bool DBIAS>
hipError_t launch_main_t(const BwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_main_kernel<D, BIAS, CAUSAL, VARLEN, ROPE, DBIAS>), dim3(a.nwg),
                     dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int D, int BIAS, bool CAUSAL, bool VARLEN>
hipError_t launch_pair(const BwdArgs &a, int phase, bool rope, bool dbias, hipStream_t s) {
  if (phase == kBwdPre) return launch_pre_t<D, BIAS, CAUSAL, VARLEN>(a, s);
  if constexpr (BIAS == kBiasT5) {
    if (dbias)
      return rope ? launch_main_t<D, BIAS, CAUSAL, VARLEN, true, true>(a, s)
                  : launch_main_t<D, BIAS, CAUSAL, VARLEN, false, true>(a, s);
  }
  return rope ? launch_main_t<D, BIAS, CAUSAL, VARLEN, true, false>(a, s)
              : launch_main_t<D, BIAS, CAUSAL, VARLEN, false, false>(a, s);
}

template <int D, int BIAS>
hipError_t launch_b(const BwdArgs &a, int phase, bool causal, bool varlen, bool rope, bool dbias,
                    hipStream_t s) {
  if (causal)
    return varlen ? launch_pair<D, BIAS, true, true>(a, phase, rope, dbias, s)
                  : launch_pair<D, BIAS, true, false>(a, phase, rope, dbias, s);
  return varlen ? launch_pair<D, BIAS, false, true>(a, phase, rope, dbias, s)
                : launch_pair<D, BIAS, false, false>(a, phase, rope, dbias, s);
}

template <int D>
hipError_t launch_d(const BwdArgs &a, int phase, int bias, bool causal, bool varlen, bool rope,
                    bool dbias, hipStream_t s) {
  switch (bias) {
    case kBiasT5: return launch_b<D, kBiasT5>(a, phase, causal, varlen, rope, dbias, s);
    case kBiasAlibi: return launch_b<D, kBiasAlibi>(a, phase, causal, varlen, rope, dbias, s);
    default: return launch_b<D, kBiasNone>(a, phase, causal, varlen, rope, dbias, s);
  }
}

}  // namespace

int bwd_tile() { return BKV; }

int64_t bwd_num_parts(const Problem &p, int nsched) {
  if (p.varlen) return nsched;
  return (int64_t)p.nbatch * p.heads * ((p.seqlen + BKV - 1) / BKV);
}

hipError_t launch_bwd_phase(const Problem &p, const BwdBuffers &b, const int4 *sched, int nsched,
                            int phase, hipStream_t s) {
  static_assert(BR == BKV, "pre-pass and main kernel share the packed-batch schedule");
  BwdArgs a;
  a.q = static_cast<const uint16_t *>(b.q);
  a.k = static_cast<const uint16_t *>(b.k);
  a.v = static_cast<const uint16_t *>(b.v);
  a.dout = static_cast<const uint16_t *>(b.dout);
  a.lse = b.lse;
  a.dk = static_cast<uint16_t *>(b.dk);
  a.dv = static_cast<uint16_t *>(b.dv);
  a.dk_acc = b.dk_acc;
  a.dq_acc = b.dq_acc;
  a.delta = b.delta;
  a.part = b.part;
  a.sched = sched;
  a.table = p.table;
  a.slopes = p.slopes;
  a.nbatch = p.nbatch;
  a.seqlen = p.seqlen;
  a.heads = p.heads;
  a.total = p.total;
  a.nb = p.bias == kBiasT5 ? (p.t5.bidir ? 2 * p.t5.nbp : p.t5.nbp) : 0;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  a.t5 = p.t5;
  if (p.varlen) {
    a.ntile = 0;
    a.nwg = nsched;
  } else {
    a.ntile = (p.seqlen + BKV - 1) / BKV;
    a.nwg = p.nbatch * p.heads * a.ntile;
  }
  if (a.nwg <= 0) return hipSuccess;
  const bool rope = p.rope_base > 0.f;
  const bool dbias = b.part != nullptr;
  if (phase == kBwdReduce) {
    if (!dbias) return hipSuccess;
    hipLaunchKernelGGL(dbias_reduce_kernel, dim3(a.nb * p.heads), dim3(256), 0, s, a.part,
                       sched, a.nwg, p.nbatch, p.heads, a.ntile, b.dtable);
    return hipGetLastError();
  }
  return p.head_dim == 64 ? launch_d<64>(a, phase, p.bias, p.causal, p.varlen, rope, dbias, s)
                          : launch_d<128>(a, phase, p.bias, p.causal, p.varlen, rope, dbias, s);
}

hipError_t launch_f32_to_bf16(const float *x, void *y, size_t n, hipStream_t s) {
  const size_t n4 = n / 4;   // n is a multiple of head_dim, hence of 4
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const float4 *>(x), static_cast<uint2 *>(y), n4);
  return hipGetLastError();
}

}  // namespace fa
