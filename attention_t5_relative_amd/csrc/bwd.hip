// Backward attention for gfx950.  The pages print no backward; this is the
// calculus of the forward they describe (FAT5 report, "Noyau CUDA"), with
// the bias table trained through the gradient of S':
//
//   dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K,
//   dTable[b, h] = sum over (i, j) with bucket b of dS_ij.
//
// Two kernels per call, each owning its outputs (no atomics):
//   dq   query-parallel, forward-shaped (128 queries per workgroup, 32 per
//        wave, 64-key tiles of K and V in LDS).  One sweep over the keys
//        recomputes P in fp32 with dP.  About a centre Dc_i = dO_i . O_i
//        (bf16 O) it accumulates D_i - Dc_i = sum_j P_ij (dP_ij - Dc_i),
//        A = K^T (P o (dP - Dc))^T and B = K^T P^T (K's operand by the
//        transposing LDS read), and ends with dQ = scale (A - (D - Dc) B).
//        D = Dc + (D - Dc) is written for the dkv kernel: it comes from the
//        recomputed P, so O's bf16 rounding, which would dominate the dQ and
//        dK errors if D were rowsum(dO * O), cancels.
//   dkv  key-parallel (128 keys per workgroup, 32 per wave): query blocks of
//        Q, dO (row-major) and their LSE and D go through double-buffered LDS;
//        S = Q K^T puts each lane on one key, so P and dS serve as MFMA B
//        operands from registers for dV^T = dO^T P and dK^T = Q^T dS, whose
//        A operands come from the same row-major tiles through the
//        transposing read.  The table gradient is binned by relative
//        distance in per-half-wave LDS bins (whole saturated blocks in
//        registers) and reduced in a fixed order.
// The large operands of the dQ and dK products (P o (dP - Dc), or dS) enter
// the MFMAs as bf16 hi + lo pairs (16 significant bits); with bf16 alone the
// gradients miss the accuracy gate.  P enters the dV product the same way:
// with bf16 P alone, dV's elementwise-normalised error reached 1.94e-2 on the
// causal S = 4096 workload, against a gate of 2e-2.
#include <type_traits>

#include "fa_device.h"

namespace fa {
namespace {

constexpr int NT = 256;
constexpr int BR = 128;    // dq: query rows per workgroup
constexpr int BC = 64;     // dq: keys per tile at head_dim 64 (32 at 128)
constexpr int BKV = 128;   // dkv: keys per workgroup

struct BwdArgs {
  const uint16_t *q, *k, *v, *o, *dout;
  const float *lse;
  const float *dlse;       // gradient with respect to lse (lse layout) or nullptr
  uint16_t *dq, *dk, *dv;  // bf16 outputs
  const double2 *rope_cs;   // RoPE: (cos, sin) [seqlen, D/2], or nullptr
  const float *fire_tab;   // FIRE segment table (fa_internal.h), or nullptr
  const float *fire_dist;  // FIRE distance table, or nullptr
  float *delta;            // -D_i, same layout as lse
  float *nls;              // -lse_i / scale, same layout (seed of the dkv kernel's S)
  float *part;             // [nb, nwg] table-gradient partials (FIRE: nb = kFireGradRows)
  const int4 *sched;       // packed batches: {token0, length, head, tile}
  const float *table, *slopes;
  const uint16_t *dense;   // dense bias bf16 [dense_batch, H, S, S]
  float *dbias;            // dense bias gradient fp32, one [S, S] per (batch, head) (the
                           // summing kernel: one per head)
  int32_t dense_batch;
  int32_t nbatch, seqlen, heads, total;
  int32_t ntile;           // dense: tiles of 128 per sequence
  int32_t nwg;
  int32_t nb;
  float scale, scale_log2;
  T5Geometry t5;
};

struct Work {
  int b, h, tile, tok0, L;   // b: batch index (dense only)
  int part;                // table-gradient partial slot (reduction order)
  size_t lse_base;         // index of row 0 in lse / delta
};

// Dense: logical id -> (batch, head, tile) with tile = g % ntile.
// Packed: the schedule entry.  Returns false for an empty entry.
template <bool VARLEN>
__device__ __forceinline__ bool locate(const BwdArgs &a, int g, Work &w) {
  if constexpr (VARLEN) {
    const int4 e = a.sched[g];
    if (e.y <= 0) return false;
    w.b = 0;
    w.tok0 = e.x;
    w.L = e.y;
    w.h = e.z;
    w.tile = e.w;
    w.part = g;
    w.lse_base = (size_t)w.h * a.total + w.tok0;
  } else {
    int pair;
    tile_order<4>(g, a.nbatch * a.heads, a.ntile, pair, w.tile);   // 2 workgroups per CU
    w.part = pair * a.ntile + w.tile;
    int b;
    pair_bh(pair, a.nbatch, a.heads, a.dense != nullptr && a.dense_batch == 1, b, w.h);
    w.b = b;
    w.tok0 = b * a.seqlen;
    w.L = a.seqlen;
    w.lse_base = ((size_t)b * a.heads + w.h) * a.seqlen;
  }
  return true;
}

// A pair (x0, x1) as bf16 hi + lo pairs: hi = the nearest bf16 values, lo =
// the rounded remainders (16 significant bits together).  The remainders
// x - bf16(x), exact in fp32, come from one bf16 dot product each against
// (-1, 0) and (0, -1): hi.lo * -1 + hi.hi * 0 + x0, instead of unpacking a
// half and subtracting it.  The two constant pairs must reach the dot
// product from registers (see NegPairs).
struct NegPairs {
  bf16x2 m10, m01;   // (-1, 0) and (0, -1)
};
__device__ __forceinline__ NegPairs neg_pairs() {
  // kept opaque: as an inline constant the hardware would read the packed
  // bf16 operand -1.0 differently
  int a = 0x0000bf80, b = (int)0xbf800000u;
  asm volatile("" : "+s"(a), "+s"(b));
  return NegPairs{__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b)};
}
__device__ __forceinline__ void split_hi_lo(float x0, float x1, uint32_t &hi, uint32_t &lo,
                                            const NegPairs &n) {
  hi = pack_bf16x2(x0, x1);
  const bf16x2 h = __builtin_bit_cast(bf16x2, hi);
  lo = pack_bf16x2(__builtin_amdgcn_fdot2_f32_bf16(h, n.m10, x0, false),
                   __builtin_amdgcn_fdot2_f32_bf16(h, n.m01, x1, false));
}

__device__ __forceinline__ bf16x8 frag(const uint32_t (&w)[4]) {
  return __builtin_bit_cast(bf16x8, i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]});
}

// RoPE: turn back the pairs of a row's gradient held in MFMA accumulators
// (lane: dims 32db + 8(r/4) + 4hl + r%4 of row t, i.e. pairs 16db + 4(r/4) +
// 2hl + {0, 1}) with the fp64 (cos, sin) table cs [npos, D/2]: a gradient
// with respect to the rotated row becomes one with respect to the row before
// the rotation.  Rows past the table read (cos, sin) = 0; they are past the
// sequence and never stored.
template <int D>
__device__ __forceinline__ void rope_unrotate_acc(f32x16 (&acc)[D / 32], const double2 *cs,
                                                  int npos, int t, int hl) {
  const rsrc_t rcs = make_rsrc(cs, (uint32_t)npos * (uint32_t)(D / 2) * 16u);
  const uint32_t t0 = ((uint32_t)t * (uint32_t)(D / 2) + 2 * hl) * 16u;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const RopeCs2 c = rope_cs2(rcs, t0 + (16 * db + 4 * rq) * 16u);
      const double a0 = acc[db][4 * rq], a1 = acc[db][4 * rq + 1], a2 = acc[db][4 * rq + 2],
                   a3 = acc[db][4 * rq + 3];
      acc[db][4 * rq] = (float)fma(a0, c.c0, a1 * c.s0);
      acc[db][4 * rq + 1] = (float)fma(a1, c.c0, -a0 * c.s0);
      acc[db][4 * rq + 2] = (float)fma(a2, c.c1, a3 * c.s1);
      acc[db][4 * rq + 3] = (float)fma(a3, c.c1, -a2 * c.s1);
    }
}

// ---------------------------------------------------------------------------
// dq kernel
// ---------------------------------------------------------------------------
// Workgroups per CU of the dq kernel (the dense bias's per-tile values and
// the FIRE lookups need more registers than two workgroups leave at
// head_dim 128).
template <int D, int BIAS>
constexpr int dq_wgs() {
  return D == 64 || (BIAS != kBiasDense && BIAS != kBiasFire) ? 2 : 1;
}

// WHOLE (dense batches with T5 at head_dim 64): the sequence length is a
// multiple of the 64-key tile, so the per-element length test of tiles near
// the diagonal drops out.
template <int D, int BIAS, bool CAUSAL, bool VARLEN, bool WHOLE = false>
__global__ __launch_bounds__(NT, (dq_wgs<D, BIAS>())) void bwd_dq_kernel(const BwdArgs a) {
  // K and V tiles, swizzled (see swz): K is read both row-wise
  // (S^T = K Q^T) and transposed (dQ^T = K^T dS^T), V row-wise.  At
  // head_dim 128 the tiles hold 32 keys and the workgroup's dO rows (the B
  // operand of dP^T) sit in LDS rather than in 32 VGPRs, which fits two
  // workgroups per CU.
  constexpr int KT = D == 64 ? BC : 32;   // keys per tile
  constexpr int NKB = KT / 32;
  constexpr bool kDoInLds = D == 128;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t dost[kDoInLds ? BR * D : 8];
  __shared__ float lut_mem[BIAS == kBiasT5 ? 2 * (kMaxDistance + kLutPad) + 1 : 1];
  const float *const lut = lut_mem + (BIAS == kBiasT5 ? a.t5.sat + kLutPad : 0);
  __shared__ float fire_mem[BIAS == kBiasFire ? kFireLds : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, il = lane & 31;
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
  const rsrc_t rdo = make_rsrc(a.dout + base, nrec);
  const rsrc_t ro = make_rsrc(a.o + base, nrec);

  const int q0 = qt * BR;
  const int wrow0 = q0 + 32 * wave;
  const int myrow = wrow0 + il;
  const bool wave_live = wrow0 < L;

  bf16x8 qf[D / 16], df[D / 16];
  i32x4 of[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint32_t off = ((uint32_t)myrow * (uint32_t)HD + 16 * s + 8 * hl) * 2u;
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    df[s] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
    of[s] = buf_load16(ro, off);
  }
  if constexpr (kDoInLds)
    dma_tile<D, BR, 4>(dma_desc(a.dout + base, nrec), HD, q0, dost, wave, lane);
  const float lse2 = myrow < L ? a.lse[w.lse_base + myrow] * kLog2e : 0.f;
  // A gradient dlse_i with respect to the returned LSE adds dlse_i P_ij to
  // dS_ij: the same as replacing D_i by D_i - dlse_i everywhere below
  // (here and, through -D, in the dkv kernel).
  const float dl = (a.dlse != nullptr && myrow < L) ? a.dlse[w.lse_base + myrow] : 0.f;

  int sat = 0;
  if constexpr (BIAS == kBiasT5) {
    // bias (log2 units) by relative position r = j - i (see kLutPad)
    sat = a.t5.sat;
    for (int x = tid; x <= 2 * (sat + kLutPad); x += NT) {
      const int r = x - sat - kLutPad;
      lut_mem[x] = (CAUSAL && r > 0) ? -INFINITY
                                     : a.table[t5_bucket_dev(r, a.t5) * a.heads + h] * kLog2e;
    }
  }
  float slope_l2 = 0.f;
  if constexpr (BIAS == kBiasAlibi) slope_l2 = -a.slopes[h] * kLog2e;
  rsrc_t rbias = make_rsrc(nullptr, 0u);
  if constexpr (BIAS == kBiasDense) {
    const size_t mat = (size_t)(a.dense_batch == 1 ? 0 : w.b) * a.heads + h;
    rbias = make_rsrc(a.dense + mat * L * L, (uint32_t)L * (uint32_t)L * 2u);
  }
  FireLane fl;
  if constexpr (BIAS == kBiasFire) {
    fire_load(a.fire_tab, h, fire_mem, tid, NT);
    fl = fire_lane(a.fire_tab, a.fire_dist, a.seqlen, fire_mem, myrow);
  }

  const int kend = CAUSAL ? min(L, q0 + BR) : L;
  const int nkt = (kend + KT - 1) / KT;
  // one key tile to LDS by buffer-to-LDS copies split over the four waves
  const i32x4 dk_src = dma_desc(a.k + base, nrec), dv_src = dma_desc(a.v + base, nrec);
  auto fill = [&](int j0, int buf) {
    dma_tile<D, KT, 4>(dk_src, HD, j0, ks[buf], wave, lane);
    dma_tile<D, KT, 4>(dv_src, HD, j0, vs[buf], wave, lane);
  };
  // row-wise operands: row il, chunk 2s + hl; transposed K operand: the two
  // halves of each 16-row group, per 32-column block
  int kof[D / 16], tro[D / 32][2];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) kof[s] = swz_off<D>(il, 2 * s + hl);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    tro[db][0] = swz_tr_off<D>(lane, 0, db);
    tro[db][1] = swz_tr_off<D>(lane, 1, db);
  }
  const float c = a.scale_log2;
  const float dscale = a.scale;
  const NegPairs negp = neg_pairs();

  // One sweep over the keys.  dQ_i = scale * sum_j P_ij (dP_ij - D_i) k_j
  // needs D_i = sum_j P_ij dP_ij, known only after the last key, so it is
  // accumulated about a per-row centre Dc_i known up front:
  //   dQ_i = scale * (A_i - (D_i - Dc_i) B_i),
  //   A_i = sum_j P_ij (dP_ij - Dc_i) k_j,  B_i = sum_j P_ij k_j,
  // with D_i - Dc_i = sum_j P_ij (dP_ij - Dc_i) (rows of P sum to one).
  // A's operand enters the MFMAs as a bf16 hi + lo pair (16 significant
  // bits); B's as bf16 alone, as its factor D_i - Dc_i is tiny.
  float dsum = 0.f;   // sum_j P_ij (dP_ij - Dc_i) over this lane's keys
  f32x16 aacc[D / 32], bacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    aacc[db] = f32x16{};
    bacc[db] = f32x16{};
  }

  wait_vmem_loads();
  // Centre Dc_i = dO_i . O_i from the bf16 O: it differs from D_i by O's
  // rounding only, so P o (dP - Dc) and the D_i - Dc_i that multiplies B are
  // both small.  Any finite Dc gives the same result up to rounding; a
  // non-finite one (O not the forward's output) falls back to 0.
  float dc = 0.f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const i32x4 d4 = __builtin_bit_cast(i32x4, df[s]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dc = fmaf(bf16_lo((uint32_t)of[s][e]), bf16_lo((uint32_t)d4[e]), dc);
      dc = fmaf(bf16_hi((uint32_t)of[s][e]), bf16_hi((uint32_t)d4[e]), dc);
    }
  }
  dc = half_sum(dc);
  if ((__builtin_bit_cast(uint32_t, dc) & 0x7f800000u) == 0x7f800000u) dc = 0.f;
  if (nkt > 0) fill(0, 0);
  wait_vmem_loads();
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int j0 = kt * KT;
    const int buf = kt & 1;
    if (kt + 1 < nkt) fill(j0 + KT, buf ^ 1);
    const bool active = wave_live && (!CAUSAL || (j0 <= wrow0 + 31));
    uint16_t bv[2][16];
    if constexpr (BIAS == kBiasDense)
      if (active) dense_row_load(rbias, myrow, L, j0, hl, bv);
    f32x16 sacc[NKB], pacc[NKB];
    if (active) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc[kb] = f32x16{};
        pacc[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&ks[buf][kof[s] + 32 * kb * D]);
          const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&vs[buf][kof[s] + 32 * kb * D]);
          bf16x8 dfs;
          if constexpr (kDoInLds)
            dfs = *reinterpret_cast<const bf16x8 *>(&dost[kof[s] + 32 * wave * D]);
          else
            dfs = df[s];
          sacc[kb] = mfma32(kf, qf[s], sacc[kb]);
          pacc[kb] = mfma32(vf, dfs, pacc[kb]);
        }
      }
    }
    if (active) {
      float bconst;
      bool fast;
      if constexpr (NKB == 2)
        fast = score_tile_T<BIAS, CAUSAL, true, false, WHOLE>(sacc, j0, wrow0, il, hl, L, c, sat,
                                                              lut, slope_l2,
                                          bconst, bv, &fl);
      else
        fast = score_block_T<BIAS, CAUSAL>(sacc[0], j0, wrow0, il, hl, L, c, sat, lut,
                                           slope_l2, bconst, bv[0], &fl);
      const float cc = fast ? c : 1.f;
      const float sub = bconst - lse2;
      // per 16-key group: P o (dP - Dc) as hi + lo fragments and P as bf16,
      // consumed at once by A^T += K^T (P o (dP - Dc))^T and B^T += K^T P^T,
      // K's operand by transposing reads
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          uint32_t xh[4], xl[4], ph[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * u + 2 * e;
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], cc, sub));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + 1], cc, sub));
            const float x0 = p0 * (pacc[kb][r] - dc), x1 = p1 * (pacc[kb][r + 1] - dc);
            dsum += x0 + x1;
            split_hi_lo(x0, x1, xh[e], xl[e], negp);
            ph[e] = pack_bf16x2(p0, p1);
          }
          const bf16x8 xhb = frag(xh), xlb = frag(xl), phb = frag(ph);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const bf16x8 kt8 =
                lds_read_tr8_at(&ks[buf][(32 * kb + 16 * u) * D], tro[db][0], tro[db][1]);
            aacc[db] = mfma32(kt8, xhb, aacc[db]);
            aacc[db] = mfma32(kt8, xlb, aacc[db]);
            bacc[db] = mfma32(kt8, phb, bacc[db]);
          }
        }
    }
    // the next tile's copies have landed (each wave waits for its own)
    wait_vmem_loads();
    __syncthreads();
  }
  const float dd = half_sum(dsum) - dl;   // D_i - dlse_i - Dc_i
  if (hl == 0 && myrow < L) {
    a.delta[w.lse_base + myrow] = -(dc + dd);
    a.nls[w.lse_base + myrow] = -a.lse[w.lse_base + myrow] / a.scale;
  }
  f32x16 qacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) qacc[db][r] = dscale * fmaf(-dd, bacc[db][r], aacc[db][r]);

  // dQ row myrow: lane holds dims 32db + 8(r/4) + 4hl + r%4.  With RoPE the
  // gradient is with respect to the rotated row: turn each pair back
  // (pairs 16db + 4(r/4) + 2hl + {0, 1}) before rounding to bf16.
  if (a.rope_cs != nullptr)
    rope_unrotate_acc<D>(qacc, a.rope_cs, a.seqlen, myrow, hl);
  const rsrc_t rdq = make_rsrc(a.dq + base, nrec);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      i32x2 w2 = {(int)pack_bf16x2(qacc[db][4 * rq], qacc[db][4 * rq + 1]),
                  (int)pack_bf16x2(qacc[db][4 * rq + 2], qacc[db][4 * rq + 3])};
      buf_store8(rdq, ((uint32_t)myrow * (uint32_t)HD + 32 * db + 8 * rq + 4 * hl) * 2u, w2);
    }
}

// ---------------------------------------------------------------------------
// FIRE parameter gradient: a query-parallel pass after the dq kernel
// ---------------------------------------------------------------------------
// The five per-(head, segment) sums of fire.hip need dS with the exact D,
// which the dq kernel knows only after its sweep.  This pass repeats the
// dq kernel's S and dP products (no dQ products, no hi/lo splits) with D
// read back, so each lane owns one query row: the row's weights (1 / log2 E,
// max(L, i) / (E ln E), [i < L]) are per-lane constants and only three sums
// per element remain (dS, dS x, dS d / e), weighted per lane when the
// wave's run in a segment ends.  Along the sweep (keys ascending) a row's x
// only falls, so a wave passes each segment about once.
template <int D, bool VARLEN>
__global__ __launch_bounds__(NT, 2) void bwd_fire_kernel(const BwdArgs a) {
  constexpr int KT = D == 64 ? BC : 32;
  constexpr int NKB = KT / 32;
  constexpr bool kDoInLds = D == 128;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t dost[kDoInLds ? BR * D : 8];
  __shared__ float fire_mem[kFireLds];
  __shared__ float fire_acc[4 * kFireGradRows];   // per wave

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, il = lane & 31;
  const int g = xcd_remap(blockIdx.x, a.nwg);
  Work w;
  if (!locate<VARLEN>(a, g, w)) return;
  const int L = w.L, h = w.h;
  const int qt = VARLEN ? w.tile : (a.ntile - 1 - w.tile);

  const int HD = a.heads * D;
  const size_t base = ((size_t)w.tok0 * a.heads + h) * D;
  const uint32_t nrec = ((uint32_t)(L - 1) * (uint32_t)HD + D) * 2u;
  const rsrc_t rq = make_rsrc(a.q + base, nrec);
  const rsrc_t rdo = make_rsrc(a.dout + base, nrec);
  const int q0 = qt * BR;
  const int wrow0 = q0 + 32 * wave;
  const int myrow = wrow0 + il;
  const bool wave_live = wrow0 < L;
  const bool row_live = myrow < L;

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint32_t off = ((uint32_t)myrow * (uint32_t)HD + 16 * s + 8 * hl) * 2u;
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    df[s] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
  }
  if constexpr (kDoInLds)
    dma_tile<D, BR, 4>(dma_desc(a.dout + base, nrec), HD, q0, dost, wave, lane);
  const float lse2 = row_live ? a.lse[w.lse_base + myrow] * kLog2e : 0.f;
  const float nd = row_live ? a.delta[w.lse_base + myrow] : 0.f;   // -D_i (dlse folded in)

  fire_load(a.fire_tab, h, fire_mem, tid, NT);
  for (int i = tid; i < 4 * kFireGradRows; i += NT) fire_acc[i] = 0.f;
  FireLane fl = fire_lane(a.fire_tab, a.fire_dist, a.seqlen, fire_mem, myrow);
  // the row's weights of dx/dc and dx/dL (see fire.hip)
  const float fc = a.fire_tab[2], fL = a.fire_tab[3];
  const float mrow = fmaxf(fL, (float)myrow);
  const float Erow = fmaf(fc, mrow, 1.f);
  const float wc = mrow * fl.inv / (Erow * kLn2);
  const float lf = (float)myrow < fL ? 1.f : 0.f;
  // Sums of the wave's current segment w_cur, per lane, until the wave's
  // keys leave it; then each lane weights its row's terms, the wave adds
  // them up (DPP moves in a fixed order) and lane 63 adds them to the
  // wave's own LDS sums: no atomics, one flush per segment change.
  float u0 = 0.f, u1 = 0.f, u2 = 0.f;
  int w_cur = -1;
  float *const my_acc = fire_acc + wave * kFireGradRows;
  auto flush = [&](int sg, float g0, float g1, float g2) {
    float t[kFireTerms] = {g0, g1, g2 * fl.inv, g1 * wc, g1 * lf};
#pragma unroll
    for (int q = 0; q < kFireTerms; ++q) t[q] = wave_sum_lane63(t[q]);
    if (lane == 63)
#pragma unroll
      for (int q = 0; q < kFireTerms; ++q) my_acc[sg * kFireTerms + q] += t[q];
  };

  const int kend = min(L, q0 + BR);
  const int nkt = (kend + KT - 1) / KT;
  const i32x4 dk_src = dma_desc(a.k + base, nrec), dv_src = dma_desc(a.v + base, nrec);
  auto fill = [&](int j0, int buf) {
    dma_tile<D, KT, 4>(dk_src, HD, j0, ks[buf], wave, lane);
    dma_tile<D, KT, 4>(dv_src, HD, j0, vs[buf], wave, lane);
  };
  int kof[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) kof[s] = swz_off<D>(il, 2 * s + hl);
  const float c = a.scale_log2;

  wait_vmem_loads();
  if (nkt > 0) fill(0, 0);
  wait_vmem_loads();
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int j0 = kt * KT;
    const int buf = kt & 1;
    if (kt + 1 < nkt) fill(j0 + KT, buf ^ 1);
    const bool active = wave_live && j0 <= wrow0 + 31;
    if (active) {
      f32x16 sacc[NKB], pacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc[kb] = f32x16{};
        pacc[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&ks[buf][kof[s] + 32 * kb * D]);
          const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&vs[buf][kof[s] + 32 * kb * D]);
          bf16x8 dfs;
          if constexpr (kDoInLds)
            dfs = *reinterpret_cast<const bf16x8 *>(&dost[kof[s] + 32 * wave * D]);
          else
            dfs = df[s];
          sacc[kb] = mfma32(kf, qf[s], sacc[kb]);
          pacc[kb] = mfma32(vf, dfs, pacc[kb]);
        }
      }
      // scores with the bias, every key's x and the lane's segment range
      constexpr int omax = 32 * NKB - 5;   // the lane's farthest key offset
      const int rbase = j0 - myrow + 4 * hl;
      const int jb = j0 + 4 * hl;
      const bool mask_l = j0 + KT > L;
      float xs[NKB][16];
      int shi;
      // (the causal mask reaches this tile when its last key follows the
      // wave's first row)
      fire_scores<NKB, true, true>(sacc, omax, rbase, mask_l ? L - jb : KT, j0 + KT - 1 > wrow0,
                                   c, fl, xs,
                                   &shi);
      const int slo = fl.seg;
      // dS
      float gs[NKB][16];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(sacc[kb][r] - lse2);
          gs[kb][r] = row_live ? p * (pacc[kb][r] + nd) : 0.f;
        }
      // the three sums of the keys at or above kink t_sg (x >= t_sg; ALL:
      // every key, with no compare); d / e from the distance table (element
      // 3 - e of the four entries from distance -rbase - 32 kb - 8 q - 3)
      auto sums_from = [&](auto all, int sg, float &g0, float &g1, float &g2) {
        constexpr bool ALL = decltype(all)::value;
        const float tlo = ALL ? -INFINITY : fl.tab[kFireOffT + sg];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 de = fire_dist4(fl, -rbase - 32 * kb - 8 * q - 3, fl.dist_half);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * q + e;
              const float x = xs[kb][r];
              const float gv = (ALL || x >= tlo) ? gs[kb][r] : 0.f;
              g0 += gv;
              g1 = fmaf(gv, x, g1);
              g2 = fmaf(gv, de[3 - e], g2);
            }
          }
      };
      // the wave's segment range over its lanes' ranges
      int wlo = slo, whi = shi;
      wave_min_max(wlo, whi);
      if (wlo == whi) {
        if (wlo != w_cur) {
          if (w_cur >= 0) flush(w_cur, u0, u1, u2);
          u0 = u1 = u2 = 0.f;
          w_cur = wlo;
        }
        sums_from(std::true_type{}, 0, u0, u1, u2);
      } else {
        if (w_cur >= 0) flush(w_cur, u0, u1, u2);
        u0 = u1 = u2 = 0.f;
        w_cur = -1;
        // from the top segment down, the sums over x >= t_sg (one compare
        // per key); a segment's own sums are the differences of consecutive
        // ones (x falls along a lane's keys, so every key lies in [wlo, whi])
        float h0 = 0.f, h1 = 0.f, h2 = 0.f;
        for (int sg = whi; sg >= wlo; --sg) {
          float c0 = 0.f, c1 = 0.f, c2 = 0.f;
          sums_from(std::false_type{}, sg, c0, c1, c2);
          flush(sg, c0 - h0, c1 - h1, c2 - h2);
          h0 = c0;
          h1 = c1;
          h2 = c2;
        }
      }
    }
    wait_vmem_loads();
    __syncthreads();
  }
  // (wave-uniform: every lane of a wave sees the same w_cur)
  if (w_cur >= 0) flush(w_cur, u0, u1, u2);
  __syncthreads();
  // the four waves' sums in a fixed order, one partial per workgroup
  for (int i = tid; i < kFireGradRows; i += NT) {
    float t = 0.f;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) t += fire_acc[w4 * kFireGradRows + i];
    a.part[(size_t)i * a.nwg + w.part] = t;
  }
}

// ---------------------------------------------------------------------------
// dkv kernel
// ---------------------------------------------------------------------------
template <int D>
struct DkvTile {
  static constexpr int QB = (D == 64) ? 64 : 32;   // query rows per block
};

// Dynamic LDS of the dkv kernel: the T5 bias table by distance (2 (sat +
// kLutPad) + 1 entries, see kLutPad), then (with the table gradient) the
// bucket of each distance in [-sat, sat], one array of
// 2 * sat + 1 distance bins per wave, and one 32 x 40 fp32 scratch tile per
// wave for the diagonal sums, with kTileGuard floats on either side of the
// tiles (the diagonal reads of masked-out rows reach up to 32 floats past a
// tile; their values are discarded).
constexpr int kTilePitch = 40;
constexpr int kTileGuard = 32;
__host__ __device__ inline size_t dkv_dyn_bytes(int sat, bool t5, bool dbias) {
  if (!t5) return 0;
  const size_t n = (size_t)(2 * sat + 1);
  const size_t nl = (size_t)(2 * (sat + kLutPad) + 1);
  return nl * 4 + (dbias ? n * 4 + 4 * n * 4 + (4 * 32 * kTilePitch + 2 * kTileGuard) * 4 : 0);
}

// Workgroups per CU.  At head_dim 128 with ALiBi or no bias the keys' V
// rows (the B operand of dP) stay in LDS and are read per block, and the
// row offsets of the Q/dO operands are computed where they are used, which
// leaves room for two workgroups per CU without spilling; the T5 (with its
// table gradient) and dense-bias variants need the registers and run one.
template <int D, int BIAS>
constexpr int dkv_wgs() {
  return D == 64 || BIAS == kBiasAlibi || BIAS == kBiasNone ? 2 : 1;
}

template <int D, int BIAS, bool CAUSAL, bool VARLEN, bool DBIAS>
__global__ __launch_bounds__(NT, (dkv_wgs<D, BIAS>())) void bwd_dkv_kernel(const BwdArgs a) {
  constexpr int QB = DkvTile<D>::QB;
  constexpr bool kVInLds = D == 128 && (BIAS == kBiasAlibi || BIAS == kBiasNone);
  __shared__ __attribute__((aligned(16))) uint16_t vtile[kVInLds ? BKV * D : 8];
  // Q and dO blocks as swizzled tiles (see swz), with the rows' -lse/scale
  // and -D (64 entries: the 4-byte copy fills one per lane)
  __shared__ __attribute__((aligned(16))) uint16_t qs[2][QB * D];
  __shared__ __attribute__((aligned(16))) uint16_t dos[2][QB * D];
  __shared__ __attribute__((aligned(16))) float nlss[2][64];
  __shared__ __attribute__((aligned(16))) float ndls[2][64];
  __shared__ float ubin[4][2];
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  constexpr bool kFire = BIAS == kBiasFire;
  __shared__ float fire_mem[kFire ? kFireLds : 1];
  __shared__ __attribute__((aligned(16))) float fire_rows[kFire ? 2 * 64 : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, il = lane & 31;
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
  const bool wave_live = kw0 < L;

  const int HD = a.heads * D;
  const size_t base = ((size_t)w.tok0 * a.heads + h) * D;
  const uint32_t nrec = ((uint32_t)(L - 1) * (uint32_t)HD + D) * 2u;
  const rsrc_t rk = make_rsrc(a.k + base, nrec);
  const rsrc_t rv = make_rsrc(a.v + base, nrec);

  // this wave's 32 keys as the B operand of S = Q K^T and dP = dO V^T
  bf16x8 kf[D / 16], vf[kVInLds ? 1 : D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint32_t off = ((uint32_t)myk * (uint32_t)HD + 16 * s + 8 * hl) * 2u;
    kf[s] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
    if constexpr (!kVInLds) vf[s] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
  }
  if constexpr (kVInLds)
    dma_tile<D, BKV, 4>(dma_desc(a.v + base, nrec), HD, kt0, vtile, wave, lane);

  int sat = 0;
  const int nlut = 2 * (a.t5.sat + kLutPad) + 1;
  float *const lut_mem = dyn;
  const float *const lut = lut_mem + (a.t5.sat + kLutPad);   // distance 0
  int *bkt = reinterpret_cast<int *>(dyn + nlut);
  const int nbin = 2 * a.t5.sat + 1;
  float *bins = dyn + nlut + nbin;
  float *const tiles = bins + 4 * nbin + kTileGuard;
  if constexpr (BIAS == kBiasT5) {
    sat = a.t5.sat;
    for (int x = tid; x < nlut; x += NT) {
      const int r = x - sat - kLutPad;
      lut_mem[x] = (CAUSAL && r > 0) ? -INFINITY
                                     : a.table[t5_bucket_dev(r, a.t5) * a.heads + h] * kLog2e;
    }
    if constexpr (DBIAS) {
      for (int x = tid; x < nbin; x += NT) {
        bkt[x] = t5_bucket_dev(x - sat, a.t5);
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) bins[w4 * nbin + x] = 0.f;
      }
    }
  }
  float slope_l2 = 0.f;
  if constexpr (BIAS == kBiasAlibi) slope_l2 = -a.slopes[h] * kLog2e;
  // dense bias: this (batch, head)'s [S, S] matrix; its gradient goes to the
  // (batch, head) matrix of a.dbias
  rsrc_t rbias = make_rsrc(nullptr, 0u), rdbias = make_rsrc(nullptr, 0u);
  if constexpr (BIAS == kBiasDense) {
    const size_t mat = (size_t)(a.dense_batch == 1 ? 0 : w.b) * a.heads + h;
    rbias = make_rsrc(a.dense + mat * L * L, (uint32_t)L * (uint32_t)L * 2u);
    if constexpr (DBIAS)
      rdbias = make_rsrc(a.dbias + ((size_t)w.b * a.heads + h) * L * L,
                         (uint32_t)L * (uint32_t)L * 4u);
  }
  float *const mybins = bins + wave * nbin;
  float *const mytile = tiles + wave * (32 * kTilePitch);
  FireLane fl;
  float fire_c = 0.f, fire_L = 0.f;
  if constexpr (kFire) {
    fire_load(a.fire_tab, h, fire_mem, tid, NT);
    fl = fire_lane(a.fire_tab, a.fire_dist, a.seqlen, fire_mem, 0);
    fire_c = a.fire_tab[2];
    fire_L = a.fire_tab[3];
  }
  // FIRE: each row's 1 / log2(c max(L, i) + 1) for the query block at q0,
  // into buffer buf
  auto fire_fill_rows = [&](int q0, int buf) {
    if constexpr (kFire) {
      if (tid < QB) {
        const int i = q0 + tid;
        fire_rows[buf * 64 + tid] =
            1.f / __builtin_amdgcn_logf(fmaf(fire_c, fmaxf(fire_L, (float)i), 1.f));
      }
    }
  };

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }
  float ub0 = 0.f, ub1 = 0.f;   // table-gradient sums of saturated blocks (low / high side)

  const float c = a.scale_log2;
  const float dscale = a.scale;
  const NegPairs negp = neg_pairs();
  const int nqb = (L + QB - 1) / QB;
  const int qb_first = CAUSAL ? (kt0 / QB) : 0;

  // one query block to LDS by buffer-to-LDS copies: Q and dO tiles split
  // over the four waves, LSE and -D one 4-byte copy each
  const i32x4 dq_src = dma_desc(a.q + base, nrec), ddo_src = dma_desc(a.dout + base, nrec);
  const i32x4 dlse_src = dma_desc(a.nls + w.lse_base, (uint32_t)L * 4u);
  const i32x4 dnd_src = dma_desc(a.delta + w.lse_base, (uint32_t)L * 4u);
  auto fill = [&](int q0, int buf) {
    dma_tile<D, QB, 4>(dq_src, HD, q0, qs[buf], wave, lane);
    dma_tile<D, QB, 4>(ddo_src, HD, q0, dos[buf], wave, lane);
    if (wave == 0) dma4(dlse_src, (uint32_t)(q0 + lane) * 4u, nlss[buf]);
    if (wave == 1) dma4(dnd_src, (uint32_t)(q0 + lane) * 4u, ndls[buf]);
  };

  // row-wise A operand: row il, chunk 2s + hl; transposed A operand: the
  // two halves of each 16-row group, per 32-column block
  int aof[kVInLds ? 1 : D / 16], tro[D / 32][2];
  if constexpr (!kVInLds) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) aof[s] = swz_off<D>(il, 2 * s + hl);
  }
  // swz_off(il, 2s + hl) = il D + 8 (hl ^ (w & 1)) + 16 (s ^ (w >> 1)), w = swz(il)
  const int aw = swz<D>(il);
  const int abase = il * D + 8 * (hl ^ (aw & 1));
  auto aoff = [&](int s) { return kVInLds ? abase + 16 * (s ^ (aw >> 1)) : aof[s]; };
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    tro[db][0] = swz_tr_off<D>(lane, 0, db);
    tro[db][1] = swz_tr_off<D>(lane, 1, db);
  }

  if (qb_first < nqb) {
    fill(qb_first * QB, 0);
    fire_fill_rows(qb_first * QB, 0);
  }
  wait_vmem_loads();
  __syncthreads();
  // S - lse/scale and dP - D of one 32-row block: each lane holds key myk
  // and rows irow0 + 8(r/4) + 4hl + r%4.  Both accumulators start at their
  // row's offset (-lse_i / scale, -D_i), read from LDS straight into the
  // MFMAs' C operands, so that P = exp2(scale log2(e) acc + bias) costs one
  // VALU operation before the exponential.
  auto block_sdp = [&](int buf, int rb, f32x16 &sacc, f32x16 &pacc) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&ndls[buf][32 * rb + 8 * qq + 4 * hl]);
      const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&nlss[buf][32 * rb + 8 * qq + 4 * hl]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pacc[4 * qq + e] = d4[e];
        sacc[4 * qq + e] = l4[e];
      }
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int at = aoff(s) + 32 * rb * D;
      sacc = mfma32(*reinterpret_cast<const bf16x8 *>(&qs[buf][at]), kf[s], sacc);
      bf16x8 vs;
      if constexpr (kVInLds)
        vs = *reinterpret_cast<const bf16x8 *>(&vtile[swz_off<D>(32 * wave + il, 2 * s + hl)]);
      else
        vs = vf[s];
      pacc = mfma32(*reinterpret_cast<const bf16x8 *>(&dos[buf][at]), vs, pacc);
    }
  };
  // P of a block whose bias is the constant bconst and that has no mask
  auto block_p_fast = [&](const f32x16 &sacc, float bconst, float (&p)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, bconst));
  };
  // dV^T += dO^T P and dK^T += Q^T dS (unscaled): P / dS from registers as
  // the B operand (k = the block's rows), as hi + lo bf16 pairs, dO^T / Q^T
  // through transposing reads of the row-major tiles.
  auto block_dvdk = [&](int buf, int rb, const float (&p)[16], const float (&ds)[16]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t pw[4], plw[4], hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        split_hi_lo(p[8 * u + 2 * e], p[8 * u + 2 * e + 1], pw[e], plw[e], negp);
        split_hi_lo(ds[8 * u + 2 * e], ds[8 * u + 2 * e + 1], hw[e], lw[e], negp);
      }
      const bf16x8 pb = frag(pw), plb = frag(plw), hb = frag(hw), lb = frag(lw);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int at = (32 * rb + 16 * u) * D;
        const bf16x8 dot8 = lds_read_tr8_at(&dos[buf][at], tro[db][0], tro[db][1]);
        const bf16x8 qt8 = lds_read_tr8_at(&qs[buf][at], tro[db][0], tro[db][1]);
        dvacc[db] = mfma32(dot8, pb, dvacc[db]);
        dvacc[db] = mfma32(dot8, plb, dvacc[db]);
        dkacc[db] = mfma32(qt8, hb, dkacc[db]);
        dkacc[db] = mfma32(qt8, lb, dkacc[db]);
      }
    }
  };

  for (int qb = qb_first; qb < nqb; ++qb) {
    const int q0 = qb * QB;
    const int buf = (qb - qb_first) & 1;
    if (qb + 1 < nqb) {
      fill(q0 + QB, buf ^ 1);
      fire_fill_rows(q0 + QB, buf ^ 1);
    }

    // Every row block takes the same path (products, P, dS, products); only
    // the computation of P branches, so the dK / dV accumulators stay in
    // place.  A block with no visible pair runs fully masked (P = 0).
    f32x16 sacc[QB / 32], pacc[QB / 32];

    // When every row block of the iteration is unmasked with a constant
    // bias (decided from positions alone), all of them go through one
    // straight-line path from the S and dP products on (no branch between
    // the blocks, so the scheduler can overlap one block's products with
    // the next block's exponentials); otherwise each block branches on its
    // own.
    bool all_fast = BIAS == kBiasT5;
    float bcv[QB / 32];
    int ulov[QB / 32];
#pragma unroll
    for (int rb = 0; rb < QB / 32; ++rb) {
      const int irow0 = q0 + 32 * rb;
      const int rmin = kw0 - (irow0 + 31), rmax = kw0 + 31 - irow0;
      bool uni = true;
      bcv[rb] = 0.f;
      ulov[rb] = 0;
      if constexpr (BIAS == kBiasT5) {
        ulov[rb] = min(max(rmin, -sat), sat);
        uni = ulov[rb] == min(max(rmax, -sat), sat);
        bcv[rb] = lut[ulov[rb]];
      }
      all_fast = all_fast && uni && wave_live && irow0 + 32 <= L && kw0 + 32 <= L &&
                 !(CAUSAL && rmax > 0);
    }
    if (all_fast) {
#pragma unroll
      for (int rb = 0; rb < QB / 32; ++rb) block_sdp(buf, rb, sacc[rb], pacc[rb]);
#pragma unroll
      for (int rb = 0; rb < QB / 32; ++rb) {
        float p[16], ds[16];
        block_p_fast(sacc[rb], bcv[rb], p);
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = p[r] * pacc[rb][r];
        if constexpr (DBIAS && BIAS == kBiasT5) {
          float t4[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) t4[k] = (ds[k] + ds[k + 4]) + (ds[k + 8] + ds[k + 12]);
          const float t = (t4[0] + t4[1]) + (t4[2] + t4[3]);
          if (ulov[rb] <= 0) ub0 += t; else ub1 += t;
        }
        block_dvdk(buf, rb, p, ds);
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < QB / 32; ++rb) block_sdp(buf, rb, sacc[rb], pacc[rb]);
    }
#pragma unroll
    for (int rb = 0; rb < QB / 32; ++rb) {
      if (all_fast) break;
      const int irow0 = q0 + 32 * rb;
      const int rmin = kw0 - (irow0 + 31), rmax = kw0 + 31 - irow0;
      const bool none = !wave_live || irow0 >= L || (CAUSAL && rmin > 0);
      const bool mask_c = CAUSAL && rmax > 0;
      const bool mask_r = irow0 + 32 > L;
      const bool mask_k = kw0 + 32 > L;
      // (with V in LDS, blocks without a bias take the masked path too: one
      // path for P keeps the register count down)
      bool uniform = (BIAS == kBiasNone) && !kVInLds;
      float bconst = 0.f;
      int ulo = 0;
      if constexpr (BIAS == kBiasT5) {
        ulo = min(max(rmin, -sat), sat);
        const int uhi = min(max(rmax, -sat), sat);
        uniform = (ulo == uhi);
        bconst = lut[ulo];
      }
      const bool fast = uniform && !none && !mask_c && !mask_r && !mask_k;
      // dense bias and its gradient: element r is row irow0 + 4hl + roff(r),
      // key myk; the lane's own part of the address is voff, the row offset
      // roff(r) * S (the same for the whole wave) goes in the scalar offset
      // (rows past the matrix fall outside the buffer: loads read 0, stores
      // are dropped; a key past S reads the next row and is masked)
      const uint32_t dvoff = (uint32_t)(irow0 + 4 * hl) * (uint32_t)L + (uint32_t)myk;
      uint16_t bkv[16];
      if constexpr (BIAS == kBiasDense) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          bkv[r] = buf_load_u16(rbias, dvoff * 2u,
                                (uint32_t)(8 * (r >> 2) + (r & 3)) * (uint32_t)L * 2u);
      }
      // The fast/slow choice is made once per block, outside the element
      // loops.
      float p[16], ds[16];
      // FIRE: x of each element (needed again by the gradient), its segment,
      // and the lane's segment range
      float fx[kFire ? 16 : 1];
      int fslo = 0, fshi = 0;
      if constexpr (kFire) {
        // element r: row irow0 + 4hl + roff, roff = 8(r/4) + r%4, key myk,
        // distance d0 + roff with d0 = irow0 + 4hl - myk; x = psi(d) / log2(E_row)
        const int d0 = irow0 + 4 * hl - myk;
        const float *rw = fire_rows + buf * 64 + 32 * rb + 4 * hl;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const f32x4 inv4 = *reinterpret_cast<const f32x4 *>(&rw[8 * qq]);
          const f32x4 ps = fire_dist4(fl, d0 + 8 * qq);
#pragma unroll
          for (int e = 0; e < 4; ++e) fx[4 * qq + e] = ps[e] * inv4[e];
        }
        // x grows with the row: elements 0 and 15 bound the lane's range
        float blo = fl.seg_lo, bhi = fl.seg_hi;
        fslo = fire_walk_cached(fl.tab, fx[0], fl.seg, blo, bhi);
        fshi = fire_walk_cached(fl.tab, fx[15], fslo, blo, bhi);
        fl.seg = fshi;
        fl.seg_lo = blo;
        fl.seg_hi = bhi;
        float fb[16];
        if (fslo == fshi) {
          const float A = fl.tab[kFireOffA + fslo], B = fl.tab[kFireOffB + fslo];
#pragma unroll
          for (int r = 0; r < 16; ++r) fb[r] = fmaf(B, fx[r], A);
        } else if (fshi == fslo + 1) {
          const float tk = fl.tab[kFireOffT + fshi];
          const float A0 = fl.tab[kFireOffA + fslo], B0 = fl.tab[kFireOffB + fslo];
          const float A1 = fl.tab[kFireOffA + fshi], B1 = fl.tab[kFireOffB + fshi];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool up = fx[r] >= tk;
            fb[r] = fmaf(up ? B1 : B0, fx[r], up ? A1 : A0);
          }
        } else {
          // the lower segment's line bent at each kink in between (the bias
          // is continuous; see fire_scores)
          const float A = fl.tab[kFireOffA + fslo], B = fl.tab[kFireOffB + fslo];
#pragma unroll
          for (int r = 0; r < 16; ++r) fb[r] = fmaf(B, fx[r], A);
          for (int k = fslo + 1; k <= fshi; ++k) {
            const float tk = fl.tab[kFireOffT + k];
            const float dB = fl.tab[kFireOffB + k] - fl.tab[kFireOffB + k - 1];
#pragma unroll
            for (int r = 0; r < 16; ++r) fb[r] = fmaf(dB, fmaxf(fx[r] - tk, 0.f), fb[r]);
          }
        }
        const int rbase = myk - (irow0 + 4 * hl);
        // masked iff roff < lo_lim (key after the query) or roff >= hi_lim
        // (row past the end), as in the generic path below
        int lo_lim = mask_c ? rbase : -1;
        const int hi_lim = mask_r ? L - (irow0 + 4 * hl) : 32;
        if (none || (mask_k && myk >= L)) lo_lim = 32;
        if (!none && !mask_c && !mask_r && !mask_k) {
#pragma unroll
          for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[rb][r], c, fb[r]));
        } else {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * qq + e, roff = 8 * qq + e;
              const float t = fmaf(sacc[rb][r], c, fb[r]);
              const bool dead = (roff < lo_lim) | (roff >= hi_lim);
              p[r] = __builtin_amdgcn_exp2f(t + (dead ? -INFINITY : 0.f));
            }
        }
      } else if (fast) {
        block_p_fast(sacc[rb], bconst, p);
      } else {
        // T5: this lane's distances are rbase - roff, roff in [0, 27]; one
        // clamped base for the block (see kLutPad), and the causal mask is
        // in the table
        const int rbase = myk - (irow0 + 4 * hl);
        const float *const lb = lut + min(max(rbase - 27, -sat - kLutPad), sat + kLutPad - 27);
        // a T5 block with no row or key past the end (the band near the
        // diagonal: the causal mask is in the table) needs no mask at all
        const bool t5_plain = BIAS == kBiasT5 && !none && !mask_r && !mask_k;
        if (t5_plain) {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              p[4 * qq + e] =
                  __builtin_amdgcn_exp2f(fmaf(sacc[rb][4 * qq + e], c, lb[27 - 8 * qq - e]));
        }
        // a dense-bias block (head_dim 64) with no mask: no compares
        const bool dense_plain =
            BIAS == kBiasDense && D == 64 && !none && !mask_c && !mask_r && !mask_k;
        if (dense_plain) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            p[r] = __builtin_amdgcn_exp2f(fmaf(bf16_bits(bkv[r]), kLog2e, sacc[rb][r] * c));
        }
        // Without T5 (whose causal mask is in its table) element r, at row
        // offset roff, is masked iff roff < lo_lim (a key after the query:
        // rbase - roff > 0) or roff >= hi_lim (a row past the end); a block
        // with no visible pair or a key past the end masks everything.  Two
        // compares per element against per-lane limits; the T5 variants keep
        // the direct form, which their register allocation prefers.
        int lo_lim = (BIAS != kBiasT5 && mask_c) ? rbase : -1;
        const int hi_lim = mask_r ? L - (irow0 + 4 * hl) : 32;
        if (none || (mask_k && myk >= L)) lo_lim = 32;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          if (t5_plain || dense_plain) break;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * qq + e;
            const int roff = 8 * qq + e;
            const int rr = rbase - roff;
            float t = sacc[rb][r] * c;
            if constexpr (BIAS == kBiasT5) t = fmaf(sacc[rb][r], c, lb[27 - roff]);
            if constexpr (BIAS == kBiasAlibi) t = fmaf(fabsf((float)rr), slope_l2, t);
            if constexpr (BIAS == kBiasDense) t = fmaf(bf16_bits(bkv[r]), kLog2e, t);
            // non-short-circuit operators keep this straight-line code
            const bool dead = BIAS == kBiasT5
                                  ? none | (mask_r & (irow0 + 4 * hl + roff >= L)) |
                                        (mask_k & (myk >= L))
                                  : (roff < lo_lim) | (roff >= hi_lim);
            // the mask as an additive -inf (exp2(-inf) = 0): a select
            // between the whole argument and -inf would be turned into a
            // branch around the table read
            p[r] = __builtin_amdgcn_exp2f(t + (dead ? -INFINITY : 0.f));
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = p[r] * pacc[rb][r];
      if constexpr (DBIAS && BIAS == kBiasDense) {
        // dL/dB = dS for every pair of the block (0 where masked)
        if (myk < L) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            buf_store_f32(rdbias, dvoff * 4u, (uint32_t)(8 * (r >> 2) + (r & 3)) * (uint32_t)L * 4u,
                          ds[r]);
        }
      }
      if constexpr (DBIAS && BIAS == kBiasT5) {
        if (fast) {
          float t4[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) t4[k] = (ds[k] + ds[k + 4]) + (ds[k + 8] + ds[k + 12]);
          const float t = (t4[0] + t4[1]) + (t4[2] + t4[3]);
          if (ulo <= 0) ub0 += t; else ub1 += t;
        } else {
          // Near the diagonal the bucket varies within the block, but it is
          // constant along each diagonal (fixed key - query).  The block's
          // dS goes to this wave's scratch tile, row = query, column = key;
          // after the block's products, lane (hl, c) sums diagonal c
          // (hl = 0: entries (row, row + c)) or c - 32 (hl = 1: entries
          // (row, row + c - 32)), reading with pitch kTilePitch + 1 - 64
          // distinct distances, so each lane owns one bin and no LDS atomics
          // are needed.  Masked pairs carry dS = 0.  LDS operations of one
          // wave complete in order, so no barrier separates the writes from
          // the reads.
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * hl + (r & 3);
            mytile[row * kTilePitch + il] = ds[r];
          }
        }
      }
      block_dvdk(buf, rb, p, ds);
      if constexpr (DBIAS && BIAS == kBiasT5) {
        if (!fast) {
          // diagonal il (hl = 0) covers rows below 32 - il, diagonal il - 32
          // (hl = 1) the others; a lane reads all 32 rows of its line (the
          // entries of the other rows lie outside the tile's row or in the
          // guard and are discarded), all reads before the masked tree sum
          float col[32];
#pragma unroll
          for (int row = 0; row < 32; ++row)
            col[row] = mytile[row * (kTilePitch + 1) + il - 32 * hl];
          // (opaque to the compiler: 32 masks hoisted out of the loop would
          // hold 64 scalar registers for the whole kernel)
          int lim = 32 - il;
          asm volatile("" : "+v"(lim));
#pragma unroll
          for (int row = 0; row < 32; ++row)
            col[row] = ((row < lim) == (hl == 0)) ? col[row] : 0.f;
#pragma unroll
          for (int w = 16; w >= 1; w >>= 1)
#pragma unroll
            for (int k = 0; k < w; ++k) col[k] += col[k + w];
          const float gsum = col[0];
          const int dd = kw0 - irow0 + (hl ? il - 32 : il);   // key - query
          if (dd <= -sat) ub0 += gsum;
          else if (dd >= sat) ub1 += gsum;
          else mybins[dd + sat] += gsum;
        }
      }
    }
    // the next block's copies have landed (each wave waits for its own)
    wait_vmem_loads();
    __syncthreads();
  }

  // dK = scale dS^T Q: the scale is applied once here
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkacc[db][r] *= dscale;
  // with RoPE, dK with respect to the unrotated key row
  if (a.rope_cs != nullptr)
    rope_unrotate_acc<D>(dkacc, a.rope_cs, a.seqlen, myk, hl);
  // dK, dV of key myk: lane holds dims 32db + 8(r/4) + 4hl + r%4
  const rsrc_t rdv = make_rsrc(a.dv + base, nrec);
  const rsrc_t rdk = make_rsrc(a.dk + base, nrec);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const uint32_t el = (uint32_t)myk * (uint32_t)HD + 32 * db + 8 * rq + 4 * hl;
      i32x2 v2 = {(int)pack_bf16x2(dvacc[db][4 * rq], dvacc[db][4 * rq + 1]),
                  (int)pack_bf16x2(dvacc[db][4 * rq + 2], dvacc[db][4 * rq + 3])};
      buf_store8(rdv, el * 2u, v2);
      i32x2 k2 = {(int)pack_bf16x2(dkacc[db][4 * rq], dkacc[db][4 * rq + 1]),
                  (int)pack_bf16x2(dkacc[db][4 * rq + 2], dkacc[db][4 * rq + 3])};
      buf_store8(rdk, el * 2u, k2);
    }

  if constexpr (DBIAS && BIAS == kBiasT5) {
    // saturated-block sums: reduce over the wave, then fold into the end bins
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
    for (int x = tid; x < nbin; x += NT) {
      float t = 0.f;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) t += bins[w4 * nbin + x];
      if (x == 0) t += ubin[0][0] + ubin[1][0] + ubin[2][0] + ubin[3][0];
      if (x == nbin - 1) t += ubin[0][1] + ubin[1][1] + ubin[2][1] + ubin[3][1];
      bins[x] = t;
    }
    __syncthreads();
    // Bin x holds relative distance r = x - sat.  On each side of r = 0 the
    // bucket is monotone in n = |r|, so bucket b covers one run of bins,
    // found from the thresholds (bucket me + j covers thr[j-1] <= n <
    // thr[j]); the bkt test keeps the sum exact whatever the run's ends.
    for (int b = tid; b < a.nb; b += NT) {
      const T5Geometry &ge = a.t5;
      const bool upper = ge.bidir && b >= ge.nbp;   // keys after the query
      const int bl = upper ? b - ge.nbp : b;
      int n0, n1;
      if (bl < ge.me) {
        n0 = n1 = bl;
      } else {
        const int j = bl - ge.me;
        n0 = j == 0 ? ge.me : ge.thr[j - 1];
        n1 = j < ge.nthr ? ge.thr[j] - 1 : sat;
      }
      n1 = min(n1, sat);
      int x0, x1;   // inclusive bin range
      if (upper) {
        x0 = sat + max(n0, 1);
        x1 = sat + n1;
      } else {
        x0 = sat - n1;
        x1 = sat - n0;
        if (!ge.bidir && b == 0) x1 = 2 * sat;   // unidirectional: r > 0 is bucket 0
      }
      float t = 0.f;
      for (int x = x0; x <= x1; ++x) t += bkt[x] == b ? bins[x] : 0.f;
      a.part[(size_t)b * a.nwg + w.part] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// Dense bias shared by the batch: its gradient summed over the batch
// ---------------------------------------------------------------------------
// dL/dB[h] = sum over b of dS[b, h] for a bias matrix [1, H, S, S].  One
// workgroup per (head, 128 x 128 output tile), lanes on keys as in the dkv
// kernel (wave w: keys 32 w .. 32 w + 31 of the tile, all 128 rows); the
// tile's sums stay in registers while the batch is the loop.  For batch b
// the tile's Q and dO rows (LDS) and the lane's K and V rows (registers)
// give S and dP, seeded with -lse/scale and -D; P takes the bias (read once,
// kept packed two per register) and dS = P (dP - D) is added in batch
// order.  After the last batch each sum is stored once: no workspace, no
// second pass over per-batch gradients, and one fixed order of the sum.
// The next batch's tiles are requested while the current one is worked on
// (two LDS buffers, two register sets; the loop is unrolled by two so each
// set is addressed statically).  head_dim 64 takes tiles of 128 rows and
// fits 256 registers (two workgroups per CU); head_dim 128, whose K/V sets
// are twice as large, takes tiles of 64 rows and a little more than 256
// registers (one workgroup, one wave per SIMD, per CU: the unrolled blocks
// give the scheduler independent MFMA and exponential work to overlap).
// Causal: only tiles with a visible pair are launched (the lower triangle
// of 128 x 128 super tiles, each cut into 128 / RT row tiles).
template <int D>
constexpr int dbias_sum_rows() { return D == 64 ? 128 : 64; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, D == 64 ? 2 : 1) void bwd_dbias_sum_kernel(const BwdArgs a) {
  constexpr int RT = dbias_sum_rows<D>();   // query rows per workgroup
  constexpr int NB = RT / 32;               // 32-row blocks
  constexpr int M = BKV / RT;               // row tiles per 128-row super tile
  constexpr int NP = RT / 64;               // 64-float pieces of -lse/scale (and of -D)
  __shared__ __attribute__((aligned(16))) uint16_t qs[2][RT * D];
  __shared__ __attribute__((aligned(16))) uint16_t dos[2][RT * D];
  __shared__ __attribute__((aligned(16))) float nlss[2][RT];
  __shared__ __attribute__((aligned(16))) float ndls[2][RT];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, il = lane & 31;
  const int L = a.seqlen, B = a.nbatch, nt = a.ntile;
  // logical id -> (head, super tile (R, kt), row tile within it); causal:
  // kt <= R, t = R (R + 1) / 2 + kt
  const int per_head = (CAUSAL ? nt * (nt + 1) / 2 : nt * nt) * M;
  const int g = xcd_remap(blockIdx.x, a.nwg);
  const int h = g / per_head;
  const int tl = g - h * per_head;
  const int t = tl / M, sub = tl - (tl / M) * M;
  int R, kt;
  if constexpr (CAUSAL) {
    R = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
    while (R > 0 && R * (R + 1) / 2 > t) --R;
    while ((R + 1) * (R + 2) / 2 <= t) ++R;
    kt = t - R * (R + 1) / 2;
  } else {
    R = t / nt;
    kt = t - R * nt;
  }
  const int row0 = R * BKV + sub * RT;
  const int kw0 = kt * BKV + 32 * wave;
  const int myk = kw0 + il;

  const int HD = a.heads * D;
  const uint32_t nrec = ((uint32_t)(L - 1) * (uint32_t)HD + D) * 2u;
  auto seq_base = [&](int b) { return ((size_t)b * L * a.heads + h) * D; };
  auto row_base = [&](int b) { return ((size_t)b * a.heads + h) * L; };
  const rsrc_t rbias = make_rsrc(a.dense + (size_t)h * L * L, (uint32_t)L * (uint32_t)L * 2u);

  const int aw = swz<D>(il);
  const int abase = il * D + 8 * (hl ^ (aw & 1));
  auto aoff = [&](int j, int s) { return j * 32 * D + abase + 16 * (s ^ (aw >> 1)); };
  const float c = a.scale_log2;
  // keys of this wave that see no row of the tile (or lie past the end):
  // its products are skipped, its sums stay 0
  const bool none = kw0 >= L || row0 >= L || (CAUSAL && kw0 > row0 + RT - 1);
  // no pair of the wave's part of the tile is masked
  const bool full = (!CAUSAL || kw0 + 31 <= row0) && row0 + RT <= L && kw0 + 32 <= L;

  auto fill = [&](int b, int buf) {
    dma_tile<D, RT, 4>(dma_desc(a.q + seq_base(b), nrec), HD, row0, qs[buf], wave, lane);
    dma_tile<D, RT, 4>(dma_desc(a.dout + seq_base(b), nrec), HD, row0, dos[buf], wave, lane);
    if (wave < 2 * NP) {
      const int which = wave / NP, piece = wave - which * NP;
      dma4(dma_desc((which ? a.delta : a.nls) + row_base(b), (uint32_t)L * 4u),
           (uint32_t)(row0 + 64 * piece + lane) * 4u, (which ? ndls[buf] : nlss[buf]) + 64 * piece);
    }
  };
  auto load_kv = [&](int b, bf16x8 (&kf)[D / 16], bf16x8 (&vf)[D / 16]) {
    const rsrc_t rk = make_rsrc(a.k + seq_base(b), nrec);
    const rsrc_t rv = make_rsrc(a.v + seq_base(b), nrec);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint32_t off = ((uint32_t)myk * (uint32_t)HD + 16 * s + 8 * hl) * 2u;
      kf[s] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
      vf[s] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
    }
  };

  // lane element r of block j: key myk, row row0 + 4 hl + roff(j, r)
  const uint32_t voff = (uint32_t)(row0 + 4 * hl) * (uint32_t)L + (uint32_t)myk;
  auto roff = [&](int j, int r) { return 32 * j + 8 * (r >> 2) + (r & 3); };
  // the first batch's tiles, then the bias, then one wait for both
  bf16x8 kfa[D / 16], vfa[D / 16], kfb[D / 16], vfb[D / 16];
  if (B > 0) {
    fill(0, 0);
    load_kv(0, kfa, vfa);
  }
  float dsum[NB * 16];
#pragma unroll
  for (int r = 0; r < NB * 16; ++r) dsum[r] = 0.f;

  // Offsets of the rows roff(j, r) walk from row to row (+1 row within a
  // group of four, +5 to the next), each step hidden from the compiler so
  // it does not turn them into one scalar constant per row, all alive
  // across the batch loop.
  auto next_row = [&](uint32_t &o, int r, uint32_t row_bytes) {
    o += ((r & 3) == 3 ? 5u : 1u) * row_bytes;
    asm volatile("" : "+v"(o));
  };
  // The bias, two rows per register (bf16 bits).  Masked pairs (key after
  // the query, row or key past the end) hold -inf instead, so P is 0 there
  // with no test in the batch loop.
  uint32_t bpk[NB * 8];
  {
    uint16_t raw[NB * 16];
    uint32_t o = voff * 2u;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        raw[16 * j + r] = buf_load_u16(rbias, o);
        next_row(o, r, (uint32_t)L * 2u);
      }
    // every load (the first batch's too) is in flight before the first use
    wait_vmem_loads();
    const int rkey = myk - (row0 + 4 * hl);   // key - first row of the lane
    const int rlim = L - (row0 + 4 * hl);     // rows past the end: roff >= rlim
    const bool part = !full;
    const bool kout = myk >= L;
    // branch-free: the masks are per element, not per wave
    auto bits = [&](int j, int r) -> uint32_t {
      const int dead = (int)part & ((int)(CAUSAL && rkey > roff(j, r)) |
                                    (int)(roff(j, r) >= rlim) | (int)kout);
      return dead ? 0xff80u : (uint32_t)raw[16 * j + r];
    };
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r2 = 0; r2 < 8; ++r2)
        bpk[8 * j + r2] = bits(j, 2 * r2) | (bits(j, 2 * r2 + 1) << 16);
  }

  // one batch: S and dP block by block, dS into the sums
  auto step = [&](int buf, const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16]) {
    if (none) return;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      f32x16 sacc, pacc;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&ndls[buf][32 * j + 8 * qq + 4 * hl]);
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&nlss[buf][32 * j + 8 * qq + 4 * hl]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pacc[4 * qq + e] = d4[e];
          sacc[4 * qq + e] = l4[e];
        }
      }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc = mfma32(*reinterpret_cast<const bf16x8 *>(&qs[buf][aoff(j, s)]), kf[s], sacc);
        pacc = mfma32(*reinterpret_cast<const bf16x8 *>(&dos[buf][aoff(j, s)]), vf[s], pacc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t w = bpk[8 * j + (r >> 1)];
        const float bias = __uint_as_float((r & 1) ? (w & 0xffff0000u) : (w << 16));
        const float p = __builtin_amdgcn_exp2f(fmaf(bias, kLog2e, sacc[r] * c));
        dsum[16 * j + r] = fmaf(p, pacc[r], dsum[16 * j + r]);
      }
    }
  };

  wait_vmem_loads();
  __syncthreads();
  for (int b = 0; b < B; b += 2) {
    // even batch: buffer 0, registers a; prefetch into buffer 1 / b
    if (b + 1 < B) {
      fill(b + 1, 1);
      load_kv(b + 1, kfb, vfb);
    }
    step(0, kfa, vfa);
    wait_vmem_loads();
    __syncthreads();
    if (b + 1 >= B) break;
    // odd batch: buffer 1, registers b; prefetch into buffer 0 / a
    if (b + 2 < B) {
      fill(b + 2, 0);
      load_kv(b + 2, kfa, vfa);
    }
    step(1, kfb, vfb);
    wait_vmem_loads();
    __syncthreads();
  }
  const rsrc_t rdbias = make_rsrc(a.dbias + (size_t)h * L * L, (uint32_t)L * (uint32_t)L * 4u);
  if (myk < L) {
    uint32_t o = voff * 4u;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        buf_store_f32(rdbias, o, dsum[16 * j + r]);
        next_row(o, r, (uint32_t)L * 4u);
      }
  }
}

// ---------------------------------------------------------------------------
// Table-gradient reduction
// ---------------------------------------------------------------------------
// dtable[b, h] = sum of the partials of head h, one workgroup per (b, h):
// strided per-thread sums, then a tree in LDS, both in a fixed order.
// Partials are stored bucket-major, part[b * nwg + slot]: the schedule
// entry for packed batches, (batch * heads + head) * ntile + key tile for
// dense ones.
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
hipError_t launch_dq_t(const BwdArgs &a, hipStream_t s) {
  if constexpr (BIAS == kBiasT5 && !VARLEN && D == 64) {
    if (a.seqlen % 64 == 0) {
      hipLaunchKernelGGL((bwd_dq_kernel<D, BIAS, CAUSAL, false, true>), dim3(a.nwg), dim3(NT), 0,
                         s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_dq_kernel<D, BIAS, CAUSAL, VARLEN>), dim3(a.nwg), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int D, int BIAS, bool CAUSAL, bool VARLEN, bool DBIAS>
hipError_t launch_dkv_t(const BwdArgs &a, hipStream_t s) {
  const size_t dyn = dkv_dyn_bytes(a.t5.sat, BIAS == kBiasT5, DBIAS);
  auto kern = bwd_dkv_kernel<D, BIAS, CAUSAL, VARLEN, DBIAS>;
  if (dyn > 16384) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)dyn);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(a.nwg), dim3(NT), dyn, s, a);
  return hipGetLastError();
}

template <int D, int BIAS, bool CAUSAL, bool VARLEN>
hipError_t launch_pair(const BwdArgs &a, int phase, bool dbias, hipStream_t s) {
  if (phase == kBwdPre) return launch_dq_t<D, BIAS, CAUSAL, VARLEN>(a, s);
  if constexpr (BIAS == kBiasT5 || BIAS == kBiasDense) {
    if (dbias) return launch_dkv_t<D, BIAS, CAUSAL, VARLEN, true>(a, s);
  }
  if constexpr (BIAS == kBiasFire && CAUSAL) {
    if (phase == kBwdFire) {
      hipLaunchKernelGGL((bwd_fire_kernel<D, VARLEN>), dim3(a.nwg), dim3(NT), 0, s, a);
      return hipGetLastError();
    }
  }
  return launch_dkv_t<D, BIAS, CAUSAL, VARLEN, false>(a, s);
}

template <int D, int BIAS>
hipError_t launch_b(const BwdArgs &a, int phase, bool causal, bool varlen, bool dbias,
                    hipStream_t s) {
  if constexpr (BIAS == kBiasDense) {   // dense entry points only
    return causal ? launch_pair<D, BIAS, true, false>(a, phase, dbias, s)
                  : launch_pair<D, BIAS, false, false>(a, phase, dbias, s);
  } else if constexpr (BIAS == kBiasFire) {   // causal only
    (void)causal;
    return varlen ? launch_pair<D, BIAS, true, true>(a, phase, dbias, s)
                  : launch_pair<D, BIAS, true, false>(a, phase, dbias, s);
  } else {
    if (causal)
      return varlen ? launch_pair<D, BIAS, true, true>(a, phase, dbias, s)
                    : launch_pair<D, BIAS, true, false>(a, phase, dbias, s);
    return varlen ? launch_pair<D, BIAS, false, true>(a, phase, dbias, s)
                  : launch_pair<D, BIAS, false, false>(a, phase, dbias, s);
  }
}

template <int D>
hipError_t launch_d(const BwdArgs &a, int phase, int bias, bool causal, bool varlen, bool dbias,
                    hipStream_t s) {
  switch (bias) {
    case kBiasT5: return launch_b<D, kBiasT5>(a, phase, causal, varlen, dbias, s);
    case kBiasAlibi: return launch_b<D, kBiasAlibi>(a, phase, causal, varlen, dbias, s);
    case kBiasDense: return launch_b<D, kBiasDense>(a, phase, causal, varlen, dbias, s);
    case kBiasFire: return launch_b<D, kBiasFire>(a, phase, causal, varlen, dbias, s);
    default: return launch_b<D, kBiasNone>(a, phase, causal, varlen, dbias, s);
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
  static_assert(BR == BKV, "dq and dkv kernels share the packed-batch schedule");
  BwdArgs a;
  a.q = static_cast<const uint16_t *>(b.q);
  a.k = static_cast<const uint16_t *>(b.k);
  a.v = static_cast<const uint16_t *>(b.v);
  a.o = static_cast<const uint16_t *>(b.o);
  a.dout = static_cast<const uint16_t *>(b.dout);
  a.lse = b.lse;
  a.dlse = b.dlse;
  a.dq = static_cast<uint16_t *>(b.dq);
  a.dk = static_cast<uint16_t *>(b.dk);
  a.dv = static_cast<uint16_t *>(b.dv);
  a.rope_cs = b.rope_cs;
  a.fire_tab = b.fire_tab;
  a.fire_dist = b.fire_dist;
  a.delta = b.delta;
  a.nls = b.delta + (size_t)p.total * p.heads;
  a.part = b.part;
  a.sched = sched;
  a.table = p.table;
  a.slopes = p.slopes;
  a.dense = p.dense;
  a.dense_batch = p.dense_batch;
  a.dbias = b.dbias;
  a.nbatch = p.nbatch;
  a.seqlen = p.seqlen;
  a.heads = p.heads;
  a.total = p.total;
  a.nb = p.bias == kBiasT5 ? (p.t5.bidir ? 2 * p.t5.nbp : p.t5.nbp)
                           : (p.bias == kBiasFire ? kFireGradRows : 0);
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  a.t5 = p.t5;
  if (p.bias != kBiasT5) a.t5.sat = 0;
  if (p.varlen) {
    a.ntile = 0;
    a.nwg = nsched;
  } else {
    a.ntile = (p.seqlen + BKV - 1) / BKV;
    a.nwg = p.nbatch * p.heads * a.ntile;
  }
  if (a.nwg <= 0) return hipSuccess;
  const bool dbias = (b.part != nullptr && p.bias != kBiasFire) || a.dbias != nullptr;
  if (phase == kBwdFire && (p.bias != kBiasFire || b.part == nullptr)) return hipSuccess;
  if (phase == kBwdDenseSum) {
    if (b.dbias_shared == nullptr) return hipSuccess;
    a.dbias = b.dbias_shared;
    const int nt = a.ntile;
    const int m = BKV / (p.head_dim == 64 ? dbias_sum_rows<64>() : dbias_sum_rows<128>());
    a.nwg = p.heads * (p.causal ? nt * (nt + 1) / 2 : nt * nt) * m;
    auto kern = p.head_dim == 64 ? (p.causal ? bwd_dbias_sum_kernel<64, true>
                                             : bwd_dbias_sum_kernel<64, false>)
                                 : (p.causal ? bwd_dbias_sum_kernel<128, true>
                                             : bwd_dbias_sum_kernel<128, false>);
    hipLaunchKernelGGL(kern, dim3(a.nwg), dim3(NT), 0, s, a);
    return hipGetLastError();
  }
  if (phase == kBwdReduce) {
    if (b.part == nullptr) return hipSuccess;
    hipLaunchKernelGGL(dbias_reduce_kernel, dim3(a.nb * p.heads), dim3(256), 0, s, a.part,
                       sched, a.nwg, p.nbatch, p.heads, a.ntile,
                       p.bias == kBiasFire ? b.fire_g : b.dtable);
    return hipGetLastError();
  }
  return p.head_dim == 64 ? launch_d<64>(a, phase, p.bias, p.causal, p.varlen, dbias, s)
                          : launch_d<128>(a, phase, p.bias, p.causal, p.varlen, dbias, s);
}

}  // namespace fa
