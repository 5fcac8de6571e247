// Forward attention for gfx950 (FAT5 report, section "Noyau CUDA", second
// kernel): per (sequence, head, 128-query tile) one workgroup streams K and V
// through LDS in 64-key tiles, forms S' = scale * Q K^T + bias on the fly from
// the per-head table (or ALiBi, or the FIRE segment table), keeps a running
// softmax, accumulates O = P V, and writes O (bf16) and the row logsumexp
// (fp32).  The score matrix never leaves registers.
//
// Layout of the work inside a workgroup (4 waves, 32 query rows each):
//   S^T (keys x queries) = K Q^T on 32x32x16 bf16 MFMA, so each lane owns one
//   query row and 32 of the tile's keys: the row max and row sum are in-lane
//   reductions plus one exchange between the two half-waves.
//   O^T (dims x queries) = V^T P^T reuses P straight from the score
//   accumulators as the MFMA B operand; its A operand (each lane: one dim,
//   the 8 keys matching its P values) comes from the row-major V tile through
//   the transposing LDS read, so K and V are staged the same way: unpadded,
//   swizzled tiles (no bank conflicts on either read) copied from global
//   memory straight into LDS.
//
// Normalisation.  O is divided by the sum of the bf16 weights that actually
// multiply V (P rounded to bf16 for the PV product), not by the fp32 sum of
// P: the rounding error of a row's dominant weight, up to 2^-9 of it, then
// cancels between numerator and denominator instead of reaching O.  (The
// lazy rescale below leaves the dominant weight at exp2 of a non-integer,
// so that error is not otherwise zero.)  The bf16 sum costs no VALU work: a
// 16x16x32 MFMA per 16-key fragment of P adds its keys against a constant
// 0/1 operand.  The LSE keeps the fp32 sum, exact to fp32.
//
// Latency.  With operands read from LDS right before each MFMA, every MFMA
// waits out an LDS round trip; measured per 64-key tile that cost more than
// the softmax itself.  So the K operands of a tile are read in one batch
// before its QK^T products, and the V operands are read before the softmax,
// whose VALU work covers their latency.  K and V tiles are requested from
// global memory one iteration ahead into double-buffered LDS.
#include "fa_device.h"

namespace fa {
namespace {

constexpr int BC = 64;    // keys per tile
constexpr int NT = 256;   // threads per workgroup (4 waves)
constexpr int BR = 128;   // query rows per workgroup (32 per wave)
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
  const uint16_t *dense;  // dense bias bf16 [dense_batch, H, S, S]
  const double2 *rope_cs;  // RoPE: (cos, sin) [seqlen, D/2], or nullptr
  const float *fire_tab;   // FIRE segment table (fa_internal.h), or nullptr
  const float *fire_dist;  // FIRE distance table, or nullptr
  int32_t dense_batch;
  int32_t nbatch, seqlen, heads, total;
  int32_t nq, nwg;
  float scale_log2;      // scale * log2(e)
  T5Geometry t5;
};

template <int D, int BIAS, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NT, D == 64 && BIAS != kBiasDense && BIAS != kBiasFire ? 3 : 2)
void fwd_kernel(
    const FwdArgs a) {
  constexpr int NVF = D / 8;                  // V operand fragments per tile
  // Register budget: at head_dim 64 the K operands of both 32-key blocks are
  // read in one batch and every V operand before the softmax; at 128 the K
  // operands go one key block at a time and a quarter of V before the softmax.
  constexpr int KBATCH = D == 64 ? 2 : 1;     // key blocks per K read batch
  constexpr int NKF = KBATCH * (D / 16);      // K fragments per batch
  constexpr int VPRE = D == 64 ? NVF : NVF / 4;
  // K and V tiles, swizzled (see swz; K read row-wise, V transposed), in a
  // ring of NBUF buffers filled NBUF - 1 tiles ahead by buffer-to-LDS copies.
  // Two buffers: at head_dim 64 that leaves LDS (and registers) for three
  // workgroups per CU, which measured faster than a deeper ring with two.
  constexpr int NBUF = 2;
  constexpr int PER_FILL = 2 * BC * D * 2 / 1024 / (NT / 64);   // copies per wave per tile
  __shared__ __attribute__((aligned(16))) uint16_t ks[NBUF][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs[NBUF][BC * D];
  __shared__ float lut_mem[BIAS == kBiasT5 ? 2 * (kMaxDistance + kLutPad) + 1 : 1];
  const float *const lut = lut_mem + (BIAS == kBiasT5 ? a.t5.sat + kLutPad : 0);
  __shared__ float fire_mem[BIAS == kBiasFire ? kFireLds : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, il = lane & 31;
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
    int pair, rank;
    tile_order<6>(g, a.nbatch * a.heads, a.nq, pair, rank);   // 3 workgroups per CU
    qt = a.nq - 1 - rank;                     // longest causal rows first
    pair_bh(pair, a.nbatch, a.heads, BIAS == kBiasDense && a.dense_batch == 1, bidx, h);
    tok0 = bidx * a.seqlen;
    L = a.seqlen;
  }

  const int HD = a.heads * D;
  const size_t base = ((size_t)tok0 * a.heads + h) * D;
  const uint32_t nrec = ((uint32_t)(L - 1) * (uint32_t)HD + D) * 2u;
  const rsrc_t rq = make_rsrc(a.q + base, nrec);
  const rsrc_t ro = make_rsrc(a.o + base, nrec);

  const int q0 = qt * BR;
  const int wrow0 = q0 + 32 * wave;           // first row of this wave
  const bool wave_live = wrow0 < L;           // rows past the end do nothing

  // Q as the B operand of S^T = K Q^T: lane (hl, il) holds row wrow0 + il,
  // dims 16s + 8hl .. +7 for k-step s.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = __builtin_bit_cast(
        bf16x8, buf_load16(rq, ((uint32_t)(wrow0 + il) * (uint32_t)HD + 16 * s + 8 * hl) * 2u));
  if (a.rope_cs != nullptr) {
    // RoPE: the row's position is its index in the sequence; fragment s holds
    // pairs 8s + 4hl .. + 3 as its four 32-bit words.  Rows past the table
    // read (cos, sin) = 0 (they are past the sequence and never stored).
    const rsrc_t rcs = make_rsrc(a.rope_cs, (uint32_t)a.seqlen * (uint32_t)(D / 2) * 16u);
    const uint32_t t0 = ((uint32_t)(wrow0 + il) * (uint32_t)(D / 2) + 4 * hl) * 16u;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      i32x4 w = __builtin_bit_cast(i32x4, qf[s]);
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const RopeCs2 c = rope_cs2(rcs, t0 + (8u * s + e) * 16u);
        w[e] = (int)rope_rotate_pair((uint32_t)w[e], c.c0, c.s0);
        w[e + 1] = (int)rope_rotate_pair((uint32_t)w[e + 1], c.c1, c.s1);
      }
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

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
  FireLane fl;
  if constexpr (BIAS == kBiasFire) {
    fire_load(a.fire_tab, h, fire_mem, tid, NT);
    fl = fire_lane(a.fire_tab, a.fire_dist, a.seqlen, fire_mem, wrow0 + il);
  }
  // dense bias: this (batch, head)'s [S, S] matrix
  rsrc_t rbias = make_rsrc(nullptr, 0u);
  if constexpr (BIAS == kBiasDense) {
    const size_t mat = (size_t)(a.dense_batch == 1 ? 0 : bidx) * a.heads + h;
    rbias = make_rsrc(a.dense + mat * L * L, (uint32_t)L * (uint32_t)L * 2u);
  }

  const int kend = CAUSAL ? min(L, q0 + BR) : L;
  const int nkt = (kend + BC - 1) / BC;

  const i32x4 dk_src = dma_desc(a.k + base, nrec), dv_src = dma_desc(a.v + base, nrec);
  auto fill = [&](int j0, int buf) {
    dma_tile<D, BC, NT / 64>(dk_src, HD, j0, ks[buf], wave, lane);
    dma_tile<D, BC, NT / 64>(dv_src, HD, j0, vs[buf], wave, lane);
  };

  // per-lane LDS offsets (elements); the rest of each address is a constant:
  // K row il, chunk 2s + hl (+ 32kb rows); V transposed, the two halves of
  // each 16-row group per 32-column block (+ 32kb + 16u rows)
  int kof[D / 16], tro[D / 32][2];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) kof[s] = swz_off<D>(il, 2 * s + hl);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    tro[db][0] = swz_tr_off<D>(lane, 0, db);
    tro[db][1] = swz_tr_off<D>(lane, 1, db);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};
  // Sum of the bf16 weights per query: P's fragment (lane (hl, il): query
  // il, 8 keys of half-wave hl), read as a 16x16x32 B operand, holds query
  // 16 ((l / 16) & 1) + (l % 16) in k-group l / 16.  With A[i][k] = 1 when
  // k-group and row agree on that query half ((k / 8) & 1 == (i / 4) & 1),
  // output row i sums the 16 keys of query 16 ((i / 4) & 1) + column, and
  // lane l's rows 4 (l / 16) .. + 3 are its own query il.
  // (At head_dim 128 the operand is rebuilt from one register in each
  // iteration: four registers held across the loop would spill the dense-
  // bias variant.  At 64 they fit, and rebuilding would cost four moves per
  // product.)
  f32x4 wsum = f32x4{};
  const int selw = (((lane >> 4) & 1) == (((lane & 15) >> 2) & 1)) ? 0x3f803f80 : 0;
  auto sel_operand = [&]() {
    int w = selw;
    if constexpr (D == 128) asm volatile("" : "+v"(w));
    return __builtin_bit_cast(bf16x8, i32x4{w, w, w, w});
  };
  const float c = a.scale_log2;

  // Tiles 0 .. NBUF - 2 are requested now.  Iteration kt requests tile
  // kt + NBUF - 1 into the buffer read in iteration kt - 1 (free since the
  // barrier that ended it) and ends once tile kt + 1 has landed: its own
  // request may stay in flight for NBUF - 2 more iterations.
  // Q (and the bias table) first: the compiler counts only its own loads,
  // so they must be retired before the copies it cannot see are in flight
  wait_vmem_loads();
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < nkt) fill(t * BC, t);
  if (NBUF == 3 && nkt > 1)
    wait_vmem_loads_but<(NBUF - 2) * PER_FILL>();
  else
    wait_vmem_loads();
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int j0 = kt * BC;
    const int buf = kt % NBUF;
    const bool ahead = kt + NBUF - 1 < nkt;
    if (ahead) fill(j0 + (NBUF - 1) * BC, (kt + NBUF - 1) % NBUF);
    // a causal wave starts work once the tile reaches its last row
    const bool active = wave_live && (!CAUSAL || (j0 <= wrow0 + 31));

    // K operands in batches of KBATCH key blocks
    const uint16_t *kb_s = ks[buf];
    auto kread = [&](bf16x8 (&kf)[NKF], int kb0) {
#pragma unroll
      for (int i = 0; i < NKF; ++i) {
        const int kb = kb0 + i / (D / 16), s = i % (D / 16);
        kf[i] = *reinterpret_cast<const bf16x8 *>(kb_s + kof[s] + 32 * kb * D);
      }
    };
    bf16x8 kf[NKF];
    if (active) kread(kf, 0);
    uint16_t bv[2][16];
    if constexpr (BIAS == kBiasDense)
      if (active) dense_row_load(rbias, wrow0 + il, L, j0, hl, bv);

    if (active) {
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb % KBATCH == 0 && kb > 0) kread(kf, kb);
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) acc = mfma32(kf[(kb % KBATCH) * (D / 16) + s], qf[s], acc);
        sacc[kb] = acc;
      }

      // V operands (fragment i: dims 32db, keys 32kb + 16u), read now so the
      // softmax below covers their latency
      const uint16_t *vt_s = vs[buf];
      auto vread = [&](int i) {
        const int db = i >> 2, kb = (i >> 1) & 1, u = i & 1;
        return lds_read_tr8_at(vt_s + (32 * kb + 16 * u) * D, tro[db][0], tro[db][1]);
      };
      bf16x8 vf[NVF];
#pragma unroll
      for (int i = 0; i < VPRE; ++i) vf[i] = vread(i);

      // Element (kb, r): key j0 + 32kb + 8(r/4) + 4hl + r%4, query wrow0 + il.
      float bconst;
      // (the linear ALiBi path would not fit the 168 VGPRs of three
      // workgroups per CU at head_dim 64)
      const bool fast = score_tile_T<BIAS, CAUSAL, D == 128, D == 64>(
          sacc, j0, wrow0, il, hl, L, c, sat, lut, slope_l2, bconst, bv, &fl);
      // row max: two chains of v_max3 (one instruction per two elements; the
      // empty asm keeps the compiler from rebalancing them into a tree of
      // two-input maxes, which takes half as many instructions again)
      float m0 = fmaxf(sacc[0][0], sacc[0][1]), m1 = fmaxf(sacc[1][0], sacc[1][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) {
        asm volatile("" : "+v"(m0), "+v"(m1));
        m0 = fmaxf(m0, fmaxf(sacc[0][r], sacc[0][r + 1]));
        m1 = fmaxf(m1, fmaxf(sacc[1][r], sacc[1][r + 1]));
      }
      const float mx = half_max(fmaxf(m0, m1));
      // c > 0, so the scaled max is the max of the scaled scores
      const float tmax = fast ? fmaf(mx, c, bconst) : mx;

      const bool need = tmax > m_run + kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - tmax) : 1.f;
        if (need) m_run = tmax;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lsum[e] *= alpha;
          wsum[e] *= alpha;
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      const float cc = fast ? c : 1.f;
      const float sub = bconst - m_use;

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
            w[e] = pack_bf16x2(p0, p1);
            // fp32 row sums (not of the bf16-rounded values): LSE stays exact
            // to fp32, which the backward's recomputed P relies on
            lsum[e] += p0 + p1;
          }
          pb[kb][u] = __builtin_bit_cast(bf16x8, i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]});
        }

#pragma unroll
      for (int i = VPRE; i < NVF; ++i) vf[i] = vread(i);
      // O^T += V^T P^T, and the bf16 weight sums
#pragma unroll
      for (int i = 0; i < NVF; ++i) {
        const int db = i >> 2, kb = (i >> 1) & 1, u = i & 1;
        oacc[db] = mfma32(vf[i], pb[kb][u], oacc[db]);
        if (db == 0) wsum = mfma16(sel_operand(), pb[kb][u], wsum);
      }
    }
    // tile kt + 1 has landed (each wave waits for its own copies)
    if (NBUF == 3 && ahead)
      wait_vmem_loads_but<(NBUF - 2) * PER_FILL>();
    else
      wait_vmem_loads();
    __syncthreads();
  }

  const int myrow = wrow0 + il;
  const float l_tot = half_sum((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]));
  const float inv = wsum[0] > 0.f ? 1.f / wsum[0] : 0.f;
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
  if constexpr (BIAS == kBiasDense) {   // dense entry points only
    return causal ? launch_t<D, BIAS, true, false>(a, grid, s)
                  : launch_t<D, BIAS, false, false>(a, grid, s);
  } else if constexpr (BIAS == kBiasFire) {   // causal only
    (void)causal;
    return varlen ? launch_t<D, BIAS, true, true>(a, grid, s)
                  : launch_t<D, BIAS, true, false>(a, grid, s);
  } else {
    if (causal)
      return varlen ? launch_t<D, BIAS, true, true>(a, grid, s)
                    : launch_t<D, BIAS, true, false>(a, grid, s);
    return varlen ? launch_t<D, BIAS, false, true>(a, grid, s)
                  : launch_t<D, BIAS, false, false>(a, grid, s);
  }
}

template <int D>
hipError_t launch_d(const FwdArgs &a, int grid, int bias, bool causal, bool varlen,
                    hipStream_t s) {
  switch (bias) {
    case kBiasT5: return launch_b<D, kBiasT5>(a, grid, causal, varlen, s);
    case kBiasAlibi: return launch_b<D, kBiasAlibi>(a, grid, causal, varlen, s);
    case kBiasDense: return launch_b<D, kBiasDense>(a, grid, causal, varlen, s);
    case kBiasFire: return launch_b<D, kBiasFire>(a, grid, causal, varlen, s);
    default: return launch_b<D, kBiasNone>(a, grid, causal, varlen, s);
  }
}

}  // namespace

int fwd_tile_rows(int) { return BR; }

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
  a.dense = p.dense;
  a.rope_cs = b.rope_cs;
  a.fire_tab = b.fire_tab;
  a.fire_dist = b.fire_dist;
  a.dense_batch = p.dense_batch;
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
