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
//   accumulators as the MFMA B operand; its A operand (each lane: one dim,
//   the 8 keys matching its P values) comes from the row-major V tile through
//   the transposing LDS read, so K and V are staged the same way.
#include "fa_device.h"

namespace fa {
namespace {

constexpr int BC = 64;    // keys per tile
constexpr int NT = 256;   // threads per workgroup (4 waves)
// Query rows per wave, in blocks of 32.  Two blocks per wave would let every
// K and V operand read from LDS feed two MFMAs, but at ~240 registers it drops
// occupancy to 2 waves per SIMD and measured slower at head_dim 64 (and does
// not fit at 128), so each wave owns one block.
template <int D>
struct FwdTile {
  static constexpr int RB = 1;                   // 32-row blocks per wave
  static constexpr int BR = 4 * 32 * RB;         // query rows per workgroup
};
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
  constexpr int RB = FwdTile<D>::RB;
  constexpr int BR = FwdTile<D>::BR;
  constexpr int WR = 32 * RB;                 // rows per wave
  constexpr int NCH = D / 8;                  // 16-byte chunks per row
  constexpr int LOADS = BC * NCH / NT;        // K (and V) chunks per thread per tile
  // Row pitches (elements).  K rows are read 16 B per lane by 8 consecutive
  // rows at once: a pitch of an odd number of 16-byte slots keeps those reads
  // on distinct banks.  V is read with the transposing read, 4 rows x 32 B per
  // 16 lanes: a pitch of 2 (mod 8) slots keeps those on distinct banks.
  constexpr int KP = D + 8;
  constexpr int VP = D + 16;
  static_assert(LOADS * NT == BC * NCH, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BC * KP];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][BC * VP];
  __shared__ float lut[BIAS == kBiasT5 ? 2 * kMaxDistance + 1 : 1];

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
  const int wrow0 = q0 + WR * wave;           // first row of this wave
  const bool wave_live = wrow0 < L;           // rows past the end do nothing

  // Q as the B operand of S^T = K Q^T: lane (hl, il) holds row
  // wrow0 + 32rb + il, dims 16s + 8hl .. +7 for k-step s.
  bf16x8 qf[RB][D / 16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[rb][s] = __builtin_bit_cast(
          bf16x8, buf_load16(rq, ((uint32_t)(wrow0 + 32 * rb + il) * (uint32_t)HD + 16 * s +
                                  8 * hl) * 2u));

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

  // staging: chunk c = tid + NT*u is row c / NCH, 16-byte column c % NCH.
  // K and V of the next tile are staged separately (K after this tile's QK
  // products, V after its PV products) so fewer staging registers are live at
  // the softmax.
  i32x4 sreg[LOADS];
  auto gload = [&](rsrc_t r, int j0) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + NT * u, row = c / NCH, col = c % NCH;
      sreg[u] = buf_load16(r, ((uint32_t)(j0 + row) * (uint32_t)HD + col * 8) * 2u);
    }
  };
  auto lstore = [&](uint16_t *dst, int pitch) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + NT * u, row = c / NCH, col = c % NCH;
      *reinterpret_cast<i32x4 *>(&dst[row * pitch + col * 8]) = sreg[u];
    }
  };

  // per-lane LDS offsets (elements); the rest of each address is a constant
  const int koff = il * KP + 8 * hl;                       // + 32kb*KP + 16s
  const int voff = tr_lane_offset(lane, VP);               // + (32kb + 16u) * VP + 32db

  f32x16 oacc[RB][D / 32];
  float m_run[RB], lsum[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[rb][db] = f32x16{};
    m_run[rb] = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) lsum[rb][e] = 0.f;
  }
  const float c = a.scale_log2;

  if (nkt > 0) {
    gload(rk, 0);
    lstore(ks[0], KP);
    gload(rv, 0);
    lstore(vs[0], VP);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int j0 = kt * BC;
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) gload(rk, j0 + BC);
    // a causal wave starts work once the tile reaches its last row
    const bool active = wave_live && (!CAUSAL || (j0 <= wrow0 + WR - 1));
    f32x16 sacc[RB][2];
    if (active) {
      const uint16_t *kb_s = ks[buf] + koff;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sacc[rb][kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kb_s + 32 * kb * KP + 16 * s);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) sacc[rb][kb] = mfma32(kf, qf[rb][s], sacc[rb][kb]);
        }
      }
    }
    if (more) {
      lstore(ks[buf ^ 1], KP);
      gload(rv, j0 + BC);
    }
    if (active) {
      const uint16_t *vt_s = vs[buf] + voff;

      bf16x8 pb[RB][2][2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // Element (kb, r) of block rb: key j0 + 32kb + 8(r/4) + 4hl + r%4,
        // query row0 + il.
        const int row0 = wrow0 + 32 * rb;
        float bconst;
        const bool fast = score_tile_T<BIAS, CAUSAL>(sacc[rb], j0, row0, il, hl, L, c, sat, lut,
                                                    slope_l2, bconst);
        float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          m0 = fmaxf(m0, fmaxf(sacc[rb][0][r], sacc[rb][0][r + 1]));
          m1 = fmaxf(m1, fmaxf(sacc[rb][1][r], sacc[rb][1][r + 1]));
        }
        float mx = fmaxf(m0, m1);
        mx = fmaxf(mx, xor32(mx));
        // c > 0, so the scaled max is the max of the scaled scores
        const float tmax = fast ? fmaf(mx, c, bconst) : mx;

        const bool need = tmax > m_run[rb] + kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(need)) {
          const float alpha = need ? __builtin_amdgcn_exp2f(m_run[rb] - tmax) : 1.f;
          if (need) m_run[rb] = tmax;
#pragma unroll
          for (int e = 0; e < 4; ++e) lsum[rb][e] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[rb][db][r] *= alpha;
        }
        const float m_use = (m_run[rb] == -INFINITY) ? 0.f : m_run[rb];
        const float cc = fast ? c : 1.f;
        const float sub = bconst - m_use;

#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 =
                  __builtin_amdgcn_exp2f(fmaf(sacc[rb][kb][8 * u + 2 * e], cc, sub));
              const float p1 =
                  __builtin_amdgcn_exp2f(fmaf(sacc[rb][kb][8 * u + 2 * e + 1], cc, sub));
              w[e] = pack_bf16x2(p0, p1);
              // fp32 row sums (not of the bf16-rounded values): LSE stays exact
              // to fp32, which the backward's recomputed P relies on
              lsum[rb][e] += p0 + p1;
            }
            pb[rb][kb][u] =
                __builtin_bit_cast(bf16x8, i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]});
          }
      }

      // O^T += V^T P^T: the A operand (dims x keys) comes straight from the
      // row-major V tile through two transposing reads per MFMA, shared by the
      // wave's row blocks.
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const bf16x8 vf = lds_read_tr8(vt_s + (32 * kb + 16 * u) * VP + 32 * db, VP);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma32(vf, pb[rb][kb][u], oacc[rb][db]);
          }
    }
    if (more) lstore(vs[buf ^ 1], VP);
    __syncthreads();
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int myrow = wrow0 + 32 * rb + il;
    const float l_run = (lsum[rb][0] + lsum[rb][1]) + (lsum[rb][2] + lsum[rb][3]);
    const float l_tot = l_run + xor32(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        i32x2 w = {(int)pack_bf16x2(oacc[rb][db][4 * rq] * inv, oacc[rb][db][4 * rq + 1] * inv),
                   (int)pack_bf16x2(oacc[rb][db][4 * rq + 2] * inv,
                                    oacc[rb][db][4 * rq + 3] * inv)};
        buf_store8(ro, ((uint32_t)myrow * (uint32_t)HD + 32 * db + 8 * rq + 4 * hl) * 2u, w);
      }
    if (hl == 0 && myrow < L) {
      const float lse = l_tot > 0.f ? (m_run[rb] + __log2f(l_tot)) * kLn2 : -INFINITY;
      size_t idx;
      if constexpr (VARLEN)
        idx = (size_t)h * a.total + tok0 + myrow;
      else
        idx = ((size_t)bidx * a.heads + h) * a.seqlen + myrow;
      a.lse[idx] = lse;
    }
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

int fwd_tile_rows(int head_dim) { return head_dim == 64 ? FwdTile<64>::BR : FwdTile<128>::BR; }

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
    const int br = fwd_tile_rows(p.head_dim);
    a.nq = (p.seqlen + br - 1) / br;
    grid = p.nbatch * p.heads * a.nq;
  }
  a.nwg = grid;
  if (grid <= 0) return hipSuccess;
  if (p.head_dim == 64) return launch_d<64>(a, grid, p.bias, p.causal, p.varlen, s);
  return launch_d<128>(a, grid, p.bias, p.causal, p.varlen, s);
}

}  // namespace fa
