// Device helpers for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Buffer resource over `bytes` bytes at `p`.  Loads past the end return 0 and
// stores past the end are dropped by the hardware range check, which handles
// ragged tiles without branches.  0x00020000 is the gfx9 dword-3 word (32-bit
// data format, no swizzle).
__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ i32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
// One bf16 (as its 16 bits) at byte offset `off`.
__device__ __forceinline__ uint16_t buf_load_u16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
// The same at byte offset voff (per lane) + soff (the same for the wave).
__device__ __forceinline__ uint16_t buf_load_u16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_store_f32(rsrc_t r, uint32_t voff, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, i32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, i32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store_f32(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, (int)off, 0, 0);
}

// Waits until every vector memory load issued so far has returned (vmcnt(0),
// other counters untouched).  Registers loaded before a loop must be waited
// for once before it: otherwise the compiler's wait insertion, which cannot
// tell across iterations that they have arrived, waits for all outstanding
// loads - including prefetches issued in the loop - at their first use.
__device__ __forceinline__ void wait_vmem_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// Wait until at most N of this wave's vector-memory loads are in flight (they
// complete in issue order, so every older one has landed).
template <int N>
__device__ __forceinline__ void wait_vmem_loads_but() {
  static_assert(N >= 0 && N <= 15, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.  Lane l holds
// row (l % 32) of A and column (l % 32) of B, each with 8 consecutive k values
// for half-wave (l / 32); the accumulator holds, in register r, the element
// (row 8*(r/4) + 4*(l/32) + r%4, column l % 32).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16), bf16 in, fp32 accumulate.  Lane l holds
// row (l % 16) of A and column (l % 16) of B, each with the 8 consecutive k
// values 8 (l / 16) .. 8 (l / 16) + 7; the accumulator holds, in register r,
// the element (row 4 (l / 16) + r, column l % 16).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}
__device__ __forceinline__ float bf16_bits(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// fp64 -> bf16 bits with one rounding to nearest, ties to even: round to
// fp32 with round-to-odd (truncate, then set the last bit if anything was
// dropped), which keeps enough information for the final fp32 -> bf16
// rounding to be the correctly rounded result.
__device__ __forceinline__ uint32_t bf16_bits_rne(double x) {
  const float f = (float)x;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != x) {
    if (fabs(back) > fabs(x)) u -= 1;   // step back toward zero
    u |= 1u;
  }
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// (cos, sin) of the RoPE angles of two consecutive pairs, fp64, from one
// 32-byte entry pair of the table.
struct RopeCs2 {
  double c0, s0, c1, s1;
};
__device__ __forceinline__ RopeCs2 rope_cs2(rsrc_t r, uint32_t off) {
  const i32x4 a = buf_load16(r, off), b = buf_load16(r, off + 16u);
  const auto da = __builtin_bit_cast(__attribute__((ext_vector_type(2))) double, a);
  const auto dbv = __builtin_bit_cast(__attribute__((ext_vector_type(2))) double, b);
  return RopeCs2{da[0], da[1], dbv[0], dbv[1]};
}

// RoPE on registers: the pair (x0, x1) held as one bf16x2 word, turned by the
// angle with (cos, sin) = (c, s): exact in fp64 (a product of bf16 and fp64
// values, summed with one fma), then rounded once to bf16, which is what a
// rotation computed exactly and stored in bf16 gives.
__device__ __forceinline__ uint32_t rope_rotate_pair(uint32_t w, double c, double s) {
  const double x0 = (double)bf16_lo(w), x1 = (double)bf16_hi(w);
  return bf16_bits_rne(fma(x0, c, -x1 * s)) | (bf16_bits_rne(fma(x0, s, x1 * c)) << 16);
}

// Max / sum of a value over the two half-waves (lanes l and l ^ 32), with
// v_permlane32_swap (a VALU lane exchange, no LDS round trip).  Both lanes of
// a pair get the same result, bit for bit.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                                  __builtin_bit_cast(int, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                                  __builtin_bit_cast(int, x), false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Sum over the 64 lanes of a wave, complete in lane 63 (the other lanes hold
// partial sums), by DPP moves within the VALU: pairs and quads by quad
// permutes, rows of 16 by two rotations, then row 0's sum broadcast into row
// 1 and row 2's into row 3, and row 1's (rows 0 + 1) into row 3.  A fixed
// order: the result does not depend on timing.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
  // lanes outside ROW_MASK take 0 (the `old` operand)
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                   CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum_lane63(float x) {
  x = dpp_add<0xb1, 0xf>(x);    // quad_perm [1, 0, 3, 2]
  x = dpp_add<0x4e, 0xf>(x);    // quad_perm [2, 3, 0, 1]
  x = dpp_add<0x124, 0xf>(x);   // row_ror 4
  x = dpp_add<0x128, 0xf>(x);   // row_ror 8: every lane holds its row's sum
  x = dpp_add<0x142, 0xa>(x);   // row_bcast 15: rows 1 and 3 add rows 0 and 2
  x = dpp_add<0x143, 0xc>(x);   // row_bcast 31: rows 2 and 3 add lane 31 (rows 0 + 1)
  return x;
}

// Minimum and maximum over the 64 lanes of a wave, returned in every lane:
// the same DPP pattern as wave_sum_lane63 (lanes outside a row mask take the
// identity), then lane 63 read back as a scalar.  The wave must be fully
// active.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_min_max(int &lo, int &hi) {
  lo = min(lo, __builtin_amdgcn_update_dpp(0x7fffffff, lo, CTRL, ROW_MASK, 0xf, false));
  hi = max(hi, __builtin_amdgcn_update_dpp(-0x7fffffff - 1, hi, CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ void wave_min_max(int &lo, int &hi) {
  dpp_min_max<0xb1, 0xf>(lo, hi);
  dpp_min_max<0x4e, 0xf>(lo, hi);
  dpp_min_max<0x124, 0xf>(lo, hi);
  dpp_min_max<0x128, 0xf>(lo, hi);
  dpp_min_max<0x142, 0xa>(lo, hi);
  dpp_min_max<0x143, 0xc>(lo, hi);
  lo = __builtin_amdgcn_readlane(lo, 63);
  hi = __builtin_amdgcn_readlane(hi, 63);
}

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8),
// each XCD with its own L2.  This remap gives every XCD a contiguous range of
// logical ids, so the query tiles of one (sequence, head) - which stream the
// same K and V - share one L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int per = n >> 3;
  if (b >= (per << 3)) return b;
  return (b & 7) * per + (b >> 3);
}

// Dense grids: logical id g -> (pair, rank), pair = (batch, head) and rank 0
// the heaviest tile of a pair (most key or query tiles to visit).  When the
// pairs split evenly over the 8 XCDs, the ids an XCD receives (a contiguous
// range, see xcd_remap) cover its own pairs in groups of G, each group
// rank-major: heavy tiles start early (longest-processing-time order; with
// plain pair-major order the heaviest tiles of the last pairs start last and
// run nearly alone at the end), while the tiles running at any time belong
// to few pairs, whose K and V stay in the XCD's L2.  Otherwise the order is
// pair-major.  The best G depends on the workgroups an XCD runs at once:
// with G pairs of 32 causal tiles per group, a group's light tiles must
// overlap the next group's heavy ones without leaving slots idle at the end
// (a list-scheduling simulation of 12 pairs per XCD: G = 4 is ideal for 64
// concurrent workgroups, G = 3 or 6 for 96; G = 6 measured best for the
// forward's 96).
// G is the largest divisor of the XCD's pair count up to GMAX.
template <int GMAX>
__device__ __forceinline__ void tile_order(int g, int npairs, int ntile, int &pair, int &rank) {
  const int pp = npairs >> 3;
  int G = GMAX;
  while (G > 1 && pp % G != 0) --G;
  if ((npairs & 7) == 0 && pp > 0) {
    const int per = pp * ntile, gsz = G * ntile;
    const int x = g / per, r = g - x * per;
    const int gi = r / gsz, rg = r - gi * gsz;
    rank = rg / G;
    pair = x * pp + gi * G + (rg - rank * G);
  } else {
    pair = g / ntile;
    rank = g - pair * ntile;
  }
}

// (batch, head) of a dense grid's pair.  Pairs run in order on each XCD
// (tile_order), so with a dense bias matrix shared by the batch the pairs of
// one head are numbered together (head-major): the tiles running at once on
// an XCD then read the same bias rows, which the XCD's L2 serves after the
// first read.  Otherwise batch-major.
__device__ __forceinline__ void pair_bh(int pair, int nbatch, int heads, bool head_major, int &b,
                                        int &h) {
  if (head_major) {
    h = pair / nbatch;
    b = pair - h * nbatch;
  } else {
    b = pair / heads;
    h = pair - b * heads;
  }
}

// T5 bucket of relative position r (key - query) from the integer thresholds.
__device__ __forceinline__ int t5_bucket_dev(int r, const T5Geometry &g) {
  int off = 0, n;
  if (g.bidir) {
    off = r > 0 ? g.nbp : 0;
    n = r > 0 ? r : -r;
  } else {
    n = r < 0 ? -r : 0;
  }
  if (n < g.me) return off + n;
  int b = g.me;
  for (int k = 0; k < g.nthr; ++k) b += (n >= g.thr[k]) ? 1 : 0;
  return off + b;
}

// The T5 bias by relative distance r (log2 units) lives in LDS for r in
// [-sat - kLutPad, sat + kLutPad]; past +-sat every entry repeats the
// saturated bucket, and under a causal mask the entries for r > 0 are -inf.
// A lane's distances in a 64-key tile are rbase + off, off in [0, 59], so
// each element reads its entry at a fixed offset from one per-lane base,
// with no clamp per element and no causal test.  The base itself is clamped
// to [-sat - kLutPad, sat + kLutPad - 59]: a clamp moves it only when all
// the lane's distances are saturated on that side (kLutPad > 59), and the
// entries it then reads hold the same saturated value.
constexpr int kLutPad = 96;

// FIRE (see fa_internal.h and fire.hip): a workgroup's LDS copy of the
// segment table (the shared part, then its head's A and B), the distance
// table, and per lane the constants of its query row and the segment its
// sweep has reached.
struct FireLane {
  const float *tab = nullptr;   // LDS, kFireLds floats
  rsrc_t dist;                  // psi(d) at [kFireDistPad + d], then d / (c d + 1)
  uint32_t dist_half = 0;       // byte offset of the d / (c d + 1) half
  float c = 0.f;                // psi(t) = log(c t + 1)
  float inv = 0.f;              // 1 / log2(c max(L, i) + 1) for the lane's row i
  int seg = -1;                 // segment of the last x looked up (-1: none yet)
  float seg_lo = 0.f, seg_hi = 0.f;   // its bounds t_seg, t_seg+1 (valid when seg >= 0)
};

__device__ __forceinline__ FireLane fire_lane(const float *gtab, const float *dist, int maxlen,
                                              const float *lds, int row) {
  FireLane fl;
  fl.tab = lds;
  const uint32_t n = (uint32_t)maxlen + 2u * kFireDistPad;
  fl.dist = make_rsrc(dist, 8u * n);
  fl.dist_half = 4u * n;
  fl.c = gtab[2];
  fl.inv = 1.f / __builtin_amdgcn_logf(fmaf(fl.c, fmaxf(gtab[3], (float)row), 1.f));
  return fl;
}

// The four table entries psi(d0) .. psi(d0 + 3) (half = 0) or d / (c d + 1)
// (half = fl.dist_half), d0 >= -kFireDistPad.
__device__ __forceinline__ f32x4 fire_dist4(const FireLane &fl, int d0, uint32_t half = 0) {
  return __builtin_bit_cast(f32x4,
                            buf_load16(fl.dist, half + 4u * (uint32_t)(kFireDistPad + d0)));
}

// Segment of x: the number of kinks t_s <= x, by a branch-free binary search
// over t_1 .. t_127 (+inf past the last kink).
__device__ __forceinline__ int fire_seg(const float *tab, float x) {
  int s = 0;
#pragma unroll
  for (int step = kFireTEnd / 2; step >= 1; step >>= 1)
    s += (x >= tab[kFireOffT + s + step]) ? step : 0;
  return min(s, kFireMaxHidden);
}

// The same, walking from a nearby segment s (x moves little between the
// tiles of one lane's sweep, so this is a read or two); s < 0 searches.
__device__ __forceinline__ int fire_walk(const float *tab, float x, int s) {
  if (s < 0) return fire_seg(tab, x);
  while (s > 0 && x < tab[kFireOffT + s]) --s;
  while (s < kFireMaxHidden && x >= tab[kFireOffT + s + 1]) ++s;
  return s;
}

// The same with segment s's bounds [lo, hi) held in registers: while x
// stays inside (most tiles) no table read waits; otherwise the walk, and lo,
// hi become the bounds of the segment found.
__device__ __forceinline__ int fire_walk_cached(const float *tab, float x, int s, float &lo,
                                                float &hi) {
  if (s >= 0 && x >= lo && x < hi) return s;
  s = fire_walk(tab, x, s);
  lo = tab[kFireOffT + s];
  hi = tab[kFireOffT + s + 1];
  return s;
}

// Copy the table's shared part and head h's coefficients into LDS (all
// threads of the workgroup; a barrier must follow before any read).
__device__ __forceinline__ void fire_load(const float *gtab, int h, float *lds, int tid, int nt) {
  for (int i = tid; i < kFireLds; i += nt)
    lds[i] = i < kFireShared ? gtab[i]
                             : gtab[kFireShared + (size_t)h * kFireHeadStride + (i - kFireShared)];
}

// Scores (log2 units, in place) of one lane's keys in a query-parallel tile
// of NKB 32-key blocks with the FIRE bias: element (kb, r) is key offset
// off = 32 kb + 8 (r / 4) + r % 4 past the lane's first key, distance
// d = -(rbase + off), x = psi(d) inv.  TABLE reads psi from the distance
// table (one 16-byte load per four keys; the tile's 32 values are held from
// load to use, which costs registers), otherwise each key takes a log2 (a
// transcendental, which the exponential of the softmax competes for).
// x is monotone in d, so the segments of the nearest and farthest keys
// (offsets 0 and omax) bound every key's: equal, the bias is A + B x; apart,
// every key adds to the lower segment's line the bend of each kink in
// between (without the table, a single kink is taken by a select).  Masked keys (causal, or off >= lim)
// become -inf.  KEEP_X also returns every key's x (0 for keys after the
// query) and the nearest key's segment (the farthest one's stays in fl.seg).
template <int NKB, bool TABLE, bool KEEP_X = false>
__device__ __forceinline__ void fire_scores(f32x16 (&sacc)[NKB], int omax, int rbase, int lim,
                                            bool mask_c, float c, FireLane &fl,
                                            float (*xkeep)[16] = nullptr, int *seg_hi = nullptr) {
  const float cn = -fl.c;
  const float u0 = fmaf(cn, (float)rbase, 1.f);
  // without the table: e of key offset 32 kb + 8 q + i is one fma per group
  // of four keys, then one add of -c i (the offsets as per-key float
  // constants would each be held in a register); the range ends use the
  // same operations
  const float ce[4] = {0.f, cn, 2.f * cn, 3.f * cn};
  f32x4 ps[TABLE ? NKB : 1][4];
  float xn, xf;
  if constexpr (TABLE) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q) ps[kb][q] = fire_dist4(fl, -rbase - 32 * kb - 8 * q - 3);
    xn = ps[0][0][3] * fl.inv;
    xf = ps[NKB - 1][3][0] * fl.inv;
  } else {
    xn = __builtin_amdgcn_logf(fmaxf(u0, 1.f)) * fl.inv;
    xf = __builtin_amdgcn_logf(fmaxf(fmaf(cn, (float)(omax - 3), u0) + ce[3], 1.f)) * fl.inv;
  }
  float lo = fl.seg_lo, hi = fl.seg_hi;
  const int shi = fire_walk_cached(fl.tab, xn, fl.seg, lo, hi);
  const int slo = fire_walk_cached(fl.tab, xf, shi, lo, hi);
  fl.seg = slo;
  fl.seg_lo = lo;
  fl.seg_hi = hi;
  if constexpr (KEEP_X) *seg_hi = shi;
  if constexpr (TABLE) {
    if (shi == slo) {
      const float A = fl.tab[kFireOffA + slo], B = fl.tab[kFireOffB + slo];
      // without KEEP_X the lane's normaliser folds into the slope: one FMA
      // per key for the bias
      const float Bi = B * fl.inv;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float psd = ps[kb][r >> 2][3 - (r & 3)];
          if constexpr (KEEP_X) {
            const float x = psd * fl.inv;
            xkeep[kb][r] = x;
            sacc[kb][r] = fmaf(sacc[kb][r], c, fmaf(B, x, A));
          } else {
            sacc[kb][r] = fmaf(sacc[kb][r], c, fmaf(Bi, psd, A));
          }
        }
    } else {
      // b(x) = A_lo + B_lo x + sum over the kinks t_k above segment lo of
      // (B_k - B_k-1) max(x - t_k, 0): b is continuous, so each kink only
      // bends the line
      const int span = shi - slo;
      const float A = fl.tab[kFireOffA + slo], B = fl.tab[kFireOffB + slo];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = ps[kb][r >> 2][3 - (r & 3)] * fl.inv;
          if constexpr (KEEP_X) xkeep[kb][r] = x;
          sacc[kb][r] = fmaf(sacc[kb][r], c, fmaf(B, x, A));
        }
      for (int j = 1; j <= span; ++j) {
        const int k = slo + j;
        const float tk = fl.tab[kFireOffT + k];
        const float dB = fl.tab[kFireOffB + k] - fl.tab[kFireOffB + k - 1];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[kb][r] = fmaf(dB, fmaxf(ps[kb][r >> 2][3 - (r & 3)] * fl.inv - tk, 0.f),
                               sacc[kb][r]);
      }
    }
  } else {
    auto e_of = [&](int kb, int q, int i, float &g) {
      if (i == 0) g = fmaf(cn, (float)(32 * kb + 8 * q), u0);
      return g + ce[i];
    };
    float g = 0.f;
    if (shi == slo) {
      const float A = fl.tab[kFireOffA + slo], Bi = fl.tab[kFireOffB + slo] * fl.inv;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float l = __builtin_amdgcn_logf(e_of(kb, r >> 2, r & 3, g));
          if constexpr (KEEP_X) xkeep[kb][r] = fmaxf(l, 0.f) * fl.inv;
          sacc[kb][r] = fmaf(sacc[kb][r], c, fmaf(Bi, l, A));
        }
    } else if (shi == slo + 1) {
      const float tk = fl.tab[kFireOffT + shi];
      const float A0 = fl.tab[kFireOffA + slo], B0 = fl.tab[kFireOffB + slo];
      const float A1 = fl.tab[kFireOffA + shi], B1 = fl.tab[kFireOffB + shi];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = __builtin_amdgcn_logf(e_of(kb, r >> 2, r & 3, g)) * fl.inv;
          if constexpr (KEEP_X) xkeep[kb][r] = fmaxf(x, 0.f);
          const bool up = x >= tk;
          sacc[kb][r] = fmaf(sacc[kb][r], c, fmaf(up ? B1 : B0, x, up ? A1 : A0));
        }
    } else {
      // the kink bends as above, one block of keys at a time holding its x
      const int span = shi - slo;
      const float A = fl.tab[kFireOffA + slo], B = fl.tab[kFireOffB + slo];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float xs[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          xs[r] = __builtin_amdgcn_logf(fmaxf(e_of(kb, r >> 2, r & 3, g), 1.f)) * fl.inv;
          if constexpr (KEEP_X) xkeep[kb][r] = xs[r];
          sacc[kb][r] = fmaf(sacc[kb][r], c, fmaf(B, xs[r], A));
        }
        for (int j = 1; j <= span; ++j) {
          const int k = slo + j;
          const float tk = fl.tab[kFireOffT + k];
          const float dB = fl.tab[kFireOffB + k] - fl.tab[kFireOffB + k - 1];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[kb][r] = fmaf(dB, fmaxf(xs[r] - tk, 0.f), sacc[kb][r]);
        }
      }
    }
  }
  // one per-lane limit: a key after the query (rbase + off > 0) or past
  // the end (off >= lim); a tile with neither mask skips the compares
  // (mask_c is per tile, and lim is below the tile width on every lane or
  // on none)
  if (mask_c || lim < 32 * NKB) {
    const int lim2 = mask_c ? min(lim, 1 - rbase) : lim;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
        if (off >= lim2) sacc[kb][r] = -INFINITY;
      }
  }
}

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// source lane s reads 4 consecutive bf16 values at its own address; lane i
// of the group receives element (i % 4) of the values read by source lanes
// 4m + i/4, m = 0..3, in that order.  So if source lane s = 4m + c points at
// row r_m, columns c0 + 4c .. c0 + 4c + 3 of a row-major tile, lane i gets
// column c0 + i of rows r_0..r_3.
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(__attribute__((address_space(3))) void *)(p));
}

// Scores of one 64-key x 32-query tile in the transposed layout used by the
// query-parallel kernels: sacc[kb][r] holds q.k (unscaled) for query
// row0 + il and key j0 + 32kb + 8(r/4) + 4hl + r%4.
//
// Returns true when the tile needs no per-element work: no mask applies and
// the bias is one value for the whole tile (no bias, or every pair saturated
// to the same T5 bucket); the log2-domain score is then fma(s, c, bconst).
// Otherwise the scores are finished in place in log2 units (scaled, biased,
// masked to -inf) and bconst is 0, so fma(s, 1, 0) gives them.
// The causal mask hides keys after the query; keys at or past L are masked.
// A dense bias arrives as the lane's own values bv (bf16 bits, same order
// as sacc; see dense_row_load).
// WHOLE: the sequence length is a multiple of 64, so no tile reaches past
// its end and the length test drops out at compile time.
template <int BIAS, bool CAUSAL, bool ALIBI_LINEAR = true, bool FIRE_TABLE = false,
          bool WHOLE = false>
__device__ __forceinline__ bool score_tile_T(f32x16 (&sacc)[2], int j0, int row0, int il, int hl,
                                             int L, float c, int sat, const float *lut,
                                             float slope_l2, float &bconst,
                                             const uint16_t (&bv)[2][16],
                                             FireLane *fl = nullptr) {
  const int rmin = j0 - (row0 + 31), rmax = j0 + 63 - row0;
  const bool mask_c = CAUSAL && rmax > 0;
  const bool mask_l = !WHOLE && j0 + 64 > L;
  bool uniform = (BIAS == kBiasNone);
  bconst = 0.f;
  if constexpr (BIAS == kBiasT5) {
    const int lo = min(max(rmin, -sat), sat), hi = min(max(rmax, -sat), sat);
    uniform = (lo == hi);
    bconst = lut[lo];
  }
  if (uniform && !mask_c && !mask_l) return true;
  bconst = 0.f;
  const int rbase = j0 - (row0 + il) + 4 * hl;
  const int jb = j0 + 4 * hl;
  if constexpr (BIAS == kBiasT5) {
    // the causal mask is in the table; the length mask is one compare per
    // element against a per-lane limit (past every offset when the tile
    // needs none)
    const float *lb = lut + min(max(rbase, -sat - kLutPad), sat + kLutPad - 59);
    const int lim = mask_l ? L - jb : 64;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
        const float t = fmaf(sacc[kb][r], c, lb[off]);
        sacc[kb][r] = off >= lim ? -INFINITY : t;
      }
    return false;
  }
  if constexpr (BIAS == kBiasFire) {
    // (the distance table where the registers allow: the forward at 64)
    fire_scores<2, FIRE_TABLE>(sacc, 59, rbase, mask_l ? L - jb : 64, mask_c, c, *fl);
    return false;
  }
  if constexpr (BIAS == kBiasAlibi && ALIBI_LINEAR) {
    // all distances of the tile on one side of 0 and no mask: the bias is
    // linear in the key offset, -slope |r| = sl (rbase + off)
    if (!mask_c && !mask_l && (rmax <= 0 || rmin >= 0)) {
      const float sl = rmax <= 0 ? -slope_l2 : slope_l2;
      const float b0 = sl * (float)rbase;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float bq = fmaf((float)(32 * kb + 8 * q), sl, b0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[kb][4 * q + e] = fmaf(sacc[kb][4 * q + e], c, fmaf((float)e, sl, bq));
        }
      return false;
    }
  }
  // one per-lane limit for both masks: offset off is a key after the query
  // (rbase + off > 0) or past the end (jb + off >= L) iff off >= lim; a
  // tile with neither mask skips the compares
  int lim = 64;
  if (mask_c) lim = min(lim, 1 - rbase);
  if (mask_l) lim = min(lim, L - jb);
  const bool masked = mask_c || mask_l;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
      const int rr = rbase + off;
      float t = sacc[kb][r] * c;
      if constexpr (BIAS == kBiasAlibi) t = fmaf(fabsf((float)rr), slope_l2, t);
      if constexpr (BIAS == kBiasDense) t = fmaf(bf16_bits(bv[kb][r]), kLog2e, t);
      sacc[kb][r] = t;
      // keep the bias-table reads from being hoisted all at once
      if ((r & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * kb + 8 * (r >> 2) + (r & 3) >= lim) sacc[kb][r] = -INFINITY;
  }
  return false;
}

// The same for one 32-key block (keys jb0 .. jb0 + 31; bv its dense bias
// values), for the query-parallel kernel's 32-key tiles.
template <int BIAS, bool CAUSAL>
__device__ __forceinline__ bool score_block_T(f32x16 &sacc, int jb0, int row0, int il, int hl,
                                              int L, float c, int sat, const float *lut,
                                              float slope_l2, float &bconst,
                                              const uint16_t (&bv)[16],
                                              FireLane *fl = nullptr) {
  const int rmin = jb0 - (row0 + 31), rmax = jb0 + 31 - row0;
  const bool mask_c = CAUSAL && rmax > 0;
  const bool mask_l = jb0 + 32 > L;
  bool uniform = (BIAS == kBiasNone);
  bconst = 0.f;
  if constexpr (BIAS == kBiasT5) {
    const int lo = min(max(rmin, -sat), sat), hi = min(max(rmax, -sat), sat);
    uniform = (lo == hi);
    bconst = lut[lo];
  }
  if (uniform && !mask_c && !mask_l) return true;
  bconst = 0.f;
  const int rbase = jb0 - (row0 + il) + 4 * hl;
  const int jb = jb0 + 4 * hl;
  if constexpr (BIAS == kBiasT5) {
    // offsets 0 .. 27 from one clamped base (see kLutPad); the length mask
    // against a per-lane limit, as in score_tile_T
    const float *lb = lut + min(max(rbase, -sat - kLutPad), sat + kLutPad - 27);
    const int lim = mask_l ? L - jb : 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 8 * (r >> 2) + (r & 3);
      const float t = fmaf(sacc[r], c, lb[off]);
      sacc[r] = off >= lim ? -INFINITY : t;
    }
    return false;
  }
  if constexpr (BIAS == kBiasFire) {
    f32x16 (&one)[1] = *reinterpret_cast<f32x16 (*)[1]>(&sacc);
    fire_scores<1, false>(one, 27, rbase, mask_l ? L - jb : 32, mask_c, c, *fl);
    return false;
  }
  if constexpr (BIAS == kBiasAlibi) {
    // one-sided and unmasked: the bias is linear in the key offset
    if (!mask_c && !mask_l && (rmax <= 0 || rmin >= 0)) {
      const float sl = rmax <= 0 ? -slope_l2 : slope_l2;
      const float b0 = sl * (float)rbase;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float bq = fmaf((float)(8 * q), sl, b0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sacc[4 * q + e] = fmaf(sacc[4 * q + e], c, fmaf((float)e, sl, bq));
      }
      return false;
    }
  }
  // one per-lane limit for both masks, as in score_tile_T
  int lim = 32;
  if (mask_c) lim = min(lim, 1 - rbase);
  if (mask_l) lim = min(lim, L - jb);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int off = 8 * (r >> 2) + (r & 3);
    const int rr = rbase + off;
    float t = sacc[r] * c;
    if constexpr (BIAS == kBiasAlibi) t = fmaf(fabsf((float)rr), slope_l2, t);
    if constexpr (BIAS == kBiasDense) t = fmaf(bf16_bits(bv[r]), kLog2e, t);
    sacc[r] = off >= lim ? -INFINITY : t;
  }
  return false;
}

// The dense bias values one lane needs for a 64-key tile of the query-
// parallel kernels: row `row` (the lane's query), keys j0 + 32kb + 8(r/4) +
// 4hl + r%4, from a buffer over one [S, S] bf16 matrix (row stride S).
// Rows past the matrix read as 0; keys past S read the next row, which the
// key mask then hides.
// When S is a multiple of 4, each group of 4 keys starts 8-byte aligned and
// is fetched with one 8-byte load.
__device__ __forceinline__ void dense_row_load(rsrc_t rb, int row, int S, int j0, int hl,
                                               uint16_t (&bv)[2][16]) {
  const uint32_t base = (uint32_t)row * (uint32_t)S + (uint32_t)(j0 + 4 * hl);
  if ((S & 3) == 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint2 w = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(rb, (int)((base + 32 * kb + 8 * g) * 2u),
                                                        0, 0));
        bv[kb][4 * g] = (uint16_t)w.x;
        bv[kb][4 * g + 1] = (uint16_t)(w.x >> 16);
        bv[kb][4 * g + 2] = (uint16_t)w.y;
        bv[kb][4 * g + 3] = (uint16_t)(w.y >> 16);
      }
  } else {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        bv[kb][r] = buf_load_u16(rb, (base + 32 * kb + 8 * (r >> 2) + (r & 3)) * 2u);
  }
}

// ---------------------------------------------------------------------------
// Unpadded bf16 tiles in LDS, swizzled by 16-byte chunk, filled straight from
// global memory by buffer-to-LDS copies.
//
// A tile row holds D bf16 (D / 8 chunks); chunk c of row r is stored at chunk
// position c ^ swz<D>(r) of that row.  gfx950's LDS has 64 four-byte banks,
// so a 256-byte line spans them all.  Both MFMA operand reads of a tile are
// then free of bank conflicts:
//   row reads        16 lanes read one chunk of 16 consecutive rows
//                    (r0 a multiple of 16): swz is a bijection on those rows
//                    within each bank line;
//   transposing      a half-wave reads the same four chunks 4g .. 4g + 3 of
//   reads            rows 4h .. 4h + 3 of an 8-row group: swz sends them to
//                    four different chunk groups (or bank-line halves).
// D = 64 (two rows per line): swz = 4 * bit1(r) + bits 2..3 of r.
// D = 128 (one row per line): swz = 4 * (r & 3) + bits 2..3 of r.
// Both depend on bits 0..3 of r only, so row offsets that are multiples of
// 16 keep a lane's swizzle.
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "head_dim");
  return D == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
}

// Element offset of chunk c of row r in a swizzled tile.
template <int D>
__device__ __forceinline__ int swz_off(int r, int c) {
  return r * D + 8 * (c ^ swz<D>(r));
}

// Element offset for the transposing read that assembles an MFMA operand of
// 8 rows x 1 column: the lane's own column is 32 db + (lane % 32) and its 8
// rows are, for k-slot v of half-wave hl, 4 hl + v (v < 4) and
// 8 + 4 hl + (v - 4) relative to a 16-row group.  half = 0 gives the offset
// for the first four rows, half = 1 for the last four, in a swizzled tile.
template <int D>
__device__ __forceinline__ int swz_tr_off(int lane, int half, int db) {
  const int i16 = lane & 15, hl = lane >> 5, b4 = (lane >> 4) & 1;
  const int r = 8 * half + 4 * hl + (i16 >> 2);
  const int c = 4 * db + 2 * b4 + ((i16 & 3) >> 1);
  return swz_off<D>(r, c) + 4 * (i16 & 1);
}

// The 8-row operand for one MFMA k-step of a swizzled tile: two transposing
// reads at the lane's offsets for the two halves of the 16-row group.
__device__ __forceinline__ bf16x8 lds_read_tr8_at(const uint16_t *base, int off0, int off1) {
  const s16x4 lo = lds_read_tr(base + off0);
  const s16x4 hi = lds_read_tr(base + off1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Global -> LDS copies.  `desc` is a raw buffer descriptor (dma_desc) over
// the source; lane l writes the bytes at byte offset `off` of the source to
// lds + 16 l (dma16) or lds + 4 l (dma4); `lds` must be the same for the
// whole wave; offsets past the descriptor's range write zeros.
//
// The copies are issued as inline assembly: the compiler's wait insertion
// cannot tell a copy's LDS destination from the tile being read and would
// wait for every copy in flight before each LDS read, which would serialise
// the prefetch.  The caller waits for its own copies (wait_vmem_loads)
// before the barrier that hands the tile to the other waves.  Copies the
// compiler does not count can only make its own count-based waits for
// other loads stricter, since loads complete in issue order.
//
// The hazard checks of the compiler do not look inside inline assembly, so
// each copy opens with the wait states the CDNA ISA requires before it:
// one after a scalar write of M0 (the LDS address of an LDS-bound buffer
// load) and five after a vector instruction that writes an SGPR the buffer
// load reads (the descriptor may be restored from a spill with
// v_readlane_b32 just before the copy).  `s_nop 4` gives five.
__device__ __forceinline__ i32x4 dma_desc(const void *p, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  return i32x4{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xffffu), (int)bytes, 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void *lds) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)lds;
}
__device__ __forceinline__ void dma16(i32x4 desc, uint32_t off, void *lds) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(desc), "{m0}"(lds_addr(lds))
               : "memory");
}
__device__ __forceinline__ void dma4(i32x4 desc, uint32_t off, void *lds) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(desc), "{m0}"(lds_addr(lds))
               : "memory");
}

// Fill the R rows of a swizzled tile from rows row0 .. row0 + R - 1 of a
// row-major bf16 matrix with row stride `stride` elements.  The tile is cut
// into 1 KB pieces (64 chunk positions); wave w of NW copies pieces w,
// w + NW, ...; lane l of a piece fetches the chunk that belongs at position l.
// Rows outside the buffer's range arrive as zeros.
template <int D, int R, int NW>
__device__ __forceinline__ void dma_tile(i32x4 src, int stride, int row0, uint16_t *tile,
                                         int wave, int lane) {
  constexpr int NPIECE = R * D * 2 / 1024;
  static_assert(NPIECE % NW == 0, "tile pieces per wave");
#pragma unroll
  for (int i = 0; i < NPIECE / NW; ++i) {
    const int piece = wave + NW * i;
    const int pos = piece * 64 + lane;
    const int r = pos / (D / 8), pc = pos % (D / 8);
    const int c = pc ^ swz<D>(r);
    dma16(src, ((uint32_t)(row0 + r) * (uint32_t)stride + 8 * c) * 2u, tile + piece * 512);
  }
}

}  // namespace fa
