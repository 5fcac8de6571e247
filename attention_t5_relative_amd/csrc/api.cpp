// C ABI of libfat5attn: argument checks, workspace layout, T5 bucket
// thresholds and dispatch to the kernel launchers.  The declarations and the
// contract of every entry point are in include/fat5attn.h.
#include "fat5attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "fa_internal.h"

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fa_status hip_fail(hipError_t e, const char *where) {
  return fail(FA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// Kernel timers (benchmark hook)
// ---------------------------------------------------------------------------
struct Timer {
  hipEvent_t start = nullptr, stop = nullptr;
};
std::mutex g_timer_mu;
Timer g_timers[FA_KERNEL_COUNT];

Timer timer_of(int id) {
  std::lock_guard<std::mutex> lock(g_timer_mu);
  return g_timers[id];
}

// Runs `launch` bracketed by the events registered for kernel `id`, if any.
template <typename F>
hipError_t timed(int id, hipStream_t s, F &&launch) {
  const Timer t = timer_of(id);
  if (t.start) {
    const hipError_t e = hipEventRecord(t.start, s);
    if (e != hipSuccess) return e;
  }
  const hipError_t e = launch();
  if (e != hipSuccess) return e;
  if (t.stop) return hipEventRecord(t.stop, s);
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// T5 thresholds by exact integer comparison.  For n >= me the T5 bucket is
// me + floor(ln(n/me) / ln(md/me) * L) (L = nb' - me) capped at nb' - 1, and
// floor(...) >= k  <=>  n^L * me^k >= md^k * me^L.  thr[k-1] is the smallest
// such n (k = 1 .. L-1), found by binary search on n in [me, md].
// ---------------------------------------------------------------------------
using Big = std::vector<uint32_t>;

void mul_small(Big &a, uint32_t m) {
  uint64_t carry = 0;
  for (auto &x : a) {
    const uint64_t t = (uint64_t)x * m + carry;
    x = (uint32_t)t;
    carry = t >> 32;
  }
  if (carry) a.push_back((uint32_t)carry);
}

int cmp_big(Big a, Big b) {
  while (a.size() > 1 && a.back() == 0) a.pop_back();
  while (b.size() > 1 && b.back() == 0) b.pop_back();
  if (a.size() != b.size()) return a.size() < b.size() ? -1 : 1;
  for (size_t i = a.size(); i-- > 0;)
    if (a[i] != b[i]) return a[i] < b[i] ? -1 : 1;
  return 0;
}

bool reaches(int n, int k, int L, int me, int md) {
  Big lhs{1}, rhs{1};
  for (int i = 0; i < L; ++i) mul_small(lhs, (uint32_t)n);
  for (int i = 0; i < k; ++i) mul_small(lhs, (uint32_t)me);
  for (int i = 0; i < k; ++i) mul_small(rhs, (uint32_t)md);
  for (int i = 0; i < L; ++i) mul_small(rhs, (uint32_t)me);
  return cmp_big(lhs, rhs) >= 0;
}

fa::T5Geometry make_geometry(int nb, int md, int bidir) {
  fa::T5Geometry g{};
  g.bidir = bidir;
  g.nbp = bidir ? nb / 2 : nb;
  g.me = g.nbp / 2;
  const int L = g.nbp - g.me;
  g.nthr = L - 1;
  for (int k = 1; k < L; ++k) {
    int lo = g.me, hi = md;
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (reaches(mid, k, L, g.me, md)) hi = mid; else lo = mid + 1;
    }
    g.thr[k - 1] = lo;
  }
  g.sat = g.nthr > 0 ? g.thr[g.nthr - 1] : g.me;
  return g;
}

const fa::T5Geometry &geometry(int nb, int md, int bidir) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int>, fa::T5Geometry> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(nb, md, bidir);
  auto it = cache.find(key);
  if (it == cache.end()) it = cache.emplace(key, make_geometry(nb, md, bidir)).first;
  return it->second;
}

// ---------------------------------------------------------------------------
// Checks
// ---------------------------------------------------------------------------
fa_status check_t5_shape(int nb, int md, int bidir) {
  if (bidir != 0 && bidir != 1) return fail(FA_ERR_INVALID, "bias.bidirectional must be 0 or 1");
  if (nb < 2 || nb > 256)
    return fail(FA_ERR_UNSUPPORTED, "bias.num_buckets=%d outside [2, 256]", nb);
  if (bidir && (nb % 2 != 0 || nb < 4))
    return fail(FA_ERR_UNSUPPORTED, "bidirectional T5 needs an even num_buckets >= 4 (got %d)",
                nb);
  const int nbp = bidir ? nb / 2 : nb, me = nbp / 2;
  if (md <= me || md > fa::kMaxDistance)
    return fail(FA_ERR_UNSUPPORTED, "bias.max_distance=%d must be in (%d, %d]", md, me,
                fa::kMaxDistance);
  return FA_OK;
}

fa_status check_common(int heads, int head_dim, int causal, float scale, float rope_base,
                       const fa_bias &bias, long long maxlen) {
  if (heads < 1) return fail(FA_ERR_INVALID, "heads=%d must be >= 1", heads);
  if (head_dim <= 0) return fail(FA_ERR_INVALID, "head_dim=%d must be > 0", head_dim);
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim=%d: only 64 and 128 are built", head_dim);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID, "causal must be 0 or 1");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "scale is not finite");
  if (!(scale > 0.f)) return fail(FA_ERR_UNSUPPORTED, "scale must be > 0");
  if (!std::isfinite(rope_base) || rope_base < 0.f)
    return fail(FA_ERR_INVALID, "rope_base must be 0 (off) or a finite positive base");
  if (maxlen > fa::kMaxSeqlen)
    return fail(FA_ERR_UNSUPPORTED, "sequence length %lld exceeds %d", maxlen, fa::kMaxSeqlen);
  if (maxlen * heads * head_dim * 2 >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "one sequence spans >= 2^31 bytes per tensor");
  switch (bias.mode) {
    case FA_BIAS_NONE: break;
    case FA_BIAS_T5: {
      if (!bias.table) return fail(FA_ERR_INVALID, "bias.table is NULL");
      const fa_status st = check_t5_shape(bias.num_buckets, bias.max_distance,
                                          bias.bidirectional);
      if (st != FA_OK) return st;
      break;
    }
    case FA_BIAS_ALIBI:
      if (!bias.slopes) return fail(FA_ERR_INVALID, "bias.slopes is NULL");
      break;
    case FA_BIAS_DENSE:
      if (!bias.dense) return fail(FA_ERR_INVALID, "bias.dense is NULL");
      if (maxlen > fa::kMaxDenseSeqlen)
        return fail(FA_ERR_UNSUPPORTED, "a dense bias needs seqlen <= %d (got %lld)",
                    fa::kMaxDenseSeqlen, maxlen);
      break;
    case FA_BIAS_FIRE:
      if (!bias.table) return fail(FA_ERR_INVALID, "bias.table (FIRE theta) is NULL");
      if (bias.fire_hidden < 1 || bias.fire_hidden > fa::kFireMaxHidden)
        return fail(FA_ERR_UNSUPPORTED, "bias.fire_hidden=%d outside [1, %d]", bias.fire_hidden,
                    fa::kFireMaxHidden);
      if (causal != 1)
        return fail(FA_ERR_UNSUPPORTED, "FIRE is defined for causal attention only");
      return FA_OK;
    default: return fail(FA_ERR_INVALID, "bias.mode=%d is not a fa_bias_mode", bias.mode);
  }
  if (bias.fire_hidden != 0) return fail(FA_ERR_INVALID, "bias.fire_hidden must be 0 unless FIRE");
  return FA_OK;
}

fa_status check_fwd_impl(const fa_fwd_params *p) {
  if (!p) return fail(FA_ERR_INVALID, "params is NULL");
  if (p->batch < 0 || p->seqlen < 0) return fail(FA_ERR_INVALID, "negative batch or seqlen");
  if (p->reserved != 0) return fail(FA_ERR_INVALID, "reserved must be 0");
  const bool empty = (long long)p->batch * p->seqlen == 0;
  if ((long long)p->batch * p->seqlen * (p->heads > 0 ? p->heads : 1) >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "batch * seqlen * heads must stay below 2^31");
  if (!empty && (!p->q || !p->k || !p->v || !p->o || !p->lse))
    return fail(FA_ERR_INVALID, "q, k, v, o and lse must be non-NULL");
  if (p->bias.mode == FA_BIAS_DENSE && p->bias.dense_batch != 1 &&
      p->bias.dense_batch != p->batch)
    return fail(FA_ERR_INVALID, "bias.dense_batch=%d must be 1 or batch=%d", p->bias.dense_batch,
                p->batch);
  if (empty && p->bias.mode == FA_BIAS_DENSE) {
    // nothing to compute, but the backward still clears a gradient of
    // dense_batch * heads * seqlen^2 floats: its size must be valid
    if (p->heads < 1) return fail(FA_ERR_INVALID, "heads=%d must be >= 1", p->heads);
    if (p->seqlen > fa::kMaxDenseSeqlen)
      return fail(FA_ERR_UNSUPPORTED, "a dense bias needs seqlen <= %d (got %d)",
                  fa::kMaxDenseSeqlen, p->seqlen);
    if (p->bias.fire_hidden != 0)
      return fail(FA_ERR_INVALID, "bias.fire_hidden must be 0 unless FIRE");
    return FA_OK;
  }
  return check_common(p->heads, p->head_dim, p->causal, p->scale, p->rope_base, p->bias,
                      p->seqlen);
}

fa_status check_varlen_fwd_impl(const fa_varlen_fwd_params *p) {
  if (!p) return fail(FA_ERR_INVALID, "params is NULL");
  if (p->nseq < 0 || p->total < 0 || p->max_seqlen < 0)
    return fail(FA_ERR_INVALID, "negative nseq, total or max_seqlen");
  if (!p->cu_seqlens) return fail(FA_ERR_INVALID, "cu_seqlens is NULL");
  if (p->total > 0 && (!p->q || !p->k || !p->v || !p->o || !p->lse))
    return fail(FA_ERR_INVALID, "q, k, v, o and lse must be non-NULL");
  if ((long long)p->total * p->heads >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "total * heads must stay below 2^31");
  // schedule entries (16 bytes each) for the smallest tile, 32 rows
  if (8LL * ((p->heads + 7) / 8) * ((long long)p->total / 32 + p->nseq + 1) >= (1LL << 27))
    return fail(FA_ERR_UNSUPPORTED, "too many sequences or tokens for the tile schedule");
  if (p->bias.mode == FA_BIAS_DENSE)
    return fail(FA_ERR_UNSUPPORTED, "a dense bias matrix is for the dense entry points only");
  return check_common(p->heads, p->head_dim, p->causal, p->scale, p->rope_base, p->bias,
                      p->max_seqlen);
}

fa_status check_bwd_ptrs(bool empty, const void *dout, const void *dq, const void *dk,
                         const void *dv) {
  if (!empty && (!dout || !dq || !dk || !dv))
    return fail(FA_ERR_INVALID, "dout, dq, dk, dv must be non-NULL");
  return FA_OK;
}

fa::Problem make_problem(const fa_fwd_params &f) {
  fa::Problem p{};
  p.varlen = 0;
  p.nbatch = f.batch;
  p.seqlen = f.seqlen;
  p.total = f.batch * f.seqlen;
  p.heads = f.heads;
  p.head_dim = f.head_dim;
  p.causal = f.causal;
  p.scale = f.scale;
  p.rope_base = f.rope_base;
  p.bias = f.bias.mode;
  p.cu_seqlens = nullptr;
  p.table = f.bias.table;
  p.slopes = f.bias.slopes;
  if (p.bias == FA_BIAS_DENSE) {
    p.dense = static_cast<const uint16_t *>(f.bias.dense);
    p.dense_batch = f.bias.dense_batch;
  }
  if (p.bias == FA_BIAS_T5)
    p.t5 = geometry(f.bias.num_buckets, f.bias.max_distance, f.bias.bidirectional);
  if (p.bias == FA_BIAS_FIRE) p.fire_hidden = f.bias.fire_hidden;
  return p;
}

fa::Problem make_problem(const fa_varlen_fwd_params &f) {
  fa::Problem p{};
  p.varlen = 1;
  p.nbatch = f.nseq;
  p.seqlen = f.max_seqlen;
  p.total = f.total;
  p.heads = f.heads;
  p.head_dim = f.head_dim;
  p.causal = f.causal;
  p.scale = f.scale;
  p.rope_base = f.rope_base;
  p.bias = f.bias.mode;
  p.cu_seqlens = f.cu_seqlens;
  p.table = f.bias.table;
  p.slopes = f.bias.slopes;
  if (p.bias == FA_BIAS_T5)
    p.t5 = geometry(f.bias.num_buckets, f.bias.max_distance, f.bias.bidirectional);
  if (p.bias == FA_BIAS_FIRE) p.fire_hidden = f.bias.fire_hidden;
  return p;
}

// ---------------------------------------------------------------------------
// Workspace layout (every region 256-byte aligned).
// ---------------------------------------------------------------------------
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  }
};

// RoPE (cos, sin) table: one fp64 pair per (position, dim pair).
size_t rope_table_bytes(const fa::Problem &p) {
  return (size_t)p.seqlen * (p.head_dim / 2) * 16;
}

struct FwdLayout {
  size_t krot = 0, rope_cs = 0, prefix = 0, sched = 0, fire_tab = 0, fire_dist = 0, total = 0;
  int nsched = 0;
};

// The forward rotates Q rows in registers from the (cos, sin) table; K,
// which every query tile streams through LDS, is rotated once into a copy.
FwdLayout fwd_layout(const fa::Problem &p) {
  FwdLayout L;
  Carve c;
  const size_t tokens = (size_t)p.total;
  if (p.rope_base > 0.f) {
    L.krot = c.take(tokens * p.heads * p.head_dim * 2);
    L.rope_cs = c.take(rope_table_bytes(p));
  }
  if (p.varlen) {
    const int br = fa::fwd_tile_rows(p.head_dim);
    L.nsched = fa::sched_entries(p.total, p.nbatch, p.heads, br);
    L.prefix = c.take((size_t)fa::sched_prefix_ints(p.nbatch) * 4);
    L.sched = c.take((size_t)L.nsched * 16);
  }
  if (p.bias == FA_BIAS_FIRE) {
    L.fire_tab = c.take(fa::fire_tab_floats(p.heads) * 4);
    L.fire_dist = c.take(fa::fire_dist_floats(p.seqlen) * 4);
  }
  L.total = c.off;
  return L;
}

struct BwdLayout {
  size_t qrot = 0, krot = 0, rope_cs = 0, delta = 0, part = 0, prefix = 0, sched = 0,
         fire_tab = 0, fire_dist = 0, fire_g = 0, total = 0;
  int nsched = 0;
  bool has_part = false;
};

BwdLayout bwd_layout(const fa::Problem &p, bool want_dtable) {
  BwdLayout L;
  Carve c;
  const size_t tokens = (size_t)p.total;
  const size_t elems = tokens * p.heads * p.head_dim;
  // Both backward kernels stream one of Q, K through LDS: each is rotated
  // once into a copy; dQ and dK are turned back in the kernels' epilogues.
  if (p.rope_base > 0.f) {
    L.qrot = c.take(elems * 2);
    L.krot = c.take(elems * 2);
    L.rope_cs = c.take(rope_table_bytes(p));
  }
  L.delta = c.take(2 * tokens * p.heads * 4);   // -D, then -lse / scale (lse layout each)
  if (p.varlen) {
    const int bt = fa::bwd_tile();
    L.nsched = fa::sched_entries(p.total, p.nbatch, p.heads, bt);
    L.prefix = c.take((size_t)fa::sched_prefix_ints(p.nbatch) * 4);
    L.sched = c.take((size_t)L.nsched * 16);
  }
  L.has_part = want_dtable && (p.bias == FA_BIAS_T5 || p.bias == FA_BIAS_FIRE);
  if (L.has_part) {
    const int nb = p.bias == FA_BIAS_FIRE ? fa::kFireGradRows
                                          : (p.t5.bidir ? 2 * p.t5.nbp : p.t5.nbp);
    L.part = c.take((size_t)fa::bwd_num_parts(p, L.nsched) * nb * 4);
  }
  if (p.bias == FA_BIAS_FIRE) {
    L.fire_tab = c.take(fa::fire_tab_floats(p.heads) * 4);
    L.fire_dist = c.take(fa::fire_dist_floats(p.seqlen) * 4);
    if (want_dtable) L.fire_g = c.take((size_t)fa::kFireGradRows * p.heads * 4);
  }
  L.total = c.off;
  return L;
}

template <typename T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

fa_status run_fwd(const fa::Problem &p, const void *q, const void *k, const void *v, void *o,
                  float *lse, void *ws, size_t ws_bytes, hipStream_t s) {
  const FwdLayout L = fwd_layout(p);
  if (L.total > 0 && (ws == nullptr || ws_bytes < L.total))
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                ws == nullptr ? (size_t)0 : ws_bytes);
  if (p.total == 0 || (!p.varlen && (p.nbatch == 0 || p.seqlen == 0))) return FA_OK;
  fa::FwdBuffers b{q, k, v, o, lse, nullptr, nullptr, nullptr};
  hipError_t e;
  if (p.bias == FA_BIAS_FIRE) {
    e = fa::launch_fire_setup(p, at<float>(ws, L.fire_tab), at<float>(ws, L.fire_dist), s);
    if (e != hipSuccess) return hip_fail(e, "FIRE tables");
    b.fire_tab = at<float>(ws, L.fire_tab);
    b.fire_dist = at<float>(ws, L.fire_dist);
  }
  if (p.rope_base > 0.f) {
    e = fa::launch_rope_table(p, at<double2>(ws, L.rope_cs), s);
    if (e == hipSuccess)
      e = fa::launch_rope_rotate(p, at<double2>(ws, L.rope_cs), k, at<void>(ws, L.krot), nullptr,
                                 nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "rope");
    b.k = at<void>(ws, L.krot);
    b.rope_cs = at<double2>(ws, L.rope_cs);
  }
  const int4 *sched = nullptr;
  if (p.varlen) {
    e = fa::launch_sched(p.cu_seqlens, p.nbatch, p.heads, fa::fwd_tile_rows(p.head_dim), L.nsched,
                         at<int32_t>(ws, L.prefix), at<int4>(ws, L.sched), s);
    if (e != hipSuccess) return hip_fail(e, "schedule");
    sched = at<int4>(ws, L.sched);
  }
  e = timed(FA_KERNEL_FWD, s, [&] { return fa::launch_fwd_impl(p, b, sched, L.nsched, s); });
  if (e != hipSuccess) return hip_fail(e, "forward");
  return FA_OK;
}

fa_status run_bwd(const fa::Problem &p, const void *q, const void *k, const void *v,
                  const void *o, const float *lse, const float *dlse, const void *dout, void *dq,
                  void *dk, void *dv, float *dtable, void *ws, size_t ws_bytes, hipStream_t s) {
  const BwdLayout L = bwd_layout(p, dtable != nullptr);
  if (L.total > 0 && (ws == nullptr || ws_bytes < L.total))
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                ws == nullptr ? (size_t)0 : ws_bytes);
  hipError_t e;
  const bool t5grad = dtable != nullptr && p.bias == FA_BIAS_T5;
  const bool densegrad = dtable != nullptr && p.bias == FA_BIAS_DENSE;
  const bool firegrad = dtable != nullptr && p.bias == FA_BIAS_FIRE;
  const int nb = p.bias == FA_BIAS_T5 ? (p.t5.bidir ? 2 * p.t5.nbp : p.t5.nbp) : 0;
  if (p.total == 0 || (!p.varlen && (p.nbatch == 0 || p.seqlen == 0))) {
    if (t5grad) {
      e = fa::launch_fill_f32(dtable, (size_t)nb * p.heads, 0.f, s);
      if (e != hipSuccess) return hip_fail(e, "fill");
    }
    if (firegrad) {
      e = fa::launch_fill_f32(dtable, (size_t)fa::fire_theta_floats(p.heads, p.fire_hidden), 0.f,
                              s);
      if (e != hipSuccess) return hip_fail(e, "fill");
    }
    if (densegrad) {   // an empty batch contributes nothing to a shared matrix
      e = fa::launch_fill_f32(dtable, (size_t)p.dense_batch * p.heads * p.seqlen * p.seqlen, 0.f,
                              s);
      if (e != hipSuccess) return hip_fail(e, "fill");
    }
    return FA_OK;
  }
  fa::BwdBuffers b{};
  b.q = q;
  b.k = k;
  b.v = v;
  b.o = o;
  b.dout = dout;
  b.lse = lse;
  b.dlse = dlse;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.delta = at<float>(ws, L.delta);
  b.part = L.has_part ? at<float>(ws, L.part) : nullptr;
  b.dtable = t5grad ? dtable : nullptr;
  if (p.bias == FA_BIAS_FIRE) {
    e = fa::launch_fire_setup(p, at<float>(ws, L.fire_tab), at<float>(ws, L.fire_dist), s);
    if (e != hipSuccess) return hip_fail(e, "FIRE tables");
    b.fire_tab = at<float>(ws, L.fire_tab);
    b.fire_dist = at<float>(ws, L.fire_dist);
    b.fire_g = firegrad ? at<float>(ws, L.fire_g) : nullptr;
  }
  // a matrix shared by a batch of several: its gradient is summed over the
  // batch by a kernel of its own; otherwise the dK/dV kernel writes dS
  const bool shared_sum = densegrad && p.dense_batch == 1 && p.nbatch > 1;
  b.dbias = densegrad && !shared_sum ? dtable : nullptr;
  b.dbias_shared = shared_sum ? dtable : nullptr;
  if (densegrad && p.causal) {
    // pairs with key > query: the key-parallel kernel skips most of them
    e = fa::launch_zero_upper(dtable, p.dense_batch * p.heads, p.seqlen, s);
    if (e != hipSuccess) return hip_fail(e, "dense bias gradient fill");
  }
  if (p.rope_base > 0.f) {
    e = fa::launch_rope_table(p, at<double2>(ws, L.rope_cs), s);
    if (e == hipSuccess)
      e = fa::launch_rope_rotate(p, at<double2>(ws, L.rope_cs), q, at<void>(ws, L.qrot), k,
                                 at<void>(ws, L.krot), s);
    if (e != hipSuccess) return hip_fail(e, "rope");
    b.q = at<void>(ws, L.qrot);
    b.k = at<void>(ws, L.krot);
    b.rope_cs = at<double2>(ws, L.rope_cs);
  }
  const int4 *sched = nullptr;
  if (p.varlen) {
    e = fa::launch_sched(p.cu_seqlens, p.nbatch, p.heads, fa::bwd_tile(), L.nsched,
                         at<int32_t>(ws, L.prefix), at<int4>(ws, L.sched), s);
    if (e != hipSuccess) return hip_fail(e, "schedule");
    sched = at<int4>(ws, L.sched);
  }
  e = timed(FA_KERNEL_BWD_DQ, s,
            [&] { return fa::launch_bwd_phase(p, b, sched, L.nsched, fa::kBwdPre, s); });
  if (e != hipSuccess) return hip_fail(e, "backward dq kernel");
  e = timed(FA_KERNEL_BWD_DKV, s,
            [&] { return fa::launch_bwd_phase(p, b, sched, L.nsched, fa::kBwdMain, s); });
  if (e != hipSuccess) return hip_fail(e, "backward dkv kernel");
  if (firegrad) {
    e = timed(FA_KERNEL_BWD_FIRE, s,
              [&] { return fa::launch_bwd_phase(p, b, sched, L.nsched, fa::kBwdFire, s); });
    if (e != hipSuccess) return hip_fail(e, "FIRE gradient sums");
  }
  e = fa::launch_bwd_phase(p, b, sched, L.nsched, fa::kBwdReduce, s);
  if (e != hipSuccess) return hip_fail(e, "table-gradient reduction");
  if (firegrad) {
    e = fa::launch_fire_grad(p, b.fire_g, dtable, s);
    if (e != hipSuccess) return hip_fail(e, "FIRE parameter gradient");
  }
  if (shared_sum) {
    e = timed(FA_KERNEL_BWD_DBIAS_SUM, s, [&] {
      return fa::launch_bwd_phase(p, b, sched, L.nsched, fa::kBwdDenseSum, s);
    });
    if (e != hipSuccess) return hip_fail(e, "dense bias gradient over the batch");
  }
  return FA_OK;
}

// ---------------------------------------------------------------------------
// Static scratch for fa_bwd_noalloc.  Each GPU holds its own copy of this
// array from the library's first use on it until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory, so the
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = FA_BWD_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;   // device ordinal -> address of its scratch

fa_status scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return FA_OK;
}

}  // namespace

extern "C" {

const char *fa_status_str(fa_status st) {
  switch (st) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP error";
    default: break;
  }
  return "unknown status";
}

const char *fa_last_error(void) { return g_last_error.c_str(); }

const char *fa_version(void) { return "0.1.0"; }

fa_status fa_set_kernel_timer(int32_t kernel, hipEvent_t start, hipEvent_t stop) {
  g_last_error.clear();
  if (kernel < 0 || kernel >= FA_KERNEL_COUNT)
    return fail(FA_ERR_INVALID, "kernel id %d is not a fa_kernel", kernel);
  std::lock_guard<std::mutex> lock(g_timer_mu);
  g_timers[kernel].start = start;
  g_timers[kernel].stop = stop;
  return FA_OK;
}

fa_status fa_check_fwd(const fa_fwd_params *p) {
  g_last_error.clear();
  return check_fwd_impl(p);
}

fa_status fa_check_varlen_fwd(const fa_varlen_fwd_params *p) {
  g_last_error.clear();
  return check_varlen_fwd_impl(p);
}

fa_status fa_check_bwd(const fa_bwd_params *p) {
  g_last_error.clear();
  if (!p) return fail(FA_ERR_INVALID, "params is NULL");
  const fa_status st = check_fwd_impl(&p->f);
  if (st != FA_OK) return st;
  return check_bwd_ptrs((long long)p->f.batch * p->f.seqlen == 0, p->dout, p->dq, p->dk, p->dv);
}

fa_status fa_check_varlen_bwd(const fa_varlen_bwd_params *p) {
  g_last_error.clear();
  if (!p) return fail(FA_ERR_INVALID, "params is NULL");
  const fa_status st = check_varlen_fwd_impl(&p->f);
  if (st != FA_OK) return st;
  return check_bwd_ptrs(p->f.total == 0, p->dout, p->dq, p->dk, p->dv);
}

size_t fa_fwd_workspace_size(const fa_fwd_params *p) {
  if (fa_check_fwd(p) != FA_OK) return (size_t)-1;
  return fwd_layout(make_problem(*p)).total;
}

size_t fa_varlen_fwd_workspace_size(const fa_varlen_fwd_params *p) {
  if (fa_check_varlen_fwd(p) != FA_OK) return (size_t)-1;
  return fwd_layout(make_problem(*p)).total;
}

size_t fa_bwd_workspace_size(const fa_bwd_params *p) {
  if (fa_check_bwd(p) != FA_OK) return (size_t)-1;
  return bwd_layout(make_problem(p->f), p->dtable != nullptr).total;
}

size_t fa_varlen_bwd_workspace_size(const fa_varlen_bwd_params *p) {
  if (fa_check_varlen_bwd(p) != FA_OK) return (size_t)-1;
  return bwd_layout(make_problem(p->f), p->dtable != nullptr).total;
}

fa_status fa_fwd(const fa_fwd_params *p, void *ws, size_t ws_bytes, hipStream_t stream) {
  const fa_status st = fa_check_fwd(p);
  if (st != FA_OK) return st;
  return run_fwd(make_problem(*p), p->q, p->k, p->v, p->o, p->lse, ws, ws_bytes, stream);
}

fa_status fa_varlen_fwd(const fa_varlen_fwd_params *p, void *ws, size_t ws_bytes,
                        hipStream_t stream) {
  const fa_status st = fa_check_varlen_fwd(p);
  if (st != FA_OK) return st;
  return run_fwd(make_problem(*p), p->q, p->k, p->v, p->o, p->lse, ws, ws_bytes, stream);
}

fa_status fa_bwd(const fa_bwd_params *p, void *ws, size_t ws_bytes, hipStream_t stream) {
  const fa_status st = fa_check_bwd(p);
  if (st != FA_OK) return st;
  return run_bwd(make_problem(p->f), p->f.q, p->f.k, p->f.v, p->f.o, p->f.lse, p->dlse,
                 p->dout, p->dq, p->dk, p->dv, p->dtable, ws, ws_bytes, stream);
}

fa_status fa_bwd_noalloc(const fa_bwd_params *p, hipStream_t stream) {
  const fa_status st = fa_check_bwd(p);
  if (st != FA_OK) return st;
  const fa::Problem pr = make_problem(p->f);
  const size_t need = bwd_layout(pr, p->dtable != nullptr).total;
  if (need > kScratchBytes)
    return fail(FA_ERR_UNSUPPORTED,
                "fa_bwd_noalloc: this problem needs %zu bytes of scratch; the static scratch "
                "holds %zu (use fa_bwd with a workspace)",
                need, kScratchBytes);
  void *ws = nullptr;
  if (need > 0) {
    const fa_status s2 = scratch_of_current_device(&ws);
    if (s2 != FA_OK) return s2;
  }
  return run_bwd(pr, p->f.q, p->f.k, p->f.v, p->f.o, p->f.lse, p->dlse, p->dout, p->dq, p->dk,
                 p->dv, p->dtable, ws, need, stream);
}

fa_status fa_varlen_bwd(const fa_varlen_bwd_params *p, void *ws, size_t ws_bytes,
                        hipStream_t stream) {
  const fa_status st = fa_check_varlen_bwd(p);
  if (st != FA_OK) return st;
  return run_bwd(make_problem(p->f), p->f.q, p->f.k, p->f.v, p->f.o, p->f.lse, p->dlse,
                 p->dout, p->dq, p->dk, p->dv, p->dtable, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// RMSNorm and cross-entropy
// ---------------------------------------------------------------------------
static fa_status check_rms_fwd(const fa_rmsnorm_fwd_params *p) {
  if (!p) return fail(FA_ERR_INVALID, "params is NULL");
  if (p->rows < 0) return fail(FA_ERR_INVALID, "rows=%d is negative", p->rows);
  if (p->dim <= 0) return fail(FA_ERR_INVALID, "dim=%d must be > 0", p->dim);
  if (p->dim % 8 != 0 || p->dim > fa::kRmsMaxDim)
    return fail(FA_ERR_UNSUPPORTED, "dim=%d must be a multiple of 8 and at most %d", p->dim,
                fa::kRmsMaxDim);
  if (!std::isfinite(p->eps) || p->eps < 0.f) return fail(FA_ERR_INVALID, "eps must be >= 0");
  if (p->reserved != 0) return fail(FA_ERR_INVALID, "reserved must be 0");
  if (p->rows > 0 && (!p->x || !p->w || !p->y || !p->rstd))
    return fail(FA_ERR_INVALID, "x, w, y and rstd must be non-NULL");
  return FA_OK;
}

static fa_status check_rms_bwd(const fa_rmsnorm_bwd_params *p) {
  if (!p) return fail(FA_ERR_INVALID, "params is NULL");
  const fa_status st = check_rms_fwd(&p->f);
  if (st != FA_OK) return st;
  if (p->f.rows > 0 && (!p->dy || !p->dx)) return fail(FA_ERR_INVALID, "dy, dx must be non-NULL");
  return FA_OK;
}

static fa_status check_ce_fwd(const fa_ce_fwd_params *p) {
  if (!p) return fail(FA_ERR_INVALID, "params is NULL");
  if (p->rows < 0) return fail(FA_ERR_INVALID, "rows=%d is negative", p->rows);
  if (p->vocab <= 0) return fail(FA_ERR_INVALID, "vocab=%d must be > 0", p->vocab);
  if (p->vocab % 8 != 0) return fail(FA_ERR_UNSUPPORTED, "vocab=%d must be a multiple of 8",
                                     p->vocab);
  if (!std::isfinite(p->z_loss) || p->z_loss < 0.f)
    return fail(FA_ERR_INVALID, "z_loss must be finite and >= 0");
  if (p->rows > 0 && (!p->logits || !p->labels || !p->loss || !p->lse))
    return fail(FA_ERR_INVALID, "logits, labels, loss and lse must be non-NULL");
  return FA_OK;
}

fa_status fa_rmsnorm_fwd(const fa_rmsnorm_fwd_params *p, hipStream_t stream) {
  g_last_error.clear();
  const fa_status st = check_rms_fwd(p);
  if (st != FA_OK) return st;
  if (p->rows == 0) return FA_OK;
  const hipError_t e = timed(FA_KERNEL_RMSNORM_FWD, stream, [&] {
    return fa::launch_rmsnorm_fwd(p->x, p->w, p->y, p->rstd, p->rows, p->dim, p->eps, stream);
  });
  return e == hipSuccess ? FA_OK : hip_fail(e, "rmsnorm forward");
}

size_t fa_rmsnorm_bwd_workspace_size(const fa_rmsnorm_bwd_params *p) {
  g_last_error.clear();
  if (check_rms_bwd(p) != FA_OK) return (size_t)-1;
  if (p->f.rows == 0 || p->dw == nullptr) return 0;
  return (size_t)fa::rmsnorm_bwd_grid(p->f.rows) * p->f.dim * 4;
}

fa_status fa_rmsnorm_bwd(const fa_rmsnorm_bwd_params *p, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  g_last_error.clear();
  const fa_status st = check_rms_bwd(p);
  if (st != FA_OK) return st;
  hipError_t e;
  if (p->f.rows == 0) {
    if (p->dw == nullptr) return FA_OK;
    e = fa::launch_fill_f32(p->dw, (size_t)p->f.dim, 0.f, stream);   // empty sum
    return e == hipSuccess ? FA_OK : hip_fail(e, "fill");
  }
  const size_t need = fa_rmsnorm_bwd_workspace_size(p);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                ws == nullptr ? (size_t)0 : ws_bytes);
  float *part = need > 0 ? static_cast<float *>(ws) : nullptr;
  e = timed(FA_KERNEL_RMSNORM_BWD, stream, [&] {
    return fa::launch_rmsnorm_bwd(p->f.x, p->f.w, p->f.rstd, p->dy, p->dx, nullptr, part,
                                  p->f.rows, p->f.dim, stream);
  });
  if (e == hipSuccess && p->dw != nullptr)
    e = fa::launch_rmsnorm_dw(part, p->dw, p->f.rows, p->f.dim, stream);
  return e == hipSuccess ? FA_OK : hip_fail(e, "rmsnorm backward");
}

fa_status fa_ce_fwd(const fa_ce_fwd_params *p, hipStream_t stream) {
  g_last_error.clear();
  const fa_status st = check_ce_fwd(p);
  if (st != FA_OK) return st;
  if (p->rows == 0) return FA_OK;
  const hipError_t e = timed(FA_KERNEL_CE_FWD, stream, [&] {
    return fa::launch_ce_fwd(p->logits, p->labels, p->loss, p->lse, p->rows, p->vocab, p->z_loss,
                             p->ignore_index, stream);
  });
  return e == hipSuccess ? FA_OK : hip_fail(e, "cross-entropy forward");
}

fa_status fa_ce_bwd(const fa_ce_bwd_params *p, hipStream_t stream) {
  g_last_error.clear();
  if (!p) return fail(FA_ERR_INVALID, "params is NULL");
  const fa_status st = check_ce_fwd(&p->f);
  if (st != FA_OK) return st;
  if (p->f.rows == 0) return FA_OK;
  if (!p->dloss || !p->dlogits) return fail(FA_ERR_INVALID, "dloss, dlogits must be non-NULL");
  const hipError_t e = timed(FA_KERNEL_CE_BWD, stream, [&] {
    return fa::launch_ce_bwd(p->f.logits, p->f.labels, p->f.lse, p->dloss, p->dlogits, p->f.rows,
                             p->f.vocab, p->f.z_loss, p->f.ignore_index, stream);
  });
  return e == hipSuccess ? FA_OK : hip_fail(e, "cross-entropy backward");
}

fa_status fa_mfma_probe(int32_t iters, float *sink, double *flops, hipStream_t stream) {
  g_last_error.clear();
  static_assert(FA_MFMA_PROBE_LANES == fa::kMfmaProbeBlocks * fa::kMfmaProbeThreads,
                "probe size");
  if (iters < 1 || iters > (1 << 20))
    return fail(FA_ERR_INVALID, "iters %d outside [1, 2^20]", iters);
  if (!sink || !flops) return fail(FA_ERR_INVALID, "sink or flops is NULL");
  const hipError_t e = fa::launch_mfma_probe(sink, iters, stream);
  if (e != hipSuccess) return hip_fail(e, "mfma_probe");
  *flops = (double)(FA_MFMA_PROBE_LANES / 64) * 4.0 * iters * (2.0 * 32 * 32 * 16);
  return FA_OK;
}

fa_status fa_t5_buckets(int32_t qlen, int32_t klen, int32_t num_buckets, int32_t max_distance,
                        int32_t bidirectional, int32_t *out, hipStream_t stream) {
  g_last_error.clear();
  if (qlen < 0 || klen < 0) return fail(FA_ERR_INVALID, "negative qlen or klen");
  if (!out && (long long)qlen * klen > 0) return fail(FA_ERR_INVALID, "out is NULL");
  const fa_status st = check_t5_shape(num_buckets, max_distance, bidirectional);
  if (st != FA_OK) return st;
  const hipError_t e = fa::launch_t5_buckets(geometry(num_buckets, max_distance, bidirectional),
                                             qlen, klen, out, stream);
  if (e != hipSuccess) return hip_fail(e, "t5_buckets");
  return FA_OK;
}

}  // extern "C"
