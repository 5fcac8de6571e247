// Host-side driver of the C ABI for the AddressSanitizer / UndefinedBehavior-
// Sanitizer build (tests/test_sanitize.py).  It runs every argument check,
// workspace-size computation and refusal path of include/fat5attn.h, and the
// T5 threshold construction over a sweep of geometries, without touching a
// GPU: every call here returns before the first HIP call.  Exit status 0 when
// every expectation holds; a sanitizer report aborts the process.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "fat5attn.h"

static int g_fail = 0;

#define EXPECT(cond)                                                             \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "%s:%d: expectation failed: %s (%s)\n", __FILE__,     \
                   __LINE__, #cond, fa_last_error());                            \
      ++g_fail;                                                                  \
    }                                                                            \
  } while (0)

static void *P(unsigned long v) { return reinterpret_cast<void *>(v); }

static fa_fwd_params dense(int B, int S, int H, int D) {
  fa_fwd_params p;
  std::memset(&p, 0, sizeof(p));
  p.batch = B;
  p.seqlen = S;
  p.heads = H;
  p.head_dim = D;
  p.scale = 1.f;
  p.q = p.k = p.v = P(0x1000);
  p.o = P(0x1000);
  p.lse = static_cast<float *>(P(0x1000));
  return p;
}

static void status_strings() {
  const fa_status all[] = {FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE,
                           FA_ERR_HIP};
  for (fa_status s : all) EXPECT(std::strlen(fa_status_str(s)) > 0);
  EXPECT(std::strlen(fa_status_str(static_cast<fa_status>(-77))) > 0);
  EXPECT(std::strlen(fa_version()) >= 5);
}

static void t5_geometries() {
  // every threshold construction the checks reach: both directions, bucket
  // counts from 2 to 256 and distances from just above the exact range to
  // the largest allowed
  const int nbs[] = {2, 3, 4, 8, 16, 31, 32, 33, 64, 100, 128, 255, 256};
  for (int bidir = 0; bidir <= 1; ++bidir)
    for (int nb : nbs) {
      const int nbp = bidir ? nb / 2 : nb, me = nbp / 2;
      const int mds[] = {me + 1, 128, 513, 1000, 1024};
      for (int md : mds) {
        fa_fwd_params p = dense(2, 300, 3, 64);
        p.bias.mode = FA_BIAS_T5;
        p.bias.num_buckets = nb;
        p.bias.max_distance = md;
        p.bias.bidirectional = bidir;
        p.bias.table = static_cast<const float *>(P(0x2000));
        const bool ok = nb >= 2 && (!bidir || (nb % 2 == 0 && nb >= 4)) && md > me &&
                        md <= 1024;
        const fa_status st = fa_check_fwd(&p);
        EXPECT((st == FA_OK) == ok);
        if (ok) {
          fa_bwd_params b;
          std::memset(&b, 0, sizeof(b));
          b.f = p;
          b.dout = b.dq = b.dk = b.dv = P(0x3000);
          b.dtable = static_cast<float *>(P(0x4000));
          EXPECT(fa_bwd_workspace_size(&b) > 0);
        }
      }
    }
}

static void dense_checks() {
  EXPECT(fa_check_fwd(nullptr) == FA_ERR_INVALID);
  EXPECT(fa_fwd(nullptr, nullptr, 0, nullptr) == FA_ERR_INVALID);
  fa_fwd_params p = dense(2, 100, 3, 64);
  EXPECT(fa_check_fwd(&p) == FA_OK);
  EXPECT(std::strlen(fa_last_error()) == 0);
  p.head_dim = 96;
  EXPECT(fa_check_fwd(&p) == FA_ERR_UNSUPPORTED);
  EXPECT(std::strlen(fa_last_error()) > 0);
  EXPECT(fa_fwd_workspace_size(&p) == (size_t)-1);
  EXPECT(fa_fwd(&p, nullptr, 0, nullptr) == FA_ERR_UNSUPPORTED);
  p = dense(2, 100, 3, 64);
  p.scale = NAN;
  EXPECT(fa_check_fwd(&p) == FA_ERR_INVALID);
  p.scale = -1.f;
  EXPECT(fa_check_fwd(&p) == FA_ERR_UNSUPPORTED);
  p = dense(2, 70000, 3, 64);
  EXPECT(fa_check_fwd(&p) == FA_ERR_UNSUPPORTED);
  p = dense(1 << 20, 4096, 1024, 128);   // sizes whose products overflow int32
  EXPECT(fa_check_fwd(&p) == FA_ERR_UNSUPPORTED);
  p = dense(-1, 10, 3, 64);
  EXPECT(fa_check_fwd(&p) == FA_ERR_INVALID);
  // an empty batch computes nothing and needs no pointers
  p = dense(0, 100, 3, 64);
  p.q = p.k = p.v = p.o = nullptr;
  p.lse = nullptr;
  EXPECT(fa_check_fwd(&p) == FA_OK);
  EXPECT(fa_fwd(&p, nullptr, 0, nullptr) == FA_OK);
  // RoPE needs a workspace; a call without one is refused before any launch
  p = dense(2, 16384, 16, 128);
  p.rope_base = 10000.f;
  const size_t ws = fa_fwd_workspace_size(&p);
  EXPECT(ws > 0 && ws != (size_t)-1);
  EXPECT(fa_fwd(&p, nullptr, 0, nullptr) == FA_ERR_WORKSPACE);
  EXPECT(fa_fwd(&p, P(0x9000), ws - 1, nullptr) == FA_ERR_WORKSPACE);
  // dense bias matrix
  p = dense(4, 1024, 2, 64);
  p.bias.mode = FA_BIAS_DENSE;
  EXPECT(fa_check_fwd(&p) == FA_ERR_INVALID);   // matrix NULL
  p.bias.dense = P(0x6000);
  p.bias.dense_batch = 1;
  EXPECT(fa_check_fwd(&p) == FA_OK);
  p.bias.dense_batch = 3;
  EXPECT(fa_check_fwd(&p) == FA_ERR_INVALID);
  p.bias.dense_batch = 1;
  fa_bwd_params b;
  std::memset(&b, 0, sizeof(b));
  b.f = p;
  b.dout = b.dq = b.dk = b.dv = P(0x3000);
  b.dtable = static_cast<float *>(P(0x4000));
  EXPECT(fa_bwd_workspace_size(&b) > 0);   // -D and -lse/scale: no per-batch gradients
  EXPECT(fa_bwd(&b, nullptr, 0, nullptr) == FA_ERR_WORKSPACE);
  p = dense(2, 16384, 16, 128);   // RoPE copies beyond the static scratch
  p.rope_base = 10000.f;
  b.f = p;
  EXPECT(fa_bwd_workspace_size(&b) > FA_BWD_NOALLOC_MAX_BYTES);
  EXPECT(fa_bwd_noalloc(&b, nullptr) == FA_ERR_UNSUPPORTED);
  b.dk = nullptr;
  EXPECT(fa_check_bwd(&b) == FA_ERR_INVALID);
  EXPECT(fa_bwd(&b, nullptr, 0, nullptr) == FA_ERR_INVALID);
  EXPECT(fa_check_bwd(nullptr) == FA_ERR_INVALID);
  // bad enums and the FIRE field outside FIRE
  p = dense(2, 100, 3, 64);
  p.bias.mode = 9;
  EXPECT(fa_check_fwd(&p) == FA_ERR_INVALID);
  p.bias.mode = FA_BIAS_NONE;
  p.bias.fire_hidden = 4;
  EXPECT(fa_check_fwd(&p) == FA_ERR_INVALID);
  p.bias.fire_hidden = 0;
  p.bias.mode = FA_BIAS_ALIBI;
  EXPECT(fa_check_fwd(&p) == FA_ERR_INVALID);   // slopes NULL
  p.bias.slopes = static_cast<const float *>(P(0x5000));
  EXPECT(fa_check_fwd(&p) == FA_OK);
}

static void fire_checks() {
  fa_fwd_params p = dense(2, 777, 5, 64);
  p.causal = 1;
  p.bias.mode = FA_BIAS_FIRE;
  p.bias.table = static_cast<const float *>(P(0x2000));
  for (int k = -1; k <= 66; ++k) {
    p.bias.fire_hidden = k;
    EXPECT((fa_check_fwd(&p) == FA_OK) == (k >= 1 && k <= 64));
  }
  p.bias.fire_hidden = 32;
  EXPECT(fa_fwd_workspace_size(&p) > 0);
  EXPECT(fa_fwd(&p, nullptr, 0, nullptr) == FA_ERR_WORKSPACE);
  p.causal = 0;
  EXPECT(fa_check_fwd(&p) == FA_ERR_UNSUPPORTED);
  p.causal = 1;
  p.bias.table = nullptr;
  EXPECT(fa_check_fwd(&p) == FA_ERR_INVALID);
  p.bias.table = static_cast<const float *>(P(0x2000));
  fa_bwd_params b;
  std::memset(&b, 0, sizeof(b));
  b.f = p;
  b.dout = b.dq = b.dk = b.dv = P(0x3000);
  const size_t without = fa_bwd_workspace_size(&b);
  b.dtable = static_cast<float *>(P(0x4000));
  EXPECT(fa_bwd_workspace_size(&b) > without);
}

static void varlen_checks() {
  fa_varlen_fwd_params p;
  std::memset(&p, 0, sizeof(p));
  p.nseq = 3;
  p.total = 300;
  p.max_seqlen = 200;
  p.heads = 4;
  p.head_dim = 128;
  p.scale = 0.1f;
  p.cu_seqlens = static_cast<const int32_t *>(P(0x5000));
  p.q = p.k = p.v = P(0x1000);
  p.o = P(0x1000);
  p.lse = static_cast<float *>(P(0x1000));
  EXPECT(fa_check_varlen_fwd(&p) == FA_OK);
  EXPECT(fa_varlen_fwd_workspace_size(&p) > 0);   // the tile schedule
  EXPECT(fa_varlen_fwd(&p, nullptr, 0, nullptr) == FA_ERR_WORKSPACE);
  p.cu_seqlens = nullptr;
  EXPECT(fa_check_varlen_fwd(&p) == FA_ERR_INVALID);
  p.cu_seqlens = static_cast<const int32_t *>(P(0x5000));
  p.nseq = 1 << 28;   // too many sequences for the schedule
  EXPECT(fa_check_varlen_fwd(&p) == FA_ERR_UNSUPPORTED);
  p.nseq = 3;
  p.bias.mode = FA_BIAS_DENSE;
  p.bias.dense = P(0x6000);
  p.bias.dense_batch = 1;
  EXPECT(fa_check_varlen_fwd(&p) == FA_ERR_UNSUPPORTED);
  p.bias.mode = FA_BIAS_NONE;
  fa_varlen_bwd_params b;
  std::memset(&b, 0, sizeof(b));
  b.f = p;
  b.dout = b.dq = b.dk = b.dv = P(0x3000);
  EXPECT(fa_check_varlen_bwd(&b) == FA_OK);
  EXPECT(fa_varlen_bwd_workspace_size(&b) > 0);
  EXPECT(fa_varlen_bwd(&b, nullptr, 0, nullptr) == FA_ERR_WORKSPACE);
  EXPECT(fa_check_varlen_bwd(nullptr) == FA_ERR_INVALID);
}

static void norm_loss_checks() {
  fa_rmsnorm_fwd_params r;
  std::memset(&r, 0, sizeof(r));
  r.rows = 16;
  r.dim = 768;
  r.eps = 1e-6f;
  r.x = r.w = P(0x1000);
  r.y = P(0x1000);
  r.rstd = static_cast<float *>(P(0x1000));
  r.dim = 9000;
  EXPECT(fa_rmsnorm_fwd(&r, nullptr) == FA_ERR_UNSUPPORTED);
  r.dim = 768;
  r.x = nullptr;
  EXPECT(fa_rmsnorm_fwd(&r, nullptr) == FA_ERR_INVALID);
  EXPECT(fa_rmsnorm_fwd(nullptr, nullptr) == FA_ERR_INVALID);
  fa_rmsnorm_bwd_params rb;
  std::memset(&rb, 0, sizeof(rb));
  rb.f = r;
  EXPECT(fa_rmsnorm_bwd_workspace_size(&rb) == (size_t)-1);
  fa_ce_fwd_params c;
  std::memset(&c, 0, sizeof(c));
  c.rows = 4;
  c.vocab = 30;   // not a multiple of 8
  c.logits = P(0x1000);
  c.labels = static_cast<const int32_t *>(P(0x1000));
  c.loss = c.lse = static_cast<float *>(P(0x1000));
  EXPECT(fa_ce_fwd(&c, nullptr) != FA_OK);
  EXPECT(fa_ce_fwd(nullptr, nullptr) == FA_ERR_INVALID);
}

static void hooks() {
  EXPECT(fa_set_kernel_timer(-1, nullptr, nullptr) == FA_ERR_INVALID);
  EXPECT(fa_set_kernel_timer(FA_KERNEL_COUNT, nullptr, nullptr) == FA_ERR_INVALID);
  for (int k = 0; k < FA_KERNEL_COUNT; ++k) EXPECT(fa_set_kernel_timer(k, nullptr, nullptr) == FA_OK);
  double flops = 0;
  EXPECT(fa_mfma_probe(0, static_cast<float *>(P(0x1000)), &flops, nullptr) == FA_ERR_INVALID);
  EXPECT(fa_mfma_probe(5, nullptr, &flops, nullptr) == FA_ERR_INVALID);
  EXPECT(fa_t5_buckets(-1, 4, 32, 128, 1, static_cast<int32_t *>(P(0x1000)), nullptr) ==
         FA_ERR_INVALID);
  EXPECT(fa_t5_buckets(4, 4, 33, 128, 1, static_cast<int32_t *>(P(0x1000)), nullptr) ==
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_t5_buckets(0, 0, 32, 128, 1, nullptr, nullptr) == FA_OK);
}

int main() {
  status_strings();
  t5_geometries();
  dense_checks();
  fire_checks();
  varlen_checks();
  norm_loss_checks();
  hooks();
  if (g_fail) std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
  else std::printf("abi sanitize driver: all expectations hold\n");
  return g_fail ? 1 : 0;
}
