/*
 * libfat5attn: exact softmax attention with the T5 relative-position bias,
 * ALiBi, FIRE and RoPE, dense or packed (cu_seqlens), forward and backward,
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (FAT5 report, section "Noyau CUDA", second kernel): for
 * every (sequence, head) the scores S = scale * Q K^T, then S' = S plus a bias
 * filled on the fly from a small per-head table T indexed by the bucket of the
 * relative position, then P = softmax(S') row by row with a running
 * ("cumulative") softmax, then O = P V.  The N x N matrices S, S', P are never
 * written to memory: memory stays linear in the sequence length, which the
 * report credits for inference on tens of thousands of tokens.  The same
 * kernel serves ALiBi and RoPE (listed beside the T5 encoding in the note
 * under that section).  Packed batches follow the flash_attn_varlen_func
 * convention of the packing blog (DataCollatorWithFlattening): tokens of
 * several examples are concatenated and attention never crosses an example
 * boundary.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers; the caller owns every buffer.  They
 *   may be NULL only when the problem is empty (B*S == 0, or total == 0).
 *   Dense tensors are [B, S, H, D] and packed tensors [T, H, D], bfloat16,
 *   contiguous (D innermost).  LSE is fp32 [B, H, S] (packed: [H, T]).  The
 *   T5 table and its gradient are fp32 [num_buckets, H] row-major; ALiBi
 *   slopes are fp32 [H].  cu_seqlens is int32 [nseq + 1] on the device.
 * - Everything is enqueued on `stream` and returns without synchronising.
 *   The library allocates no device memory: scratch space is the caller's
 *   workspace, sized by the matching *_workspace_size call (0 means none is
 *   needed and `ws` may be NULL).
 * - The params struct is only read during the call.  Outputs (O, LSE, dQ,
 *   dK, dV, dtable) are fully overwritten, never accumulated into.
 * - A validation failure returns a negative status before anything is
 *   enqueued; fa_last_error() then names the offending field.  A failed
 *   launch returns FA_ERR_HIP with the HIP error text in fa_last_error().
 *   Device faults surface at the caller's next synchronisation.
 * - head_dim must be 64 or 128; scale must be finite and > 0; the sequence
 *   length (dense S, packed max_seqlen) is at most 65536 and a single
 *   sequence times H*D*2 bytes must stay below 2^31.
 * - cu_seqlens is trusted: it must start at 0, be non-decreasing, end at
 *   `total`, and no sequence may be longer than max_seqlen.  It is not read
 *   on the host (no device-to-host copy).
 * - Buckets (FA_BIAS_T5): relative position r = key index - query index.
 *   Bidirectional: num_buckets/2 buckets per side, keys after the query use
 *   the upper half, n = |r|.  Unidirectional: n = max(-r, 0).  With nb' the
 *   buckets per side and me = nb'/2, n < me maps to bucket n, larger n to
 *   me + floor(ln(n/me)/ln(max_distance/me) * (nb'-me)), capped at nb'-1 (the
 *   T5 scheme, cited by the report; it prints no formula).  The kernels decide
 *   each boundary exactly with integer thresholds.  Requires num_buckets in
 *   [2, 256] (even when bidirectional), me < max_distance <= 1024.
 * - ALiBi (FA_BIAS_ALIBI): bias = -slope[h] * |i - j|.
 * - RoPE (rope_base > 0): interleaved pairs (2p, 2p+1) of q and k at
 *   position t (0-based, local to each packed sequence) are rotated by the
 *   angle t * rope_base^(-2p/D) before the scores; gradients are returned
 *   with respect to the unrotated q and k.  RoPE combines with any bias mode.
 * - Causal: key j is visible to query i iff j <= i (self-attention only:
 *   queries and keys share one length).
 */
#ifndef FAT5ATTN_H
#define FAT5ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID = -1,     /* a NULL pointer, a negative size, a bad enum value */
  FA_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement   */
  FA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required     */
  FA_ERR_HIP = -4,         /* a HIP launch failed                            */
  FA_STATUS_MAX_ENUM = 0x7fffffff   /* not a status: gives the type the range of
                                       int32, so any int32 passed as an fa_status
                                       (fa_status_str) is a valid value        */
} fa_status;

typedef enum {
  FA_BIAS_NONE = 0,
  FA_BIAS_T5 = 1,
  FA_BIAS_ALIBI = 2,
  FA_BIAS_DENSE = 3,
  FA_BIAS_FIRE = 4
} fa_bias_mode;

/* Additive score bias.  FAT5 report, "Noyau CUDA": the second kernel is
 * handed the compact bucket tensor T instead of a dense bias matrix; the
 * first kernel was handed the bias matrix B itself (FA_BIAS_DENSE: memory
 * quadratic in the sequence length, dense entry points only).
 *
 * FA_BIAS_FIRE: the FIRE bias (listed with RoPE and ALiBi in the note under
 * "Noyau CUDA"; definition from the FIRE paper it cites), causal attention
 * only.  For query i and key j <= i (positions local to each sequence):
 *   x = log(c (i - j) + 1) / log(c max(L, i) + 1),
 *   bias_h = b2_h + sum_k w2_hk relu(w1_k x + b1_k)   (K = fire_hidden units).
 * `table` points to theta, device fp32
 *   [w1 (K), b1 (K), w2 (H * K, row h at h * K), b2 (H), c, L]
 * with c > 0 and L > 0 (trusted: not read on the host).  The backward's
 * dtable is d(theta) in the same layout, summed over the batch and heads.
 * K <= 64. */
typedef struct {
  int32_t mode;            /* fa_bias_mode                                     */
  int32_t num_buckets;     /* T5 only                                          */
  int32_t max_distance;    /* T5 only                                          */
  int32_t bidirectional;   /* T5 only: 1 encoder style, 0 decoder style        */
  const float *table;      /* T5: device fp32 [num_buckets, H]; FIRE: theta    */
  const float *slopes;     /* ALiBi: device fp32 [H]                           */
  const void *dense;       /* DENSE: device bf16 [dense_batch, H, S, S], row =
                              query, column = key, added to scale * Q K^T     */
  int32_t dense_batch;     /* DENSE: 1 (one matrix per head, shared by the
                              batch) or B; S <= 16384                         */
  int32_t fire_hidden;     /* FIRE: hidden units K in [1, 64]; else 0          */
} fa_bias;

/* Dense forward: q, k, v [B, S, H, D] bf16 in; o [B, S, H, D] bf16 and
 * lse [B, H, S] fp32 out (lse_i = log sum_j exp(S'_ij), natural log). */
typedef struct {
  int32_t batch;
  int32_t seqlen;
  int32_t heads;
  int32_t head_dim;
  int32_t causal;
  float scale;             /* multiplies Q K^T; the bias is added unscaled     */
  float rope_base;         /* > 0 enables RoPE, 0 disables it                  */
  int32_t reserved;        /* must be 0                                        */
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;
  fa_bias bias;
} fa_fwd_params;

/* Dense backward.  `f` describes the forward; f.lse and f.o are READ here
 * (the forward's outputs for the same inputs).  D_i = sum_j P_ij dP_ij is
 * recomputed from fp32 P; dO_i . O_i only centres that sum, so an O other than
 * the forward's costs accuracy, not correctness (a non-finite centre is
 * dropped).  dout [B, S, H, D] bf16 in; dq, dk,
 * dv [B, S, H, D] bf16 out.  dtable is the bias gradient (may be NULL to skip
 * it): T5, fp32 [num_buckets, H], the sum over the batch and over every
 * visible (query, key) pair in bucket b of dL/dS'; DENSE, fp32
 * [dense_batch, H, S, S], dL/dS' itself (0 for masked pairs), summed over
 * the batch in batch order when dense_batch is 1 (no workspace: a kernel of
 * its own sums each element in registers); FIRE, d(theta) (see fa_bias);
 * other modes ignore it. */
typedef struct {
  fa_fwd_params f;
  const void *dout;
  void *dq;
  void *dk;
  void *dv;
  float *dtable;
  const float *dlse;       /* may be NULL: gradient of the loss with respect to
                              f.lse, fp32 [B, H, S]; LSE_i's derivative with
                              respect to S'_ij is P_ij, so it adds dlse_i P_ij
                              to dS_ij                                        */
} fa_bwd_params;

/* Packed forward: q, k, v, o [total, H, D] bf16; lse [H, total] fp32;
 * sequence s holds tokens cu_seqlens[s] .. cu_seqlens[s+1]-1.  max_seqlen is
 * a host-side upper bound on every sequence length. */
typedef struct {
  int32_t nseq;
  int32_t total;
  int32_t max_seqlen;
  int32_t heads;
  int32_t head_dim;
  int32_t causal;
  float scale;
  float rope_base;
  const int32_t *cu_seqlens;
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;
  fa_bias bias;
} fa_varlen_fwd_params;

typedef struct {
  fa_varlen_fwd_params f;
  const void *dout;
  void *dq;
  void *dk;
  void *dv;
  float *dtable;
  const float *dlse;       /* may be NULL: fp32 [H, total], as in fa_bwd_params */
} fa_varlen_bwd_params;

/* Host-only argument checks (no HIP call, nothing enqueued). */
fa_status fa_check_fwd(const fa_fwd_params *p);
fa_status fa_check_bwd(const fa_bwd_params *p);
fa_status fa_check_varlen_fwd(const fa_varlen_fwd_params *p);
fa_status fa_check_varlen_bwd(const fa_varlen_bwd_params *p);

/* Workspace bytes the matching call needs (0 when none); (size_t)-1 when the
 * params fail the checks above. */
size_t fa_fwd_workspace_size(const fa_fwd_params *p);
size_t fa_bwd_workspace_size(const fa_bwd_params *p);
size_t fa_varlen_fwd_workspace_size(const fa_varlen_fwd_params *p);
size_t fa_varlen_bwd_workspace_size(const fa_varlen_bwd_params *p);

/* Forward attention (FAT5 report, "Noyau CUDA", kernel v2 forward steps). */
fa_status fa_fwd(const fa_fwd_params *p, void *ws, size_t ws_bytes, hipStream_t stream);
/* Backward: dQ, dK, dV and the table gradient (the report trains T, so its
 * gradient is implied; it prints no backward). */
fa_status fa_bwd(const fa_bwd_params *p, void *ws, size_t ws_bytes, hipStream_t stream);
/* Backward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same contract and results as fa_bwd, bit for bit,
 * except that its scratch space (the same layout fa_bwd_workspace_size
 * sizes) lives in a static device array of FA_BWD_NOALLOC_MAX_BYTES inside
 * the library: each GPU the library runs on holds one until the process
 * ends.  Problems needing more scratch return FA_ERR_UNSUPPORTED before
 * anything is enqueued (RoPE, and a dense bias matrix shared by a batch of
 * more than one, need workspaces of their own size: use fa_bwd).  Every call
 * on one GPU uses that GPU's array, so calls that overlap in time on one GPU
 * (two streams, two threads) race and must be serialised by the caller.
 * The call itself allocates nothing; its first call on a device looks up
 * the array's device address once. */
#define FA_BWD_NOALLOC_MAX_BYTES (16u << 20)
fa_status fa_bwd_noalloc(const fa_bwd_params *p, hipStream_t stream);

/* Packed variants (packing blog: flash_attn_varlen_func semantics). */
fa_status fa_varlen_fwd(const fa_varlen_fwd_params *p, void *ws, size_t ws_bytes,
                        hipStream_t stream);
fa_status fa_varlen_bwd(const fa_varlen_bwd_params *p, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The report's two other fused kernels (FAT5 report, section on the Triton
 * kernels; benchmarks under "Torch vs Triton").  Both entry points take a
 * stream, allocate nothing and follow the conventions above.
 * ------------------------------------------------------------------------- */

/* RMSNorm (the layer of Zhang & Sennrich the report cites, as T5 uses it: no
 * mean subtraction, no bias): y = x / sqrt(mean_j x_j^2 + eps) * w per row.
 * x, y bf16 [rows, dim]; w bf16 [dim]; rstd fp32 [rows] out, the reciprocal
 * root mean square the backward reads.  dim a multiple of 8, at most 8192;
 * eps finite and >= 0. */
typedef struct {
  int32_t rows;
  int32_t dim;
  float eps;
  int32_t reserved;        /* must be 0                                        */
  const void *x;
  const void *w;
  void *y;
  float *rstd;
} fa_rmsnorm_fwd_params;

/* RMSNorm backward: dy bf16 [rows, dim] in; dx bf16 [rows, dim] out and dw
 * fp32 [dim] out (the sum over rows; may be NULL).  f.rstd is READ (the
 * forward's output for the same x); f.y is not used.  With dw, the call
 * needs fa_rmsnorm_bwd_workspace_size bytes of workspace (one fp32 row of
 * partial sums per workgroup, added in a fixed order). */
typedef struct {
  fa_rmsnorm_fwd_params f;
  const void *dy;
  void *dx;
  float *dw;
} fa_rmsnorm_bwd_params;

fa_status fa_rmsnorm_fwd(const fa_rmsnorm_fwd_params *p, hipStream_t stream);
size_t fa_rmsnorm_bwd_workspace_size(const fa_rmsnorm_bwd_params *p);
fa_status fa_rmsnorm_bwd(const fa_rmsnorm_bwd_params *p, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* Cross-entropy with z-loss (the z-loss of de Brebisson & Vincent the report
 * cites), per row of bf16 logits z [rows, vocab] with int32 label y:
 * lse = log sum_v exp z_v, loss = lse - z_y + z_loss * lse^2.  Rows whose
 * label equals ignore_index or lies outside [0, vocab) get loss 0 and no
 * gradient (their lse is still written).  loss, lse fp32 [rows] out; the
 * mean over rows is the caller's.  vocab a multiple of 8; logits finite;
 * z_loss finite and >= 0. */
typedef struct {
  int32_t rows;
  int32_t vocab;
  float z_loss;
  int32_t ignore_index;
  const void *logits;
  const int32_t *labels;
  float *loss;
  float *lse;
} fa_ce_fwd_params;

/* Backward: dloss fp32 [rows] in (dL/dloss per row, e.g. 1/count for a
 * mean); dlogits bf16 [rows, vocab] out = dloss * (softmax(z) * (1 + 2 z_loss
 * lse) - onehot(y)), 0 for ignored rows.  f.lse is READ (the forward's);
 * f.loss is not used.  dlogits may be f.logits itself (in place). */
typedef struct {
  fa_ce_fwd_params f;
  const float *dloss;
  void *dlogits;
} fa_ce_bwd_params;

fa_status fa_ce_fwd(const fa_ce_fwd_params *p, hipStream_t stream);
fa_status fa_ce_bwd(const fa_ce_bwd_params *p, hipStream_t stream);

/* Test hook: out[i * klen + j] = T5 bucket of (query i, key j), computed on
 * the device by the same threshold code the attention kernels use.  out is a
 * device int32 [qlen, klen]. */
fa_status fa_t5_buckets(int32_t qlen, int32_t klen, int32_t num_buckets, int32_t max_distance,
                        int32_t bidirectional, int32_t *out, hipStream_t stream);

/* Benchmark hook: the chip's sustained dense bf16 MFMA rate, to set a
 * kernel's achieved rate beside.  Launches FA_MFMA_PROBE_LANES lanes (8 per
 * SIMD) whose waves each issue 4 * iters v_mfma_f32_32x32x16_bf16 with no
 * memory traffic; time the call with events on `stream`.  *flops receives the
 * call's flop count (2 * 32 * 32 * 16 per MFMA).  sink: device float
 * [FA_MFMA_PROBE_LANES], overwritten.  FA_ERR_INVALID for iters outside
 * [1, 1 << 20] or a NULL sink / flops. */
#define FA_MFMA_PROBE_LANES (2048 * 256)
fa_status fa_mfma_probe(int32_t iters, float *sink, double *flops, hipStream_t stream);

/* Kernels that fa_set_kernel_timer can bracket. */
typedef enum {
  FA_KERNEL_FWD = 0,       /* the attention forward kernel                       */
  FA_KERNEL_BWD_DQ = 1,    /* backward, query-parallel: D_i and dQ               */
  FA_KERNEL_BWD_DKV = 2,   /* backward, key-parallel: dK, dV and table gradient  */
  FA_KERNEL_RMSNORM_FWD = 3,
  FA_KERNEL_RMSNORM_BWD = 4, /* dx and the dw partials (not their final sum)     */
  FA_KERNEL_CE_FWD = 5,
  FA_KERNEL_CE_BWD = 6,
  FA_KERNEL_BWD_DBIAS_SUM = 7, /* backward, a dense bias shared by the batch:
                                  its gradient summed over the batch       */
  FA_KERNEL_BWD_FIRE = 8,  /* backward, FIRE: the parameter-gradient sums    */
  FA_KERNEL_COUNT = 9
} fa_kernel;

/* Benchmark hook.  While set, every launch of `kernel` is bracketed by
 * hipEventRecord(start) and hipEventRecord(stop) on the stream it is launched
 * on, so a caller can time that kernel alone.  NULL events clear the hook.
 * The setting is process-wide: change it only while no other thread is inside
 * the library.  Returns FA_ERR_INVALID for an unknown kernel id. */
fa_status fa_set_kernel_timer(int32_t kernel, hipEvent_t start, hipEvent_t stop);

/* Static text for a status code. */
const char *fa_status_str(fa_status st);
/* Detail of the last failure on the calling thread ("" if none). */
const char *fa_last_error(void);
/* Library version, "major.minor.patch". */
const char *fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FAT5ATTN_H */
