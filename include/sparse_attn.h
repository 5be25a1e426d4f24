/*
 * sparse_attn.h -- C ABI of the block-sparse attention library for MI355X
 * (gfx950).  Training-free block-sparse attention in two calls:
 *
 *   sparse_attn_predict   stage one: block-mean pooled Q and K, a compressed
 *                         Q.K^T that predicts the block attention map, and a
 *                         per-query-block cumulative-mass mask written as a
 *                         kept-block list per query block.
 *   sparse_attn_forward   stage two: block-sparse flash attention over the
 *                         kept lists, skipping a tile's P.V product for a
 *                         group of rows when the tile cannot matter there
 *                         (the softmax-aware lambda test inside the online
 *                         softmax).  Native precision (bf16 / fp32) or the
 *                         quantised variants (INT8 or 4-bit Q.K^T, FP8 e4m3
 *                         P.V).
 *
 * Sources: the SpargeAttn abstract (taxoreview.com page; also on the
 * huggingface-mirror search page) defines the two-stage online filter --
 * predict the attention map to skip products, then an online softmax-aware
 * filter that skips more -- and calls the attention quantized.  The iCATS
 * abstract (arxivdaily.com page) describes the pipeline as estimating the
 * importance of query-key regions, deriving a sparse mask and computing only
 * the important candidates, with a top-p rule.  The DynSparse story
 * (embedding.report page) adds the cumulative-energy threshold and notes
 * that masks can be precomputed, which is why the mask is an explicit,
 * reusable object passed between the two calls.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Device pointers unless marked "host".  Q, K, V, O are [B, H, N, D]
 *   tensors of `dtype` with D contiguous (O is fp32 when o_fp32 is set);
 *   element strides of the B, H and N dimensions come from sa_params
 *   (0 = packed B,H,N,D).  All four share the strides, counted in elements
 *   of their own type.  Base pointers must be 16-byte aligned and strides must
 *   keep every row 16-byte aligned.
 * - The caller owns every buffer (inputs, outputs, mask, workspace).  The
 *   library allocates no device memory and keeps no pointer after a call
 *   returns.  Calls are asynchronous on `stream` (a hipStream_t passed as
 *   void*; NULL = the default stream).
 * - Arguments are validated on the host before anything is enqueued.  On
 *   any error nothing is enqueued and the call returns a non-zero sa_status;
 *   sparse_attn_last_error() then returns a message (thread-local).
 *   SA_ERR_HIP reports a failed kernel launch.  No C++ exception crosses the
 *   ABI.  NaN/Inf inside Q, K, V are not checked and propagate.
 * - An empty problem (B, H or N equal to 0) is valid and enqueues nothing.
 * - Supported: D in {64, 128}; block_q = 128, block_k = 64; skip groups of
 *   16, 32, 64 or 128 rows; N <= 262144 (4096 key blocks); one
 *   head's rows (N + 64) * stride_n elements under 2 GiB.  The
 *   quantised variants need dtype = SA_BF16 (D 64 or 128).  Anything else
 *   returns SA_ERR_UNSUPPORTED.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSE_ATTN_VERSION 8

#if defined(__GNUC__)
#define SA_API __attribute__((visibility("default")))
#else
#define SA_API
#endif

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = 1,   /* bad pointer, shape, stride or parameter     */
  SA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (D, block sizes)  */
  SA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required  */
  SA_ERR_HIP = 4            /* the HIP runtime reported a launch failure   */
} sa_status;

/* Storage type of Q, K, V and O. */
enum { SA_F32 = 0, SA_BF16 = 1 };
/* Arithmetic of stage two: native (bf16 MFMA / fp32 MFMA) or INT8 Q.K^T with
 * FP8 e4m3 P.V (per-block scales: Q and K absmax/127, V absmax/448 per key
 * block; P pre-scaled by 2^8).  SA_PREC_I4_FP8 is the same with 4-bit Q and
 * K codes (scale absmax/7, codes in [-7, 7]), the INT4 attention the PARO
 * abstract (huggingface-mirror search page) reports after token
 * reordering; gfx950 has no INT4 MFMA, so the codes run on the INT8 MFMA and
 * the mode changes accuracy, not speed.  SA_PREC_I8_MXFP8 is SA_PREC_I8_FP8
 * with a power-of-two V scale per key block: 2^e with e the smallest integer
 * such that absmax <= 448 * 2^e (the E8M0 block scale of the OCP
 * microscaling formats; the pages fix no V scale), V codes e4m3(V / 2^e); the
 * scaled FP8 MFMA applies it in hardware, so the mode is the faster one.  It
 * also normalises differently: l (the divisor of O and the l of lse) is the
 * sum of the quantised weights e4m3(2^8 P) / 2^8 over the kept tiles,
 * skipped ones included, instead of the sum of P, so that without skips O is
 * an exact weighted average of V's dequantised codes; the skip decisions are
 * taken as in SA_PREC_I8_FP8 (SA_SKIP_RECALL's energies from P itself). */
enum { SA_PREC_NATIVE = 0, SA_PREC_I8_FP8 = 1, SA_PREC_I4_FP8 = 2, SA_PREC_I8_MXFP8 = 3 };
/* Mask rule of stage one.  TOPCDF: P-hat = softmax of the block scores over
 * the admissible key blocks.  ENERGY: P-hat_j proportional to
 * n_j * exp(s_j), n_j the number of keys in block j (a cumulative-energy
 * target; equal to TOPCDF when every block is full).  TOPK: a fixed budget
 * of `topk_blocks` key blocks per query block in the same processing order
 * (the fixed-budget comparator the DynSparse story sets against top-p);
 * P-hat as for TOPCDF. */
enum { SA_RULE_TOPCDF = 0, SA_RULE_ENERGY = 1, SA_RULE_TOPK = 2 };
/* Skip rule of stage two (see sparse_attn_forward).  LAMBDA: the static
 * threshold `lambda` on (tile max - running max), the SpargeAttn abstract's
 * stage-two filter.  RECALL: a dynamic threshold from the cumulative energy
 * the online softmax already holds, keeping at least a share `recall` of
 * each row's energy over the kept tiles (the DynSparse story's "cumulative
 * energy filtering" with a fixed recall). */
enum { SA_SKIP_LAMBDA = 0, SA_SKIP_RECALL = 1 };

typedef struct sa_params {
  int32_t B, H, N, D;          /* batch, heads, tokens, head dimension         */
  int32_t block_q, block_k;    /* query / key block rows: 128 and 64           */
  int32_t causal;              /* 1: key c visible to row r only if c <= r     */
  int32_t dtype;               /* SA_F32 | SA_BF16                             */
  int32_t prec;                /* SA_PREC_NATIVE | SA_PREC_I8_FP8 |            */
                               /* SA_PREC_I4_FP8 | SA_PREC_I8_MXFP8            */
  int32_t rule;                /* SA_RULE_TOPCDF | SA_RULE_ENERGY |            */
                               /* SA_RULE_TOPK                                 */
  float tau;                   /* cumulative-mass target in (0, 1]; >= 1 keeps */
                               /* every admissible block                       */
  float lambda;                /* skip threshold, natural-log units of the     */
                               /* scaled logits; -INFINITY never skips; NaN is */
                               /* invalid                                      */
  float sm_scale;              /* softmax scale; 0 -> 1/sqrt(D)                */
  int32_t keep_prefix_kblocks; /* leading key blocks that are always kept      */
  int32_t lambda_group_rows;   /* rows G per skip group: 16, 32, 64 or 128;    */
                               /* 0 -> 32 (one wavefront's rows)               */
  int32_t o_fp32;              /* 1: O is written as fp32 whatever `dtype` is; */
                               /* 0: O has `dtype` (bf16 O = the fp32 result  */
                               /* rounded to nearest even)                    */
  int64_t stride_b, stride_h, stride_n;  /* element strides; 0 -> packed       */
  int32_t skip_rule;           /* SA_SKIP_LAMBDA | SA_SKIP_RECALL              */
  float recall;                /* SA_SKIP_RECALL: target share rho in (0, 1]   */
                               /* of each row's energy; ignored otherwise      */
  int32_t topk_blocks;         /* SA_RULE_TOPK: key blocks kept per query      */
                               /* block (>= 1; the forced blocks are kept even */
                               /* beyond it); ignored otherwise                */
} sa_params;

/* The mask: output of predict, input of forward.  Caller-allocated; sizes
 * from sparse_attn_mask_shape().
 *   kept_idx   int32 [B, H, NQB, NKB]: for query block i the first
 *              kept_cnt[b,h,i] entries are the kept key blocks in processing
 *              order (forced blocks first, then predicted score descending,
 *              then index ascending); later entries are not written.
 *   kept_cnt   int32 [B, H, NQB].
 *   block_prob optional float [B, H, NQB, NKB] predicted map P-hat in key
 *              block order (0 for inadmissible blocks); NULL skips it. */
typedef struct sa_mask {
  int32_t* kept_idx;
  int32_t* kept_cnt;
  float* block_prob;
} sa_mask;

/* Host.  NQB = ceil(N / block_q), NKB = ceil(N / block_k). */
SA_API sa_status sparse_attn_mask_shape(const sa_params* p, int64_t* nqb, int64_t* nkb);

/* Host.  Workspace bytes needed by predict and by forward (either output
 * pointer may be NULL).  Layouts (offsets rounded up to 256 bytes):
 *   predict: qbar float [B,H,NQB,D], then kbar float [B,H,NKB,D] -- the
 *            block means, left in place after the call.
 *   forward, the quantised precisions: Q codes int8 [B,H,N,D], K
 *            codes int8 [B,H,N,D] (in [-7, 7] for SA_PREC_I4_FP8),
 *            V codes e4m3 [B,H,NKB,D,64] (each key block stored transposed,
 *            keys permuted: byte (d, p) of block j holds key
 *            j*64 + 32t + 8g + 4h + e for p = 32h + 16t + 4g + e, with
 *            h, t in {0,1} and g, e in {0..3}), then float scales
 *            sq [B,H,NQB], sk [B,H,NKB], sv [B,H,NKB].
 *   forward, SA_PREC_NATIVE: 0 bytes. */
SA_API sa_status sparse_attn_workspace_size(const sa_params* p, size_t* predict_ws,
                                     size_t* forward_ws);

/* Stage one.  Reads Q and K; writes out->kept_idx, out->kept_cnt and, if
 * non-NULL, out->block_prob.  Steps, per (b, h):
 *   block means qbar_i (query block rows valid only) and kbar_j;
 *   admissible key blocks A_i (all; causal: first key <= last row of R_i);
 *   scores s_ij = sm * qbar_i . kbar_j  (fp32 means, fp64 dot product);
 *   weights P-hat per `rule`, in fp64;
 *   forced blocks F_i: j < keep_prefix_kblocks, and under causality the key
 *   blocks that reach the query block's diagonal;
 *   order: forced first, s descending, j ascending;
 *   cut: the shortest prefix whose fp64 running sum of P-hat reaches tau,
 *   never fewer than |F_i|; tau >= 1 keeps all of A_i; under SA_RULE_TOPK
 *   the first min(|A_i|, max(|F_i|, topk_blocks)) entries instead.
 * `ws` must hold the predict workspace. */
SA_API sa_status sparse_attn_predict(const sa_params* p, const void* q, const void* k,
                              const sa_mask* out, void* ws, size_t ws_bytes,
                              void* stream);

/* sparse_attn_predict for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same stage one, with the workspace taken from a static
 * scratch array inside the library (64 MiB per GPU, held until the process
 * ends; the address of each GPU's copy is looked up once, on the first call
 * on that device).  The caller still passes Q, K and the mask.  Problems
 * whose predict workspace (sparse_attn_workspace_size) exceeds 64 MiB are
 * rejected with SA_ERR_WORKSPACE before anything is enqueued.  The call
 * allocates nothing.  All calls on one GPU share its scratch: calls that
 * overlap on one GPU (on different streams, or from different threads
 * without ordering) race, and the block means of a call are overwritten by
 * the next one.  Arguments and errors otherwise as for sparse_attn_predict. */
SA_API sa_status sparse_attn_predict_noalloc(const sa_params* p, const void* q,
                                             const void* k, const sa_mask* out,
                                             void* stream);

/* Stage one's first step alone: the block means qbar (query blocks of
 * block_q rows) and kbar (key blocks of block_k rows), written to `ws` in
 * the predict layout (sparse_attn_workspace_size), each the fp32 mean of
 * its block's valid rows.  The SpargeAttn abstract's first stage predicts
 * the attention map quickly; the iCATS abstract describes the prior work's
 * estimate from query and key tokens grouped independently, of which a
 * contiguous block is the simplest grouping.  This is the HBM-bound part of
 * stage one (every element of Q and K read once), exposed for callers that
 * reuse the means and for measuring it on its own; sparse_attn_predict
 * runs it as its first step.  Arguments and errors as for
 * sparse_attn_predict without the mask. */
SA_API sa_status sparse_attn_pool(const sa_params* p, const void* q, const void* k, void* ws,
                                  size_t ws_bytes, void* stream);

/* Stage two.  For each query block, processes mask->kept_idx in list order
 * with an online softmax (running max m, running sum l).  For each group of
 * G = lambda_group_rows consecutive rows of the block (counted from its
 * first row; the SpargeAttn abstract's filter reads as a test per
 * wavefront, G = 32, the default) and each tile:
 *   SA_SKIP_LAMBDA: delta = max over the group's rows of (tile max - new
 *     running max); when delta < lambda the group skips the tile's P.V
 *     product;
 *   SA_SKIP_RECALL: each row also keeps d, the energy it has dropped so far
 *     (rescaled with l when m moves); with E the row's energy in the tile
 *     (sum of exp(S - m)) and l already including it, the group skips when
 *     d + E <= (1 - recall) * l for every row, and each row then adds E to
 *     d.  So every row drops at most a share 1 - recall of its energy.
 * m and l are updated either way.  Writes
 *   o          [B,H,N,D] dtype (fp32 if o_fp32): acc / l;
 *   lse        optional float [B,H,N]: m + log(l) in natural-log units;
 *   skip_bits  optional uint32 [B,H,NQB,128/G,ceil(NKB/32)]: bit (t % 32)
 *              of word t / 32 of group g is 1 when group g skipped the P.V
 *              product of list entry t; only words that cover entries
 *              t < kept_cnt are written, with zero bits past kept_cnt.
 *              Groups past the last row of a partial block hold no rows
 *              and read as skipped.
 * Every kept_idx entry must be an admissible key block for its query block
 * (causal) and kept_cnt must lie in [1, NKB]; predict produces such masks.
 * `ws` must hold the forward workspace (none for SA_PREC_NATIVE). */
SA_API sa_status sparse_attn_forward(const sa_params* p, const void* q, const void* k,
                              const void* v, const sa_mask* mask, void* o,
                              float* lse, uint32_t* skip_bits, void* ws,
                              size_t ws_bytes, void* stream);

/* Mask reuse across a sequence of calls (e.g. the denoising steps of a
 * diffusion model), for sparse_attn_step.  The pages note that attention
 * patterns stay similar across denoising steps and can be precomputed once
 * and reused (SparseD and LiteAttention abstracts on the search page; the
 * DynSparse story: combinable with pre-computed masks), and that early steps
 * are critical (SparseD runs them dense).  The iCATS abstract adds that the
 * tolerance to sparse approximation error varies across denoising timesteps
 * and schedules the sparsity by the signal-to-noise ratio: `tau_by_step`
 * carries such a schedule, one tau per call, computed by the caller from its
 * own noise schedule (the pages give no formula).  Caller-owned; set step = 0
 * to start a sequence. */
typedef struct sa_schedule {
  int32_t refresh_every;  /* >= 1: sparse calls predict a new mask on their   */
                          /* first call and every refresh_every-th after, and */
                          /* reuse the caller's mask in between              */
  int32_t dense_steps;    /* >= 0: the first dense_steps calls keep every     */
                          /* admissible block and skip nothing (exact up to   */
                          /* rounding)                                        */
  int32_t step;           /* calls made so far; incremented on success        */
  int32_t refreshed;      /* out: 1 if this call ran stage one                */
  const float* tau_by_step; /* host, optional: a sparse call s predicts with  */
                          /* tau = tau_by_step[min(s, n_tau - 1)] instead of  */
                          /* params->tau (same rules); NULL keeps params->tau */
  int32_t n_tau;          /* entries of tau_by_step (>= 1 when it is given)   */
} sa_schedule;

/* One call of a sequence: stage one when the schedule says so (writing
 * *mask), then stage two with *mask.  Call number s = sched->step runs
 *   s <  dense_steps: predict and forward with tau = 1 and no skip (every
 *                     admissible block kept, also under SA_RULE_TOPK);
 *   s >= dense_steps: predict iff (s - dense_steps) % refresh_every == 0,
 *                     then forward, with *p as given except tau, taken
 *                     from tau_by_step when the schedule has one (a reused
 *                     mask keeps the tau it was predicted with).
 * A reused mask must come from a call with the same shapes and causality
 * (every entry admissible), which the sequence guarantees when the caller
 * keeps `mask` between calls.  Every argument is validated before anything
 * is enqueued.  Workspaces as for sparse_attn_predict / sparse_attn_forward. */
SA_API sa_status sparse_attn_step(const sa_params* p, sa_schedule* sched, const void* q,
                           const void* k, const void* v, const sa_mask* mask, void* o,
                           float* lse, uint32_t* skip_bits, void* predict_ws,
                           size_t predict_ws_bytes, void* forward_ws,
                           size_t forward_ws_bytes, void* stream);

/* Token reordering ahead of the two stages.  The iCATS abstract
 * (arxivdaily.com page): block scores estimated from tokens grouped by their
 * query-key dot-product interaction are more accurate than from query and
 * key tokens grouped independently by feature similarity, and that
 * objective is a simple quadratic form; irregular cluster sizes are handled
 * by merging tails instead of padding.  The PARO abstract (huggingface-mirror
 * search page): reordering tokens turns the attention pattern block-wise.
 *
 * Readings.  Replacing a query x by a representative c moves its logit with
 * key k by sm (x - c) . k; the mean square of that move over the N keys is
 * sm^2 (x - c)^T M_K (x - c) with M_K = K^T K / N.  SA_METRIC_INTERACTION
 * clusters queries under that quadratic form and keys under the one of
 * M_Q = Q^T Q / N; SA_METRIC_FEATURE uses M = I (plain feature k-means, the
 * baseline the abstract compares against).  Per (b, h) and side, with C
 * clusters: centroid m starts at token floor((2m + 1) N / (2C)); `iters`
 * Lloyd passes each give every token the cluster m minimising
 * (x - c_m)^T M (x - c_m) (ties to the smaller m), and between passes each
 * centroid becomes the mean of its members (a cluster without members keeps
 * its centroid).  The order lists the tokens by (cluster, position):
 * clusters packed back to back with no padding, so the fixed block_q /
 * block_k blocks cut from it merge one cluster's tail with the next
 * cluster's head.  Arithmetic: M and the member sums in fp32; the cluster
 * decision compares c_m^T M c_m - 2 x^T M c_m in fp32 with x^T M c_m from
 * bf16 MFMA over x (exact in bf16) and M c_m split into two bf16 parts. */
enum { SA_METRIC_FEATURE = 0, SA_METRIC_INTERACTION = 1 };

typedef struct sa_cluster_params {
  int32_t clusters_q;  /* query clusters per head, in [1, min(N, 4096)]      */
  int32_t clusters_k;  /* key clusters per head, in [1, min(N, 4096)]        */
  int32_t iters;       /* Lloyd passes, in [1, 64]                           */
  int32_t metric;      /* SA_METRIC_FEATURE | SA_METRIC_INTERACTION          */
} sa_cluster_params;

/* Outputs of sparse_attn_cluster, caller-allocated, int32 [B, H, N]:
 *   perm_q    perm_q[b,h,r] = the query token at reordered position r
 *   perm_k    the same for keys (and values)
 *   labels_q  optional: the cluster of each query token, in token order
 *   labels_k  optional: the same for keys */
typedef struct sa_reorder {
  int32_t* perm_q;
  int32_t* perm_k;
  int32_t* labels_q;
  int32_t* labels_k;
} sa_reorder;

/* Host.  Workspace bytes of sparse_attn_cluster.  Needs dtype = SA_BF16 and
 * causal = 0 besides the sa_params rules. */
SA_API sa_status sparse_attn_cluster_workspace_size(const sa_params* p,
                                                    const sa_cluster_params* cp,
                                                    size_t* ws);

/* Clusters the query and the key tokens of every head and writes the orders
 * (and labels) to *out.  Reads q and k ([B,H,N,D] bf16, strides of *p).
 * Deterministic: the same inputs give the same outputs bit for bit.  Causal
 * attention is rejected (its mask is defined on the original positions); f32
 * inputs return SA_ERR_UNSUPPORTED.  The reordered attention is: permute Q by
 * perm_q and K, V by perm_k (sparse_attn_permute), run predict and forward on
 * the permuted tensors, and scatter O back by perm_q (inverse = 1). */
SA_API sa_status sparse_attn_cluster(const sa_params* p, const sa_cluster_params* cp,
                                     const void* q, const void* k, const sa_reorder* out,
                                     void* ws, size_t ws_bytes, void* stream);

/* Row permutation of a [B,H,N,D] tensor with the strides of *p and elements
 * of elem_bytes (2 or 4; e.g. 4 for an fp32 O).  inverse = 0 gathers,
 * y[b,h,r] = x[b,h,perm[b,h,r]]; inverse = 1 scatters, y[b,h,perm[b,h,r]] =
 * x[b,h,r].  perm is int32 [B,H,N] and should be a permutation of [0, N):
 * entries outside [0, N) are skipped (their rows are not written), repeated
 * entries leave the affected rows undefined.  x and y must not overlap. */
SA_API sa_status sparse_attn_permute(const sa_params* p, const void* x, const int32_t* perm,
                                     int32_t inverse, int32_t elem_bytes, void* y,
                                     void* stream);

/* Host.  Checks a mask held in host memory (copies of kept_idx
 * [B,H,NQB,NKB] and kept_cnt [B,H,NQB]) against the rules forward relies on:
 * for every query block i, kept_cnt in [max(1, |F_i|), |A_i|]; the first
 * kept_cnt entries distinct admissible key blocks (A_i: all, or under
 * causality those whose first key is not after the block's last row); the
 * |F_i| forced blocks (the keep_prefix_kblocks leading blocks, and under
 * causality the blocks that reach the diagonal) first.  Masks from
 * sparse_attn_predict pass; the check is for masks built or edited by the
 * caller.  Returns SA_ERR_INVALID_ARG naming the first offending row (its
 * flat index [B,H,NQB] in *bad_row, -1 if none; bad_row may be NULL).  With
 * the environment variable SA_CHECK_MASK=1, sparse_attn_forward and
 * sparse_attn_step run the same check on their device mask before any
 * launch (copying it to the host, which synchronises the stream). */
SA_API sa_status sparse_attn_check_mask(const sa_params* p, const int32_t* kept_idx,
                                        const int32_t* kept_cnt, int64_t* bad_row);

/* Host.  Library defaults and version (either pointer may be NULL). */
SA_API sa_status sparse_attn_info(int32_t* default_group_rows, int32_t* version);

/* Host.  Static string naming a status code. */
SA_API const char* sparse_attn_status_str(int32_t status);

/* Host.  Message describing the last failed call on this thread ("" if the
 * last call succeeded).  Valid until the next call on this thread. */
SA_API const char* sparse_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
