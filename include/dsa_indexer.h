/*
 * dsa_indexer.h -- C ABI of the MI355X (gfx950) lightning indexer with exact
 * per-query Top-K and certified (DoSA) pruning.
 *
 * What is computed (DeepSeek DSA FLOPs notes, section "Lightning Indexer
 * FLOPs", the index-score equation; query t, key s):
 *
 *     I[t,s] = sum_{j<H} w[t,j] * ReLU(q[t,j,:] . k[s,:])
 *
 * with H = 64 indexer heads of d = 128, one key row shared by all heads
 * (section "Notation", indexer tensors Q^I (T,H^I,d^I), K^I (T,d^I),
 * W^I (T,H^I)).  Key s is visible to query row t iff s <= positions[t]
 * (section "Causal token-pair 数": the diagonal counts), and each row keeps
 * the min(k, visible) best visible keys (the N_sel equation there).
 * The pages fix no tie rule; this library orders by score descending, then
 * key index ascending, in every path.
 *
 * For fp8 inputs (OCP e4m3fn codes), q_scale[t] (one per query token, shared
 * by its heads) and k_scale[s] (one per key row) are the dequantisation
 * scales: the score is the equation above on scale * code values, computed as
 * (q_scale[t] * k_scale[s]) * sum_j w[t,j] ReLU(q8[t,j,:] . k8[s,:]),
 * exact for positive scales.
 *
 * Conventions shared by all entry points
 *  - Every array pointer is DEVICE memory owned by the caller, row-major and
 *    contiguous, innermost dimension last, 16-byte aligned.  The library
 *    never allocates, frees or synchronises (one exception: the first
 *    dsa_indexer_project call on a thread creates a rocBLAS handle); work is
 *    enqueued on `stream` (a hipStream_t; NULL is the default stream) and
 *    returns at once.
 *  - Scores are fp32 computed with fp32 accumulation; every path uses the
 *    same instruction sequence for a (t, s) pair, so a score is bit-identical
 *    whichever entry point or tile produced it.
 *  - Return value: DSA_OK (0) or an error code; the call enqueues nothing
 *    when it returns an argument, support or workspace error.
 *    dsa_indexer_last_error() gives a thread-local detail string.
 *  - Device data (positions, finiteness of inputs) are preconditions and are
 *    not inspected on the host.  Inputs must be finite.
 *  - Calls on one stream are ordered; calls that share a workspace must not
 *    run concurrently on different streams.
 */
#ifndef DSA_INDEXER_H_
#define DSA_INDEXER_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { DSA_BF16 = 0, DSA_FP8_E4M3 = 1 };

enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer, scales wrong for dtype */
  DSA_ERR_UNSUPPORTED = 2, /* heads != 64, head_dim != 128, unknown dtype, topk out of range */
  DSA_ERR_WORKSPACE = 3,   /* workspace smaller than dsa_indexer_workspace_bytes() */
  DSA_ERR_HIP = 4          /* a HIP launch reported an error */
};

/* Shared inputs.  B = batch (independent sequences), Q = query rows per
 * sequence, N = keys per sequence.
 *   q          [B,Q,H,d]  bf16 bits (uint16) or e4m3fn codes (uint8)
 *   k          [B,N,d]    same dtype as q
 *   w          [B,Q,H]    fp32 head weights, any sign
 *   q_scale    [B,Q]      fp32 > 0, fp8 only (must be NULL for bf16)
 *   k_scale    [B,N]      fp32 > 0, fp8 only (must be NULL for bf16)
 *   positions  [B,Q]      int32 absolute position of each query row; the
 *                         row sees keys 0..min(positions, N-1); a negative
 *                         position sees no key.                            */
typedef struct dsa_indexer_inputs {
  int32_t batch, num_q, num_k, heads, head_dim, dtype;
  const void* q;
  const void* k;
  const float* w;
  const float* q_scale;
  const float* k_scale;
  const int32_t* positions;
  uint32_t flags; /* 0, or DSA_FLAG_* bits below; other bits are DSA_ERR_INVALID_ARG */
} dsa_indexer_inputs;

/* flags: Top-K route of dsa_indexer_topk (at most one of the two; 0 lets the
 * library choose: the key-split route when the rows are too few to fill the
 * GPU with one workgroup per 8 rows and their score rows fit in 8 GiB, else
 * the streaming route).  Both routes return the same index set; the flags
 * exist so that callers and tests can pin one.  The workspace size depends on
 * the route, so pass the same flags to dsa_indexer_workspace_bytes. */
enum {
  DSA_FLAG_ROUTE_STREAM = 1u << 0, /* fused score + streaming Top-K, no score rows stored */
  DSA_FLAG_ROUTE_SPLIT = 1u << 1   /* key-split score rows in the workspace, then a per-row select */
};

/* Full score matrix (the index-score equation for every pair).
 *   scores [B,Q,N] fp32 out; -inf where the key is not visible.
 * Intended for checking and small shapes: it writes B*Q*N floats.          */
int dsa_indexer_scores(const dsa_indexer_inputs* in, float* scores, void* stream);

/* Exact Top-K per query row.  Prefill blocks are scored and selected in one
 * pass that never stores the score matrix; for few rows (decode: one row per
 * sequence against a long cache) whole score rows go to the workspace and a
 * per-row select follows, which fills the GPU with key-split workgroups.
 *   topk       1..4096
 *   out_idx    [B,Q,topk] int32 out: the min(topk, visible) selected key
 *              indices first (in no particular order), then -1 padding
 *   out_score  [B,Q,topk] fp32 out (score of each index; -inf at padding),
 *              or NULL
 *   workspace  device scratch of at least
 *              dsa_indexer_workspace_bytes(DSA_OP_TOPK, in, topk, NULL) bytes,
 *              256-byte aligned; contents on entry are ignored.
 * Selection ties are broken by the smaller key index.                       */
int dsa_indexer_topk(const dsa_indexer_inputs* in, int32_t topk, int32_t* out_idx,
                     float* out_score, void* workspace, size_t workspace_bytes, void* stream);

/* dsa_indexer_topk with no workspace argument and no allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops that forbid hipMalloc).  The workspace is a fixed device array of
 * DSA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * library's load until the process ends; its address on the current device
 * is looked up on the first call on that device (hipGetSymbolAddress).
 * Same inputs, route flags, outputs and results as dsa_indexer_topk.
 * Returns DSA_ERR_WORKSPACE, enqueuing nothing, when the call needs more than
 * DSA_NOALLOC_SCRATCH_BYTES of workspace (dsa_indexer_workspace_bytes with
 * DSA_OP_TOPK tells: e.g. 64 decode rows over 131072 keys need 32.5 MiB, the
 * streaming route (4*topk + 640)*8 bytes per row).  Every call on one GPU
 * uses that GPU's one array: calls that can overlap in time on one GPU
 * (different streams, or host threads) race and must be serialised by the
 * caller.  Calls on one stream are ordered and safe.  The stream must belong
 * to the current device.                                                     */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dsa_indexer_topk_noalloc(const dsa_indexer_inputs* in, int32_t topk, int32_t* out_idx, float* out_score,
                             void* stream);

/* Options of the pruned path (host struct; pass NULL for defaults).
 *   num_seeds     seeds per sequence (0 -> 12288), clamped to the common
 *                 visible prefix; seeds rescored with all heads fix the
 *                 starting threshold tau (DoSA reading notes, annotation
 *                 LBKERZAW, step 1)
 *   num_retained  positive-weight heads whose dot products the bound uses
 *                 directly (0 -> 30, range 1..30, else DSA_ERR_UNSUPPORTED;
 *                 fewer if the row has fewer positive heads, and at most 28
 *                 for fp8 inputs); the bound also uses one folded
 *                 negative-head row (every negative-weight head, folded by
 *                 |w|) and one linear row that carries the projected
 *                 positive heads (32 rows in all).  For fp8 inputs these two
 *                 rows are stored as high and low e4m3 parts: the low parts
 *                 take plan rows 28 and 29
 *   seed_idx      [B,num_seeds] int32 device array of ascending, distinct
 *                 key indices, or NULL for evenly spaced seeds
 *                 floor(i*(p0+1)/S) over the common prefix 0..p0
 *   force_recover [B,Q] uint8 device mask, or NULL: rows marked non-zero
 *                 take the recovery (unpruned) path; for tests
 *   flags         0, or DSA_PRUNE_* bits below; other bits are
 *                 DSA_ERR_INVALID_ARG
 *
 * Starting threshold.  The pages start the running threshold at tau, the
 * K-th best seed score.  By default a row starts higher, at its m-th best
 * seed record with m = ceil(mu + 5 sqrt(mu)) + 1 and mu = K * (its visible
 * seeds) / (its visible keys): with evenly spread seeds about mu seeds lie
 * at or above the K-th score, so the m-th one is an estimate of a score
 * that at least K keys reach.  Only rows with m < K start raised.  A key
 * below the start is excluded with the same certified bound test, so
 * every key whose exact score reaches the start is found.  If at least K
 * do, the Top-K is exact as before; if fewer do, the row is recomputed by
 * the unpruned path (statistics: recovered = 2).  The results are the same
 * index set either way.  DSA_PRUNE_START_AT_TAU starts every row at tau.
 *
 * Candidate records.  By default a kept candidate is a 64-bit record (the
 * score's monotone 32-bit code, then the inverted key index), which orders
 * candidates exactly.  DSA_PRUNE_COMPACT_RECORDS keeps 32-bit records
 * instead (DoSA reading notes, annotation TMIF4XYF; 机器之心 DoSA article,
 * section 04): the low kb bits hold the key index (kb = bits of N - 1) and
 * the high 32 - kb bits a score code relative to the row, c = min(2^(32-kb)
 * - 1, (code(s) - code(start)) >> shift), with the shift fitted at the start
 * so that twice the row's best seed score still fits.  Records of different
 * codes are ordered by score; the Top-K boundary code is resolved by
 * rescoring its keys with all heads (all selected keys when out_score is
 * requested).  A row whose boundary or buffer cannot be resolved in the
 * workspace is recomputed by the unpruned path (recovered = 3).  Needs
 * N <= 2^24 (else DSA_ERR_UNSUPPORTED).  Same index set and scores.
 *
 * Anchor seeds.  DSA_PRUNE_ANCHOR_SEEDS takes the seeds from a few anchor
 * queries instead of spacing them evenly (机器之心 DoSA article, section 03,
 * seed sources): A = num_seeds / K anchor rows per sequence (at least 1, at
 * most Q), the rows floor((2i + 1) Q / (2A)), i < A, have their exact Top-K
 * computed first by the unpruned path, and the sequence's seeds are the
 * distinct keys of those Top-K sets, ascending (at most A * K <= num_seeds).
 * Such seeds are not an even sample, so every row starts at tau (the flag
 * implies DSA_PRUNE_START_AT_TAU); a row that sees fewer than K seeds starts
 * with no threshold.  Needs num_seeds >= K and seed_idx == NULL (else
 * DSA_ERR_INVALID_ARG).  Same index set and scores. */
enum {
  DSA_PRUNE_START_AT_TAU = 1u << 0,
  DSA_PRUNE_COMPACT_RECORDS = 1u << 1,
  DSA_PRUNE_ANCHOR_SEEDS = 1u << 2
};
typedef struct dsa_prune_opts {
  int32_t num_seeds;
  int32_t num_retained;
  const int32_t* seed_idx;
  const uint8_t* force_recover;
  uint32_t flags;
} dsa_prune_opts;

/* Optional per-row statistics of the pruned path (device pointers, each may
 * be NULL):
 *   tau        [B,Q] fp32  threshold from the seeds (K-th seed score)
 *   screened   [B,Q] int32 non-seed visible keys that were bounded
 *   survivors  [B,Q] int32 keys whose bound reached the running threshold
 *   recovered  [B,Q] uint8 0, or the reason the row was recomputed by the
 *              unpruned path: 1 its plan or seeds (or force_recover), 2
 *              fewer than K exact scores reached its raised start, 3 its
 *              compact records did not fit the workspace
 *   upper_bound [B,Q,N] fp32 debug: the bound of every non-seed visible key
 *              (NaN elsewhere); small shapes only, costs one extra pass
 *   plan_rows  [B,Q,32,128] debug: each row's bound plan, in the input dtype
 *              (bf16 bits or e4m3 codes): rows 0..29 the retained heads'
 *              query rows (zero past the row's retained count; fp8: rows
 *              28 and 29 the low parts of E and q_neg), row 30 the folded
 *              negative-head row q_neg, row 31 the linear row E (fp8: their
 *              high parts)
 *   plan_coef  [B,Q,32] fp32 debug: c_0..c_29 (the |d_i| coefficients), the
 *              q_neg multiplier, the E multiplier
 *   plan_misc  [B,Q,2] fp32 debug: kappa (the |k| coefficient, guard
 *              included) and e_neg (the |k| coefficient of q_neg's
 *              rounding).  With d_i = plan_rows[i] . k in code units, the
 *              screen's bound is (for fp8 times q_scale * k_scale)
 *                U = sum_i c_i |d_i| + c_31 d_31 - ReLU(c_30 d_30 - e_neg |k|)
 *                    + kappa |k|                                            */
typedef struct dsa_prune_stats {
  float* tau;
  int32_t* screened;
  int32_t* survivors;
  uint8_t* recovered;
  float* upper_bound;
  void* plan_rows;
  float* plan_coef;
  float* plan_misc;
} dsa_prune_stats;

/* Exact Top-K with certified pruning (DoSA reading notes, annotation
 * LBKERZAW; 机器之心 DoSA article, sections 03-04): seeds fix a threshold,
 * a per-key upper bound from a few retained heads, projected positive heads
 * with a residual term and a folded negative-head penalty excludes keys that
 * cannot reach the Top-K, and survivors are rescored with all heads.
 * Returns the same index set as dsa_indexer_topk, bit for bit.  Rows whose
 * seeds are invalid (not ascending or duplicated), whose plan is not finite,
 * or that are forced by opts->force_recover are recomputed by the unpruned
 * path on the device.  Arguments as for dsa_indexer_topk, plus opts and
 * stats; workspace from dsa_indexer_workspace_bytes(DSA_OP_TOPK_PRUNED, ...). */
int dsa_indexer_topk_pruned(const dsa_indexer_inputs* in, int32_t topk, const dsa_prune_opts* opts,
                            int32_t* out_idx, float* out_score, const dsa_prune_stats* stats,
                            void* workspace, size_t workspace_bytes, void* stream);

enum { DSA_OP_SCORES = 0, DSA_OP_TOPK = 1, DSA_OP_TOPK_PRUNED = 2 };

/* Workspace bytes an entry point needs for these inputs (0 for scores).
 * Returns 0 and sets the last error if the arguments are invalid.          */
size_t dsa_indexer_workspace_bytes(int op, const dsa_indexer_inputs* in, int32_t topk,
                                   const dsa_prune_opts* opts);

/* ------------------------------------------------------------ projections
 *
 * The indexer projections that produce the inputs above (DeepSeek DSA FLOPs
 * notes, section "Indexer projections"): with T tokens,
 *     Q^I = C^Q W_IQ   (T,d_qc) x (d_qc, H d)  -> (T, H, d)
 *     K^I = X   W_IK   (T,d)    x (d, d)       -> (T, d)      (d = 128 here)
 *     W^I = X   W_IW   (T,d)    x (d, H)       -> (T, H)
 * followed by the output conversion of q and k.  All inputs are bf16 bits
 * (uint16), device, row-major:
 *   c_q   [T, q_latent]        the MLA query latent C^Q of each token
 *   x     [T, hidden]          the hidden state X of each token
 *   w_iq  [heads*head_dim, q_latent]  W_IQ stored out-feature major: row o
 *                              holds column o of W_IQ (output o = head o/128,
 *                              dimension o%128)
 *   w_ik  [head_dim, hidden]   W_IK, same layout
 *   w_iw  [heads, hidden]      W_IW, same layout
 * heads must be 64 and head_dim 128; hidden and q_latent are multiples of 8
 * in 8..65536 (DeepSeek-V3.2: hidden 7168, q_latent 1536); num_tokens is
 * 1..4194304.                                                            */
typedef struct dsa_proj_inputs {
  int32_t num_tokens, hidden, q_latent, heads, head_dim;
  int32_t block_tokens; /* tokens per query-GEMM block (64..262144), or 0 for 65536;
                           capped at num_tokens; sets the workspace size */
  const void* c_q;
  const void* x;
  const void* w_iq;
  const void* w_ik;
  const void* w_iw;
} dsa_proj_inputs;

enum { DSA_F32 = 2 }; /* projection outputs only: the raw fp32 projections */

/* Projections with fp32 accumulation of exact bf16 products, then per token:
 *   out_dtype DSA_FP8_E4M3: q_out [T,64,128] and k_out [T,128] e4m3fn codes
 *     (uint8); q_scale [T] / k_scale [T] fp32.  One scale per token for its
 *     8192 query values (shared by its heads) and one for its 128 key values:
 *     scale = amax / 448 and code = e4m3fn round-to-nearest-even of
 *     x * (448 / amax), saturated to +-448, each fp32 step IEEE-rounded to
 *     nearest even; a row of zeros gets scale 1.  (The pages say the indexer
 *     runs in FP8 and fix no scaling rule; this per-token rule is the one the
 *     fp8 inputs of dsa_indexer_inputs take.)
 *   out_dtype DSA_BF16: q_out, k_out bf16 bits, rounded to nearest even;
 *     q_scale and k_scale must be NULL.
 *   out_dtype DSA_F32: q_out, k_out fp32 (the projections themselves);
 *     q_scale and k_scale must be NULL.
 *   w_out [T,64] fp32, the head weights W^I, in every mode.
 * For one sequence the outputs are the q, k, w, q_scale, k_scale of
 * dsa_indexer_inputs (batch 1: each token is both a query row and a key).
 * workspace: at least dsa_indexer_project_workspace_bytes(in) bytes,
 * 256-byte aligned; it holds the fp32 projections of a block of tokens and
 * the GEMM scratch.  The three products run as two rocBLAS GEMMs per token
 * block (X is read once for W_IK and W_IW together) on `stream`; the first
 * call on a thread and device creates that thread's rocBLAS handle, whose
 * state rocBLAS allocates then; after that the call allocates nothing.  A
 * first call on a stream that is capturing a HIP graph returns
 * DSA_ERR_UNSUPPORTED (it would allocate): make one call outside capture
 * first, after which captured calls are fine.
 * Results are bit-reproducible for a given shape: rocBLAS atomics are off.
 * Errors as for the other entry points; a rocBLAS failure is DSA_ERR_HIP.   */
int dsa_indexer_project(const dsa_proj_inputs* in, int32_t out_dtype, void* q_out, float* q_scale, void* k_out,
                        float* k_scale, float* w_out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of dsa_indexer_project (0 and the last error set if the
 * inputs are invalid).                                                      */
size_t dsa_indexer_project_workspace_bytes(const dsa_proj_inputs* in);

/* ---------------------------------------------------------- sparse MLA
 *
 * The core attention that consumes the selected indices (DeepSeek DSA FLOPs
 * notes, section "Core Sparse Attention FLOPs"): MLA in MQA mode, every head
 * reading the same latent cache row [C^KV | K^R] of each selected position.
 * For query row t with selected positions S_t (the Top-K output):
 *     s[h,i] = q[t,h,:] . kv[S_t[i],:]      (content score S^A plus RoPE score S^R)
 *     P[h,:] = softmax_i(sm_scale * s[h,:])
 *     Z[t,h,:] = sum_i P[h,i] * kv[S_t[i], 0:latent_dim]
 *     lse[t,h] = log(sum_i exp(sm_scale * s[h,i]))   (natural log)
 * Inputs (device):
 *   q        [B,Q,heads,latent_dim+rope_dim] bf16 bits: [Q^A | Q^R] per head
 *   kv       [B,N,latent_dim+rope_dim]       bf16 bits: [C^KV | K^R] per position
 *   indices  [B,Q,topk] int32: positions into the row's sequence; entries
 *            outside 0..N-1 (the Top-K's -1 padding) are skipped, others are
 *            used as given (a repeated entry counts twice)
 * Paged cache (page_table non-NULL): kv is instead a pool
 *   kv          [num_pages, page_size, latent_dim+rope_dim] bf16, and
 *   page_table  [B, pages_per_seq] int32: the pool page holding positions
 *               j*page_size .. (j+1)*page_size-1 of sequence b
 * (pages_per_seq >= ceil(N / page_size), num_pages * page_size <= 2^31);
 * page ids outside 0..num_pages-1 are clamped into it, so a bad table reads
 * wrong rows but never outside the pool.  With page_table NULL the three
 * paging fields are ignored and kv is [B,N,latent_dim+rope_dim].
 * heads must be 128, latent_dim 512, rope_dim 64 (DeepSeek-V3.2); topk is
 * 1..2048.                                                                  */
typedef struct dsa_mla_inputs {
  int32_t batch, num_q, num_k, heads, latent_dim, rope_dim, topk;
  int32_t num_splits; /* work units per query row, 1..8 (each takes a share of the row's
                         selected tiles, merged by log-sum-exp), or 0 to choose: 1 when
                         there are at least 256 rows, else enough to give ~512 units;
                         sets the workspace size */
  const void* q;
  const void* kv;
  const int32_t* indices;
  const int32_t* page_table;
  int32_t page_size, pages_per_seq, num_pages;
} dsa_mla_inputs;

/* Sparse MLA attention over the selected positions.
 *   sm_scale   finite, >= 0 (the pages' formula has 1; scaled-dot-product
 *              attention over 576-value rows takes 1/sqrt(576))
 *   out        [B,Q,heads,latent_dim] bf16 out (Z, rounded to nearest even);
 *              zeros for a row with no selected position
 *   lse        [B,Q,heads] fp32 out, or NULL; -inf for a row with nothing
 *              selected
 *   workspace  dsa_sparse_mla_workspace_bytes(in) bytes, 256-byte aligned:
 *              per-row softmax maxima for the rare rows whose scores span
 *              more than 2^32 in weight, which a second launch recomputes
 * Scores accumulate in fp32 (exact bf16 products), the weights enter the
 * weighted sum as bf16, the sums accumulate in fp32.                       */
int dsa_sparse_mla(const dsa_mla_inputs* in, float sm_scale, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Workspace bytes of dsa_sparse_mla (0 and the last error set if the inputs
 * are invalid).                                                             */
size_t dsa_sparse_mla_workspace_bytes(const dsa_mla_inputs* in);

/* Static name of an error code, and the calling thread's last error detail. */
const char* dsa_indexer_error_string(int code);
const char* dsa_indexer_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_INDEXER_H_ */
