// kernels.h -- host-side launchers of the HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace dsa {

// Optional per-kernel event timing (see dsa_indexer_profile.h): a launcher
// brackets its launch with prof_open / prof_close on the launch stream.
int prof_open(const char* name, hipStream_t st);
void prof_close(int slot, hipStream_t st);

struct Problem {
  int B, Q, N, dtype;
  const uint8_t* q;
  const uint8_t* k;
  const float* w;
  const float* q_scale;
  const float* k_scale;
  const int32_t* pos;
};

// Full [B,Q,N] score matrix, -inf where not visible.  If row_hist is not
// null it is set to the [B*Q][kRowHistBins] histogram of each row's visible
// scores over the leading 11 bits of their monotone codes (the first digit
// of the row select).
constexpr int kRowHistBins = 2048;
hipError_t launch_scores(const Problem& p, float* scores, uint32_t* row_hist, hipStream_t st);

// Exact Top-K of every row of a [B*Q, N] score matrix (visibility from pos);
// row_hist (nullable) is launch_scores' histogram of the same rows.
hipError_t launch_select_rows(const Problem& p, const float* scores, const uint32_t* row_hist, int topk,
                              int32_t* out_idx, float* out_score, hipStream_t st);

// Streaming Top-K: scores key tiles and keeps per-row candidate records in
// `cand` ([B*Q][cap] uint64), never storing the score matrix.
hipError_t launch_topk_stream(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx,
                              float* out_score, hipStream_t st);

// Streaming Top-K of the rows whose row_flag[b*Q + t] is non-zero only (the
// pruned path's recovery); other rows' outputs are left as they are.
hipError_t launch_topk_stream_rows(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx,
                                   float* out_score, const int32_t* row_flag, const char* prof_name, hipStream_t st);

// ---------------------------------------------------------------- pruned path

// Per-row state of the pruned path between its launches (device memory).
struct PruneRowCtl {
  uint64_t thr;       // running threshold record
  int32_t cnt;        // records in the row's candidate buffer
  uint32_t base;      // threshold histogram: code of bin 0
  int32_t shift;      // threshold histogram: log2 of the bin width
  int32_t added;      // records kept since the last threshold raise
  int32_t screened;   // statistics: bounded keys
  int32_t survived;   // statistics: keys whose bound reached the threshold
  float tau;          // threshold from the seeds
  int32_t raised;     // 1: the row started above tau (needs K records at its start)
  uint32_t cbase;     // compact records: monotone code of the row's start
  int32_t cshift;     // compact records: score code = (monotone code - cbase) >> cshift
  int32_t reason;     // 0, or why the streaming Top-K recomputes the row (statistics)
  int32_t pad[3];
};

// Key bytes of the longest chunk of the screen/refine schedule: a chunk's
// key rows then fit one XCD's 4 MiB L2, so the row groups that screen it
// after the first ones read it from there (16384 bf16 or 32768 fp8 keys).
constexpr int kPruneChunkBytes = 4 << 20;
// Bitmask words per row: the longest chunk of the schedule for N keys of
// row_bytes each (256 bf16, 128 fp8), / 64.
int prune_mask_words(int N, int row_bytes);

// Device buffers of the pruned Top-K (workspace carve-up and optional stats).
struct PrunedBuffers {
  uint8_t* plan_rows;  // [B*Q][32][128] dtype
  float* plan_coef;    // [B*Q][32]
  float* plan_misc;    // [B*Q][4]
  int32_t* plan_flag;  // [B*Q]
  float* knorm;        // [B][N]
  int32_t* seeds;      // [B][seed_stride]
  int32_t* seed_count; // [B]
  int seed_stride;
  uint32_t* seed_bits; // [B][bits_stride]
  int bits_stride;
  int32_t* batch_flag; // [B]
  uint8_t* seed_keys;     // [B][seed_stride] key rows (dtype): the seeds packed
  float* seed_kscale;     // [B][seed_stride] their fp8 key scales
  int32_t* seed_pos;      // [B*Q]: (number of the row's visible seeds) - 1
  int32_t* seed_top_idx;  // [B*Q][topk]: the row's exact seed Top-K (seed numbers, -1 padded)
  float* seed_top_score;  // [B*Q][topk]: their scores
  PruneRowCtl* ctl;       // [B*Q]
  uint32_t* hist;         // [B*Q][256]
  uint64_t* mask;         // [B*Q][mask_stride]
  int mask_stride;
  float* st_tau;
  int32_t* st_screened;
  int32_t* st_surv;
  uint8_t* st_rec;
  float* st_ub;
  int raised_start;       // 1: rows start above tau (verified at the end; misses recover)
  int compact;            // 1: 32-bit candidate records (score code + key), boundary resolved by rescoring
};

hipError_t launch_seed_prep(const Problem& p, int S, const int32_t* user_seeds, int32_t* seeds, int32_t* seed_count,
                            uint32_t* bits, int32_t* batch_flag, hipStream_t st);
hipError_t launch_key_norms(const Problem& p, float* knorm, hipStream_t st);
// Anchor seeds: flag[b*Q + t] = 1 on the A anchor rows of every sequence,
// else 0; then, from the anchor rows' Top-K (top_idx, [B*Q][topk]), each
// sequence's seeds (the distinct keys, ascending, at most S), count, bitmap.
hipError_t launch_anchor_rows(const Problem& p, int A, int32_t* flag, hipStream_t st);
hipError_t launch_anchor_seeds(const Problem& p, int A, int topk, const int32_t* top_idx, int S, int32_t* seeds,
                               int32_t* seed_count, uint32_t* bits, int32_t* batch_flag, hipStream_t st);
// Packs the seed keys (and fp8 scales) of every sequence and counts each
// row's visible seeds, so the streaming Top-K can score the seeds.
hipError_t launch_seed_pack(const Problem& p, const int32_t* seeds, const int32_t* seed_count, int seed_stride,
                            uint8_t* seed_keys, float* seed_kscale, int32_t* seed_pos, hipStream_t st);
hipError_t launch_plan(const Problem& p, int nret, const int32_t* seeds, const int32_t* seed_count, int seed_stride,
                       const int32_t* batch_flag, const uint8_t* force_recover, uint8_t* plan_rows, float* plan_coef,
                       float* plan_misc, int32_t* plan_flag, hipStream_t st);
hipError_t launch_topk_pruned(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx, float* out_score,
                              const PrunedBuffers& pb, hipStream_t st);

// ---------------------------------------------------------------- projections

// bf16 operands of the indexer projections (weights out-feature major).
struct ProjProblem {
  int T, hidden, q_latent, block_tokens;
  const uint16_t* c_q;   // [T][q_latent]
  const uint16_t* x;     // [T][hidden]
  const uint16_t* w_iq;  // [8192][q_latent]
  const uint16_t* w_ik;  // [128][hidden]
  const uint16_t* w_iw;  // [64][hidden]
};
// Device scratch handed to rocBLAS from the workspace.
constexpr size_t kProjBlasScratch = size_t(32) << 20;
// Tokens per GEMM block (the fp32 staging rows held at once): `requested`
// if positive, else 65536, capped at T.
int proj_block_tokens(int T, int requested);
size_t proj_workspace_bytes(int T, int hidden, int block_tokens);
// The GEMMs and the output pass; out 0 = fp8 + scales, 1 = bf16, 2 = fp32.
// Returns 0; 1 with *err set on a HIP or rocBLAS failure; 2 with *err set
// if the call would have to create the thread's rocBLAS handle while `st`
// is capturing a graph.
int run_projection(const ProjProblem& p, int out, uint8_t* q_out, float* q_scale, uint8_t* k_out, float* k_scale,
                   float* w_out, uint8_t* ws, hipStream_t st, std::string* err);

// ---------------------------------------------------------------- sparse MLA

// Core attention over selected positions: q [B*Q][128][576], kv [B][N][576]
// (bf16, [latent 512 | RoPE 64]), indices [B*Q][topk] (topk <= 2048).
struct MlaProblem {
  int B, Q, N, topk;
  const uint16_t* q;
  const uint16_t* kv;  // [B][N][576], or a page pool [num_pages][page_size][576]
  const int32_t* indices;
  const int32_t* page_table;  // [B][pages_per_seq], or null for the flat layout
  int page_size, pages_per_seq, num_pages;
};
// Work units per row: `requested` (capped at kMaxSplits = 8) if positive,
// else 1, or (few rows) a split of each row's tiles.
int mla_splits(int rows, int requested);
// out [B*Q][128][512] bf16, lse [B*Q][128] fp32 (may be null); scratch:
// row_max [units][128] fp32 and retry [units] int32 (the second pass), and
// for nsplit > 1 part_o [units][128][512] and part_ml [units][128][2] fp32.
hipError_t launch_sparse_mla(const MlaProblem& p, float sm_scale, uint16_t* out, float* lse, float* row_max,
                             int32_t* retry, int nsplit, float* part_o, float* part_ml, hipStream_t st);

// ---------------------------------------------------------------- sustained-rate probe

// Workgroups of the probe launch: two per compute unit of the current device
// (-1 on a HIP error).
int mfma_ceiling_workgroups();
// The score step on synthetic operands held in registers and LDS; mode 0:
// MFMAs and key-fragment reloads only, mode 1: with the head sum and the
// combine.  `out`: workgroups * 256 floats (per-lane sinks).
hipError_t launch_mfma_ceiling(int dtype, int mode, int iters, int workgroups, float* out, hipStream_t st);

// ---------------------------------------------------------------- fixed scratch

// Bytes of the per-device scratch array behind dsa_indexer_topk_noalloc.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// Device address of that array on the current device (resolved once per
// device with hipGetSymbolAddress).  Returns 0, or 1 with *err set.
int noalloc_scratch(void** ptr, std::string* err);

// Candidate capacity (records per row) used by the streaming Top-K: a cut
// keeps at most topk + 512 records, so one more tile of up to 128 keys always
// fits behind it.
inline int stream_capacity(int topk) { return 4 * topk + 640; }

}  // namespace dsa
